"""The allocation-free prefill entry point (kda_chunk_prefill_noalloc) against
kda_chunk_prefill with a caller workspace.

Both run the same kernels; only where the chunk records and segment states live
differs (the library's fixed per-device scratch instead of a workspace).  Each call
is compared with the workspace call bit for bit and with the fp64 oracle to the
parity bar, on consecutive calls whose second is smaller than the first (the scratch
keeps the previous call's contents), including one that runs the segment-parallel
scan (its states also live in the scratch).
"""

import numpy as np
import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import chunk_prefill, chunk_prefill_noalloc, prefill_workspace_bytes
from linear_attention_rule_amd import noalloc_scratch_bytes
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _args(d):
    return (d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
            d["lower_bound"], d["cu_seqlens"])


def _oracle(data):
    f = W.to_f64
    init = data["initial_state"]
    idx = data["initial_state_idx"]
    return O.chunk_prefill(f(data["q"]), f(data["k"]), f(data["v"]), f(data["g"]),
                           f(data["beta_logits"]), f(data["A_log"]), f(data["dt_bias"]),
                           data["lower_bound"], data["cu_seqlens"].numpy(),
                           None if init is None else init.numpy(),
                           None if idx is None else idx.numpy(), scale=data["scale"])


CASES = [
    # larger first: 8 x 16 heads x (4800 / 64 + 3) chunk slots of records
    W.PrefillCase("noalloc_first", [3000, 1700, 100], 8, init="per_seq", seed=5101),
    # then smaller calls over the same scratch: plain scan, then the segment-parallel scan
    W.PrefillCase("noalloc_second", [130, 7, 64], 2, init=None, seed=5102),
    W.PrefillCase("noalloc_segmented", [64 * 40 + 17], 2, init="pool", pool_slots=3, seed=5103),
]


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    sizes = []
    for case in CASES:
        print(f"case {case.name} lens {case.seq_lens} heads {case.heads}", flush=True)
        data = W.make_prefill(case)
        d = _dev(data)
        T, H = d["q"].shape[:2]
        N = d["cu_seqlens"].numel() - 1
        need = prefill_workspace_bytes(N, T, H)
        assert 0 < need <= noalloc_scratch_bytes()
        sizes.append(need)
        kw = dict(initial_state=d["initial_state"], initial_state_idx=d["initial_state_idx"],
                  scale=d["scale"])
        ref_out, ref_fin = chunk_prefill(*_args(d), **kw)
        out = torch.full((T, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
        fin = torch.full((N, H, 128, 128), 7.0, dtype=torch.float32, device="cuda")
        o, f = chunk_prefill_noalloc(*_args(d), out=out, final_state=fin, **kw)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr() and f.data_ptr() == fin.data_ptr()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(fin, ref_fin)
        o_ref, f_ref = _oracle(data)
        e = TOL.assert_output_ok(out, o_ref)
        r = TOL.assert_state_ok(fin, f_ref)
        print(f"  bitwise equal to the workspace call; oracle excess/RMS "
              f"{e['excess_over_rms']:.2e}, state rel L2 {r:.2e}", flush=True)
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # 4 x 8192 tokens at 16 heads needs ~492 MiB of records: refused before any launch.
    q = torch.zeros((32768, 16, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 8192, 16384, 24576, 32768], dtype=torch.int32, device="cuda")
    A = torch.zeros(16, dtype=torch.float32, device="cuda")
    dt = torch.zeros((16, 128), dtype=torch.float32, device="cuda")
    b = torch.zeros((32768, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="KDA_ERR_UNSUPPORTED"):
        chunk_prefill_noalloc(q, q, q, q, b, A, dt, -5.0, cu)
