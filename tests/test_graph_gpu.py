"""Prefill and verify calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library validates on host integers only and issues no synchronisation, memset or
allocation, so a call with caller-provided buffers captures as plain kernel nodes.
Each graph is replayed several times, with eager work (fills of the outputs) and
synchronisations between replays, and every replay must reproduce the eager call
bit for bit; the eager call itself is checked against the oracle.
"""

import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import chunk_prefill, prefill_workspace_bytes, recurrent_verify
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu
REPLAYS = 3


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _capture(fn):
    # torch's capture recipe: one warm-up call on a side stream before capturing.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def _replay_and_compare(graph, outputs, refs):
    for i in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan") if t.dtype == torch.float32 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, refs):
            assert torch.equal(t, r), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("lens,H", [([200, 64, 1, 90], 2),      # plain scan
                                    ([64 * 40 + 17], 2)])       # segment-parallel scan
def test_prefill_graph_replays_match_eager(lens, H):
    case = W.PrefillCase(f"graph_{len(lens)}x{H}", lens, H, init="per_seq", seed=3400 + len(lens))
    print(f"case {case.name} lens {lens}", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    T, N = d["q"].shape[0], len(lens)
    ws = torch.empty(prefill_workspace_bytes(N, T, H), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")

    def call():
        chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
                      d["lower_bound"], d["cu_seqlens"], initial_state=d["initial_state"],
                      scale=d["scale"], out=out, final_state=fin, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_fin = out.clone(), fin.clone()
    f = W.to_f64
    o_ref, s_ref = O.chunk_prefill(f(data["q"]), f(data["k"]), f(data["v"]), f(data["g"]),
                                   f(data["beta_logits"]), f(data["A_log"]), f(data["dt_bias"]),
                                   data["lower_bound"], data["cu_seqlens"].numpy(),
                                   data["initial_state"].numpy(), None, scale=data["scale"])
    TOL.assert_output_ok(ref_out, o_ref)
    TOL.assert_state_ok(ref_fin, s_ref)
    graph = _capture(call)
    _replay_and_compare(graph, [out, fin], [ref_out, ref_fin])


@pytest.mark.parametrize("B,H", [(10, 3), (36, 16)])   # block form; looping step form
def test_verify_graph_replays_match_eager(B, H):
    T = 8
    case = W.VerifyCase(f"graph_v{B}x{H}", B, T, H, pool_slots=64, seed=4400 + B,
                        padding_rows=[3])
    data = W.make_verify(case)
    d = _dev(data)
    out = torch.empty((B * T, H, 128), dtype=torch.bfloat16, device="cuda")
    inter = torch.empty((B, T, H, 128, 128), dtype=torch.float32, device="cuda")

    def call():
        recurrent_verify(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"],
                         d["dt_bias"], d["lower_bound"], d["state_pool"], d["state_idx"], T,
                         scale=d["scale"], out=out, intermediate=inter)

    call()
    torch.cuda.synchronize()
    f = W.to_f64
    o_ref, i_ref = O.recurrent_verify(f(data["q"]), f(data["k"]), f(data["v"]), f(data["g"]),
                                      f(data["beta_logits"]), f(data["A_log"]),
                                      f(data["dt_bias"]), data["lower_bound"],
                                      data["state_pool"].numpy(), data["state_idx"].numpy(), T,
                                      scale=data["scale"])
    TOL.assert_output_ok(out, o_ref)
    live = [b for b in range(B) if b != 3]
    TOL.assert_state_ok(inter[live], i_ref[live])
    # padding row 3 writes no state rows: keep what the eager call left there
    ref_out, ref_inter = out.clone(), inter.clone()
    graph = _capture(call)
    for i in range(REPLAYS):
        out.fill_(0)
        inter[live] = float("nan")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: outputs differ"
        assert torch.equal(inter[live], ref_inter[live]), f"replay {i}: states differ"
