"""GPU parity of verify with the output-gate sigmoid RMSNorm fused into its store
(kda_recurrent_verify_gated) against the fp64 oracle's composition
gated_rmsnorm(recurrent_verify(...)).

Bar, from the arithmetic: the output o of the fp32 recurrence carries at most a few
1e-6 of RMS(o) error, the fused norm adds an fp32 128-term sum of squares, an rsqrt and
three products, and y is rounded to bf16 once; so each element must satisfy
|y - y_ref| <= ulp_bf16(y_ref)/2 + 1e-4 RMS(y_ref), and rstd must match to 2e-5
relative.  The per-step states are unchanged by the fusion: with the same 128-column
tiles they equal the plain verify's bit for bit.
"""

import numpy as np
import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import recurrent_verify, recurrent_verify_gated
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu
Y_ABS_RMS = 1e-4
RSTD_REL = 2e-5
EPS = 1e-6


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _args(d):
    return (d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
            d["lower_bound"], d["state_pool"], d["state_idx"], d["num_steps"])


def _gate_weight(rows, H, seed):
    nd = W.make_norm(W.NormCase("verify_gate", rows, H, eps=EPS, seed=seed))
    return nd["gate"], nd["weight"]


def _reference(data, gate, weight, out_index=None, rows=None):
    """y, rstd by output row (rows without a token: None)."""
    f = W.to_f64
    o_ref, i_ref = O.recurrent_verify(f(data["q"]), f(data["k"]), f(data["v"]), f(data["g"]),
                                      f(data["beta_logits"]), f(data["A_log"]), f(data["dt_bias"]),
                                      data["lower_bound"], data["state_pool"].numpy(),
                                      data["state_idx"].numpy(), data["num_steps"],
                                      scale=data["scale"])
    if out_index is not None:
        full = np.zeros((rows,) + o_ref.shape[1:])
        idx = out_index.numpy()
        ok = (idx >= 0) & (idx < rows)
        full[idx[ok]] = o_ref[ok]
        o_ref = full
    y_ref, r_ref = O.gated_rmsnorm(o_ref, f(gate), weight.numpy(), EPS)
    return y_ref, r_ref, i_ref


def _check(y, rstd, y_ref, r_ref, rows_written):
    yg = TOL.to_np64(y)[rows_written]
    yr = y_ref[rows_written]
    rms = float(np.sqrt(np.mean(yr ** 2)))
    err = np.abs(yg - yr)
    bound = TOL.bf16_half_ulp(yr) + Y_ABS_RMS * rms
    assert np.all(err <= bound), float(np.max(err / rms))
    if rstd is not None:
        rg = TOL.to_np64(rstd)[rows_written]
        rr = r_ref[rows_written]
        assert np.all(np.abs(rg - rr) <= RSTD_REL * rr), float(np.max(np.abs(rg - rr) / rr))
    return float(np.max(err / rms))


@pytest.mark.parametrize("case", [W.VERIFY, W.VERIFY_B1], ids=lambda c: c.name)
def test_verify_gated_matches_oracle_composition(case):
    print(f"case {case.name} seed {case.seed}", flush=True)
    data = W.make_verify(case)
    d = _dev(data)
    B, T, H = case.batch, case.steps, case.heads
    gate, weight = _gate_weight(B * T, H, 4400 + case.seed)
    y, inter, rstd = recurrent_verify_gated(*_args(d), gate.cuda(), weight.cuda(), EPS,
                                            scale=d["scale"])
    torch.cuda.synchronize()
    y_ref, r_ref, i_ref = _reference(data, gate, weight)
    worst = _check(y, rstd, y_ref, r_ref, np.arange(B * T))
    ic = inter.cpu().numpy()
    for b in range(B):
        assert TOL.state_rel_l2(ic[b], i_ref[b]) <= 2e-5
    if B * H >= 256 or B * H <= 64:
        # the same form as the plain verify (the step form's 128-column tiles, or the
        # block form's row split): per-step states bit for bit
        _, inter_plain = recurrent_verify(*_args(d), scale=d["scale"])
        torch.cuda.synchronize()
        assert torch.equal(inter, inter_plain)
    print(f"  worst |y - y_ref| / RMS {worst:.2e}", flush=True)


# T = 19: three blocks of the block form, the last one partial
@pytest.mark.parametrize("T", [5, 19])
def test_verify_gated_padding_scatter_strided_gate_no_rstd(T):
    case = W.VerifyCase(f"gated_small_t{T}", 6, T, 3, pool_slots=9, seed=4501 + T,
                        padding_rows=[1, 4])
    data = W.make_verify(case)
    d = _dev(data)
    B, T, H = case.batch, case.steps, case.heads
    rows = B * T + 7
    rng = np.random.default_rng(4502)
    out_index = torch.from_numpy(rng.permutation(rows)[:B * T].astype(np.int32))
    out_index[3] = rows + 5            # a token whose output row lies outside: not written
    gate, weight = _gate_weight(rows, H, 4503)
    # the gate read in place from a wider fused buffer (token stride 2 H 128)
    fused = torch.zeros((rows, 2 * H, 128), dtype=torch.bfloat16)
    fused[:, H:] = gate
    gate_view = fused.cuda()[:, H:]
    out = torch.full((rows, H, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((rows, H), -1.0, dtype=torch.float32, device="cuda")
    y, _, r = recurrent_verify_gated(*_args(d), gate_view, weight.cuda(), EPS, out=out,
                                     rstd=rstd, scale=d["scale"],
                                     out_token_index=out_index.cuda())
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr() and r.data_ptr() == rstd.data_ptr()
    idx = out_index.numpy()
    written = np.array(sorted(i for i in idx if 0 <= i < rows))
    untouched = np.setdiff1d(np.arange(rows), written)
    y_ref, r_ref, _ = _reference(data, gate, weight, out_index, rows)
    _check(y, rstd, y_ref, r_ref, written)
    # padding rows' outputs are zero (norm of a zero row), their rstd 1/sqrt(eps)
    pad_rows = [idx[b * T + t] for b in case.padding_rows for t in range(T)
                if 0 <= idx[b * T + t] < rows]
    assert torch.all(y[torch.as_tensor(pad_rows).long()].float() == 0)
    assert np.allclose(rstd.cpu().numpy()[pad_rows], 1.0 / np.sqrt(EPS), rtol=RSTD_REL)
    # rows no token maps to stay untouched
    assert torch.all(out[torch.as_tensor(untouched).long()].float() == 3.0)
    assert torch.all(rstd[torch.as_tensor(untouched).long()] == -1.0)
    # without rstd the outputs are the same
    y2, _, r2 = recurrent_verify_gated(*_args(d), gate_view, weight.cuda(), EPS,
                                       out=torch.empty_like(out), want_rstd=False,
                                       scale=d["scale"], out_token_index=out_index.cuda())
    torch.cuda.synchronize()
    assert r2 is None
    assert torch.equal(y2[torch.as_tensor(written).long()].view(torch.int16),
                       y[torch.as_tensor(written).long()].view(torch.int16))
