"""GPU parity of the fused multi-step verify against the fp64 oracle.

Every case goes through the C ABI (via the ctypes binding) on seeded inputs
from linear_attention_rule_amd.workloads, and is compared element by element
with oracle.kda_oracle.recurrent_verify.  The verify path is fp32 end to end,
so beyond the project bar (tolerances.py) the tests also hold it to a bound
derived from fp32 arithmetic: relative state error <= 2e-5 over 64 steps.
"""

import numpy as np
import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import recurrent_verify
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu
FP32_STATE_BOUND = 2e-5


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _oracle(data):
    f = W.to_f64
    return O.recurrent_verify(f(data["q"]), f(data["k"]), f(data["v"]), f(data["g"]),
                              f(data["beta_logits"]), f(data["A_log"]), f(data["dt_bias"]),
                              data["lower_bound"], data["state_pool"].numpy(),
                              data["state_idx"].numpy(), data["num_steps"], scale=data["scale"])


def _call(d, **kw):
    return recurrent_verify(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"],
                            d["dt_bias"], d["lower_bound"], d["state_pool"], d["state_idx"],
                            d["num_steps"], scale=d["scale"], **kw)


def _check(data, out, inter):
    o_ref, i_ref = _oracle(data)
    e = TOL.assert_output_ok(out, o_ref)
    live = [b for b in range(data["state_idx"].numel())
            if 0 <= int(data["state_idx"][b]) < data["state_pool"].shape[0]]
    inter_np = inter.cpu().numpy()
    worst = 0.0
    for b in live:
        r = TOL.state_rel_l2(inter_np[b], i_ref[b])
        worst = max(worst, r)
    assert worst <= min(TOL.STATE_TOL, FP32_STATE_BOUND), worst
    return e, worst


def test_verify_64x8_h16_pool256():
    case = W.VERIFY
    print(f"case {case.name} seed {case.seed}", flush=True)
    data = W.make_verify(case)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    e, worst = _check(data, out, inter)
    print("output", e, "state", worst)


def test_verify_1x8_latency_case():
    data = W.make_verify(W.VERIFY_B1)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    _check(data, out, inter)


def test_verify_saturated_and_degenerate_inputs():
    """Zero q or k rows, gate logits past both ends of the sigmoid and beta at 1 or ~0."""
    data = W.make_verify(W.VerifyCase("saturated", 12, 8, 2, 16, seed=4106))
    n = data["q"].shape[0]
    t = torch.arange(n)
    data["q"][t % 11 == 3] = 0
    data["k"][t % 13 == 5] = 0
    data["g"][t % 4 == 0, 0] = 64.0
    data["g"][t % 4 == 1, 1] = -64.0
    data["beta_logits"][t % 7 == 0] = 32.0
    data["beta_logits"][t % 7 == 1] = -32.0
    print("case saturated B 12 T 8 H 2", flush=True)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(inter).all()
    _check(data, out, inter)


@pytest.mark.parametrize("B", [2, 40])
def test_verify_strongest_decay_at_the_lower_bound(B):
    """Gate logits that saturate the sigmoid at the API's lower bound -5: every step
    decays by e^-5, so over an 8-step block the block form's 1/Gamma reaches 2^57.7 (its
    largest value) on the channels where the gate saturates; both launch forms (B = 2:
    block, B = 40: step) against the oracle."""
    case = W.VerifyCase(f"v_lb5_{B}", B, 16, 3, pool_slots=B + 2, seed=2500 + B, lower_bound=-5.0)
    data = W.make_verify(case)
    n = data["g"].shape[0]
    t = torch.arange(n)
    data["g"][t % 3 != 1] = 60.0            # sigmoid -> 1 on every channel
    data["g"][t % 3 == 1, :, :64] = 60.0    # and on half of them in the other steps
    print(f"case lb=-5 B {B} T 16 H 3", flush=True)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(inter).all()
    _check(data, out, inter)


@pytest.mark.parametrize("B,T,H", [(3, 1, 1), (5, 3, 2), (2, 16, 3), (1, 64, 2), (40, 8, 8)])
def test_verify_small_shapes(B, T, H):
    case = W.VerifyCase(f"v_{B}x{T}_h{H}", B, T, H, pool_slots=B + 5, seed=2000 + B * 100 + T + H)
    data = W.make_verify(case)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    _check(data, out, inter)


# (row, head) pair counts on both sides of the launcher's switches: the block form up to
# 96 pairs, the step form with 32-column tiles below 256 and with whole rows from 256
# on, each with a padding row.
@pytest.mark.parametrize("B,H", [(1, 16), (3, 12), (6, 16), (7, 14), (15, 17), (16, 16), (9, 30)])
def test_verify_every_launch_form(B, H):
    case = W.VerifyCase(f"v_tiles_{B}x8_h{H}", B, 8, H, pool_slots=B + 2, seed=2300 + 10 * B + H,
                        padding_rows=[B - 1] if B > 1 else [])
    data = W.make_verify(case)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    _check(data, out, inter)


@pytest.mark.parametrize("seed", range(4300, 4306))
def test_verify_random_shapes(seed):
    """Seeded random shapes: 1-20 rows, 1-16 draft steps (64 at times), 1-6 heads, a few
    padding rows, and a pool of states larger than the batch."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 21))
    T = 64 if rng.random() < 0.15 else int(rng.integers(1, 17))
    H = int(rng.integers(1, 7))
    pad = sorted(set(int(x) for x in rng.integers(0, B, size=int(rng.integers(0, 3)))))
    if len(pad) == B:
        pad = pad[:-1]
    case = W.VerifyCase(f"vrand_{seed}", B, T, H, pool_slots=B + 3, seed=seed, padding_rows=pad)
    print(f"case {case.name} B {B} T {T} H {H} padding {pad}", flush=True)
    data = W.make_verify(case)
    d = _dev(data)
    out, inter = _call(d)
    torch.cuda.synchronize()
    _check(data, out, inter)
    for b in pad:   # padding rows: zero outputs
        assert torch.count_nonzero(out[b * T:(b + 1) * T]) == 0


def test_verify_padding_rows_untouched():
    case = W.VerifyCase("v_pad", 6, 4, 2, pool_slots=8, seed=2101, padding_rows=[1])
    data = W.make_verify(case)
    data["state_idx"][4] = 8          # == num_slots: out of range, treated as padding
    d = _dev(data)
    sentinel = 7.25
    inter = torch.full((6, 4, 2, 128, 128), sentinel, dtype=torch.float32, device="cuda")
    out = torch.full((24, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    _call(d, intermediate=inter, out=out)
    torch.cuda.synchronize()
    _check(data, out, inter)
    for b in (1, 4):
        assert torch.all(out[b * 4:(b + 1) * 4] == 0)
        assert torch.all(inter[b] == sentinel)


@pytest.mark.parametrize("B,T", [(33, 8), (40, 8), (32, 19)])
def test_verify_looping_workgroups_with_padding_rows(B, T):
    """B x 16 heads at 128-column tiles is at least two items per CU on 256 CUs (528, 640
    and 512 items): each workgroup loops over items and prefetches the next item's state
    (T = 19: a longer step loop per item).  Padding rows (slot -1 and slot ==
    num_slots) sit among them; their outputs are zero and their state rows untouched, and
    every live row matches the oracle."""
    case = W.VerifyCase(f"v_loop{B}x{T}", B, T, 16, pool_slots=64, seed=2110 + B + T,
                        padding_rows=[0, 7, B - 1])
    data = W.make_verify(case)
    data["state_idx"][12] = 64        # == num_slots: out of range, treated as padding
    print(f"case {case.name} seed {case.seed}", flush=True)
    d = _dev(data)
    sentinel = -2.5
    inter = torch.full((B, T, 16, 128, 128), sentinel, dtype=torch.float32, device="cuda")
    out = torch.full((B * T, 16, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    _call(d, intermediate=inter, out=out)
    torch.cuda.synchronize()
    _check(data, out, inter)
    for b in (0, 7, 12, B - 1):
        assert torch.all(out[b * T:(b + 1) * T] == 0)
        assert torch.all(inter[b] == sentinel)


def test_verify_strided_fused_projection_inputs():
    """q/k/v/g read in place from one fused [tokens, 4*H*128] projection buffer."""
    case = W.VerifyCase("v_strided", 8, 8, 4, pool_slots=16, seed=2102)
    data = W.make_verify(case)
    d = _dev(data)
    BT, H = 64, 4
    fused = torch.empty((BT, 4 * H * 128), dtype=torch.bfloat16, device="cuda")
    views = {}
    for i, name in enumerate(("q", "k", "v", "g")):
        fused[:, i * H * 128:(i + 1) * H * 128] = d[name].reshape(BT, H * 128)
        views[name] = fused[:, i * H * 128:(i + 1) * H * 128].view(BT, H, 128)
    assert views["q"].stride(0) == 4 * H * 128
    out_dense, inter_dense = _call(d)
    ds = dict(d, **views)
    out_s, inter_s = _call(ds)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_dense)
    assert torch.equal(inter_s, inter_dense)


def test_verify_single_steps_match_one_call():
    """T one-step calls, each seeded from the previous call's state row, agree with one
    T-step call to fp32 rounding: the multi-step call takes its steps' key-direction sums
    from the state at the start of each 8-step block, so the sums run in another order.
    States within 1e-6 relative (L2), outputs within one bf16 step."""
    case = W.VerifyCase("v_steps", 4, 6, 2, pool_slots=8, seed=2103)
    data = W.make_verify(case)
    d = _dev(data)
    out_all, inter_all = _call(d)
    B, T = 4, 6
    pool = d["state_pool"]
    idx = d["state_idx"]
    for t in range(T):
        rows = torch.arange(B, device="cuda") * T + t
        dt = dict(d, q=d["q"][rows], k=d["k"][rows], v=d["v"][rows], g=d["g"][rows],
                  beta_logits=d["beta_logits"][rows], state_pool=pool, state_idx=idx, num_steps=1)
        o1, i1 = _call(dt)
        a, c = o1.float(), out_all[rows].float()
        assert torch.all((a - c).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), c.abs()) + 1e-6)
        for r in range(B):
            err = TOL.state_rel_l2(i1[r, 0].cpu().numpy(), inter_all[r, t].cpu().numpy())
            assert err <= 1e-6, (t, r, err)
        pool = i1[:, 0].contiguous()
        idx = torch.arange(B, dtype=torch.int32, device="cuda")


def test_verify_deterministic():
    data = W.make_verify(W.VerifyCase("v_det", 16, 8, 16, pool_slots=32, seed=2104))
    d = _dev(data)
    o1, i1 = _call(d)
    o2, i2 = _call(d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(i1, i2)
