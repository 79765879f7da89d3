"""The operand formats of the GPU prefill, re-derived on the CPU.

tests/precision_emulator.py replays the chunked prefill with the kernels' rounding
points.  Against the fp64 oracle it must show that
  * the formats the kernels use (bf16 G, three-product bf16 P, fp16 scan operands)
    meet the parity bar with margin;
  * plain bf16 P, or bf16 scan operands, do not -- the reason for each choice;
  * the fp16 operands (S, X = V - K_Gamma S, U = T'X) stay far inside fp16 range for
    |v| up to 2^14, the input range the library documents, and overflow well beyond it.
"""

import numpy as np
import pytest

import precision_emulator as E
import tolerances as TOL
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

FP16_MAX = 65504.0


def _case(lens, H, init, seed, v_max=None):
    d = W.make_prefill(W.PrefillCase("precision_map", lens, H, init=init, seed=seed))
    f = W.to_f64
    v = f(d["v"])
    if v_max is not None:
        # bf16-exact rescaling by a power of two keeps v on the bf16 grid
        v = v * 2.0 ** np.floor(np.log2(v_max / np.max(np.abs(v))))
    args = (f(d["q"]), f(d["k"]), v, f(d["g"]), f(d["beta_logits"]), f(d["A_log"]),
            f(d["dt_bias"]), d["lower_bound"], d["cu_seqlens"].numpy())
    init_np = None if d["initial_state"] is None else d["initial_state"].numpy()
    return args, init_np, d["scale"]


def _errors(lens, H, init, seed, variant, v_max=None):
    args, init_np, scale = _case(lens, H, init, seed, v_max)
    o_ref, f_ref = O.chunk_prefill(*args, init_np, scale=scale)
    o, fin, stats = E.emulate_prefill(*args, init_np, scale=scale, variant=variant)
    return TOL.output_errors(o, o_ref), TOL.state_rel_l2(fin, f_ref), stats, args


@pytest.mark.parametrize("lens,H,init", [([1024], 2, None), ([2048], 2, "per_seq"),
                                         ([300, 77], 2, "per_seq")])
def test_kernel_formats_meet_the_bar(lens, H, init):
    e, r, _, _ = _errors(lens, H, init, 7000 + sum(lens), "gpu")
    print("kernel formats", e, r)
    # measured 2.8e-3 .. 4.3e-3 output excess and 3.3e-4 .. 3.7e-4 state error
    assert e["excess_over_rms"] <= 0.5 * TOL.OUT_TOL
    assert r <= 0.5 * TOL.STATE_TOL


def test_fp16_off_diagonal_blocks_cost_nothing():
    # off the diagonal both Gram factors are <= 1: fp16 (one product) is as good as bf16
    for lb in (-5.0, 0.0):
        d = W.make_prefill(W.PrefillCase("offdiag", [1024], 2, seed=7124, lower_bound=lb))
        f = W.to_f64
        args = (f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["beta_logits"]), f(d["A_log"]),
                f(d["dt_bias"]), d["lower_bound"], d["cu_seqlens"].numpy())
        o_ref, f_ref = O.chunk_prefill(*args, None, scale=d["scale"])
        res = {}
        for var in ("gpu", "bf16_offdiag"):
            o, fin, _ = E.emulate_prefill(*args, None, scale=d["scale"], variant=var)
            res[var] = (TOL.output_errors(o, o_ref)["excess_over_rms"], TOL.state_rel_l2(fin, f_ref))
        print(lb, res)
        assert res["gpu"][0] <= 1.05 * res["bf16_offdiag"][0]
        assert res["gpu"][1] <= 1.05 * res["bf16_offdiag"][1]


def test_plain_bf16_P_fails_the_output_bar():
    e, r, _, _ = _errors([2048], 2, "per_seq", 9048, "plain_bf16_P")
    e_ok, _, _, _ = _errors([2048], 2, "per_seq", 9048, "gpu")
    print("plain bf16 P", e, "kernel formats", e_ok)
    assert e["excess_over_rms"] > TOL.OUT_TOL
    assert e["excess_over_rms"] > 4 * e_ok["excess_over_rms"]
    assert r <= TOL.STATE_TOL            # P never reaches the state


def test_bf16_scan_operands_fail_both_bars():
    e, r, _, _ = _errors([1024], 2, None, 8024, "bf16_scan")
    print("bf16 scan operands", e, r)
    assert e["excess_over_rms"] > TOL.OUT_TOL
    assert r > TOL.STATE_TOL


def test_fp16_operands_stay_in_range_up_to_v_2_14():
    e, r, stats, args = _errors([2048], 2, "per_seq", 9148, "gpu", v_max=2.0 ** 14)
    assert 2.0 ** 13 <= np.max(np.abs(args[2])) <= 2.0 ** 14
    print("max |v| 2^14:", stats, e, r)
    assert max(stats.values()) < FP16_MAX / 2
    assert e["excess_over_rms"] <= TOL.OUT_TOL and r <= TOL.STATE_TOL
    # far past the documented range the fp16 operands overflow
    _, _, stats, _ = _errors([2048], 2, "per_seq", 9148, "gpu", v_max=2.0 ** 17)
    assert max(stats["X"], stats["U"]) > FP16_MAX
