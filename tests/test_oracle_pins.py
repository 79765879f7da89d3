"""Pins for the CPU oracle: each checks it against something other than itself.

Kinds of pin (closed forms, invariants, exact rational brute force with a
different formula, an independently ordered chunked computation, and
equivalences between calls).  The last group plants mistakes in the oracle's
step (on the CPU) and checks that the pins catch each one.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import chunkform_fp64
from oracle import kda_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(7)


def _rand_inputs(T, H, K, V, rng, lb=-5.0):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = rng.standard_normal((T, H, K))
    bl = rng.standard_normal((T, H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt = 0.1 * rng.standard_normal((H, K))
    return q, k, v, g, bl, A_log, dt, lb


# ---------------------------------------------------------------- gate / beta / norm

def _read_gate_golden():
    env = {"log": math.log}
    rows = []
    with open(os.path.join(GOLDEN, "gate_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([float(eval(tok, {"__builtins__": {}}, env)) for tok in line.split()])
    return rows


def test_gate_closed_forms_golden():
    rows = _read_gate_golden()
    assert len(rows) >= 6
    for A_log, g, dt, lb, want in rows:
        got = O.gate_log_alpha(np.array([[g]]), np.array([A_log]), np.array([[dt]]), lb)
        assert abs(got.item() - want) < 1e-12, (A_log, g, dt, lb, got, want)


def test_gate_range_and_lb_zero():
    g = 30.0 * RNG.standard_normal((50, 3, 8))
    A_log = np.log(RNG.uniform(1, 16, 3))
    dt = RNG.standard_normal((3, 8))
    la = O.gate_log_alpha(g, A_log, dt, -5.0)
    alpha = np.exp(la)
    assert np.all(alpha >= math.exp(-5.0)) and np.all(alpha <= 1.0)
    assert np.all(O.gate_log_alpha(g, A_log, dt, 0.0) == 0.0)
    # Monotone in g for lb < 0: larger g -> stronger decay.
    la1 = O.gate_log_alpha(np.full((1, 1, 1), 0.3), np.zeros(1), np.zeros((1, 1)), -5.0)
    la2 = O.gate_log_alpha(np.full((1, 1, 1), 0.4), np.zeros(1), np.zeros((1, 1)), -5.0)
    assert la2.item() < la1.item() < 0


def test_beta_closed_form_and_range():
    assert O.beta_from_logits(np.array([0.0])).item() == 0.5
    assert abs(O.beta_from_logits(np.array([math.log(3.0)])).item() - 0.75) < 1e-15
    b = O.beta_from_logits(RNG.standard_normal(1000) * 3)
    assert np.all((b > 0) & (b < 1))
    # Symmetry sigma(-x) = 1 - sigma(x), and no overflow at extremes.
    x = RNG.standard_normal(100) * 50
    assert np.allclose(O.sigmoid(-x), 1 - O.sigmoid(x), atol=1e-15)
    assert O.sigmoid(np.array([-800.0])).item() == 0.0 and O.sigmoid(np.array([800.0])).item() == 1.0


def test_l2norm_invariants():
    x = RNG.standard_normal((20, 128))
    n = np.linalg.norm(O.l2_normalize(x), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-7)
    assert np.allclose(O.l2_normalize(3.5 * x), O.l2_normalize(x), atol=1e-9)
    assert np.all(O.l2_normalize(np.zeros((2, 128))) == 0.0)
    # eps appears exactly as sqrt(sum + eps): a unit vector maps to 1/sqrt(1+eps).
    e = np.zeros((1, 4)); e[0, 2] = 1.0
    assert abs(O.l2_normalize(e)[0, 2] - 1 / math.sqrt(1 + O.L2NORM_EPS)) < 1e-15


# ---------------------------------------------------------------- closed forms of the step

def _run_core(S0, qn, kn, v, alpha, beta, scale, step=None):
    """Drive the step for one head over T tokens: returns (outs [T,V], states [T,K,V])."""
    step = step or O.kda_step
    S = S0[None].copy()
    outs, states = [], []
    for t in range(qn.shape[0]):
        S, o = step(S, qn[t][None], kn[t][None], v[t][None], alpha[t][None],
                    np.array([beta[t]]), scale)
        outs.append(o[0]); states.append(S[0].copy())
    return np.array(outs), np.array(states)


def pin_pure_decay(step=None):
    """beta = 0: S_t = Diag(exp(sum la)) S_0 and o_t = scale * S_0^T (Gamma_t * q_t)."""
    rng = np.random.default_rng(1)
    T, K, V = 12, 16, 8
    S0 = rng.standard_normal((K, V))
    qn = O.l2_normalize(rng.standard_normal((T, K)))
    kn = O.l2_normalize(rng.standard_normal((T, K)))
    v = rng.standard_normal((T, V))
    la = -rng.uniform(0, 2, (T, K))
    outs, states = _run_core(S0, qn, kn, v, np.exp(la), np.zeros(T), 0.3, step)
    gam = np.exp(np.cumsum(la, axis=0))
    err = 0.0
    for t in range(T):
        err = max(err, np.abs(states[t] - gam[t][:, None] * S0).max())
        err = max(err, np.abs(outs[t] - 0.3 * S0.T @ (gam[t] * qn[t])).max())
    return err


def pin_delta_rule(step=None):
    """alpha = 1, beta = 1: S_1 = S_0 + k (v - S_0^T k)^T, so S_1^T k = v; o = scale S_1^T q."""
    rng = np.random.default_rng(2)
    K, V = 16, 8
    S0 = rng.standard_normal((K, V))
    kn = O.l2_normalize(rng.standard_normal((1, K)))
    qn = O.l2_normalize(rng.standard_normal((1, K)))
    v = rng.standard_normal((1, V))
    outs, states = _run_core(S0, qn, kn, v, np.ones((1, K)), np.ones(1), 0.5, step)
    # With ||k|| = 1 - O(eps), S_1^T k = v up to the norm's eps term.
    kk = float(kn[0] @ kn[0])
    S1 = S0 + np.outer(kn[0], v[0] - S0.T @ kn[0])
    err = np.abs(states[0] - S1).max()
    err = max(err, np.abs(states[0].T @ kn[0] - (v[0] * kk + (1 - kk) * (S0.T @ kn[0]))).max())
    err = max(err, np.abs(outs[0] - 0.5 * S1.T @ qn[0]).max())
    # Zero start: o = scale (k.q) v
    outs0, _ = _run_core(np.zeros((K, V)), qn, kn, v, np.ones((1, K)), np.ones(1), 0.5, step)
    err = max(err, np.abs(outs0[0] - 0.5 * float(kn[0] @ qn[0]) * v[0]).max())
    return err


def pin_orthonormal(step=None):
    """alpha = 1, beta = 1, orthonormal keys: S_T = S_0 + sum_i k_i (v_i - S_0^T k_i)^T."""
    rng = np.random.default_rng(3)
    K, V, T = 16, 8, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    kn = Qm[:, :T].T                                  # exactly orthonormal rows
    qn = O.l2_normalize(rng.standard_normal((T, K)))
    v = rng.standard_normal((T, V))
    S0 = rng.standard_normal((K, V))
    _, states = _run_core(S0, qn, kn, v, np.ones((T, K)), np.ones(T), 1.0, step)
    want = S0 + sum(np.outer(kn[i], v[i] - S0.T @ kn[i]) for i in range(T))
    return np.abs(states[-1] - want).max()


def pin_repeated_key(step=None):
    """alpha = 1, beta = 1, the same unit key at t1 < t2: S_t2^T k = v_t2 (overwrite)."""
    rng = np.random.default_rng(4)
    K, V, T = 16, 8, 7
    kn = O.l2_normalize(rng.standard_normal((T, K)))
    kn = kn / np.linalg.norm(kn, axis=1, keepdims=True)
    kn[5] = kn[1]
    qn = O.l2_normalize(rng.standard_normal((T, K)))
    v = rng.standard_normal((T, V))
    _, states = _run_core(rng.standard_normal((K, V)), qn, kn, v, np.ones((T, K)), np.ones(T), 1.0, step)
    return np.abs(states[5].T @ kn[5] - v[5]).max()


def test_pure_decay_closed_form():
    assert pin_pure_decay() < 1e-13


def test_single_token_delta_rule_closed_form():
    assert pin_delta_rule() < 1e-13


def test_orthonormal_keys_closed_form():
    assert pin_orthonormal() < 1e-12


def test_repeated_key_overwrite():
    assert pin_repeated_key() < 1e-12


# ---------------------------------------------------------------- exact brute force

def _frac_inputs(rng, T, K, V):
    def fr(lo, hi, den):
        return Fraction(int(rng.integers(lo, hi)), den)
    k = [[fr(-6, 7, 5) for _ in range(K)] for _ in range(T)]
    q = [[fr(-6, 7, 5) for _ in range(K)] for _ in range(T)]
    v = [[fr(-9, 10, 4) for _ in range(V)] for _ in range(T)]
    alpha = [[Fraction(int(rng.integers(1, 8)), 8) for _ in range(K)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 6)), 6) for _ in range(T)]
    S0 = [[fr(-4, 5, 3) for _ in range(V)] for _ in range(K)]
    return q, k, v, alpha, beta, S0


def _product_formula(q, k, v, alpha, beta, S0, scale):
    """S_T = M_T...M_1 S_0 + sum_t M_T...M_{t+1} beta_t k_t v_t^T, M_t = (I - beta_t k_t k_t^T) Diag(alpha_t).

    Evaluated with plain Python lists of Fractions (no numpy), step by explicit matrix products.
    """
    T, K, V = len(k), len(k[0]), len(v[0])

    def matmul(A, B):
        return [[sum(A[i][p] * B[p][j] for p in range(len(B))) for j in range(len(B[0]))]
                for i in range(len(A))]

    def M(t):
        return [[((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) * alpha[t][j]
                 for j in range(K)] for i in range(K)]

    outs, states = [], []
    for T_ in range(1, T + 1):
        # propagate S_0 through M_1..M_T_
        acc = [row[:] for row in S0]
        for t in range(T_):
            acc = matmul(M(t), acc)
        for t in range(T_):
            term = [[beta[t] * k[t][i] * v[t][j] for j in range(V)] for i in range(K)]
            for s in range(t + 1, T_):
                term = matmul(M(s), term)
            acc = [[acc[i][j] + term[i][j] for j in range(V)] for i in range(K)]
        states.append(acc)
        outs.append([scale * sum(acc[i][j] * q[T_ - 1][i] for i in range(K)) for j in range(V)])
    return outs, states


@pytest.mark.parametrize("K,V,T", [(2, 2, 4), (3, 2, 5), (4, 3, 6)])
def test_exact_bruteforce_product_formula(K, V, T):
    rng = np.random.default_rng(100 + K * 10 + T)
    q, k, v, alpha, beta, S0 = _frac_inputs(rng, T, K, V)
    scale = Fraction(1, 3)
    want_o, want_S = _product_formula(q, k, v, alpha, beta, S0, scale)
    # (1) The oracle's step run on exact rationals agrees exactly.
    obj = lambda x: np.array(x, dtype=object)
    S = obj([S0])
    for t in range(T):
        S, o = O.kda_step(S, obj([q[t]]), obj([k[t]]), obj([v[t]]), obj([alpha[t]]),
                          obj([beta[t]]), scale)
        assert all(o[0][j] == want_o[t][j] for j in range(V))
        assert all(S[0][i][j] == want_S[t][i][j] for i in range(K) for j in range(V))
    # (2) The float64 step agrees to rounding.
    f = lambda x: np.array(x, dtype=np.float64)
    outs, states = _run_core(f(S0), f(q), f(k), f(v), f(alpha), f(beta), float(scale))
    assert np.abs(outs - f(want_o)).max() < 1e-12
    assert np.abs(states - f(want_S)).max() < 1e-12


# ---------------------------------------------------------------- invariants of a full call

def test_linearity_and_column_independence():
    T, H, K, V = 40, 2, 16, 12
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(T, H, K, V, np.random.default_rng(5))
    cu = np.array([0, 17, 40])
    S_a = RNG.standard_normal((2, H, K, V)); S_b = RNG.standard_normal((2, H, K, V))
    v_b = RNG.standard_normal(v.shape)
    oa, fa = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, S_a)
    ob, fb = O.chunk_prefill(q, k, v_b, g, bl, A_log, dt, lb, cu, S_b)
    oc, fc = O.chunk_prefill(q, k, 2 * v - 3 * v_b, g, bl, A_log, dt, lb, cu, 2 * S_a - 3 * S_b)
    assert np.abs(oc - (2 * oa - 3 * ob)).max() < 1e-11
    assert np.abs(fc - (2 * fa - 3 * fb)).max() < 1e-11
    # Columns of S (value channels) evolve independently.
    o1, f1 = O.chunk_prefill(q, k, v[..., :5], g, bl, A_log, dt, lb, cu, S_a[..., :5])
    assert np.abs(o1 - oa[..., :5]).max() < 1e-12
    assert np.abs(f1 - fa[..., :5]).max() < 1e-12


# C = 8 is the block form of the verify kernel for few (row, head) pairs.
@pytest.mark.parametrize("C", [1, 8, 16, 64])
def test_chunk_form_matches_token_loop(C):
    T, H, K, V = 150, 2, 32, 24
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(T, H, K, V, np.random.default_rng(6))
    cu = np.array([0, 64, 65, 150])          # full chunk, 1-token seq, ragged tail
    S0 = 0.05 * RNG.standard_normal((3, H, K, V))
    o_ref, f_ref = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, S0)
    o_ch, f_ch = chunkform_fp64.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, S0, C=C)
    assert np.abs(o_ch - o_ref).max() < 1e-10
    assert np.abs(f_ch - f_ref).max() < 1e-10


def test_chunk_form_full_size_head():
    """Same equivalence at the real head size (K = V = 128), lb = -5, chunk 64."""
    T, H, K, V = 200, 1, 128, 128
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(T, H, K, V, np.random.default_rng(8))
    cu = np.array([0, T])
    o_ref, f_ref = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu)
    o_ch, f_ch = chunkform_fp64.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, C=64)
    assert np.abs(o_ch - o_ref).max() < 1e-10
    assert np.abs(f_ch - f_ref).max() < 1e-10


def test_varlen_equals_separate_and_resume():
    T, H, K, V = 90, 2, 16, 16
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(T, H, K, V, np.random.default_rng(9))
    cu = np.array([0, 30, 30, 90])           # includes a zero-length sequence
    S0 = RNG.standard_normal((3, H, K, V))
    o, f = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, S0)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        o1, f1 = O.chunk_prefill(q[s:e], k[s:e], v[s:e], g[s:e], bl[s:e], A_log, dt, lb,
                                 np.array([0, e - s]), S0[n:n + 1])
        if e > s:
            assert np.abs(o1 - o[s:e]).max() < 1e-13
        assert np.abs(f1[0] - f[n]).max() < 1e-13
    assert np.array_equal(f[1], S0[1])       # empty sequence: state untouched
    # Resume: split sequence 2 at 47 and carry the state.
    a = 47
    oA, fA = O.chunk_prefill(q[30:a], k[30:a], v[30:a], g[30:a], bl[30:a], A_log, dt, lb,
                             np.array([0, a - 30]), S0[2:3])
    oB, fB = O.chunk_prefill(q[a:90], k[a:90], v[a:90], g[a:90], bl[a:90], A_log, dt, lb,
                             np.array([0, 90 - a]), fA)
    assert np.abs(np.concatenate([oA, oB]) - o[30:90]).max() < 1e-12
    assert np.abs(fB[0] - f[2]).max() < 1e-12


def test_state_index_gather():
    T, H, K, V = 20, 2, 8, 8
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(T, H, K, V, np.random.default_rng(10))
    pool = RNG.standard_normal((5, H, K, V))
    o, f = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, np.array([0, 20]), pool,
                           initial_state_idx=np.array([3]))
    o2, f2 = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, np.array([0, 20]), pool[3:4])
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


def test_out_of_range_indices():
    """Verify: an index outside [0, slots) is a padding row (zero output, zero rows).
    Prefill: a start index outside the pool starts from the zero state."""
    B, T, H, K, V = 3, 4, 1, 8, 8
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(B * T, H, K, V, np.random.default_rng(12))
    pool = RNG.standard_normal((2, H, K, V))
    o, inter = O.recurrent_verify(q, k, v, g, bl, A_log, dt, lb, pool, np.array([1, 2, -3]), T)
    assert np.all(o[T:] == 0) and np.all(inter[1:] == 0) and np.any(o[:T] != 0)
    cu = np.array([0, 5, 12])
    o1, f1 = O.chunk_prefill(q[:12], k[:12], v[:12], g[:12], bl[:12], A_log, dt, lb, cu, pool,
                             initial_state_idx=np.array([7, -1]))
    o2, f2 = O.chunk_prefill(q[:12], k[:12], v[:12], g[:12], bl[:12], A_log, dt, lb, cu, None)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_verify_equals_prefill_and_rows():
    B, T, H, K, V = 3, 5, 2, 16, 16
    q, k, v, g, bl, A_log, dt, lb = _rand_inputs(B * T, H, K, V, np.random.default_rng(11))
    pool = RNG.standard_normal((7, H, K, V))
    idx = np.array([4, -1, 0])
    o, inter = O.recurrent_verify(q, k, v, g, bl, A_log, dt, lb, pool, idx, T)
    cu = np.arange(0, B * T + 1, T)
    op, fp = O.chunk_prefill(q, k, v, g, bl, A_log, dt, lb, cu, pool,
                             initial_state_idx=np.array([4, 0, 0]))
    for b in (0, 2):
        assert np.abs(o[b * T:(b + 1) * T] - op[b * T:(b + 1) * T]).max() < 1e-13
        assert np.abs(inter[b, T - 1] - fp[b]).max() < 1e-13
        for t in range(T):   # row t is the state after tokens 0..t
            s = b * T
            _, ft = O.chunk_prefill(q[s:s + t + 1], k[s:s + t + 1], v[s:s + t + 1],
                                    g[s:s + t + 1], bl[s:s + t + 1], A_log, dt, lb,
                                    np.array([0, t + 1]), pool[idx[b]:idx[b] + 1])
            assert np.abs(inter[b, t] - ft[0]).max() < 1e-13
    assert np.all(o[T:2 * T] == 0) and np.all(inter[1] == 0)   # padding row
    # T single-step calls chained through the state == one call.
    S = pool.copy()
    for t in range(T):
        rows = np.arange(B) * T + t
        ot, it = O.recurrent_verify(q[rows], k[rows], v[rows], g[rows], bl[rows], A_log, dt, lb,
                                    S, np.array([0, -1, 2]) if t else idx, 1)
        if t == 0:
            S = np.zeros((B, H, K, V)); S[0] = it[0, 0]; S[2] = it[2, 0]
        else:
            S[0] = it[0, 0]; S[2] = it[2, 0]
        for b in (0, 2):
            assert np.abs(ot[b] - o[b * T + t]).max() < 1e-13
            assert np.abs(it[b, 0] - inter[b, t]).max() < 1e-13


# ---------------------------------------------------------------- planted mistakes are caught

def _step_output_before_update(S, q, k, v, a, b, scale):
    S = a[:, :, None] * S
    o = scale * np.einsum("bkv,bk->bv", S, q)
    r = np.einsum("bkv,bk->bv", S, k)
    return S + b[:, None, None] * k[:, :, None] * (v - r)[:, None, :], o


def _step_decay_after_delta(S, q, k, v, a, b, scale):
    r = np.einsum("bkv,bk->bv", S, k)
    S = S + b[:, None, None] * k[:, :, None] * (v - r)[:, None, :]
    S = a[:, :, None] * S
    return S, scale * np.einsum("bkv,bk->bv", S, q)


def _step_decay_columns(S, q, k, v, a, b, scale):
    S = a[:, None, :S.shape[2]] * S                 # decays value channels instead of key channels
    r = np.einsum("bkv,bk->bv", S, k)
    S = S + b[:, None, None] * k[:, :, None] * (v - r)[:, None, :]
    return S, scale * np.einsum("bkv,bk->bv", S, q)


def _step_sign_flip(S, q, k, v, a, b, scale):
    S = a[:, :, None] * S
    r = np.einsum("bkv,bk->bv", S, k)
    S = S + b[:, None, None] * k[:, :, None] * (v + r)[:, None, :]
    return S, scale * np.einsum("bkv,bk->bv", S, q)


def _step_no_beta(S, q, k, v, a, b, scale):
    S = a[:, :, None] * S
    r = np.einsum("bkv,bk->bv", S, k)
    S = S + k[:, :, None] * (v - r)[:, None, :]
    return S, scale * np.einsum("bkv,bk->bv", S, q)


def _bruteforce_error(step):
    rng = np.random.default_rng(123)
    q, k, v, alpha, beta, S0 = _frac_inputs(rng, 5, 3, 2)
    want_o, want_S = _product_formula(q, k, v, alpha, beta, S0, Fraction(1, 3))
    f = lambda x: np.array(x, dtype=np.float64)
    outs, states = _run_core(f(S0), f(q), f(k), f(v), f(alpha), f(beta), 1 / 3, step)
    return max(np.abs(outs - f(want_o)).max(), np.abs(states - f(want_S)).max())


@pytest.mark.parametrize("bad", [_step_output_before_update, _step_decay_after_delta,
                                 _step_decay_columns, _step_sign_flip, _step_no_beta])
def test_planted_mistakes_are_caught(bad):
    errs = {
        "bruteforce": _bruteforce_error(bad),
        "pure_decay": pin_pure_decay(bad),
        "delta_rule": pin_delta_rule(bad),
        "orthonormal": pin_orthonormal(bad),
        "repeated_key": pin_repeated_key(bad),
    }
    assert max(errs.values()) > 1e-3, errs
    # The exact brute force alone catches every one of these.
    assert errs["bruteforce"] > 1e-3, errs
