"""Pins for the oracle's mixed speculative step pieces: the scatter of outputs by token
index and the rollback commit after verify.

The commit is pinned to the recurrence through a different computation: the state a
row commits after accepting n draft tokens must equal the final state of a prefill
over those n tokens from the same pool slot, computed by the independent chunked
fp64 form (tests/chunkform_fp64.py).  Planted off-by-one commits must fail that pin.
"""

import numpy as np
import pytest

import chunkform_fp64 as CF
from oracle import kda_oracle as O


def _inputs(T, H, K, V, rng, lb=-5.0):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = rng.standard_normal((T, H, K))
    bl = rng.standard_normal((T, H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt = 0.1 * rng.standard_normal((H, K))
    return q, k, v, g, bl, A_log, dt, lb


def _commit_next_row(pool, inter, idx, nacc):
    """Planted mistake: commits the state after n+1 tokens (clamped)."""
    pool = np.array(pool, copy=True)
    T = inter.shape[1]
    for b in range(inter.shape[0]):
        s, n = int(idx[b]), int(nacc[b])
        if 0 <= s < pool.shape[0] and 1 <= n <= T:
            pool[s] = inter[b, min(n, T - 1)]
    return pool


def _commit_row_zero(pool, inter, idx, nacc):
    """Planted mistake: always commits the first intermediate row."""
    pool = np.array(pool, copy=True)
    for b in range(inter.shape[0]):
        s, n = int(idx[b]), int(nacc[b])
        if 0 <= s < pool.shape[0] and 1 <= n <= inter.shape[1]:
            pool[s] = inter[b, 0]
    return pool


CASE = dict(B=5, T=6, H=2, K=8, V=8, slots=7)
IDX = np.array([3, 0, 6, 9, 2])      # 9 lies outside the pool: a padding row
NACC = np.array([2, 4, 6, 3, 0])     # 0: nothing accepted


def _prefix_mismatch(commit_fn):
    rng = np.random.default_rng(11)
    B, T, H, K, V, slots = (CASE[x] for x in ("B", "T", "H", "K", "V", "slots"))
    q, k, v, g, bl, A, dt, lb = _inputs(B * T, H, K, V, rng)
    pool = 0.3 * rng.standard_normal((slots, H, K, V))
    _, inter = O.recurrent_verify(q, k, v, g, bl, A, dt, lb, pool, IDX, T)
    new = commit_fn(pool, inter, IDX, NACC)
    worst = 0.0
    for b in range(B):
        s, n = int(IDX[b]), int(NACC[b])
        if not (0 <= s < slots and 1 <= n <= T):
            continue
        rows = slice(b * T, b * T + n)
        _, fin = CF.chunk_prefill(q[rows], k[rows], v[rows], g[rows], bl[rows], A, dt, lb,
                                  [0, n], initial_state=pool, initial_state_idx=[s], C=4)
        worst = max(worst, float(np.abs(new[s] - fin[0]).max()))
    return worst, pool, new


def test_commit_equals_prefill_of_accepted_prefix():
    worst, pool, new = _prefix_mismatch(O.commit_accepted)
    assert worst < 1e-10
    # Slots no valid row names (and slot 2, whose row accepted nothing) are unchanged.
    for s in range(CASE["slots"]):
        if s not in (3, 0, 6):
            assert np.array_equal(new[s], pool[s])


@pytest.mark.parametrize("bad", [_commit_next_row, _commit_row_zero])
def test_planted_commit_mistakes_are_caught(bad):
    worst, _, _ = _prefix_mismatch(bad)
    assert worst > 1e-3


def test_commit_returns_a_copy_and_ignores_out_of_range_counts():
    rng = np.random.default_rng(3)
    pool = rng.standard_normal((4, 1, 2, 2))
    inter = rng.standard_normal((3, 2, 1, 2, 2))
    before = pool.copy()
    new = O.commit_accepted(pool, inter, np.array([0, 1, 2]), np.array([3, -1, 2]))
    assert np.array_equal(pool, before)                 # the input pool is not modified
    assert np.array_equal(new[0], pool[0]) and np.array_equal(new[1], pool[1])
    assert np.array_equal(new[2], inter[2, 1]) and np.array_equal(new[3], pool[3])


def test_scatter_rows_places_and_drops():
    rng = np.random.default_rng(5)
    R, n = 20, 12
    vals = rng.standard_normal((n, 2, 4))
    perm = rng.permutation(R)[:n]
    out = O.scatter_rows(vals, perm, R)
    assert np.array_equal(out[perm], vals)
    rest = np.setdiff1d(np.arange(R), perm)
    assert np.all(out[rest] == 0)
    idx = perm.copy()
    idx[0], idx[1] = -1, R                               # dropped
    base = np.full((R, 2, 4), 7.0)
    out2 = O.scatter_rows(vals, idx, R, base)
    assert np.array_equal(out2[idx[2:]], vals[2:])
    kept = np.setdiff1d(np.arange(R), idx[2:])
    assert np.all(out2[kept] == 7.0)


def test_mixed_step_rows_equal_separate_requests():
    """A step carrying a prefill segment and spec rows: each request's rows of the
    merged output equal that request processed alone (requests are independent)."""
    rng = np.random.default_rng(9)
    H, K, V = 2, 8, 8
    lens = [5, 9]
    Tp = sum(lens)
    B, T, slots = 3, 2, 4
    qp, kp, vp, gp, blp, A, dt, lb = _inputs(Tp, H, K, V, rng)
    qs, ks, vs, gs, bls, _, _, _ = _inputs(B * T, H, K, V, rng)
    pool = 0.3 * rng.standard_normal((slots, H, K, V))
    sidx = np.array([1, 3, 0])
    R = Tp + B * T
    order = rng.permutation(R)
    non_spec, spec = order[:Tp], order[Tp:]
    op, _ = O.chunk_prefill(qp, kp, vp, gp, blp, A, dt, lb, [0, lens[0], Tp])
    ov, _ = O.recurrent_verify(qs, ks, vs, gs, bls, A, dt, lb, pool, sidx, T)
    merged = O.scatter_rows(ov, spec, R, O.scatter_rows(op, non_spec, R))
    s0 = slice(0, lens[0])
    alone, _ = O.chunk_prefill(qp[s0], kp[s0], vp[s0], gp[s0], blp[s0], A, dt, lb, [0, lens[0]])
    assert np.allclose(merged[non_spec[s0]], alone, atol=1e-12, rtol=0)
    r1 = slice(T, 2 * T)
    alone_v, _ = O.recurrent_verify(qs[r1], ks[r1], vs[r1], gs[r1], bls[r1], A, dt, lb, pool,
                                    sidx[1:2], T)
    assert np.allclose(merged[spec[r1]], alone_v, atol=1e-12, rtol=0)
