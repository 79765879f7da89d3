"""Independent float64 chunked (WY / UT-transform) form of the KDA recurrence.

Test infrastructure: a second, differently-ordered computation of the same
result as the token-loop oracle, used only to pin the oracle (chunked vs
sequential equivalence).  It imports nothing from the oracle or the HIP path.

Derivation (unrolling the per-token step inside one chunk of C tokens, with
a_t the per-channel log-decay, b_t = a_1 + ... + a_t and Gamma_t = exp(b_t)):

    S_t = Diag(Gamma_t) S_0 + sum_{i<=t} Diag(exp(b_t - b_i)) k_i u_i^T
    u_t = beta_t (v_t - S_0^T (Gamma_t * k_t) - sum_{i<t} G_ti u_i)
    G_ti = sum_c k_tc k_ic exp(b_tc - b_ic)

so (I + diag(beta) strict(G)) U = diag(beta)(V - K_Gamma S_0), i.e.
U = T diag(beta) V - T diag(beta) K_Gamma S_0 with T = (I + A)^-1, and

    O   = scale * (Q_Gamma S_0 + tril(P) U),   P_ti = sum_c q_tc k_ic exp(b_tc - b_ic)
    S_C = Diag(Gamma_C) S_0 + K_C^T U,          K_C[i] = exp(b_C - b_i) * k_i
"""

from __future__ import annotations

import math

import numpy as np


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))   # a different closed form from the oracle's


def _normalize(x, eps=1e-6):
    n2 = np.einsum("...k,...k->...", x, x)
    return x / np.sqrt(n2 + eps)[..., None]


def chunk_forward_head(qn, kn, v, la, beta, S0, scale, C):
    """One (sequence, head): qn, kn, la [T, K]; v [T, V]; beta [T]; S0 [K, V]."""
    T, K = qn.shape
    out = np.zeros((T, v.shape[1]))
    S = S0.copy()
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        q_, k_, v_, a_, be = qn[c0:c1], kn[c0:c1], v[c0:c1], la[c0:c1], beta[c0:c1]
        n = c1 - c0
        b = np.cumsum(a_, axis=0)                       # [n, K]
        gam = np.exp(b)
        diff = b[:, None, :] - b[None, :, :]            # [t, i, K] = b_t - b_i
        dec = np.exp(np.minimum(diff, 0.0))             # only i <= t is used
        G = np.einsum("tc,ic,tic->ti", k_, k_, dec)
        P = np.einsum("tc,ic,tic->ti", q_, k_, dec)
        A = be[:, None] * np.tril(G, -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))  # (I + A)^-1
        W = Tm @ (be[:, None] * (k_ * gam))
        Ut = Tm @ (be[:, None] * v_)
        U = Ut - W @ S
        out[c0:c1] = scale * ((q_ * gam) @ S + np.tril(P) @ U)
        KC = np.exp(b[-1][None, :] - b) * k_
        S = gam[-1][:, None] * S + KC.T @ U
    return out, S


def chunk_prefill(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                  initial_state=None, initial_state_idx=None, scale=None, C=64):
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    Tt, H, K = q.shape
    V = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    N = len(cu) - 1
    qn, kn = _normalize(q), _normalize(k)
    expA = np.exp(np.asarray(A_log, np.float64))[:, None]
    la = lower_bound * _sigmoid(expA * (g + np.asarray(dt_bias, np.float64)))
    beta = _sigmoid(np.asarray(beta_logits, np.float64))
    out = np.zeros((Tt, H, V))
    final = np.zeros((N, H, K, V))
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        for h in range(H):
            if initial_state is None:
                S0 = np.zeros((K, V))
            else:
                row = n if initial_state_idx is None else int(initial_state_idx[n])
                S0 = np.asarray(initial_state[row, h], np.float64)
            if e == s:
                final[n, h] = S0
                continue
            o, S = chunk_forward_head(qn[s:e, h], kn[s:e, h], v[s:e, h], la[s:e, h],
                                      beta[s:e, h], S0, scale, C)
            out[s:e, h] = o
            final[n, h] = S
    return out, final
