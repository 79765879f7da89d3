"""Operand-precision model of the GPU prefill (test infrastructure, CPU only).

The GPU prefill evaluates the chunked form of the KDA recurrence with its MFMA
operands rounded to 16-bit formats.  This module replays that chunked form in
float64 with exactly those rounding points, so the error each format choice costs
can be measured against the fp64 token-loop oracle without a GPU:

* G (k.k Gram, feeds the UT transform): bf16 operands, one product, on the diagonal
  16-token blocks; fp16 operands off them (both factors <= 1 there);
* P (q.k Gram, feeds the output directly): bf16 hi/lo split, three products, on the
  diagonal blocks; one fp16 product off them;
* T = (I + diag(beta) strict(G))^-1 and everything on the fp32 VALU: kept in float64;
* the scan operands -K_Gamma, T diag(beta), scale Q_Gamma, scale tril(P), K_C^T and
  the per-chunk S, X = V - K_Gamma S, U = T'X: fp16, with fp32 accumulation;
* the output: bf16 round-to-nearest-even.

Variants swap one choice to show what it costs: "bf16_offdiag" (the off-diagonal blocks
in bf16 like the diagonal ones), "plain_bf16_P" (no split anywhere), "bf16_scan" (bf16 scan
operands).
The chunked form itself is derived from the recurrence in tests/chunkform_fp64.py's
terms; the 16-token row blocks with block-start references are how the GPU keeps
every exponential inside the bf16/fp16 exponent range.  Nothing here is shared with
the HIP sources or with the oracle: it imports neither.

`emulate_prefill` also reports the largest magnitude that reaches each fp16 operand
(S, X, U), which is what bounds the inputs' admissible range.
"""

from __future__ import annotations

import numpy as np

CHUNK = 64
BLOCK = 16
EPS = 1e-6


def bf16(x):
    """Round float64 values to bf16 (round to nearest, ties to even) via fp32 bits."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if np.any(nan):
        out[nan] = np.nan
    return out


def f16(x):
    """Round float64 values to fp16 (round to nearest even; overflow gives inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _split_bf16(x):
    hi = bf16(x)
    return hi, bf16(x - hi)


def _token_prologue(q, k, g, beta_logits, A_log_h, dt_h, lower_bound):
    qn = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + EPS)
    kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + EPS)
    la2 = lower_bound * np.log2(np.e) / (1.0 + np.exp(-np.exp(A_log_h) * (g + dt_h)))
    beta = 1.0 / (1.0 + np.exp(-beta_logits))
    return qn, kn, la2, beta


def _chunk_record(qn, kn, la2, beta, scale, variant):
    """What the intra-chunk kernel stores for one chunk of L <= 64 tokens (one head)."""
    L = qn.shape[0]
    nb = (L + BLOCK - 1) // BLOCK
    blk = np.arange(L) // BLOCK
    bl = np.zeros_like(la2)                       # in-block inclusive cumulative log2 decay
    base = np.zeros((nb + 1, la2.shape[1]))       # block bases; base[nb] = chunk total
    for m in range(nb):
        rows = slice(m * BLOCK, min(L, (m + 1) * BLOCK))
        bl[rows] = np.cumsum(la2[rows], axis=0)
        base[m + 1] = base[m] + bl[rows][-1]
    Lf, Rf = 2.0 ** bl, 2.0 ** (-bl)
    kl = kn * Lf                                  # k^ 2^(b_t - base_m)
    ql = scale * qn * Lf
    kr = kn * Rf                                  # k^ 2^(base_m - b_t)
    KL = bf16(kl)
    QLh, QLl = _split_bf16(ql)
    G = np.zeros((L, L))
    P = np.zeros((L, L))
    for m in range(nb):
        tr = slice(m * BLOCK, min(L, (m + 1) * BLOCK))
        for w in range(m + 1):
            ic = slice(w * BLOCK, min(L, (w + 1) * BLOCK))
            right = kr[ic] * 2.0 ** (base[m] - base[w])       # re-referenced to block m
            if variant in ("gpu", "bf16_scan") and w < m:
                # both factors <= 1 off the diagonal: one fp16 product each for G and P
                Rf16 = f16(right)
                G[tr, ic] = f16(kl[tr]) @ Rf16.T
                P[tr, ic] = f16(ql[tr]) @ Rf16.T
                continue
            Rh, Rl = _split_bf16(right)
            G[tr, ic] = KL[tr] @ Rh.T
            if variant == "plain_bf16_P":
                P[tr, ic] = bf16(ql[tr]) @ Rh.T
            else:
                P[tr, ic] = QLh[tr] @ Rh.T + QLh[tr] @ Rl.T + QLl[tr] @ Rh.T
    A = beta[:, None] * np.tril(G, -1)
    T = np.linalg.inv(np.eye(L) + A)
    rnd = bf16 if variant == "bf16_scan" else f16
    Eb = 2.0 ** base[blk]                         # 2^(base_m) per token row
    KCb = 2.0 ** (base[nb][None, :] - base[blk])  # 2^(total - base_m)
    return dict(
        TP=rnd(np.tril(T) * beta[None, :]),
        PM=rnd(np.tril(P)),
        KG=rnd(-kl * Eb),                         # -K_Gamma
        QG=rnd(ql * Eb),                          # scale Q_Gamma
        KC=rnd(kr * KCb),                         # K_C (rows: tokens)
        gamma_C=2.0 ** base[nb],
        rnd=rnd,
    )


def emulate_prefill(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                    initial_state=None, scale=None, variant="gpu"):
    """Chunked prefill with the GPU's operand rounding.

    Arrays as in the oracle (float64 values of the bf16 inputs): q, k, g [T, H, 128];
    v [T, H, 128]; beta_logits [T, H]; A_log [H]; dt_bias [H, 128]; cu_seqlens [N+1];
    initial_state [N, H, 128, 128] or None.  variant: "gpu" (the formats the kernels
    use), "bf16_offdiag", "plain_bf16_P" or "bf16_scan".
    Returns (out [T, H, 128] bf16-rounded, final [N, H, 128, 128], stats) where stats
    holds the largest |value| entering each fp16 operand: "S", "X", "U".
    """
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    beta_logits = np.asarray(beta_logits, dtype=np.float64)
    T_total, H, K = q.shape
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    N = len(cu) - 1
    scale = 1.0 / np.sqrt(K) if scale is None else scale
    out = np.zeros((T_total, H, K))
    final = np.zeros((N, H, K, K))
    stats = {"S": 0.0, "X": 0.0, "U": 0.0}
    with np.errstate(over="ignore", invalid="ignore"):    # fp16 overflow is reported, not raised
        _scan(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu, initial_state, scale,
              variant, out, final, stats)
    return out, final, stats


def _scan(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu, initial_state, scale,
          variant, out, final, stats):
    H, K = q.shape[1], q.shape[2]
    for n in range(len(cu) - 1):
        for h in range(H):
            S = np.zeros((K, K)) if initial_state is None else \
                np.array(initial_state[n, h], dtype=np.float64)
            qn, kn, la2, beta = _token_prologue(q[cu[n]:cu[n + 1], h], k[cu[n]:cu[n + 1], h],
                                                g[cu[n]:cu[n + 1], h],
                                                beta_logits[cu[n]:cu[n + 1], h],
                                                float(np.asarray(A_log)[h]),
                                                np.asarray(dt_bias)[h], lower_bound)
            for c0 in range(0, cu[n + 1] - cu[n], CHUNK):
                c1 = min(cu[n + 1] - cu[n], c0 + CHUNK)
                rec = _chunk_record(qn[c0:c1], kn[c0:c1], la2[c0:c1], beta[c0:c1], scale,
                                    variant)
                rnd = rec["rnd"]
                stats["S"] = max(stats["S"], float(np.max(np.abs(S))))
                Sf = rnd(S)
                X = v[cu[n] + c0:cu[n] + c1, h] + rec["KG"] @ Sf
                stats["X"] = max(stats["X"], float(np.max(np.abs(X))))
                Xf = rnd(X)
                U = rec["TP"] @ Xf
                stats["U"] = max(stats["U"], float(np.max(np.abs(U))))
                Uf = rnd(U)
                out[cu[n] + c0:cu[n] + c1, h] = bf16(rec["QG"] @ Sf + rec["PM"] @ Uf)
                S = rec["gamma_C"][:, None] * S + rec["KC"].T @ Uf
            final[n, h] = S
