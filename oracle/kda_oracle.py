"""Plain CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no helpers, tables, constants or pre/post-processing).

What it computes (the plain definition, token by token, in float64):

* Gate -- vLLM PR #55737 "Use FlashKDA for KDA chunked prefill", opening
  commit message and the "Purpose" section: the bounded gate is
  ``lower_bound * sigmoid(exp(A_log) * (g + dt_bias))``; q and k are
  L2-normalised inside the kernel; beta arrives as raw logits.  We read the
  gate value as the natural log of the per-key-channel decay alpha, so
  alpha = exp(gate) lies in [exp(lower_bound), 1].
* Recurrence -- the same page states that FlashKDA and the Triton chunk path
  compute one and the same bounded-gate KDA recurrence, but no page writes the
  step out.  The step used here is the gated delta rule with a per-key-channel
  gate: decay the rows of the state S[K, V] by alpha, apply the delta rule
  on the decayed state, then read the output from the updated state:
      S <- Diag(alpha) S
      S <- S + beta * k (v - S^T k)^T
      o  = scale * S^T q
* Verify -- TensorRT-LLM PR #21179 "GLM-5.3-Flash FP8 performance fixes on
  Hopper", the fused-verify commit message: one call seeds each batch row from
  the state pool and writes step t's state to row (b, t) of the per-step state
  buffer; the pool stays read-only.  Reading used: row t holds the state after
  token t (0-based), so the last row is the all-accepted state.

* Short causal conv -- TensorRT-LLM PR #21179 (fused-verify commit message) and vLLM
  PR #55737 ("Notes for review"): depthwise causal conv of width W <= 4 per channel
  with optional bias and SiLU, windows of the W-1 previous inputs.
* Gated output norm -- SGLang PR #42489 "Improve GLM-5.3-Flash DFlash decoding
  on B300": a sigmoid RMSNorm over D = 128 rows with output and rstd parity.
  Reading used: y = x / sqrt(mean(x^2) + eps) * weight * sigmoid(gate).
* Mixed speculative step and commit -- vLLM PR #55737, the "...code steps too"
  commit message: outputs of the prefill segment and of the spec tokens are
  scattered into one layer output by their token indices, and spec rows keep
  the state their accepted tokens reached (num_accepted_tokens rollback).
  Reading used: num_accepted counts the accepted tokens n of a row, so the
  committed state is intermediate[b, n-1]; n = 0 (or more than T) commits
  nothing.

Readings taken where the pages are silent:
L2 norm is x / sqrt(sum(x^2) + 1e-6); scale defaults to 1/sqrt(d_k); state
layout is [K, V] (rows are key channels, the ones the gate decays); a
zero-length sequence leaves its state untouched; in verify, a state index
outside [0, slots) marks a padding row whose outputs are zero and whose
states are not written; in prefill, a start-state index outside the pool
starts that sequence from the zero state.

Parity pins for every function here live in ``tests/test_oracle_pins.py`` (recurrence,
prefill, verify), ``tests/test_oracle_mixed_pins.py`` (scatter, commit),
``tests/test_oracle_norm_pins.py`` and ``tests/test_oracle_conv_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

L2NORM_EPS = 1e-6


# ---------------------------------------------------------------------------
# Elementwise pieces (vLLM PR #55737, opening commit / "Purpose")
# ---------------------------------------------------------------------------

def sigmoid(x):
    """Logistic function in float64, written in the overflow-free two-branch form."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def l2_normalize(x, eps: float = L2NORM_EPS):
    """Row-wise x / sqrt(sum(x^2) + eps) over the last axis (q/k L2 norm)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gate_log_alpha(g, A_log, dt_bias, lower_bound: float):
    """Bounded gate: lower_bound * sigmoid(exp(A_log) * (g + dt_bias)).

    g: [..., H, K]; A_log: [H]; dt_bias: [H, K].  Returns log(alpha) with the
    same shape as g (natural log, per key channel).
    """
    g = np.asarray(g, dtype=np.float64)
    a = np.exp(np.asarray(A_log, dtype=np.float64))[:, None]          # [H, 1]
    return float(lower_bound) * sigmoid(a * (g + np.asarray(dt_bias, np.float64)))


def beta_from_logits(beta_logits):
    """beta = sigmoid(beta logit); the kernel receives logits (vLLM PR #55737)."""
    return sigmoid(beta_logits)


# ---------------------------------------------------------------------------
# One recurrence step (the definition).  Works on float64 arrays and, for the
# exact brute-force pins, on object arrays of fractions.Fraction.
# ---------------------------------------------------------------------------

def kda_step(S, q_hat, k_hat, v, alpha, beta, scale):
    """One token of the gated delta rule for a batch of independent heads.

    S: [B, K, V]; q_hat, k_hat, alpha: [B, K]; v: [B, V]; beta: [B].
    Returns (S_new, o) with o: [B, V].
    """
    S = alpha[:, :, None] * S                                      # S <- Diag(alpha) S
    r = np.einsum("bkv,bk->bv", S, k_hat)                          # S^T k
    S = S + beta[:, None, None] * k_hat[:, :, None] * (v - r)[:, None, :]
    o = scale * np.einsum("bkv,bk->bv", S, q_hat)                  # o = scale S^T q
    return S, o


# ---------------------------------------------------------------------------
# Modes
# ---------------------------------------------------------------------------

def _as64(x):
    return np.asarray(x, dtype=np.float64)


def chunk_prefill(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                  initial_state=None, initial_state_idx=None, scale=None):
    """Varlen prefill, token by token.

    q, k, g: [T_total, H, K]; v: [T_total, H, V]; beta_logits: [T_total, H];
    A_log: [H]; dt_bias: [H, K]; cu_seqlens: [N+1] ints (cu[0] = 0, non-decreasing).
    initial_state: None (zeros) or [rows, H, K, V]; row n is used for sequence n,
    or row initial_state_idx[n] when an index vector is given.
    Returns (out [T_total, H, V] float64, final_state [N, H, K, V] float64).
    """
    q, k, v, g = _as64(q), _as64(k), _as64(v), _as64(g)
    T_total, H, K = q.shape
    V = v.shape[-1]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = np.zeros((T_total, H, V), dtype=np.float64)
    final = np.zeros((N, H, K, V), dtype=np.float64)

    qn = l2_normalize(q)
    kn = l2_normalize(k)
    alpha = np.exp(gate_log_alpha(g, A_log, dt_bias, lower_bound))
    beta = beta_from_logits(_as64(beta_logits))

    # Sequences of equal length are stepped together (they are independent).
    by_len = {}
    for n in range(N):
        by_len.setdefault(cu[n + 1] - cu[n], []).append(n)
    for length, seqs in by_len.items():
        S = np.zeros((len(seqs), H, K, V), dtype=np.float64)
        if initial_state is not None:
            init = _as64(initial_state)
            for j, n in enumerate(seqs):
                row = n if initial_state_idx is None else int(initial_state_idx[n])
                if 0 <= row < init.shape[0]:
                    S[j] = init[row]
        S = S.reshape(len(seqs) * H, K, V)
        starts = np.array([cu[n] for n in seqs])
        for t in range(length):
            rows = starts + t
            S, o = kda_step(S, qn[rows].reshape(-1, K), kn[rows].reshape(-1, K),
                            v[rows].reshape(-1, V), alpha[rows].reshape(-1, K),
                            beta[rows].reshape(-1), scale)
            out[rows] = o.reshape(len(seqs), H, V)
        final[seqs] = S.reshape(len(seqs), H, K, V)
    return out, final


def recurrent_verify(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound,
                     state_pool, state_idx, num_steps, scale=None):
    """Multi-step verify: B rows of num_steps tokens each (token b*T + t).

    state_pool: [slots, H, K, V] (read only); state_idx: [B] ints, outside [0, slots) = padding.
    Returns (out [B*T, H, V], intermediate [B, T, H, K, V]) where
    intermediate[b, t] is the state after token t of row b.  Padding rows give
    zero outputs and zero intermediate rows (the GPU leaves them unwritten).
    """
    q, k, v, g = _as64(q), _as64(k), _as64(v), _as64(g)
    BT, H, K = q.shape
    V = v.shape[-1]
    T = int(num_steps)
    B = BT // T
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    idx = np.asarray(state_idx).reshape(-1)
    out = np.zeros((BT, H, V), dtype=np.float64)
    inter = np.zeros((B, T, H, K, V), dtype=np.float64)
    pool = np.asarray(state_pool)
    live = [b for b in range(B) if 0 <= int(idx[b]) < pool.shape[0]]
    if not live:
        return out, inter
    S = np.stack([pool[int(idx[b])].astype(np.float64) for b in live]).reshape(-1, K, V)

    qn = l2_normalize(q)
    kn = l2_normalize(k)
    alpha = np.exp(gate_log_alpha(g, A_log, dt_bias, lower_bound))
    beta = beta_from_logits(_as64(beta_logits))
    live_arr = np.array(live)
    for t in range(T):
        rows = live_arr * T + t
        S, o = kda_step(S, qn[rows].reshape(-1, K), kn[rows].reshape(-1, K),
                        v[rows].reshape(-1, V), alpha[rows].reshape(-1, K),
                        beta[rows].reshape(-1), scale)
        out[rows] = o.reshape(len(live), H, V)
        inter[live_arr, t] = S.reshape(len(live), H, K, V)
    return out, inter


# ---------------------------------------------------------------------------
# Mixed speculative step and commit (vLLM PR #55737, the "...code steps too"
# commit message: in a step that carries both kinds of tokens the prefill
# segment's outputs are scattered into the layer output by the non-spec token
# indices and the spec tokens' outputs by the spec token indices; spec tokens
# keep the recurrent kernel with num_accepted_tokens rollback).
# ---------------------------------------------------------------------------

def scatter_rows(values, index, num_rows, base=None):
    """Row t of `values` placed at row index[t] of a [num_rows, ...] array.

    Rows of `base` (zeros when None) that no index names are kept; an index
    outside [0, num_rows) drops its row.  Indices are taken as distinct.
    """
    values = np.asarray(values)
    out = (np.zeros((num_rows,) + values.shape[1:], dtype=values.dtype) if base is None
           else np.array(base, copy=True))
    for t, r in enumerate(np.asarray(index).reshape(-1)):
        if 0 <= int(r) < num_rows:
            out[int(r)] = values[t]
    return out


def commit_accepted(state_pool, intermediate, state_idx, num_accepted):
    """Rollback commit after verify, returning the updated pool (a copy).

    Row b accepted n = num_accepted[b] of its T draft tokens; its pool slot
    state_idx[b] takes the state after those n tokens, intermediate[b, n-1].
    Rows with a slot outside the pool, or n outside [1, T], change nothing.
    """
    pool = np.array(state_pool, copy=True)
    inter = np.asarray(intermediate)
    B, T = inter.shape[:2]
    idx = np.asarray(state_idx).reshape(-1)
    nacc = np.asarray(num_accepted).reshape(-1)
    for b in range(B):
        s, n = int(idx[b]), int(nacc[b])
        if 0 <= s < pool.shape[0] and 1 <= n <= T:
            pool[s] = inter[b, n - 1]
    return pool


# ---------------------------------------------------------------------------
# Output-gate sigmoid RMSNorm (SGLang PR #42489 "Improve GLM-5.3-Flash DFlash
# decoding on B300", "Modifications" and "Accuracy Tests": the sigmoid RMSNorm
# dispatch for bf16, D = 128 rows, checked for output and rstd parity; the page
# never writes the formula).  Reading used: per row of D channels (one token and
# head), y = x / sqrt(mean(x^2) + eps) * weight * sigmoid(gate), and rstd is the
# row's 1 / sqrt(mean(x^2) + eps).
# ---------------------------------------------------------------------------

def gated_rmsnorm(x, gate, weight, eps):
    """Returns (y, rstd) in float64 for x, gate [..., D] and weight [D]."""
    x = np.asarray(x, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    y = x * rstd[..., None] * w * sigmoid(gate)
    return y, rstd


# ---------------------------------------------------------------------------
# Short causal convolution on the q / k / v projections (TensorRT-LLM PR #21179,
# fused-verify commit message: three short convolutions per draft step, run as
# one packed causal_conv1d_update that writes each step's window into
# intermediate_conv_window from a gathered copy of the pool rows, inputs read
# in place from the fused projection; vLLM PR #55737, "Notes for review": the
# short conv per q/k/v into separate buffers).  Readings used: a depthwise causal
# convolution of width W <= 4 per channel c,
#     y_t[c] = act(bias[c] + sum_{i<W} weight[c, i] * x_{t-W+1+i}[c]),
# where inputs before a sequence's first token come from its window (the W-1
# previous inputs, oldest first; zeros when the window index is out of range),
# act is SiLU (x * sigmoid(x)) or the identity, and the window after a token is
# the last W-1 inputs up to and including it.
# ---------------------------------------------------------------------------

def _conv_run(xs, window, weight, bias, silu):
    """Token loop over one sequence.  xs [L, C], window [W-1, C] -> (y [L, C], windows
    [L, W-1, C] after each token)."""
    W = weight.shape[1]
    hist = [window[i] for i in range(W - 1)]
    ys, wins = [], []
    for t in range(xs.shape[0]):
        taps = hist + [xs[t]]                       # oldest first, W entries
        acc = np.zeros(xs.shape[1]) if bias is None else np.array(bias, dtype=np.float64)
        for i in range(W):
            acc = acc + weight[:, i] * taps[i]
        ys.append(acc * sigmoid(acc) if silu else acc)
        hist = taps[1:]
        wins.append(np.stack(hist) if W > 1 else np.zeros((0, xs.shape[1])))
    y = np.stack(ys) if ys else np.zeros((0, xs.shape[1]))
    win = np.stack(wins) if wins else np.zeros((0, W - 1, xs.shape[1]))
    return y, win


def conv1d_prefill(x, weight, bias, cu_seqlens, state, state_idx, silu=True):
    """Varlen causal conv.  x [T, C]; weight [C, W]; bias [C] or None; state [slots, W-1, C]
    (windows, or None for zeros); state_idx [N] or None (row n).  Returns (y [T, C],
    new_state [slots, W-1, C]: each in-range indexed window replaced by the window after
    its sequence)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    W = w.shape[1]
    C = x.shape[1]
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    y = np.zeros_like(x)
    new_state = None if state is None else np.array(state, dtype=np.float64, copy=True)
    for n in range(len(cu) - 1):
        row = n if state_idx is None else int(np.asarray(state_idx).reshape(-1)[n])
        in_pool = state is not None and 0 <= row < state.shape[0]
        win0 = (np.asarray(state[row], dtype=np.float64) if in_pool else np.zeros((W - 1, C)))
        ys, wins = _conv_run(x[cu[n]:cu[n + 1]], win0, w, bias, silu)
        y[cu[n]:cu[n + 1]] = ys
        if in_pool and len(ys):
            new_state[row] = wins[-1]
    return y, new_state


def conv1d_update(x, weight, bias, state_pool, state_idx, num_steps, silu=True):
    """Multi-step update: B rows of T tokens (token b*T + t) from pool windows (read only).
    Returns (y [B*T, C], intermediate [B, T, W-1, C]: the window after token t).  A row whose
    index lies outside the pool is padding: zero outputs and zero windows (the GPU leaves
    its windows unwritten)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    W = w.shape[1]
    T = int(num_steps)
    B = x.shape[0] // T
    C = x.shape[1]
    y = np.zeros_like(x)
    inter = np.zeros((B, T, W - 1, C))
    idx = np.asarray(state_idx).reshape(-1)
    for b in range(B):
        s = int(idx[b])
        if not 0 <= s < state_pool.shape[0]:
            continue
        ys, wins = _conv_run(x[b * T:(b + 1) * T], np.asarray(state_pool[s], np.float64), w, bias,
                             silu)
        y[b * T:(b + 1) * T] = ys
        inter[b] = wins
    return y, inter
