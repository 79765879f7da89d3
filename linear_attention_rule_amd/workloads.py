"""Seeded synthetic inputs shaped like the KDA workloads on the pages.

This module holds no arithmetic of the method: it only draws random numbers
and rounds them to bf16.  The same host bytes feed both the HIP library and
the CPU oracle.

Shapes follow vLLM PR #55737 ("Purpose": H=16 heads per rank, head_dim 128,
prefill at 2048x8, 8192x4 and 16384x1 tokens) and the verify block of the
sglang DFlash and TensorRT-LLM verify pages (8 draft tokens per row).
Distributions (q, k, v, g, beta logits ~ N(0, 1); A_log = log U(1, 16) per
head; dt_bias ~ N(0, 0.1) per key channel; states ~ N(0, 0.05)) are this
build's stand-ins: the pages name no input distribution.

Draw order is fixed: q, k, v, g, beta_logits, A_log, dt_bias, then the
initial states or the pool, then the state indices.  Values are drawn in
float32 with ``numpy.random.default_rng(seed)`` and rounded to bf16
(round-to-nearest-even) by torch on the CPU.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
LOWER_BOUND = -5.0


@dataclass
class PrefillCase:
    name: str
    seq_lens: list
    heads: int
    init: str | None = None        # None (zero), "per_seq", or "pool"
    pool_slots: int = 0
    seed: int = 1000
    lower_bound: float = LOWER_BOUND
    head_dim: int = HEAD_DIM


@dataclass
class VerifyCase:
    name: str
    batch: int
    steps: int
    heads: int
    pool_slots: int
    seed: int = 1004
    lower_bound: float = LOWER_BOUND
    head_dim: int = HEAD_DIM
    padding_rows: list = field(default_factory=list)


# The workload table.  Index = the seed offset (seed = 1000 + index).
TINY = PrefillCase("tiny_1x256_h2", [256], 2, init=None, seed=1000)
VARLEN = PrefillCase("varlen_8x2048_h16", [2048] * 8, 16, init="per_seq", seed=1001)
LONG = PrefillCase("long_4x8192_h16", [8192] * 4, 16, init=None, seed=1002)
SINGLE_LONG = PrefillCase("single_16384_h16_pool64", [16384], 16, init="pool",
                          pool_slots=64, seed=1003)
VERIFY = VerifyCase("verify_64x8_h16_pool256", 64, 8, 16, 256, seed=1004)
VERIFY_B1 = VerifyCase("verify_1x8_h16_pool256", 1, 8, 16, 256, seed=1005)

PREFILL_CASES = {c.name: c for c in (TINY, VARLEN, LONG, SINGLE_LONG)}
VERIFY_CASES = {c.name: c for c in (VERIFY, VERIFY_B1)}


@dataclass
class MixedCase:
    """One serving step carrying a prefill segment and speculative rows (MTP k draft
    tokens per row: steps = k + 1), merged into one layer output of R rows."""
    name: str
    prefill: PrefillCase
    spec: VerifyCase
    extra_rows: int = 0            # rows of the layer output no token names
    seed: int = 1006


# Prefill segment 8 x 2048 with 64 spec rows of MTP k = 1 (2 tokens each), 16 heads.
MIXED = MixedCase("mixed_8x2048_spec64x2_h16",
                  PrefillCase("mixed_prefill_8x2048_h16", [2048] * 8, 16, init=None, seed=1007),
                  VerifyCase("mixed_spec_64x2_h16_pool256", 64, 2, 16, 256, seed=1008))


def _bf16(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16)


def _gate_params(rng, heads, d):
    a_log = np.log(rng.uniform(1.0, 16.0, size=heads)).astype(np.float32)
    dt_bias = (rng.standard_normal(size=(heads, d), dtype=np.float32) * np.float32(0.1))
    return torch.from_numpy(a_log), torch.from_numpy(dt_bias)


def make_prefill(case: PrefillCase):
    """Draw one prefill workload.  Returns a dict of CPU tensors.

    q, k, v, g: bf16 [T, H, D]; beta_logits: bf16 [T, H]; A_log: f32 [H];
    dt_bias: f32 [H, D]; cu_seqlens: int32 [N+1]; initial_state: f32 or None;
    initial_state_idx: int32 [N] or None.
    """
    rng = np.random.default_rng(case.seed)
    lens = [int(x) for x in case.seq_lens]
    T = int(sum(lens))
    H, D = case.heads, case.head_dim
    q = _bf16(rng, (T, H, D))
    k = _bf16(rng, (T, H, D))
    v = _bf16(rng, (T, H, D))
    g = _bf16(rng, (T, H, D))
    beta_logits = _bf16(rng, (T, H))
    A_log, dt_bias = _gate_params(rng, H, D)
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.tensor(np.cumsum(lens), dtype=torch.int32)
    init = None
    init_idx = None
    if case.init == "per_seq":
        init = torch.from_numpy(
            rng.standard_normal(size=(len(lens), H, D, D), dtype=np.float32) * np.float32(0.05))
    elif case.init == "pool":
        init = torch.from_numpy(
            rng.standard_normal(size=(case.pool_slots, H, D, D), dtype=np.float32) * np.float32(0.05))
        init_idx = torch.from_numpy(
            rng.integers(0, case.pool_slots, size=len(lens)).astype(np.int32))
    return dict(q=q, k=k, v=v, g=g, beta_logits=beta_logits, A_log=A_log, dt_bias=dt_bias,
                cu_seqlens=cu, initial_state=init, initial_state_idx=init_idx,
                lower_bound=case.lower_bound, scale=1.0 / math.sqrt(D))


def make_verify(case: VerifyCase):
    """Draw one verify workload: B rows of `steps` tokens (token b*steps + t)."""
    rng = np.random.default_rng(case.seed)
    B, T, H, D = case.batch, case.steps, case.heads, case.head_dim
    q = _bf16(rng, (B * T, H, D))
    k = _bf16(rng, (B * T, H, D))
    v = _bf16(rng, (B * T, H, D))
    g = _bf16(rng, (B * T, H, D))
    beta_logits = _bf16(rng, (B * T, H))
    A_log, dt_bias = _gate_params(rng, H, D)
    pool = torch.from_numpy(
        rng.standard_normal(size=(case.pool_slots, H, D, D), dtype=np.float32) * np.float32(0.05))
    idx = rng.permutation(case.pool_slots)[:B].astype(np.int32)
    for b in case.padding_rows:
        idx[b] = -1
    return dict(q=q, k=k, v=v, g=g, beta_logits=beta_logits, A_log=A_log, dt_bias=dt_bias,
                state_pool=pool, state_idx=torch.from_numpy(idx), num_steps=T,
                lower_bound=case.lower_bound, scale=1.0 / math.sqrt(D))


@dataclass
class NormCase:
    name: str
    tokens: int
    heads: int
    eps: float = 1e-6
    seed: int = 1009
    head_dim: int = HEAD_DIM


# The gated output norm at the size of the 4 x 8192 prefill output (16 heads).
NORM = NormCase("gated_norm_32768x16", 32768, 16, seed=1009)


def make_norm(case: NormCase):
    """x, gate bf16 [T, H, D] ~ N(0, 1); weight f32 [D] ~ U(0.5, 1.5)."""
    rng = np.random.default_rng(case.seed)
    T, H, D = case.tokens, case.heads, case.head_dim
    x = _bf16(rng, (T, H, D))
    gate = _bf16(rng, (T, H, D))
    weight = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    return dict(x=x, gate=gate, weight=weight, eps=case.eps)


@dataclass
class ConvCase:
    name: str
    seq_lens: list                 # prefill: sequence lengths; update: ignored
    channels: int
    width: int = 4
    pool_slots: int = 0            # windows in the pool (0: no windows)
    batch: int = 0                 # update: B rows
    steps: int = 0                 # update: T tokens per row
    bias: bool = True
    seed: int = 1010


# Short conv on the packed q|k|v columns (3 x 16 heads x 128 channels) at the 4 x 8192
# prefill size, and its multi-step update at the 64 x 8 verify size.
CONV_PREFILL = ConvCase("conv_prefill_4x8192_c6144_w4", [8192] * 4, 3 * 16 * 128, 4,
                        pool_slots=4, seed=1010)
CONV_UPDATE = ConvCase("conv_update_64x8_c6144_w4_pool256", [], 3 * 16 * 128, 4,
                       pool_slots=256, batch=64, steps=8, seed=1011)


def make_conv(case: ConvCase):
    """x bf16 [T, C] ~ N(0, 1); weight bf16 [C, W] ~ N(0, 0.5^2); bias bf16 [C] ~ N(0, 0.1^2)
    (or None); windows bf16 [slots, W-1, C] ~ N(0, 1); window indices: a seeded
    permutation (prefill: one per sequence; update: one per row)."""
    rng = np.random.default_rng(case.seed)
    C, W = case.channels, case.width
    update = case.batch > 0
    T = case.batch * case.steps if update else int(sum(case.seq_lens))
    x = _bf16(rng, (T, C))
    weight = _bf16(rng, (C, W), std=0.5)
    bias = _bf16(rng, (C,), std=0.1) if case.bias else None
    state = _bf16(rng, (case.pool_slots, W - 1, C)) if case.pool_slots else None
    rows = case.batch if update else len(case.seq_lens)
    idx = None
    if case.pool_slots:
        perm = rng.permutation(max(case.pool_slots, rows))[:rows]
        idx = torch.from_numpy(perm.astype(np.int32))
    out = dict(x=x, weight=weight, bias=bias, state=state, state_idx=idx, width=W)
    if update:
        out["num_steps"] = case.steps
    else:
        lens = [int(v) for v in case.seq_lens]
        out["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return out


def make_mixed(case: MixedCase):
    """Draw one mixed step: the prefill and spec workloads, the token order of the merged
    layer output (non_spec_idx [T_prefill], spec_idx [B*T], int32, disjoint), the output
    row count, and the accepted-token counts num_accepted [B] in 1..T."""
    pre = make_prefill(case.prefill)
    spec = make_verify(case.spec)
    rng = np.random.default_rng(case.seed)
    Tp = int(pre["q"].shape[0])
    Ts = int(spec["q"].shape[0])
    rows = Tp + Ts + case.extra_rows
    order = rng.permutation(rows)[:Tp + Ts].astype(np.int32)
    nacc = rng.integers(1, case.spec.steps + 1, size=case.spec.batch).astype(np.int32)
    return dict(prefill=pre, spec=spec, out_rows=rows,
                non_spec_idx=torch.from_numpy(order[:Tp].copy()),
                spec_idx=torch.from_numpy(order[Tp:].copy()),
                num_accepted=torch.from_numpy(nacc))


def to_f64(t):
    """Widen a CPU tensor (bf16 / f32 / int) to a numpy array for the oracle."""
    if t is None:
        return None
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.to(torch.float64).numpy()
