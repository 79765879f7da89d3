"""ctypes binding for libkda: argument marshalling only.

Every step of the KDA path runs in the library's HIP kernels; this module
checks torch dtypes/devices/shapes, turns tensors into pointers and strides,
passes torch's current HIP stream, and raises on a non-OK status.  torch is
used only for device memory and streams.  There is no CPU fallback: if the
library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "kda.h")
HEAD_DIM = 128
# Magnitude bound on v and the prefill state (fp16 MFMA operands in the scan).
FP16_RANGE_LIMIT = 2.0 ** 14

KDA_OK = 0
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
                3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}


class PrefillDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("num_state_rows", ctypes.c_int32),
                ("q_token_stride", ctypes.c_int64), ("k_token_stride", ctypes.c_int64),
                ("v_token_stride", ctypes.c_int64), ("g_token_stride", ctypes.c_int64),
                ("beta_token_stride", ctypes.c_int64), ("out_token_stride", ctypes.c_int64),
                ("out_token_index", ctypes.c_void_p), ("out_rows", ctypes.c_int64)]


class VerifyDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_steps", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("num_slots", ctypes.c_int32),
                ("q_token_stride", ctypes.c_int64), ("k_token_stride", ctypes.c_int64),
                ("v_token_stride", ctypes.c_int64), ("g_token_stride", ctypes.c_int64),
                ("beta_token_stride", ctypes.c_int64), ("out_token_stride", ctypes.c_int64),
                ("out_token_index", ctypes.c_void_p), ("out_rows", ctypes.c_int64)]


class OutputNorm(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("gate_token_stride", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("eps", ctypes.c_float), ("rstd", ctypes.c_void_p)]


class CommitDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_steps", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_slots", ctypes.c_int32)]


class NormDesc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("eps", ctypes.c_float),
                ("x_token_stride", ctypes.c_int64), ("gate_token_stride", ctypes.c_int64),
                ("y_token_stride", ctypes.c_int64)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("num_steps", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("num_state_slots", ctypes.c_int32),
                ("silu", ctypes.c_int32), ("x_token_stride", ctypes.c_int64),
                ("y_token_stride", ctypes.c_int64)]


ABI_VERSION = 2
_lib = None


class KDAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: str | None = None):
    """Load libkda.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libkda is not built ({path} missing); run "
                           "`python -m linear_attention_rule_amd.build` first")
    lib = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_chunk_prefill_workspace_size.restype = sz
    lib.kda_chunk_prefill_workspace_size.argtypes = [i32, i32, i32, i32]
    for name in ("kda_chunk_prefill", "kda_chunk_prefill_intra", "kda_chunk_prefill_scan"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, sz,
                       ctypes.POINTER(PrefillDesc), vp]
    lib.kda_chunk_prefill_noalloc.restype = ctypes.c_int
    lib.kda_chunk_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                              ctypes.POINTER(PrefillDesc), vp]
    lib.kda_recurrent_verify.restype = ctypes.c_int
    lib.kda_recurrent_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                                         ctypes.POINTER(VerifyDesc), vp]
    lib.kda_recurrent_verify_gated.restype = ctypes.c_int
    lib.kda_recurrent_verify_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                                               ctypes.POINTER(OutputNorm),
                                               ctypes.POINTER(VerifyDesc), vp]
    lib.kda_commit_accepted.restype = ctypes.c_int
    lib.kda_commit_accepted.argtypes = [vp, vp, vp, vp, ctypes.POINTER(CommitDesc), vp]
    lib.kda_causal_conv1d_prefill.restype = ctypes.c_int
    lib.kda_causal_conv1d_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.POINTER(ConvDesc), vp]
    lib.kda_causal_conv1d_update.restype = ctypes.c_int
    lib.kda_causal_conv1d_update.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.POINTER(ConvDesc), vp]
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(NormDesc), vp]
    if lib.kda_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libkda ABI version {lib.kda_abi_version()}, binding expects "
                           f"{ABI_VERSION}")
    _lib = lib
    return lib


def header_entry_points() -> list[str]:
    """Names of the functions include/kda.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def _ptr(t):
    # an int: the argtypes (and the descriptors' pointer fields) are c_void_p
    return None if t is None else t.data_ptr()


# torch's current HIP stream of a device as a raw handle; the private accessor skips
# building a Stream object (a few microseconds per call on the latency-bound verify).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device):
    if _raw_stream is not None:
        index = device.index if device.index is not None else torch.cuda.current_device()
        return _raw_stream(index)
    return torch.cuda.current_stream(device).cuda_stream


def _check(status):
    if status != KDA_OK:
        raise KDAError(status, _lib.kda_last_error().decode())


def _token_tensor(name, t, heads, width):
    """A [tokens, heads, width] (or [tokens, heads] when width is None) view with dense heads."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    shape = t.shape
    if width is None:
        if len(shape) != 2 or shape[1] != heads:
            raise ValueError(f"{name} must be [tokens, {heads}]")
        if t.numel() == 0:
            return 0
        st = t.stride()
        if st[1] != 1:
            raise ValueError(f"{name} must have contiguous heads")
    else:
        if len(shape) != 3 or shape[1] != heads or shape[2] != width:
            raise ValueError(f"{name} must be [tokens, {heads}, {width}]")
        if t.numel() == 0:
            return 0
        st = t.stride()
        if st[2] != 1 or st[1] != width:
            raise ValueError(f"{name} must have dense heads")
    return st[0]


def _f32(name, t, shape):
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _i32(name, t, n):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
        raise TypeError(f"{name} must be a contiguous 1-D int32 device tensor")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} entries")


def prefill_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int) -> int:
    lib = load_library()
    return int(lib.kda_chunk_prefill_workspace_size(num_seqs, total_tokens, num_heads, HEAD_DIM))


def _out_index(out, out_token_index, tokens, H):
    """Validates out against an optional scatter index; returns (token stride, rows, ptr)."""
    os_ = _token_tensor("out", out, H, HEAD_DIM)
    if out_token_index is None:
        if out.shape[0] != tokens:
            raise ValueError(f"out must have {tokens} tokens")
        return os_, 0, None
    _i32("out_token_index", out_token_index, tokens)
    return os_, int(out.shape[0]), _ptr(out_token_index)


def noalloc_scratch_bytes() -> int:
    """Size of the fixed per-device scratch behind chunk_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES)."""
    with open(HEADER_PATH) as f:
        m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \((\d+)ll \* 1024 \* 1024\)", f.read())
    return int(m.group(1)) << 20


def chunk_prefill(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens, *,
                  initial_state=None, initial_state_idx=None, out=None, final_state=None,
                  write_final_state=True, scale=None, workspace=None, check=False,
                  phase="both", out_token_index=None):
    """Varlen chunked KDA prefill.  Returns (out, final_state or None).

    phase: "both" (kda_chunk_prefill), "intra" / "scan" for the two halves of the
    same call (kda_chunk_prefill_intra / kda_chunk_prefill_scan), which must then be
    given the same workspace, or "noalloc" (kda_chunk_prefill_noalloc: no workspace,
    the library's fixed per-device scratch instead).

    out_token_index: optional int32 [T] on the device; token t's output goes to row
    out_token_index[t] of `out` (which must then be given: the layer buffer), rows
    outside [0, out.shape[0]) are not written.

    q, k, v, g: bf16 [T, H, 128] (token stride free, heads dense); beta_logits bf16 [T, H];
    A_log f32 [H]; dt_bias f32 [H, 128]; cu_seqlens int32 [N+1] on the device.
    N comes from cu_seqlens.numel() and T from q.shape[0]: both host values.
    """
    lib = load_library()
    T, H = int(q.shape[0]), int(q.shape[1])
    N = int(cu_seqlens.numel()) - 1
    qs = _token_tensor("q", q, H, HEAD_DIM)
    ks = _token_tensor("k", k, H, HEAD_DIM)
    vs = _token_tensor("v", v, H, HEAD_DIM)
    gs = _token_tensor("g", g, H, HEAD_DIM)
    bs = _token_tensor("beta_logits", beta_logits, H, None)
    for name, t in (("k", k), ("v", v), ("g", g), ("beta_logits", beta_logits)):
        if t.shape[0] != T:
            raise ValueError(f"{name} has {t.shape[0]} tokens, q has {T}")
    _f32("A_log", A_log, (H,))
    _f32("dt_bias", dt_bias, (H, HEAD_DIM))
    _i32("cu_seqlens", cu_seqlens, None)
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    dev = q.device
    rows = 0
    if initial_state is not None:
        if initial_state.dim() != 4:
            raise ValueError("initial_state must be [rows, H, 128, 128]")
        rows = int(initial_state.shape[0])
        _f32("initial_state", initial_state, (rows, H, HEAD_DIM, HEAD_DIM))
    if initial_state_idx is not None:
        _i32("initial_state_idx", initial_state_idx, N)
    if out is None:
        if out_token_index is not None:
            raise ValueError("out_token_index needs the destination buffer `out`")
        out = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    os_, out_rows, oidx = _out_index(out, out_token_index, T, H)
    if final_state is None and write_final_state:
        final_state = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    if final_state is not None:
        _f32("final_state", final_state, (N, H, HEAD_DIM, HEAD_DIM))
    if phase not in ("both", "intra", "scan", "noalloc"):
        raise ValueError(f"unknown phase {phase!r}")
    need = int(lib.kda_chunk_prefill_workspace_size(N, T, H, HEAD_DIM))
    if phase == "noalloc":
        if workspace is not None:
            raise ValueError("phase='noalloc' takes no workspace")
    elif workspace is None:
        if phase != "both":
            # The scan reads the records the intra phase left in this same buffer.
            raise ValueError(f"phase={phase!r} needs the workspace shared by both phases")
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if check:
        cu = cu_seqlens.cpu()
        if int(cu[0]) != 0 or int(cu[-1]) != T or bool((cu[1:] < cu[:-1]).any()):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
        # The scan's fp16 MFMA operands hold v, the state and values a small multiple of
        # them: inputs at or past 2^14 may overflow fp16 (FP16_RANGE_LIMIT in kda.h).
        if T > 0 and not bool((v.abs() < FP16_RANGE_LIMIT).all()):
            raise ValueError(f"|v| must stay below {FP16_RANGE_LIMIT:g} (fp16 scan operands)")
        if initial_state is not None and initial_state.numel() and \
                not bool((initial_state.abs() < FP16_RANGE_LIMIT).all()):
            raise ValueError(f"|initial_state| must stay below {FP16_RANGE_LIMIT:g} "
                             "(fp16 scan operands)")
    desc = PrefillDesc(N, T, H, HEAD_DIM, float(scale) if scale else 0.0, rows,
                       qs, ks, vs, gs, bs, os_, oidx, out_rows)
    if phase == "noalloc":
        st = lib.kda_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta_logits),
                                           _ptr(A_log), _ptr(dt_bias), float(lower_bound),
                                           _ptr(cu_seqlens), _ptr(initial_state),
                                           _ptr(initial_state_idx), _ptr(out), _ptr(final_state),
                                           ctypes.byref(desc), _stream_handle(dev))
    else:
        fn = {"both": lib.kda_chunk_prefill, "intra": lib.kda_chunk_prefill_intra,
              "scan": lib.kda_chunk_prefill_scan}[phase]
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta_logits), _ptr(A_log),
                _ptr(dt_bias), float(lower_bound), _ptr(cu_seqlens), _ptr(initial_state),
                _ptr(initial_state_idx), _ptr(out), _ptr(final_state), _ptr(workspace),
                workspace.numel() * workspace.element_size(), ctypes.byref(desc),
                _stream_handle(dev))
    _check(st)
    return out, final_state


def chunk_prefill_noalloc(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                          **kw):
    """kda_chunk_prefill_noalloc: chunk_prefill with the library's fixed per-device scratch
    in place of a workspace (no device allocation in the call itself, given `out` and
    `final_state`).  Same arguments as chunk_prefill, without workspace and phase."""
    return chunk_prefill(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                         phase="noalloc", **kw)


def recurrent_verify(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, state_pool, state_idx,
                     num_steps, *, intermediate=None, out=None, scale=None, out_token_index=None):
    """Fused multi-step verify.  Returns (out [B*T, H, 128] bf16, intermediate [B, T, H, 128, 128] f32).

    out_token_index: as in chunk_prefill, for token b*T + t.
    """
    lib = load_library()
    BT, H = int(q.shape[0]), int(q.shape[1])
    T = int(num_steps)
    if T < 1 or BT % T:
        raise ValueError("token count must be a multiple of num_steps")
    B = BT // T
    qs = _token_tensor("q", q, H, HEAD_DIM)
    ks = _token_tensor("k", k, H, HEAD_DIM)
    vs = _token_tensor("v", v, H, HEAD_DIM)
    gs = _token_tensor("g", g, H, HEAD_DIM)
    bs = _token_tensor("beta_logits", beta_logits, H, None)
    _f32("A_log", A_log, (H,))
    _f32("dt_bias", dt_bias, (H, HEAD_DIM))
    slots = int(state_pool.shape[0])
    _f32("state_pool", state_pool, (slots, H, HEAD_DIM, HEAD_DIM))
    _i32("state_idx", state_idx, B)
    dev = q.device
    if out is None:
        if out_token_index is not None:
            raise ValueError("out_token_index needs the destination buffer `out`")
        out = torch.empty((BT, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    os_, out_rows, oidx = _out_index(out, out_token_index, BT, H)
    if intermediate is None:
        intermediate = torch.empty((B, T, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    _f32("intermediate", intermediate, (B, T, H, HEAD_DIM, HEAD_DIM))
    desc = VerifyDesc(B, T, H, HEAD_DIM, float(scale) if scale else 0.0, slots,
                      qs, ks, vs, gs, bs, os_, oidx, out_rows)
    st = lib.kda_recurrent_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta_logits),
                                  _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(state_pool),
                                  _ptr(state_idx), _ptr(intermediate), _ptr(out),
                                  ctypes.byref(desc), _stream_handle(dev))
    _check(st)
    return out, intermediate


def recurrent_verify_gated(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, state_pool,
                           state_idx, num_steps, out_gate, norm_weight, norm_eps, *,
                           intermediate=None, out=None, rstd=None, want_rstd=True, scale=None,
                           out_token_index=None):
    """Fused multi-step verify with the output-gate sigmoid RMSNorm applied to each output
    row before it is stored (kda_recurrent_verify_gated).  Returns (y [B*T or rows, H, 128]
    bf16, intermediate, rstd [rows, H] f32 or None).

    out_gate: bf16 [rows, H, 128] (token stride free, heads dense), one row per output row
    (rows = B*T, or out.shape[0] with out_token_index); norm_weight: f32 [128].
    """
    lib = load_library()
    BT, H = int(q.shape[0]), int(q.shape[1])
    T = int(num_steps)
    if T < 1 or BT % T:
        raise ValueError("token count must be a multiple of num_steps")
    B = BT // T
    qs = _token_tensor("q", q, H, HEAD_DIM)
    ks = _token_tensor("k", k, H, HEAD_DIM)
    vs = _token_tensor("v", v, H, HEAD_DIM)
    gs = _token_tensor("g", g, H, HEAD_DIM)
    bs = _token_tensor("beta_logits", beta_logits, H, None)
    _f32("A_log", A_log, (H,))
    _f32("dt_bias", dt_bias, (H, HEAD_DIM))
    slots = int(state_pool.shape[0])
    _f32("state_pool", state_pool, (slots, H, HEAD_DIM, HEAD_DIM))
    _i32("state_idx", state_idx, B)
    _f32("norm_weight", norm_weight, (HEAD_DIM,))
    dev = q.device
    if out is None:
        if out_token_index is not None:
            raise ValueError("out_token_index needs the destination buffer `out`")
        out = torch.empty((BT, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    os_, out_rows, oidx = _out_index(out, out_token_index, BT, H)
    rows = int(out.shape[0])
    ogs = _token_tensor("out_gate", out_gate, H, HEAD_DIM)
    if out_gate.shape[0] != rows:
        raise ValueError(f"out_gate must have {rows} rows (one per output row)")
    if intermediate is None:
        intermediate = torch.empty((B, T, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    _f32("intermediate", intermediate, (B, T, H, HEAD_DIM, HEAD_DIM))
    if rstd is None and want_rstd:
        rstd = torch.empty((rows, H), dtype=torch.float32, device=dev)
    if rstd is not None:
        _f32("rstd", rstd, (rows, H))
    norm = OutputNorm(_ptr(out_gate), ogs, _ptr(norm_weight), float(norm_eps), _ptr(rstd))
    desc = VerifyDesc(B, T, H, HEAD_DIM, float(scale) if scale else 0.0, slots,
                      qs, ks, vs, gs, bs, os_, oidx, out_rows)
    st = lib.kda_recurrent_verify_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta_logits),
                                        _ptr(A_log), _ptr(dt_bias), float(lower_bound),
                                        _ptr(state_pool), _ptr(state_idx), _ptr(intermediate),
                                        _ptr(out), ctypes.byref(norm), ctypes.byref(desc),
                                        _stream_handle(dev))
    _check(st)
    return out, intermediate, rstd


def commit_accepted(intermediate, state_idx, num_accepted, state_pool):
    """Rollback commit after verify: state_pool[state_idx[b]] <- intermediate[b, num_accepted[b]-1]
    for rows with an in-range slot and 1 <= num_accepted[b] <= T.  Updates state_pool in place
    and returns it."""
    lib = load_library()
    if intermediate.dim() != 5:
        raise ValueError("intermediate must be [B, T, H, 128, 128]")
    B, T, H = (int(x) for x in intermediate.shape[:3])
    _f32("intermediate", intermediate, (B, T, H, HEAD_DIM, HEAD_DIM))
    slots = int(state_pool.shape[0])
    _f32("state_pool", state_pool, (slots, H, HEAD_DIM, HEAD_DIM))
    _i32("state_idx", state_idx, B)
    _i32("num_accepted", num_accepted, B)
    desc = CommitDesc(B, T, H, HEAD_DIM, slots)
    st = lib.kda_commit_accepted(_ptr(intermediate), _ptr(state_idx), _ptr(num_accepted),
                                 _ptr(state_pool), ctypes.byref(desc),
                                 _stream_handle(intermediate.device))
    _check(st)
    return state_pool


def gated_rmsnorm(x, gate, weight, eps, *, out=None, rstd=None, want_rstd=True):
    """Output-gate sigmoid RMSNorm over rows of 128 channels.  Returns (y, rstd or None).

    x, gate: bf16 [T, H, 128] (token stride free, heads dense); weight: f32 [128].
    out may be x itself (in place).
    """
    lib = load_library()
    T, H = int(x.shape[0]), int(x.shape[1])
    xs = _token_tensor("x", x, H, HEAD_DIM)
    gs = _token_tensor("gate", gate, H, HEAD_DIM)
    if gate.shape[0] != T:
        raise ValueError("gate must have as many tokens as x")
    _f32("weight", weight, (HEAD_DIM,))
    dev = x.device
    if out is None:
        out = torch.empty((T, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    ys = _token_tensor("out", out, H, HEAD_DIM)
    if out.shape[0] != T:
        raise ValueError("out must have as many tokens as x")
    if rstd is None and want_rstd:
        rstd = torch.empty((T, H), dtype=torch.float32, device=dev)
    if rstd is not None:
        _f32("rstd", rstd, (T, H))
    desc = NormDesc(T, H, HEAD_DIM, float(eps), xs, gs, ys)
    st = lib.kda_gated_rmsnorm(_ptr(x), _ptr(gate), _ptr(weight), _ptr(out), _ptr(rstd),
                               ctypes.byref(desc), _stream_handle(dev))
    _check(st)
    return out, rstd


def _rows_tensor(name, t, width):
    """A bf16 [tokens, width] view with contiguous channels; returns its token stride."""
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 device tensor")
    if t.dim() != 2 or t.shape[1] != width:
        raise ValueError(f"{name} must be [tokens, {width}]")
    if t.numel() == 0:
        return 0
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous channels")
    return t.stride(0)


def _conv_weights(weight, bias, C):
    if weight.dtype != torch.bfloat16 or not weight.is_cuda or not weight.is_contiguous() \
            or weight.dim() != 2 or weight.shape[0] != C:
        raise TypeError(f"weight must be a contiguous bf16 device tensor [{C}, W]")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_cuda or
                             not bias.is_contiguous() or tuple(bias.shape) != (C,)):
        raise TypeError(f"bias must be a contiguous bf16 device tensor [{C}]")
    return int(weight.shape[1])


def _windows(name, t, W, C, rows=None):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous bf16 device tensor")
    if t.shape[-2:] != (W - 1, C) or (rows is not None and t.shape[0] != rows):
        raise ValueError(f"{name} must be [{rows or 'slots'}, {W - 1}, {C}]")


def causal_conv1d_prefill(x, weight, bias, cu_seqlens, *, conv_state=None, state_idx=None,
                          out=None, silu=True):
    """Short causal conv over N packed sequences.  Returns y [T, C] (bf16).

    x: bf16 [T, C] (token stride free); weight bf16 [C, W]; bias bf16 [C] or None;
    conv_state: bf16 [slots, W-1, C] windows, updated in place; state_idx int32 [N] or None.
    """
    lib = load_library()
    T, C = int(x.shape[0]), int(x.shape[1])
    xs = _rows_tensor("x", x, C)
    W = _conv_weights(weight, bias, C)
    _i32("cu_seqlens", cu_seqlens, None)
    N = int(cu_seqlens.numel()) - 1
    slots = 0
    if conv_state is not None:
        _windows("conv_state", conv_state, W, C)
        slots = int(conv_state.shape[0])
    if state_idx is not None:
        _i32("state_idx", state_idx, N)
    if out is None:
        out = torch.empty((T, C), dtype=torch.bfloat16, device=x.device)
    ys = _rows_tensor("out", out, C)
    desc = ConvDesc(N, T, 0, C, W, slots, 1 if silu else 0, xs, ys)
    st = lib.kda_causal_conv1d_prefill(_ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens),
                                       _ptr(conv_state), _ptr(state_idx), _ptr(out),
                                       ctypes.byref(desc), _stream_handle(x.device))
    _check(st)
    return out


def causal_conv1d_update(x, weight, bias, conv_state, state_idx, num_steps, *,
                         intermediate=None, out=None, silu=True):
    """Multi-step conv update for verify.  Returns (y [B*T, C], intermediate [B, T, W-1, C]).

    The pool conv_state [slots, W-1, C] is only read; state_idx int32 [B] (out of range =
    padding row)."""
    lib = load_library()
    BT, C = int(x.shape[0]), int(x.shape[1])
    T = int(num_steps)
    if T < 1 or BT % T:
        raise ValueError("token count must be a multiple of num_steps")
    B = BT // T
    xs = _rows_tensor("x", x, C)
    W = _conv_weights(weight, bias, C)
    _windows("conv_state", conv_state, W, C)
    _i32("state_idx", state_idx, B)
    if intermediate is None:
        intermediate = torch.empty((B, T, W - 1, C), dtype=torch.bfloat16, device=x.device)
    _windows("intermediate", intermediate.view(B * T, W - 1, C), W, C, B * T)
    if out is None:
        out = torch.empty((BT, C), dtype=torch.bfloat16, device=x.device)
    ys = _rows_tensor("out", out, C)
    desc = ConvDesc(B, BT, T, C, W, int(conv_state.shape[0]), 1 if silu else 0, xs, ys)
    st = lib.kda_causal_conv1d_update(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
                                      _ptr(state_idx), _ptr(intermediate), _ptr(out),
                                      ctypes.byref(desc), _stream_handle(x.device))
    _check(st)
    return out, intermediate


def default_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)
