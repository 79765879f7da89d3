"""Host-only checks of libkda: it loads, exports what include/kda.h declares,
and its host-side validation rejects bad arguments before touching a GPU.

No compute call is made here (no GPU in this process); every call below
returns from argument validation.
"""

import ctypes

import pytest

import linear_attention_rule_amd as L
from linear_attention_rule_amd import _binding as B

KDA_OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def test_exports_every_declared_symbol(lib):
    names = L.header_entry_points()
    assert set(names) >= {"kda_chunk_prefill", "kda_recurrent_verify", "kda_last_error",
                          "kda_abi_version", "kda_chunk_prefill_workspace_size",
                          "kda_commit_accepted", "kda_gated_rmsnorm",
                          "kda_causal_conv1d_prefill", "kda_causal_conv1d_update"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_workspace_size(lib):
    assert lib.kda_abi_version() == 2 == B.ABI_VERSION
    rec = 61 * 1024
    # chunk slots = floor(T/64) + N
    assert lib.kda_chunk_prefill_workspace_size(4, 32768, 16, 128) == (512 + 4) * 16 * rec
    # few (sequence, head) pairs: room for the segment-parallel scan's states as well
    seg = 19 * 128 * 128 * 4
    assert lib.kda_chunk_prefill_workspace_size(1, 100, 2, 128) == (1 + 1) * 2 * rec + 2 * seg
    assert lib.kda_chunk_prefill_workspace_size(2, 640, 16, 128) == (10 + 2) * 16 * rec + 32 * seg
    assert lib.kda_chunk_prefill_workspace_size(3, 640, 16, 128) == (10 + 3) * 16 * rec
    assert lib.kda_chunk_prefill_workspace_size(1, 100, 2, 64) == 0
    assert lib.kda_chunk_prefill_workspace_size(0, 0, 1, 128) == 0


def _fake(n=1):
    # Non-null, 16-byte-aligned host addresses.  Validation never dereferences
    # them; every case below fails before a launch.
    return ctypes.c_void_p(0x10000 * n)


def _prefill(lib, desc, lb=-5.0, ws_bytes=1 << 40, null_q=False, null_desc=False):
    f = _fake
    return lib.kda_chunk_prefill(None if null_q else f(1), f(2), f(3), f(4), f(5), f(6), f(7), lb,
                                 f(8), None, None, f(9), f(10), f(11), ws_bytes,
                                 None if null_desc else ctypes.byref(desc), None)


def _pdesc(N=1, T=64, H=2, D=128):
    return B.PrefillDesc(N, T, H, D, 0.0, 0, 0, 0, 0, 0, 0, 0)


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, _pdesc(), null_desc=True) == INVALID
    assert _prefill(lib, _pdesc(D=64)) == UNSUPPORTED
    assert b"head_dim" in lib.kda_last_error()
    assert _prefill(lib, _pdesc(), lb=-6.0) == UNSUPPORTED
    assert _prefill(lib, _pdesc(), lb=0.5) == UNSUPPORTED
    assert _prefill(lib, _pdesc(), lb=float("nan")) == UNSUPPORTED
    assert _prefill(lib, _pdesc(), null_q=True) == INVALID
    assert _prefill(lib, _pdesc(H=0)) == INVALID
    assert _prefill(lib, _pdesc(), ws_bytes=100) == WS_SMALL
    assert b"workspace" in lib.kda_last_error()
    d = _pdesc()
    d.q_token_stride = 100          # < H*128
    assert _prefill(lib, d) == INVALID
    d = _pdesc()
    d.q_token_stride = 260          # >= H*128 but not a multiple of 8
    assert _prefill(lib, d) == INVALID


def test_prefill_rejects_out_overlapping_input(lib):
    d = _pdesc(T=64, H=2)
    f = _fake
    st = lib.kda_chunk_prefill(f(1), f(2), f(3), f(4), f(5), f(6), f(7), -5.0, f(8), None, None,
                               f(1), f(10), f(11), 1 << 40, ctypes.byref(d), None)
    assert st == INVALID and b"overlap" in lib.kda_last_error()


def _vdesc(Bn=2, T=8, H=2, D=128, slots=4):
    return B.VerifyDesc(Bn, T, H, D, 0.0, slots, 0, 0, 0, 0, 0, 0)


def _verify(lib, desc, lb=-5.0, inter=None):
    f = _fake
    return lib.kda_recurrent_verify(f(1), f(2), f(3), f(4), f(5), f(6), f(7), lb, f(20), f(9),
                                    inter if inter is not None else f(40), f(50),
                                    ctypes.byref(desc), None)


def test_verify_rejects_bad_arguments(lib):
    assert _verify(lib, _vdesc(D=96)) == UNSUPPORTED
    assert _verify(lib, _vdesc(T=0)) == UNSUPPORTED
    assert _verify(lib, _vdesc(T=65)) == UNSUPPORTED
    assert _verify(lib, _vdesc(Bn=(1 << 26), T=64)) == UNSUPPORTED   # 2^32 tokens
    assert b"exceeds" in lib.kda_last_error()
    assert _verify(lib, _vdesc(slots=0)) == INVALID
    assert _verify(lib, _vdesc(), lb=-7.0) == UNSUPPORTED
    # intermediate overlapping the pool
    assert _verify(lib, _vdesc(), inter=_fake(20)) == INVALID
    assert b"overlap" in lib.kda_last_error()


def test_zero_sized_calls_are_ok_without_launch(lib):
    # N = 0 prefill and B = 0 verify enqueue nothing and succeed.
    assert _prefill(lib, _pdesc(N=0, T=0), ws_bytes=0) == KDA_OK
    assert _verify(lib, _vdesc(Bn=0)) == KDA_OK
    assert lib.kda_last_error() == b""


def test_scatter_index_validation(lib):
    # out_rows < 0 with an index
    d = _pdesc(T=64, H=2)
    d.out_token_index = 0x120000
    d.out_rows = -1
    assert _prefill(lib, d) == INVALID and b"out_rows" in lib.kda_last_error()
    # misaligned index
    d.out_rows = 10
    d.out_token_index = 0x120002
    assert _prefill(lib, d) == INVALID and b"aligned" in lib.kda_last_error()
    # the index inside the output rows (out = fake(9), 10 rows of 256 bf16)
    d.out_token_index = 0x90000 + 64
    assert _prefill(lib, d) == INVALID and b"out_token_index" in lib.kda_last_error()
    v = _vdesc()
    v.out_token_index = 0x320000 + 16   # out = fake(50)
    v.out_rows = 4
    assert _verify(lib, v) == INVALID and b"out_token_index" in lib.kda_last_error()


def _cdesc(Bn=2, T=8, H=2, D=128, slots=4):
    return B.CommitDesc(Bn, T, H, D, slots)


def _commit(lib, desc, inter=None, pool=None, null_idx=False):
    f = _fake
    return lib.kda_commit_accepted(inter if inter is not None else f(40), None if null_idx else f(7),
                                   f(8), pool if pool is not None else f(20), ctypes.byref(desc),
                                   None)


def test_commit_rejects_bad_arguments(lib):
    assert _commit(lib, _cdesc(D=64)) == UNSUPPORTED
    assert _commit(lib, _cdesc(T=0)) == INVALID
    assert _commit(lib, _cdesc(slots=0)) == INVALID
    assert _commit(lib, _cdesc(H=0)) == INVALID
    assert _commit(lib, _cdesc(), null_idx=True) == INVALID
    assert _commit(lib, _cdesc(), inter=_fake(20)) == INVALID
    assert b"overlap" in lib.kda_last_error()
    assert lib.kda_commit_accepted(_fake(40), _fake(7), _fake(8), _fake(20), None, None) == INVALID
    assert _commit(lib, _cdesc(Bn=0)) == KDA_OK


def _ndesc(T=4, H=2, D=128, eps=1e-6):
    return B.NormDesc(T, H, D, eps, 0, 0, 0)


def _norm(lib, desc, x=None, gate=None, y=None):
    f = _fake
    return lib.kda_gated_rmsnorm(x if x is not None else f(1), gate if gate is not None else f(2),
                                 f(3), y if y is not None else f(4), None, ctypes.byref(desc), None)


def test_norm_rejects_bad_arguments(lib):
    assert _norm(lib, _ndesc(D=64)) == UNSUPPORTED
    assert _norm(lib, _ndesc(eps=-1.0)) == INVALID
    assert _norm(lib, _ndesc(eps=float("inf"))) == INVALID
    assert _norm(lib, _ndesc(H=0)) == INVALID
    assert _norm(lib, _ndesc(), y=_fake(2)) == INVALID          # y over gate
    assert b"gate" in lib.kda_last_error()
    d = _ndesc()
    d.y_token_stride = 512                                     # y == x but another stride
    assert _norm(lib, d, y=_fake(1)) == INVALID
    assert _norm(lib, _ndesc(T=0)) == KDA_OK


def test_norm_launch_size_limit(lib):
    # One short-lived workgroup per 32 rows: more than 2^24 - 1 workgroups is refused.
    far = lambda k: ctypes.c_void_p(k << 44)
    over = _ndesc(T=2**31 - 1, H=1)
    assert _norm(lib, over, x=far(1), gate=far(2), y=far(3)) == UNSUPPORTED
    assert b"workgroups" in lib.kda_last_error()
    at = _ndesc(T=32 * (2**24 - 1) // 16, H=16)              # exactly 2^24 - 1 workgroups
    assert _norm(lib, at, x=far(1), gate=far(2), y=far(3)) not in (INVALID, UNSUPPORTED)


def test_norm_accepts_interleaved_views(lib):
    # x and gate interleaved rows of one fused buffer (stride 3*H*128), y in place over x:
    # validation passes (without a GPU the call then fails at the launch).
    d = _ndesc(T=4, H=2)
    d.x_token_stride = d.gate_token_stride = d.y_token_stride = 3 * 2 * 128
    st = _norm(lib, d, x=_fake(1), gate=ctypes.c_void_p(0x10000 + 2 * 128 * 2), y=_fake(1))
    assert st not in (INVALID, UNSUPPORTED), lib.kda_last_error()
    # gate one row later than x (same stride) still overlaps
    d2 = _ndesc(T=4, H=2)
    d2.x_token_stride = d2.gate_token_stride = d2.y_token_stride = 2 * 2 * 128
    st = _norm(lib, d2, x=_fake(1), gate=ctypes.c_void_p(0x10000 + 100), y=_fake(1))
    assert st == INVALID


def _cvdesc(N=2, T=16, steps=0, C=64, W=4, slots=4, silu=1):
    return B.ConvDesc(N, T, steps, C, W, slots, silu, 0, 0)


def test_conv_rejects_bad_arguments(lib):
    f = _fake
    pre = lambda d, y=None: lib.kda_causal_conv1d_prefill(f(1), f(2), None, f(3), f(4), None,
                                                          y if y is not None else f(8),
                                                          ctypes.byref(d), None)
    upd = lambda d, inter=None: lib.kda_causal_conv1d_update(f(1), f(2), None, f(4), f(5),
                                                             inter if inter is not None else f(9),
                                                             f(12), ctypes.byref(d), None)
    assert pre(_cvdesc(W=5)) == UNSUPPORTED
    assert pre(_cvdesc(C=12)) == INVALID                  # not a multiple of 8
    assert pre(_cvdesc(slots=1)) == INVALID               # fewer windows than sequences
    assert pre(_cvdesc(), y=f(1)) == INVALID and b"overlap" in lib.kda_last_error()
    assert upd(_cvdesc(N=2, T=16, steps=8)) not in (INVALID, UNSUPPORTED)   # passes checks
    assert upd(_cvdesc(N=2, T=15, steps=8)) == INVALID    # total != B * T
    assert upd(_cvdesc(N=2, T=16, steps=8), inter=f(4)) == INVALID   # windows overlap the pool
    assert pre(_cvdesc(N=0, T=0)) == KDA_OK


def test_conv_prefill_launch_size_limit(lib):
    # One workgroup per (16-token row slot, 2048-channel block) in a 1-D grid: more than
    # 2^24 - 1 workgroups is refused on the host.  x and y sit far apart so that only the
    # size check can object.
    def pre(T, C):
        d = _cvdesc(N=1, T=T, C=C, slots=0)
        return lib.kda_causal_conv1d_prefill(ctypes.c_void_p(1 << 46), _fake(2), None, _fake(3),
                                             None, None, ctypes.c_void_p(1 << 47),
                                             ctypes.byref(d), None)
    assert pre(2**31 - 1, 6144) == UNSUPPORTED and b"workgroups" in lib.kda_last_error()
    limit_T = 16 * ((2**24 - 1) // 3 - 1)                  # (T/16 + 1) * 3 <= 2^24 - 1
    assert pre(limit_T, 6144) not in (INVALID, UNSUPPORTED)
    assert pre(limit_T + 16 * 2, 6144) == UNSUPPORTED


def test_noalloc_prefill_rejects_shapes_beyond_its_scratch(lib):
    f = _fake
    limit = B.noalloc_scratch_bytes()
    assert limit == 128 << 20

    def call(desc):
        # fake buffers 2^32 bytes apart, so no two of them overlap at these sizes
        g = lambda n: ctypes.c_void_p(n << 32)
        return lib.kda_chunk_prefill_noalloc(g(1), g(2), g(3), g(4), g(5), g(6), g(7), -5.0, g(8),
                                             None, None, g(9), g(10), ctypes.byref(desc), None)

    # 4 x 8192 tokens at 16 heads: (512 + 4) x 16 records of 61 KiB, far beyond the scratch.
    assert lib.kda_chunk_prefill_workspace_size(4, 32768, 16, 128) > limit
    assert call(_pdesc(N=4, T=32768, H=16)) == UNSUPPORTED
    assert b"fixed scratch" in lib.kda_last_error()
    assert lib.kda_chunk_prefill_noalloc(f(1), f(2), f(3), f(4), f(5), f(6), f(7), -5.0, f(8),
                                         None, None, f(9), f(10), None, None) == INVALID
    assert call(_pdesc(D=64)) == UNSUPPORTED
    # Inside the limit the checks are kda_chunk_prefill's, all made before the scratch is
    # looked up (no GPU in this process, so a lookup would fail with KDA_ERR_HIP).
    assert lib.kda_chunk_prefill_workspace_size(1, 64, 2, 128) <= limit
    d = _pdesc(N=1, T=64, H=2)
    assert lib.kda_chunk_prefill_noalloc(f(1), f(2), f(3), f(4), f(5), f(6), f(7), -7.0, f(8),
                                         None, None, f(9), f(10), ctypes.byref(d), None) \
        == UNSUPPORTED
    assert lib.kda_chunk_prefill_noalloc(None, f(2), f(3), f(4), f(5), f(6), f(7), -5.0, f(8),
                                         None, None, f(9), f(10), ctypes.byref(d), None) \
        == INVALID
    d.q_token_stride = 100
    assert lib.kda_chunk_prefill_noalloc(f(1), f(2), f(3), f(4), f(5), f(6), f(7), -5.0, f(8),
                                         None, None, f(9), f(10), ctypes.byref(d), None) \
        == INVALID


def test_prefill_alignment_and_state_overlap_checks(lib):
    g = lambda n: ctypes.c_void_p(n << 32)      # fake buffers 4 GiB apart
    d = _pdesc(N=2, T=128, H=2)
    d.num_state_rows = 2

    def call(dt=g(7), A=g(6), init=None, idx=None, out=g(9), fin=g(10), q=g(1), ws_bytes=1 << 40):
        return lib.kda_chunk_prefill(q, g(2), g(3), g(4), g(5), A, dt, -5.0, g(8), init, idx,
                                     out, fin, g(11), ws_bytes, ctypes.byref(d), None)

    # dt_bias is read as 16-byte vectors, A_log as words
    assert call(dt=ctypes.c_void_p((7 << 32) + 8)) == INVALID
    assert b"dt_bias" in lib.kda_last_error()
    assert call(A=ctypes.c_void_p((6 << 32) + 2)) == INVALID
    # final_state sharing bytes with an input, with out, or partly with initial_state
    assert call(fin=ctypes.c_void_p((1 << 32) + 4096)) == INVALID
    assert b"final_state overlaps an input" in lib.kda_last_error()
    assert call(fin=ctypes.c_void_p((5 << 32) + 16)) == INVALID      # beta logits
    assert call(fin=ctypes.c_void_p((9 << 32) - 65536)) == INVALID   # runs into out
    assert call(init=g(12), fin=ctypes.c_void_p((12 << 32) + 65536)) == INVALID
    assert b"initial_state" in lib.kda_last_error()
    # out over the start states
    assert call(init=g(12), out=ctypes.c_void_p((12 << 32) + 1024)) == INVALID
    # in place over the start states is allowed only when indexed by sequence
    assert call(init=g(12), fin=g(12), idx=g(13)) == INVALID
    assert call(init=g(12), fin=g(12), ws_bytes=100) == WS_SMALL     # every other check passed


def test_verify_rejects_out_over_beta_and_states_over_inputs(lib):
    f = _fake
    d = _vdesc(Bn=2, T=8, H=2)
    # beta logits [16, 2] bf16 at f(5); out starting inside them
    st = lib.kda_recurrent_verify(f(1), f(2), f(3), f(4), f(5), f(6), f(7), -5.0, f(20), f(9),
                                  f(40), ctypes.c_void_p(0x50000 + 32), ctypes.byref(d), None)
    assert st == INVALID and b"beta_logits" in lib.kda_last_error()
    # per-step states written over q
    st = lib.kda_recurrent_verify(ctypes.c_void_p(0x400000 + 4096), f(2), f(3), f(4), f(5), f(6),
                                  f(7), -5.0, f(20), f(9), ctypes.c_void_p(0x400000), f(50),
                                  ctypes.byref(d), None)
    assert st == INVALID and b"intermediate_state overlaps" in lib.kda_last_error()
