// libkda C ABI: host-side validation, workspace sizing and kernel launches.
//
// Every check here uses host integers only (shapes, strides, pointer values);
// no device memory is read and no stream is synchronised, so a call can be
// captured into a HIP graph.  Status codes and messages follow include/kda.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/kda.h"
#include "kda_internal.h"

static_assert(KDA_NOALLOC_SCRATCH_BYTES == kda::NOALLOC_SCRATCH_BYTES,
              "kda.h and kda_internal.h disagree on the fixed scratch size");

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kda_status ok() {
  g_last_error.clear();
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

// Bytes touched by a token-strided tensor of `tokens` rows of `row_elems` elements.
Span span_of(const void* base, int64_t tokens, int64_t stride, int64_t row_elems, int64_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
  if (tokens <= 0) return {lo, lo};
  return {lo, lo + static_cast<uintptr_t>(((tokens - 1) * stride + row_elems) * esize)};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Whether two token-strided tensors of `tokens` rows share a byte.  With equal strides
// the rows of one sit at a fixed offset from the rows of the other, so interleaved
// views of one fused buffer are told apart exactly; otherwise the byte spans decide.
bool rows_overlap(const void* a, const void* b, int64_t tokens, int64_t stride, int64_t b_stride,
                  int64_t row_elems, int64_t esize) {
  const Span sa = span_of(a, tokens, stride, row_elems, esize);
  const Span sb = span_of(b, tokens, b_stride, row_elems, esize);
  if (!overlaps(sa, sb)) return false;
  if (stride != b_stride) return true;
  const int64_t period = stride * esize, width = row_elems * esize;
  const int64_t d = static_cast<int64_t>(reinterpret_cast<uintptr_t>(b)) -
                    static_cast<int64_t>(reinterpret_cast<uintptr_t>(a));
  const int64_t m = ((d % period) + period) % period;   // offset of b's rows past a's
  return m < width || m > period - width;
}

// Validates one token-strided bf16 input: returns the effective stride (0 -> dense default).
kda_status check_stride(const char* name, int64_t stride, int64_t dense, int64_t row_elems,
                        int64_t* eff) {
  if (stride == 0) stride = dense;
  if (stride < row_elems) return fail(KDA_ERR_INVALID_ARGUMENT, "%s token stride %lld < %lld", name,
                                      static_cast<long long>(stride), static_cast<long long>(row_elems));
  // Kernels address up to 64 rows of a chunk with 32-bit byte offsets.
  if (stride > (int64_t{1} << 24))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s token stride %lld exceeds 2^24 elements", name,
                static_cast<long long>(stride));
  *eff = stride;
  return KDA_OK;
}

// Output rows reachable through an optional scatter index (tokens rows when none).
kda_status check_out_index(const int32_t* idx, int64_t rows, int64_t tokens, int64_t* out_rows) {
  if (!idx) {
    *out_rows = tokens;
    return KDA_OK;
  }
  if (rows < 0 || rows > INT32_MAX)
    return fail(KDA_ERR_INVALID_ARGUMENT, "out_rows %lld outside [0, 2^31)",
                static_cast<long long>(rows));
  if (tokens > 0 && (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "out_token_index must be 4-byte aligned");
  *out_rows = rows;
  return KDA_OK;
}

kda_status check_lower_bound(float lb) {
  if (!std::isfinite(lb)) return fail(KDA_ERR_UNSUPPORTED, "lower_bound must be finite");
  // The intra-chunk factorisation keeps every exponential of a 16-token block
  // within fp32/bf16 range only while 16 * |lower_bound| * log2(e) < 127.
  if (lb < -5.0f || lb > 0.0f)
    return fail(KDA_ERR_UNSUPPORTED, "lower_bound %g outside the supported range [-5, 0]", lb);
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_last_error.c_str(); }

size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                        int32_t head_dim) {
  if (num_seqs < 0 || total_tokens < 0 || num_heads < 1 || head_dim != KDA_HEAD_DIM) return 0;
  const int64_t rec = kda::prefill_record_bytes(num_seqs, total_tokens, num_heads);
  if (rec == 0) return 0;
  return static_cast<size_t>(rec + kda::prefill_segment_bytes(num_seqs, num_heads));
}

}  // extern "C"

namespace {

kda_status prefill_phases(const void* q, const void* k, const void* v, const void* g,
                          const void* beta_logits, const float* A_log, const float* dt_bias,
                          float lower_bound, const int32_t* cu_seqlens,
                          const float* initial_state, const int32_t* initial_state_idx,
                          void* out, float* final_state, void* workspace,
                          size_t workspace_bytes, const kda_prefill_desc* desc, void* stream,
                          int phases, bool use_scratch = false) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int N = desc->num_seqs, T = desc->total_tokens, H = desc->num_heads;
  if (desc->head_dim != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", desc->head_dim);
  if (N < 0 || T < 0 || H < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes N=%d T_total=%d H=%d", N, T, H);
  if (kda_status s = check_lower_bound(lower_bound)) return s;
  if (kda::chunk_slots(N, T) * H > INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "%lld chunk-heads exceed one launch",
                static_cast<long long>(kda::chunk_slots(N, T) * H));
  if (!A_log || !dt_bias) return fail(KDA_ERR_INVALID_ARGUMENT, "A_log / dt_bias is NULL");
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (T > 0 && (!q || !k || !v || !g || !beta_logits || !out))
    return fail(KDA_ERR_INVALID_ARGUMENT, "an input or output pointer is NULL");
  if (initial_state_idx && !initial_state)
    return fail(KDA_ERR_INVALID_ARGUMENT, "initial_state_idx given without initial_state");
  if (initial_state && desc->num_state_rows < (initial_state_idx ? 1 : N))
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_state_rows %d too small", desc->num_state_rows);
  const int64_t HD = static_cast<int64_t>(H) * KDA_HEAD_DIM;
  int64_t qs, ks, vs, gs, bs, os;
  if (kda_status s = check_stride("q", desc->q_token_stride, HD, HD, &qs)) return s;
  if (kda_status s = check_stride("k", desc->k_token_stride, HD, HD, &ks)) return s;
  if (kda_status s = check_stride("v", desc->v_token_stride, HD, HD, &vs)) return s;
  if (kda_status s = check_stride("g", desc->g_token_stride, HD, HD, &gs)) return s;
  if (kda_status s = check_stride("beta_logits", desc->beta_token_stride, H, H, &bs)) return s;
  if (kda_status s = check_stride("out", desc->out_token_stride, HD, HD, &os)) return s;
  int64_t orows;
  if (kda_status s = check_out_index(desc->out_token_index, desc->out_rows, T, &orows)) return s;
  if (T > 0) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(out))
      return fail(KDA_ERR_INVALID_ARGUMENT, "q/k/v/g/out must be 16-byte aligned");
    if ((qs | ks | vs | gs | os) & 7)
      return fail(KDA_ERR_INVALID_ARGUMENT, "q/k/v/g/out token strides must be multiples of 8");
    const Span so = span_of(out, orows, os, HD, 2);
    if (desc->out_token_index && overlaps(so, span_of(desc->out_token_index, T, 1, 1, 4)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps out_token_index");
    const void* ins[4] = {q, k, v, g};
    const int64_t sts[4] = {qs, ks, vs, gs};
    for (int i = 0; i < 4; ++i)
      if (overlaps(so, span_of(ins[i], T, sts[i], HD, 2)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps an input");
    if (overlaps(so, span_of(beta_logits, T, bs, H, 2)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps beta_logits");
  }
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "state buffers must be 16-byte aligned");
  // The intra kernel reads dt_bias rows as 16-byte vectors.
  if (!aligned16(dt_bias) || (reinterpret_cast<uintptr_t>(A_log) & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "dt_bias must be 16-byte and A_log 4-byte aligned");
  {
    // States: the final states are written while other workgroups still read the
    // inputs and the start states, so they may share no byte with them, except that
    // final_state may be initial_state itself when both are indexed by sequence (each
    // workgroup reads its start columns before it writes them).
    const int64_t state_elems = static_cast<int64_t>(KDA_HEAD_DIM) * KDA_HEAD_DIM;
    const Span s_init = initial_state
                            ? span_of(initial_state, desc->num_state_rows, H * state_elems,
                                      H * state_elems, 4)
                            : Span{0, 0};
    const Span s_fin = final_state ? span_of(final_state, N, H * state_elems, H * state_elems, 4)
                                   : Span{0, 0};
    if (final_state && initial_state && overlaps(s_fin, s_init) &&
        !(final_state == initial_state && !initial_state_idx))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "final_state overlaps initial_state (only final_state == initial_state "
                  "without initial_state_idx is allowed)");
    if (T > 0) {
      const void* ins[5] = {q, k, v, g, beta_logits};
      const int64_t sts[5] = {qs, ks, vs, gs, bs};
      const int64_t widths[5] = {HD, HD, HD, HD, H};
      const Span so = span_of(out, orows, os, HD, 2);
      for (int i = 0; i < 5; ++i)
        if (final_state && overlaps(s_fin, span_of(ins[i], T, sts[i], widths[i], 2)))
          return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps an input");
      if (final_state && overlaps(s_fin, so))
        return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps out");
      if (initial_state && overlaps(s_init, so))
        return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps initial_state");
    }
  }
  const size_t need = kda_chunk_prefill_workspace_size(N, T, H, KDA_HEAD_DIM);
  if (use_scratch) {
    // kda_chunk_prefill_noalloc: the same bytes from the library's fixed per-device array,
    // looked up only once every other check has passed.
    if (need > static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES))
      return fail(KDA_ERR_UNSUPPORTED,
                  "N=%d T_total=%d H=%d needs %zu bytes of scratch; the fixed scratch holds %zu",
                  N, T, H, need, static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES));
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0 && N > 0) {
      const hipError_t e = kda::noalloc_scratch(&workspace);
      if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "scratch lookup failed: %s", hipGetErrorString(e));
      workspace_bytes = need;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (need > 0 && !aligned16(workspace))
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (N == 0) return ok();

  kda::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g);
  p.beta = static_cast<const uint16_t*>(beta_logits);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.cu = cu_seqlens;
  p.init = initial_state;
  p.init_idx = initial_state_idx;
  p.out = static_cast<uint16_t*>(out);
  p.out_idx = desc->out_token_index;
  p.out_rows = orows;
  p.final_state = final_state;
  p.work = static_cast<unsigned char*>(workspace);
  p.seg_ws = kda::prefill_segment_bytes(N, H) > 0 && kda::prefill_record_bytes(N, T, H) > 0
                 ? reinterpret_cast<float*>(p.work + kda::prefill_record_bytes(N, T, H))
                 : nullptr;
  p.seg_G = 1;
  p.lb_log2e = lower_bound * kda::LOG2E;
  p.scale = desc->scale > 0.f ? desc->scale : 1.0f / std::sqrt(static_cast<float>(KDA_HEAD_DIM));
  p.N = N;
  p.T_total = T;
  p.H = H;
  p.num_slots_chunk = static_cast<int>(kda::chunk_slots(N, T));
  p.init_rows = desc->num_state_rows;
  p.q_st = qs; p.k_st = ks; p.v_st = vs; p.g_st = gs; p.b_st = bs; p.o_st = os;
  const hipError_t e = kda::launch_prefill(p, phases, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

#define KDA_PREFILL_ARGS                                                                      \
  const void *q, const void *k, const void *v, const void *g, const void *beta_logits,       \
      const float *A_log, const float *dt_bias, float lower_bound, const int32_t *cu_seqlens, \
      const float *initial_state, const int32_t *initial_state_idx, void *out,               \
      float *final_state, void *workspace, size_t workspace_bytes,                           \
      const kda_prefill_desc *desc, void *stream
#define KDA_PREFILL_FWD                                                                     \
  q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens, initial_state,          \
      initial_state_idx, out, final_state, workspace, workspace_bytes, desc, stream

kda_status kda_chunk_prefill(KDA_PREFILL_ARGS) {
  return prefill_phases(KDA_PREFILL_FWD, kda::PHASE_INTRA | kda::PHASE_SCAN);
}
kda_status kda_chunk_prefill_intra(KDA_PREFILL_ARGS) {
  return prefill_phases(KDA_PREFILL_FWD, kda::PHASE_INTRA);
}
kda_status kda_chunk_prefill_scan(KDA_PREFILL_ARGS) {
  return prefill_phases(KDA_PREFILL_FWD, kda::PHASE_SCAN);
}

kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta_logits, const float* A_log,
                                     const float* dt_bias, float lower_bound,
                                     const int32_t* cu_seqlens, const float* initial_state,
                                     const int32_t* initial_state_idx, void* out,
                                     float* final_state, const kda_prefill_desc* desc,
                                     void* stream) {
  return prefill_phases(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, cu_seqlens,
                        initial_state, initial_state_idx, out, final_state, nullptr, 0, desc,
                        stream, kda::PHASE_INTRA | kda::PHASE_SCAN, /*use_scratch=*/true);
}

}  // extern "C"

namespace {

kda_status verify_impl(const void* q, const void* k, const void* v, const void* g,
                       const void* beta_logits, const float* A_log, const float* dt_bias,
                       float lower_bound, const float* state_pool, const int32_t* state_idx,
                       float* intermediate_state, void* out, const kda_output_norm* norm,
                       const kda_verify_desc* desc, void* stream) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int B = desc->batch, T = desc->num_steps, H = desc->num_heads;
  if (desc->head_dim != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", desc->head_dim);
  if (B < 0 || H < 1 || desc->num_slots < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d slots=%d", B, H, desc->num_slots);
  if (T < 1 || T > KDA_MAX_VERIFY_STEPS)
    return fail(KDA_ERR_UNSUPPORTED, "num_steps %d outside 1..%d", T, KDA_MAX_VERIFY_STEPS);
  // The kernel numbers a row's tokens b*T + t in 32-bit integers.
  if (static_cast<int64_t>(B) * T > INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "batch %d x num_steps %d exceeds 2^31 - 1 tokens", B, T);
  if (kda_status s = check_lower_bound(lower_bound)) return s;
  if (!A_log || !dt_bias || !state_pool)
    return fail(KDA_ERR_INVALID_ARGUMENT, "A_log / dt_bias / state_pool is NULL");
  if (B > 0 && (!q || !k || !v || !g || !beta_logits || !state_idx || !intermediate_state || !out))
    return fail(KDA_ERR_INVALID_ARGUMENT, "an input or output pointer is NULL");
  const int64_t HD = static_cast<int64_t>(H) * KDA_HEAD_DIM;
  int64_t qs, ks, vs, gs, bs, os;
  if (kda_status s = check_stride("q", desc->q_token_stride, HD, HD, &qs)) return s;
  if (kda_status s = check_stride("k", desc->k_token_stride, HD, HD, &ks)) return s;
  if (kda_status s = check_stride("v", desc->v_token_stride, HD, HD, &vs)) return s;
  if (kda_status s = check_stride("g", desc->g_token_stride, HD, HD, &gs)) return s;
  if (kda_status s = check_stride("beta_logits", desc->beta_token_stride, H, H, &bs)) return s;
  if (kda_status s = check_stride("out", desc->out_token_stride, HD, HD, &os)) return s;
  int64_t orows;
  if (kda_status s = check_out_index(desc->out_token_index, desc->out_rows,
                                     static_cast<int64_t>(B) * T, &orows))
    return s;
  if (B == 0) return ok();
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(out) ||
      !aligned16(state_pool) || !aligned16(intermediate_state) || !aligned16(dt_bias))
    return fail(KDA_ERR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
  if ((qs | ks | vs | gs | os) & 7)
    return fail(KDA_ERR_INVALID_ARGUMENT, "q/k/v/g/out token strides must be multiples of 8");
  const int64_t BT = static_cast<int64_t>(B) * T;
  const int64_t state_elems = static_cast<int64_t>(KDA_HEAD_DIM) * KDA_HEAD_DIM;
  const Span s_pool = span_of(state_pool, desc->num_slots, H * state_elems, H * state_elems, 4);
  const Span s_int = span_of(intermediate_state, BT, H * state_elems, H * state_elems, 4);
  if (overlaps(s_pool, s_int))
    return fail(KDA_ERR_INVALID_ARGUMENT, "intermediate_state overlaps state_pool");
  const Span so = span_of(out, orows, os, HD, 2);
  if (desc->out_token_index && overlaps(so, span_of(desc->out_token_index, BT, 1, 1, 4)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps out_token_index");
  const void* ins[4] = {q, k, v, g};
  const int64_t sts[4] = {qs, ks, vs, gs};
  for (int i = 0; i < 4; ++i)
    if (overlaps(so, span_of(ins[i], BT, sts[i], HD, 2)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps an input");
  if (overlaps(so, s_int) || overlaps(so, s_pool))
    return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps a state buffer");
  if (overlaps(so, span_of(beta_logits, BT, bs, H, 2)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps beta_logits");
  for (int i = 0; i < 4; ++i)
    if (overlaps(s_int, span_of(ins[i], BT, sts[i], HD, 2)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "intermediate_state overlaps an input");
  if (overlaps(s_int, span_of(beta_logits, BT, bs, H, 2)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "intermediate_state overlaps beta_logits");
  int64_t ngs = 0;
  if (norm) {
    // The fused output norm reads the gate rows of the output rows and writes rstd rows.
    if (!norm->gate || !norm->weight)
      return fail(KDA_ERR_INVALID_ARGUMENT, "norm gate / weight is NULL");
    if (!std::isfinite(norm->eps) || norm->eps < 0.f)
      return fail(KDA_ERR_INVALID_ARGUMENT, "norm eps must be finite and >= 0");
    if (kda_status st = check_stride("norm gate", norm->gate_token_stride, HD, HD, &ngs)) return st;
    if (!aligned16(norm->gate) || !aligned16(norm->weight) || (ngs & 7))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "norm gate / weight must be 16-byte aligned, gate stride a multiple of 8");
    if (norm->rstd && (reinterpret_cast<uintptr_t>(norm->rstd) & 3u))
      return fail(KDA_ERR_INVALID_ARGUMENT, "rstd must be 4-byte aligned");
    const Span s_gate = span_of(norm->gate, orows, ngs, HD, 2);
    if (overlaps(so, s_gate)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps the norm gate");
    if (overlaps(s_int, s_gate))
      return fail(KDA_ERR_INVALID_ARGUMENT, "intermediate_state overlaps the norm gate");
    if (norm->rstd) {
      const Span s_r = span_of(norm->rstd, orows * H, 1, 1, 4);
      if (overlaps(s_r, so) || overlaps(s_r, s_gate) || overlaps(s_r, s_int) ||
          overlaps(s_r, s_pool))
        return fail(KDA_ERR_INVALID_ARGUMENT, "rstd overlaps out, the gate or a state buffer");
    }
  }

  kda::VerifyParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g);
  p.beta = static_cast<const uint16_t*>(beta_logits);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.pool = state_pool;
  p.idx = state_idx;
  p.inter = intermediate_state;
  p.out = static_cast<uint16_t*>(out);
  p.out_idx = desc->out_token_index;
  p.out_rows = orows;
  p.lb_log2e = lower_bound * kda::LOG2E;
  p.scale = desc->scale > 0.f ? desc->scale : 1.0f / std::sqrt(static_cast<float>(KDA_HEAD_DIM));
  p.B = B;
  p.T = T;
  p.H = H;
  p.slots = desc->num_slots;
  p.q_st = qs; p.k_st = ks; p.v_st = vs; p.g_st = gs; p.b_st = bs; p.o_st = os;
  if (norm) {
    p.out_gate = static_cast<const uint16_t*>(norm->gate);
    p.norm_w = norm->weight;
    p.rstd = norm->rstd;
    p.norm_eps = norm->eps;
    p.og_st = ngs;
  }
  const hipError_t e = kda::launch_verify(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "verify launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const void* g,
                                const void* beta_logits, const float* A_log, const float* dt_bias,
                                float lower_bound, const float* state_pool,
                                const int32_t* state_idx, float* intermediate_state, void* out,
                                const kda_verify_desc* desc, void* stream) {
  return verify_impl(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, state_pool, state_idx,
                     intermediate_state, out, nullptr, desc, stream);
}

kda_status kda_recurrent_verify_gated(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta_logits, const float* A_log,
                                      const float* dt_bias, float lower_bound,
                                      const float* state_pool, const int32_t* state_idx,
                                      float* intermediate_state, void* out,
                                      const kda_output_norm* norm, const kda_verify_desc* desc,
                                      void* stream) {
  if (!norm) return fail(KDA_ERR_INVALID_ARGUMENT, "norm is NULL");
  return verify_impl(q, k, v, g, beta_logits, A_log, dt_bias, lower_bound, state_pool, state_idx,
                     intermediate_state, out, norm, desc, stream);
}

}  // extern "C"

namespace {

// Host checks shared by the two conv entry points; fills the common fields of p.
kda_status conv_common(const void* x, const void* weight, const void* bias, const void* y,
                       const kda_conv_desc* desc, int64_t tokens, kda::ConvParams* p) {
  const int C = desc->channels, W = desc->width;
  if (C < 8 || C % 8) return fail(KDA_ERR_INVALID_ARGUMENT, "channels %d: positive multiple of 8", C);
  if (W < 1 || W > 4) return fail(KDA_ERR_UNSUPPORTED, "width %d outside 1..4", W);
  if (desc->num_state_slots < 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_state_slots %d < 0", desc->num_state_slots);
  int64_t xs, ys;
  if (kda_status s = check_stride("x", desc->x_token_stride, C, C, &xs)) return s;
  if (kda_status s = check_stride("y", desc->y_token_stride, C, C, &ys)) return s;
  if (tokens > 0) {
    if (!x || !weight || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "x / weight / y is NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(weight) || (bias && !aligned16(bias)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "x / y / weight / bias must be 16-byte aligned");
    if ((xs | ys) & 7) return fail(KDA_ERR_INVALID_ARGUMENT, "token strides must be multiples of 8");
    if (rows_overlap(y, x, tokens, ys, xs, C, 2))
      return fail(KDA_ERR_INVALID_ARGUMENT, "y overlaps x");
  }
  p->x = static_cast<const uint16_t*>(x);
  p->weight = static_cast<const uint16_t*>(weight);
  p->bias = static_cast<const uint16_t*>(bias);
  p->y = static_cast<uint16_t*>(const_cast<void*>(y));
  p->C = C;
  p->W = W;
  p->slots = desc->num_state_slots;
  p->silu = desc->silu != 0;
  p->x_st = xs;
  p->y_st = ys;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_causal_conv1d_prefill(const void* x, const void* weight, const void* bias,
                                     const int32_t* cu_seqlens, void* conv_state,
                                     const int32_t* state_idx, void* y,
                                     const kda_conv_desc* desc, void* stream) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int N = desc->num_seqs, T = desc->total_tokens;
  if (N < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes N=%d T_total=%d", N, T);
  kda::ConvParams p{};
  if (kda_status s = conv_common(x, weight, bias, y, desc, T, &p)) return s;
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (conv_state && desc->width > 1) {
    if (!aligned16(conv_state))
      return fail(KDA_ERR_INVALID_ARGUMENT, "conv_state must be 16-byte aligned");
    if (desc->num_state_slots < (state_idx ? 1 : N))
      return fail(KDA_ERR_INVALID_ARGUMENT, "num_state_slots %d too small", desc->num_state_slots);
    const int64_t win = static_cast<int64_t>(desc->width - 1) * desc->channels;
    if (T > 0 && overlaps(span_of(conv_state, desc->num_state_slots, win, win, 2),
                          span_of(y, T, p.y_st, desc->channels, 2)))
      return fail(KDA_ERR_INVALID_ARGUMENT, "y overlaps conv_state");
  }
  if (N == 0) return ok();
  // One 256-thread workgroup per (16-token row slot, 2048-channel block), in a 1-D grid.
  if (kda::conv_prefill_workgroups(N, T, desc->channels) > (int64_t{1} << 24) - 1)
    return fail(KDA_ERR_UNSUPPORTED, "conv prefill of %d tokens x %d channels: too many workgroups",
                T, desc->channels);
  p.cu = cu_seqlens;
  p.state = desc->width > 1 ? static_cast<uint16_t*>(conv_state) : nullptr;
  p.state_idx = state_idx;
  p.N = N;
  p.T_total = T;
  const hipError_t e = kda::launch_conv_prefill(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv launch failed: %s", hipGetErrorString(e));
  return ok();
}

kda_status kda_causal_conv1d_update(const void* x, const void* weight, const void* bias,
                                    const void* conv_state, const int32_t* state_idx,
                                    void* intermediate_window, void* y,
                                    const kda_conv_desc* desc, void* stream) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int B = desc->num_seqs, T = desc->num_steps;
  if (B < 0 || T < 1 || T > KDA_MAX_VERIFY_STEPS)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes B=%d num_steps=%d", B, T);
  if (static_cast<int64_t>(B) * T != desc->total_tokens)
    return fail(KDA_ERR_INVALID_ARGUMENT, "total_tokens must be B * num_steps");
  kda::ConvParams p{};
  if (kda_status s = conv_common(x, weight, bias, y, desc, static_cast<int64_t>(B) * T, &p))
    return s;
  if (B == 0) return ok();
  if (!state_idx || (desc->width > 1 && (!conv_state || !intermediate_window)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_idx / conv_state / intermediate_window is NULL");
  if (desc->num_state_slots < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_state_slots < 1");
  if (desc->width > 1) {
    if (!aligned16(conv_state) || !aligned16(intermediate_window))
      return fail(KDA_ERR_INVALID_ARGUMENT, "windows must be 16-byte aligned");
    const int64_t win = static_cast<int64_t>(desc->width - 1) * desc->channels;
    const Span s_pool = span_of(conv_state, desc->num_state_slots, win, win, 2);
    const Span s_int = span_of(intermediate_window, static_cast<int64_t>(B) * T, win, win, 2);
    const Span s_y = span_of(y, static_cast<int64_t>(B) * T, p.y_st, desc->channels, 2);
    if (overlaps(s_pool, s_int) || overlaps(s_y, s_int) || overlaps(s_y, s_pool))
      return fail(KDA_ERR_INVALID_ARGUMENT, "windows overlap each other or y");
  }
  p.state = const_cast<uint16_t*>(static_cast<const uint16_t*>(conv_state));
  p.state_idx = state_idx;
  p.inter = static_cast<uint16_t*>(intermediate_window);
  p.N = B;
  p.T = T;
  p.T_total = B * T;
  const hipError_t e = kda::launch_conv_update(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv launch failed: %s", hipGetErrorString(e));
  return ok();
}

kda_status kda_gated_rmsnorm(const void* x, const void* gate, const float* weight, void* y,
                             float* rstd, const kda_norm_desc* desc, void* stream) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int T = desc->tokens, H = desc->num_heads;
  if (desc->head_dim != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", desc->head_dim);
  if (T < 0 || H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes tokens=%d H=%d", T, H);
  if (!std::isfinite(desc->eps) || desc->eps < 0.f)
    return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  const int64_t HD = static_cast<int64_t>(H) * KDA_HEAD_DIM;
  int64_t xs, gs, ys;
  if (kda_status s = check_stride("x", desc->x_token_stride, HD, HD, &xs)) return s;
  if (kda_status s = check_stride("gate", desc->gate_token_stride, HD, HD, &gs)) return s;
  if (kda_status s = check_stride("y", desc->y_token_stride, HD, HD, &ys)) return s;
  if (T == 0) return ok();
  if (!x || !gate || !weight || !y)
    return fail(KDA_ERR_INVALID_ARGUMENT, "x / gate / weight / y is NULL");
  if (!aligned16(x) || !aligned16(gate) || !aligned16(weight) || !aligned16(y))
    return fail(KDA_ERR_INVALID_ARGUMENT, "x / gate / weight / y must be 16-byte aligned");
  if ((xs | gs | ys) & 7)
    return fail(KDA_ERR_INVALID_ARGUMENT, "token strides must be multiples of 8");
  if (rstd && (reinterpret_cast<uintptr_t>(rstd) & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "rstd must be 4-byte aligned");
  const Span sy = span_of(y, T, ys, HD, 2);
  if (rows_overlap(y, gate, T, ys, gs, HD, 2))
    return fail(KDA_ERR_INVALID_ARGUMENT, "y overlaps gate");
  if (rows_overlap(y, x, T, ys, xs, HD, 2) && !(y == x && ys == xs))
    return fail(KDA_ERR_INVALID_ARGUMENT, "y overlaps x (only y == x with equal strides is allowed)");
  if (rstd && overlaps(span_of(rstd, static_cast<int64_t>(T) * H, 1, 1, 4), sy))
    return fail(KDA_ERR_INVALID_ARGUMENT, "rstd overlaps y");
  if (kda::norm_workgroups(static_cast<int64_t>(T) * H) > (int64_t{1} << 24) - 1)
    return fail(KDA_ERR_UNSUPPORTED, "norm over %d x %d rows: too many workgroups", T, H);
  kda::NormParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.gate = static_cast<const uint16_t*>(gate);
  p.weight = weight;
  p.y = static_cast<uint16_t*>(y);
  p.rstd = rstd;
  p.eps = desc->eps;
  p.tokens = T;
  p.H = H;
  p.x_st = xs; p.g_st = gs; p.y_st = ys;
  const hipError_t e = kda::launch_gated_rmsnorm(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "norm launch failed: %s", hipGetErrorString(e));
  return ok();
}

kda_status kda_commit_accepted(const float* intermediate_state, const int32_t* state_idx,
                               const int32_t* num_accepted, float* state_pool,
                               const kda_commit_desc* desc, void* stream) {
  if (!desc) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  const int B = desc->batch, T = desc->num_steps, H = desc->num_heads;
  if (desc->head_dim != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", desc->head_dim);
  if (B < 0 || T < 1 || H < 1 || desc->num_slots < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes B=%d T=%d H=%d slots=%d", B, T, H,
                desc->num_slots);
  if (B == 0) return ok();
  if (!intermediate_state || !state_idx || !num_accepted || !state_pool)
    return fail(KDA_ERR_INVALID_ARGUMENT, "a pointer is NULL");
  if (!aligned16(intermediate_state) || !aligned16(state_pool))
    return fail(KDA_ERR_INVALID_ARGUMENT, "state buffers must be 16-byte aligned");
  if (static_cast<int64_t>(B) * H > INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "B*H exceeds one launch");
  const int64_t state_elems = static_cast<int64_t>(KDA_HEAD_DIM) * KDA_HEAD_DIM;
  const Span s_pool = span_of(state_pool, desc->num_slots, H * state_elems, H * state_elems, 4);
  const Span s_int = span_of(intermediate_state, static_cast<int64_t>(B) * T, H * state_elems,
                             H * state_elems, 4);
  if (overlaps(s_pool, s_int))
    return fail(KDA_ERR_INVALID_ARGUMENT, "intermediate_state overlaps state_pool");
  if (overlaps(s_pool, span_of(state_idx, B, 1, 1, 4)) ||
      overlaps(s_pool, span_of(num_accepted, B, 1, 1, 4)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_pool overlaps an index array");
  kda::CommitParams p{};
  p.inter = intermediate_state;
  p.idx = state_idx;
  p.n_acc = num_accepted;
  p.pool = state_pool;
  p.B = B;
  p.T = T;
  p.H = H;
  p.slots = desc->num_slots;
  const hipError_t e = kda::launch_commit(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "commit launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
