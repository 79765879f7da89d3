// Output-gate sigmoid RMSNorm for gfx950: the sigmoid RMSNorm of SGLang PR #42489
// ("Improve GLM-5.3-Flash DFlash decoding on B300": bf16, D = 128 rows, output and
// rstd checked), taken as y = x / sqrt(mean(x^2) + eps) * weight * sigmoid(gate) per
// row of 128 channels (one token and head), rstd = 1 / sqrt(mean(x^2) + eps).
// Bound by HBM: each row moves 3 x 256 bytes.  Sixteen lanes own one row, 8 channels
// (16 bytes) each, so a wave reads and writes whole 1 KiB runs of 4 rows and the row
// sum needs four lane exchanges inside each 16-lane group.  Workgroups are short-lived:
// each wave takes NORM_UNROLL groups of 4 consecutive rows and issues all their loads
// before any arithmetic (on MI355X at 32768 x 16 rows: 80 us against 87 us for a
// grid-stride loop of long-lived workgroups with one group in flight per wave).
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int NORM_THREADS = 256;
constexpr int ROWS_PER_WAVE = 4;
constexpr int NORM_UNROLL = 2;

__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
  f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
  f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
  f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
}

__global__ __launch_bounds__(NORM_THREADS) void gated_rmsnorm_kernel(NormParams p) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;                 // row of this 16-lane group within a group of 4
  const int c0 = 8 * (lane & 15);            // its 8 channels
  const int64_t rows = static_cast<int64_t>(p.tokens) * p.H;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * (NORM_THREADS / 64) + (threadIdx.x >> 6);
  const int64_t row0 = wave_id * (NORM_UNROLL * ROWS_PER_WAVE) + sub;
  float w[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(p.weight + c0);
    const float4 b = *reinterpret_cast<const float4*>(p.weight + c0 + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  // Loads first.  Rows past the end re-read the last row (in bounds) and store nothing;
  // every lane runs the exchanges below, so they only ever read active lanes.
  uint4 xw[NORM_UNROLL], gw[NORM_UNROLL];
  int64_t tt[NORM_UNROLL];
  int hh[NORM_UNROLL];
#pragma unroll
  for (int u = 0; u < NORM_UNROLL; ++u) {
    const int64_t r = min(row0 + u * ROWS_PER_WAVE, rows - 1);
    tt[u] = r / p.H;
    hh[u] = static_cast<int>(r - tt[u] * p.H);
    xw[u] = *reinterpret_cast<const uint4*>(p.x + tt[u] * p.x_st + hh[u] * D + c0);
    gw[u] = *reinterpret_cast<const uint4*>(p.gate + tt[u] * p.g_st + hh[u] * D + c0);
  }
#pragma unroll
  for (int u = 0; u < NORM_UNROLL; ++u) {
    const int64_t r = row0 + u * ROWS_PER_WAVE;
    float x[8], g[8];
    unpack8(xw[u], x);
    unpack8(gw[u], g);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * rstd * w[i] * sigmoid_f32(g[i]);
    if (r < rows) {
      *reinterpret_cast<uint4*>(p.y + tt[u] * p.y_st + hh[u] * D + c0) =
          make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                     pack_bf16x2(y[6], y[7]));
      if (p.rstd && (lane & 15) == 0) p.rstd[r] = rstd;
    }
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.tokens) * p.H;
  if (rows == 0) return hipSuccess;
  static_assert(NORM_ROWS_PER_WG == (NORM_THREADS / 64) * ROWS_PER_WAVE * NORM_UNROLL, "rows per workgroup");
  const int64_t wgs = norm_workgroups(rows);
  hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3(static_cast<unsigned>(wgs)), dim3(NORM_THREADS), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace kda
