// Output-gate sigmoid RMSNorm for gfx950: the sigmoid RMSNorm of SGLang PR #42489
// ("Improve GLM-5.3-Flash DFlash decoding on B300": bf16, D = 128 rows, output and
// rstd checked), taken as y = x / sqrt(mean(x^2) + eps) * weight * sigmoid(gate) per
// row of 128 channels (one token and head), rstd = 1 / sqrt(mean(x^2) + eps).
// Bound by HBM: each row moves 3 x 256 bytes.  Sixteen lanes own one row, 8 channels
// (16 bytes) each, so a wave reads and writes whole 1 KiB runs of 4 rows and the row
// sum needs four lane exchanges inside each 16-lane group.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int NORM_THREADS = 256;
constexpr int ROWS_PER_WAVE = 4;

__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
  f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
  f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
  f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
}

__global__ __launch_bounds__(NORM_THREADS) void gated_rmsnorm_kernel(NormParams p) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;                 // row of this 16-lane group within the wave
  const int c0 = 8 * (lane & 15);            // its 8 channels
  const int64_t rows = static_cast<int64_t>(p.tokens) * p.H;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (NORM_THREADS / 64);
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * (NORM_THREADS / 64) + (threadIdx.x >> 6);
  float w[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(p.weight + c0);
    const float4 b = *reinterpret_cast<const float4*>(p.weight + c0 + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  // Every lane of a 16-lane group takes the same trip count, so the exchanges below
  // only ever read lanes of an active group.
  for (int64_t r = wave_id * ROWS_PER_WAVE + sub; r < rows; r += waves * ROWS_PER_WAVE) {
    const int64_t t = r / p.H;
    const int h = static_cast<int>(r - t * p.H);
    const uint4 xw = *reinterpret_cast<const uint4*>(p.x + t * p.x_st + h * D + c0);
    const uint4 gw = *reinterpret_cast<const uint4*>(p.gate + t * p.g_st + h * D + c0);
    float x[8], g[8];
    unpack8(xw, x);
    unpack8(gw, g);
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
    *reinterpret_cast<uint4*>(p.y + t * p.y_st + h * D + c0) =
        make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                   pack_bf16x2(y[6], y[7]));
    if (p.rstd && (lane & 15) == 0) p.rstd[r] = rstd;
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormParams& p, int cus, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.tokens) * p.H;
  if (rows == 0) return hipSuccess;
  const int64_t per_wg = (NORM_THREADS / 64) * ROWS_PER_WAVE;
  const int64_t wgs = std::min<int64_t>((rows + per_wg - 1) / per_wg,
                                        static_cast<int64_t>(std::max(cus, 1)) * 8);
  hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3(static_cast<unsigned>(wgs)), dim3(NORM_THREADS), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace kda
