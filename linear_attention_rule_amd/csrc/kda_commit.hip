// Commit after verify for gfx950: the num_accepted_tokens rollback of vLLM PR #55737
// ("...code steps too" commit message).  Each verify row b that accepted n of its T
// draft tokens moves state row (b, n-1) of the verify call's intermediate buffer into
// its pool slot state_idx[b], for every head.  A pure copy of 64 KiB per (row, head),
// so the kernel is bound by HBM.  Two workgroups per CU loop over the (row, head) items:
// each loads its next item (non-temporal loads: the source is read once) before storing
// the current one (ordinary stores: the next verify reads the pool), so reads and writes
// stay interleaved.  64 x 8 x 16 heads (1024 items, 128 MiB moved): 22.9 us against
// 26.4 us with one workgroup per item; 256, 384, 640 or 768 workgroups: 29.4, 25.4,
// 24.1, 24.5 us.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int COMMIT_THREADS = 256;
constexpr int COMMIT_VEC = D * D / 4 / COMMIT_THREADS;   // float4 per thread (16)

__global__ __launch_bounds__(COMMIT_THREADS) void commit_kernel(CommitParams p) {
  const int64_t HDD = static_cast<int64_t>(D) * D;
  const int items = p.B * p.H;
  // Source of item (b, h), or null when row b commits nothing (padding slot or no
  // accepted token in range).
  auto src_of = [&](int it) -> const f32x4* {
    const int b = it / p.H, h = it % p.H;
    const int slot = p.idx[b], n = p.n_acc[b];
    if (slot < 0 || slot >= p.slots || n < 1 || n > p.T) return nullptr;
    return reinterpret_cast<const f32x4*>(
        p.inter + ((static_cast<int64_t>(b) * p.T + (n - 1)) * p.H + h) * HDD);
  };
  auto load = [&](const f32x4* src, f32x4 (&v)[COMMIT_VEC]) {
#pragma unroll
    for (int i = 0; i < COMMIT_VEC; ++i)
      v[i] = __builtin_nontemporal_load(src + threadIdx.x + COMMIT_THREADS * i);
  };
  f32x4 cur[COMMIT_VEC], nxt[COMMIT_VEC];
  if (const f32x4* src = src_of(blockIdx.x)) load(src, cur);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int nx = it + gridDim.x;
    if (const f32x4* nsrc = nx < items ? src_of(nx) : nullptr) load(nsrc, nxt);
    if (src_of(it)) {
      const int b = it / p.H, h = it % p.H;
      f32x4* dst = reinterpret_cast<f32x4*>(p.pool + (static_cast<int64_t>(p.idx[b]) * p.H + h) * HDD);
#pragma unroll
      for (int i = 0; i < COMMIT_VEC; ++i) dst[threadIdx.x + COMMIT_THREADS * i] = cur[i];
    }
#pragma unroll
    for (int i = 0; i < COMMIT_VEC; ++i) cur[i] = nxt[i];
  }
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  int cus = 0;
  const hipError_t e = current_device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t items = static_cast<int64_t>(p.B) * p.H;
  const int64_t cap = 2 * static_cast<int64_t>(cus);
  const dim3 grid(static_cast<unsigned>(cap > 0 && items > cap ? cap : items));
  hipLaunchKernelGGL(commit_kernel, grid, dim3(COMMIT_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace kda
