// Commit after verify for gfx950: the num_accepted_tokens rollback of vLLM PR #55737
// ("...code steps too" commit message).  Each verify row b that accepted n of its T
// draft tokens moves state row (b, n-1) of the verify call's intermediate buffer into
// its pool slot state_idx[b], for every head.  A pure copy of 64 KiB per (row, head),
// so the kernel is bound by HBM: one workgroup per (row, head) streams the source with
// non-temporal loads (it is read once) and writes the pool with ordinary stores (the
// next verify reads it).
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int COMMIT_THREADS = 256;
constexpr int COMMIT_VEC = D * D / 4 / COMMIT_THREADS;   // float4 per thread (16)

__global__ __launch_bounds__(COMMIT_THREADS) void commit_kernel(CommitParams p) {
  const int b = blockIdx.x / p.H;
  const int h = blockIdx.x % p.H;
  const int slot = p.idx[b];
  const int n = p.n_acc[b];
  if (slot < 0 || slot >= p.slots || n < 1 || n > p.T) return;   // uniform per workgroup
  const int64_t HDD = static_cast<int64_t>(D) * D;
  const f32x4* src = reinterpret_cast<const f32x4*>(
      p.inter + ((static_cast<int64_t>(b) * p.T + (n - 1)) * p.H + h) * HDD);
  f32x4* dst = reinterpret_cast<f32x4*>(p.pool + (static_cast<int64_t>(slot) * p.H + h) * HDD);
  f32x4 v[COMMIT_VEC];
#pragma unroll
  for (int i = 0; i < COMMIT_VEC; ++i)
    v[i] = __builtin_nontemporal_load(src + threadIdx.x + COMMIT_THREADS * i);
#pragma unroll
  for (int i = 0; i < COMMIT_VEC; ++i) dst[threadIdx.x + COMMIT_THREADS * i] = v[i];
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.H));
  hipLaunchKernelGGL(commit_kernel, grid, dim3(COMMIT_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace kda
