// Short causal convolution on the q / k / v projections for gfx950: the depthwise
// causal conv of TensorRT-LLM PR #21179 (fused-verify commit message: three short
// convolutions per draft step, run as one packed causal_conv1d_update that writes
// each step's window into intermediate_conv_window from a gathered copy of the pool
// rows, inputs read in place from the fused projection) and vLLM PR #55737 ("Notes for
// review": the conv per q/k/v into separate buffers).  Per channel c, with W <= 4 taps,
//     y_t[c] = act(bias[c] + sum_{i<W} weight[c, i] * x_{t-W+1+i}[c]),
// act = SiLU or the identity; a window holds the W-1 previous inputs, oldest first.
// All three kernels are bound by HBM; each thread owns 8 consecutive channels
// (16 bytes per token row), so a wave moves 1 KiB runs of a token row.
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int CONV_THREADS = 256;
constexpr int CONV_CPT = 8;                                 // channels per thread
static_assert(CONV_CPB == CONV_THREADS * CONV_CPT, "channels per workgroup");
static_assert(CONV_ROWS >= 3, "a row slot after the first reads its W - 1 <= 3 history rows from x");
constexpr int CONV_BATCH = 16;                              // token rows loaded at once

__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
  f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
  f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
  f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
}

struct ConvTaps {
  float w[CONV_CPT][4];   // [channel][tap], taps >= W are zero
  float b[CONV_CPT];
};

template <int W>
__device__ __forceinline__ void load_taps(const ConvParams& p, int c0, ConvTaps& k) {
  // weight [C, W] row-major: the 8 channels' taps are 8W contiguous bf16 = W x 16 bytes.
  const uint4* wp = reinterpret_cast<const uint4*>(p.weight + static_cast<int64_t>(c0) * W);
  float all[8 * W];
#pragma unroll
  for (int q = 0; q < W; ++q) unpack8(wp[q], all + 8 * q);
#pragma unroll
  for (int c = 0; c < CONV_CPT; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) k.w[c][i] = (i < W) ? all[c * W + i] : 0.f;
  if (p.bias) {
    float bb[8];
    unpack8(*reinterpret_cast<const uint4*>(p.bias + c0), bb);
#pragma unroll
    for (int c = 0; c < CONV_CPT; ++c) k.b[c] = bb[c];
  } else {
#pragma unroll
    for (int c = 0; c < CONV_CPT; ++c) k.b[c] = 0.f;
  }
}

// One output row from the current input and the W-1 previous ones (hist[0] oldest),
// hist and x as raw bf16 words; returns the packed bf16 outputs.
template <int W>
__device__ __forceinline__ uint4 conv_row(const ConvTaps& k, const uint4 (&hist)[3], uint4 x,
                                          bool silu) {
  float taps[4][8];
  unpack8(hist[0], taps[0]);
  unpack8(hist[1], taps[1]);
  unpack8(hist[2], taps[2]);
  unpack8(x, taps[3]);
  float y[8];
#pragma unroll
  for (int c = 0; c < CONV_CPT; ++c) {
    // Tap i of W meets input slot 4 - W + i (slots 0..2 history, 3 current).
    float acc = k.b[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < W) acc += k.w[c][i] * taps[4 - W + i][c];
    }
    y[c] = silu ? acc * sigmoid_f32(acc) : acc;
  }
  return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                    pack_bf16x2(y[6], y[7]));
}

// hist <- (hist minus its oldest entry) + x, over the last W-1 slots.
__device__ __forceinline__ void push_hist(uint4 (&hist)[3], uint4 x) {
  hist[0] = hist[1];
  hist[1] = hist[2];
  hist[2] = x;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Prefill outputs: one short-lived workgroup per (16-token row slot, channel block),
// channel blocks fastest in a 1-D grid, so the workgroups running at any moment read
// and write whole token rows; the W-1 history rows before a slot are re-read (mostly
// from L2).  On MI355X at 4 x 8192 tokens x 6144 channels this runs at 160 us against
// 188 us for 64-token slots with the slots fastest.
template <int W>
__global__ __launch_bounds__(CONV_THREADS) void conv_prefill_kernel(ConvParams p) {
  const int cblocks = (p.C + CONV_CPB - 1) / CONV_CPB;
  const int slot = blockIdx.x / cblocks;
  const int c0 = (blockIdx.x % cblocks) * CONV_CPB + threadIdx.x * CONV_CPT;
  // Row-slot map: sequence n owns slots [cu[n]/16 + n, ...); the last n whose first slot
  // is <= this one (binary search on the device, no host sync).
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] / CONV_ROWS + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int cs = p.cu[n], ce = p.cu[n + 1];
  const int jc = slot - (cs / CONV_ROWS + n);
  if (jc * CONV_ROWS >= ce - cs || c0 >= p.C) return;
  const int t0 = cs + jc * CONV_ROWS;
  const int L = min(CONV_ROWS, ce - t0);
  ConvTaps k;
  load_taps<W>(p, c0, k);
  // History: the W-1 inputs before t0 (slots 3 - (W-1) .. 2 of hist; the rest zero).
  uint4 hist[3] = {zero4(), zero4(), zero4()};
  int row = -1;
  if (jc == 0 && p.state) {
    row = p.state_idx ? p.state_idx[n] : n;
    if (row < 0 || row >= p.slots) row = -1;
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int back = 3 - i;                       // hist[i] holds input t0 - back
    if (back > W - 1) continue;
    if (jc > 0) {
      hist[i] = *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(t0 - back) * p.x_st + c0);
    } else if (row >= 0) {
      // window entry (W-1) - back of the sequence's start window
      hist[i] = *reinterpret_cast<const uint4*>(
          p.state + (static_cast<int64_t>(row) * (W - 1) + (W - 1 - back)) * p.C + c0);
    }
  }
  for (int tb = 0; tb < L; tb += CONV_BATCH) {
    uint4 xb[CONV_BATCH];
#pragma unroll
    for (int u = 0; u < CONV_BATCH; ++u) {
      const int t = min(tb + u, L - 1);           // clamped in bounds; extra rows unused
      xb[u] = *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(t0 + t) * p.x_st + c0);
    }
#pragma unroll
    for (int u = 0; u < CONV_BATCH; ++u) {
      if (tb + u < L) {
        *reinterpret_cast<uint4*>(p.y + static_cast<int64_t>(t0 + tb + u) * p.y_st + c0) =
            conv_row<W>(k, hist, xb[u], p.silu);
        push_hist(hist, xb[u]);
      }
    }
  }
}

// Prefill windows: after the outputs (which read the old windows), each in-range window
// becomes the W-1 inputs ending at its sequence's last token, earlier entries coming
// from the old window when the sequence is shorter.  All reads precede the writes of a
// thread, so in-place pools are safe.
template <int W>
__global__ __launch_bounds__(CONV_THREADS) void conv_state_kernel(ConvParams p) {
  const int n = blockIdx.x;
  const int c0 = blockIdx.y * CONV_CPB + threadIdx.x * CONV_CPT;
  if (c0 >= p.C) return;
  const int row = p.state_idx ? p.state_idx[n] : n;
  if (row < 0 || row >= p.slots) return;
  const int cs = p.cu[n], len = p.cu[n + 1] - cs;
  if (len == 0) return;
  constexpr int Wm = W - 1;
  uint4 v[3];
  uint16_t* base = p.state + static_cast<int64_t>(row) * Wm * p.C + c0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    if (j >= Wm) continue;
    const int u = len - Wm + j;                   // token of the sequence, or before it
    v[j] = (u >= 0) ? *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(cs + u) * p.x_st + c0)
                    : *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(j + len) * p.C);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < Wm) *reinterpret_cast<uint4*>(base + static_cast<int64_t>(j) * p.C) = v[j];
}

// Multi-step update: one thread per (row b, step t, 8 channels).  Given its inputs, every
// step of a row is independent: step t reads x_t and the W-1 inputs before it, from the
// row's earlier tokens or, before its first token, from the pool window (read only), and
// writes its output and the window after it.  On MI355X at 64 rows x 8 steps x 6144
// channels: 8.9 us against 11.4 us for one thread per (row, 8 channels) running the
// steps in order (rocprofv3 kernel times; outputs and windows bit-identical).
template <int W>
__global__ __launch_bounds__(CONV_THREADS) void conv_update_kernel(ConvParams p) {
  const int b = blockIdx.x;
  const int t = blockIdx.z;
  const int c0 = blockIdx.y * CONV_CPB + threadIdx.x * CONV_CPT;
  if (c0 >= p.C) return;
  const int T = p.T;
  const int64_t tok = static_cast<int64_t>(b) * T + t;
  const int s = p.state_idx[b];
  if (s < 0 || s >= p.slots) {                    // padding row: zero outputs only
    *reinterpret_cast<uint4*>(p.y + tok * p.y_st + c0) = zero4();
    return;
  }
  ConvTaps k;
  load_taps<W>(p, c0, k);
  constexpr int Wm = W - 1;
  uint4 hist[3] = {zero4(), zero4(), zero4()};   // hist[i] holds input t - (3 - i)
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int back = 3 - i;
    if (back > Wm) continue;
    const int u = t - back;
    hist[i] = (u >= 0)
                  ? *reinterpret_cast<const uint4*>(p.x + (static_cast<int64_t>(b) * T + u) * p.x_st + c0)
                  : *reinterpret_cast<const uint4*>(
                        p.state + (static_cast<int64_t>(s) * Wm + (Wm + u)) * p.C + c0);
  }
  const uint4 xt = *reinterpret_cast<const uint4*>(p.x + tok * p.x_st + c0);
  *reinterpret_cast<uint4*>(p.y + tok * p.y_st + c0) = conv_row<W>(k, hist, xt, p.silu);
  push_hist(hist, xt);
  uint16_t* win = p.inter + (tok * Wm) * p.C + c0;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < Wm) *reinterpret_cast<uint4*>(win + static_cast<int64_t>(j) * p.C) = hist[3 - Wm + j];
}

template <int W>
hipError_t conv_prefill_w(const ConvParams& p, hipStream_t s) {
  const unsigned cblocks = static_cast<unsigned>((p.C + CONV_CPB - 1) / CONV_CPB);
  if (p.T_total > 0) {
    const dim3 grid(static_cast<unsigned>(conv_prefill_workgroups(p.N, p.T_total, p.C)));
    hipLaunchKernelGGL(conv_prefill_kernel<W>, grid, dim3(CONV_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (W > 1 && p.state) {
    hipLaunchKernelGGL(conv_state_kernel<W>, dim3(static_cast<unsigned>(p.N), cblocks),
                       dim3(CONV_THREADS), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int W>
hipError_t conv_update_w(const ConvParams& p, hipStream_t s) {
  const unsigned cblocks = static_cast<unsigned>((p.C + CONV_CPB - 1) / CONV_CPB);
  hipLaunchKernelGGL(conv_update_kernel<W>,
                     dim3(static_cast<unsigned>(p.N), cblocks, static_cast<unsigned>(p.T)),
                     dim3(CONV_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  switch (p.W) {
    case 1: return conv_prefill_w<1>(p, s);
    case 2: return conv_prefill_w<2>(p, s);
    case 3: return conv_prefill_w<3>(p, s);
    default: return conv_prefill_w<4>(p, s);
  }
}

hipError_t launch_conv_update(const ConvParams& p, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  switch (p.W) {
    case 1: return conv_update_w<1>(p, s);
    case 2: return conv_update_w<2>(p, s);
    case 3: return conv_update_w<3>(p, s);
    default: return conv_update_w<4>(p, s);
  }
}

}  // namespace kda
