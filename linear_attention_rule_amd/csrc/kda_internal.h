// Internal declarations shared by the libkda host code and its HIP kernels.
// Device helpers here are small bit-level conversions and the fp32 gate /
// sigmoid / norm pieces every KDA kernel needs (vLLM PR #55737, opening commit
// message: bounded gate, in-kernel q/k L2 norm, beta from raw logits).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

namespace kda {

constexpr int D = 128;             // head_dim (key and value channels)
constexpr int CHUNK = 64;          // prefill chunk length (tokens)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2_EPS = 1e-6f;
constexpr int KDA_MAX_STEPS_INTERNAL = 64;   // == KDA_MAX_VERIFY_STEPS in include/kda.h

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2 (low half = a) with the gfx950 conversion instruction
// (round to nearest even).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)); saturates to exactly 0 or 1 at the ends.
__device__ __forceinline__ float sigmoid_f32(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * LOG2E));
}

// ---------------------------------------------------------------- per-device host state
// One-time set-up per device (function attributes, device properties), kept for the
// life of the process so that no call pays a runtime query after the first one on a
// device.  Only successful results are kept.
constexpr int KDA_MAX_DEVICES = 64;
struct PerDeviceOnce {
  std::mutex mu;
  bool done[KDA_MAX_DEVICES] = {};
  int value[KDA_MAX_DEVICES] = {};
  // Runs f(&value) for the current device unless it already succeeded there.
  template <class F>
  hipError_t run(F&& f, int* out = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= KDA_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
      int v = 0;
      e = f(dev, &v);
      if (e != hipSuccess) return e;
      value[dev] = v;
      done[dev] = true;
    }
    if (out) *out = value[dev];
    return hipSuccess;
  }
};

// Compute units of the current device (looked up once per device).
hipError_t current_device_cus(int* cus);

// ---------------------------------------------------------------- launch parameters
struct VerifyParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  const float* pool;
  const int32_t* idx;
  float* inter;
  uint16_t* out;
  const int32_t* out_idx;  // output row of each token, or null (row = token)
  int64_t out_rows;        // rows of out addressable through out_idx
  float lb_log2e;      // lower_bound * log2(e): gate computed in log2 units
  float scale;
  int B, T, H, slots;
  int64_t q_st, k_st, v_st, g_st, b_st, o_st;
  // Output-gate sigmoid RMSNorm fused into the output store (null gate: plain output).
  // gate and rstd rows are the output rows the tokens' outputs go to.
  const uint16_t* out_gate;
  const float* norm_w;
  float* rstd;
  float norm_eps;
  int64_t og_st;
};

struct NormParams {
  const uint16_t* x;
  const uint16_t* gate;
  const float* weight;
  uint16_t* y;
  float* rstd;
  float eps;
  int tokens, H;
  int64_t x_st, g_st, y_st;
};

// Conv prefill work split: one workgroup per (CONV_ROWS-token row slot, CONV_CPB-channel
// block); sequence n owns row slots from cu[n] / CONV_ROWS + n on.
constexpr int CONV_ROWS = 16;
constexpr int CONV_CPB = 2048;
inline int64_t conv_prefill_workgroups(int N, int T_total, int C) {
  return (static_cast<int64_t>(T_total) / CONV_ROWS + N) * ((C + CONV_CPB - 1) / CONV_CPB);
}

struct ConvParams {
  const uint16_t* x;
  const uint16_t* weight;    // [C, W] bf16
  const uint16_t* bias;      // [C] bf16 or null
  const int32_t* cu;         // prefill: cu_seqlens
  uint16_t* state;           // windows [slots, W-1, C] (prefill: updated; update: read only)
  const int32_t* state_idx;
  uint16_t* inter;           // update: windows after each token [B, T, W-1, C]
  uint16_t* y;
  int N, T_total, T, C, W, slots;
  bool silu;
  int64_t x_st, y_st;
};

struct CommitParams {
  const float* inter;
  const int32_t* idx;
  const int32_t* n_acc;
  float* pool;
  int B, T, H, slots;
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu;
  const float* init;
  const int32_t* init_idx;
  uint16_t* out;
  const int32_t* out_idx;  // output row of each token, or null (row = token)
  int64_t out_rows;        // rows of out addressable through out_idx
  float* final_state;
  float* seg_ws;           // segment-parallel scan states, or null (not available)
  int seg_G;               // segments per sequence (set by launch_prefill; 1 = none)
  unsigned char* work;  // chunk records
  float lb_log2e;
  float scale;
  int N, T_total, H, num_slots_chunk, init_rows;
  int64_t q_st, k_st, v_st, g_st, b_st, o_st;
};

// Chunk record written by the intra-chunk kernel and read by the state-scan kernel.
// 60 fp16 MFMA fragments of 1 KiB (64 lanes x 8 halves) + Gamma_C (128 fp32) + pad.
constexpr int REC_FRAGS = 60;
constexpr int REC_BYTES = 61 * 1024;
constexpr int FR_KG = 0;    // -(k^ * Gamma), A operand [token x key], (tb, s): 16
constexpr int FR_TP = 16;   // T' = (I+A)^-1 diag(beta), A operand [token x token]: 6
constexpr int FR_QG = 22;   // scale * q^ * Gamma, B operand of O^T [key x token]: 16
constexpr int FR_PM = 38;   // scale * tril(P), B operand of O^T [token x token]: 6
constexpr int FR_KC = 44;   // K_C^T, A operand [key x token], (cb, s'): 16
constexpr int REC_GAMMA_OFF = REC_FRAGS * 1024;

inline int64_t chunk_slots(int N, int T_total) { return static_cast<int64_t>(T_total / CHUNK) + N; }

// Launchers (enqueue only; return the hipGetLastError() of the launch).
hipError_t launch_verify(const VerifyParams& p, hipStream_t s);
hipError_t launch_commit(const CommitParams& p, hipStream_t s);
// Gated RMSNorm: one short-lived workgroup per NORM_ROWS_PER_WG rows.
constexpr int NORM_ROWS_PER_WG = 32;
inline int64_t norm_workgroups(int64_t rows) { return (rows + NORM_ROWS_PER_WG - 1) / NORM_ROWS_PER_WG; }
hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t s);
hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t s);
hipError_t launch_conv_update(const ConvParams& p, hipStream_t s);
// Prefill phases: bit 0 = intra-chunk kernel, bit 1 = state-scan kernel.
constexpr int PHASE_INTRA = 1;
constexpr int PHASE_SCAN = 2;
hipError_t launch_prefill(const PrefillParams& p, int phases, hipStream_t s);
// The intra-chunk kernel alone (called by launch_prefill).
hipError_t launch_prefill_intra(const PrefillParams& p, hipStream_t s);

// Segment-parallel scan: at most SEG_MAX segments per sequence, used only when
// N * H <= SEG_MAX_PAIRS (the workspace holds SEG_SLOTS states per pair then).
constexpr int SEG_MAX = 8;
constexpr int SEG_SLOTS = 3 * SEG_MAX - 5;
constexpr int SEG_MIN_CHUNKS = 4;
constexpr int SEG_MAX_PAIRS = 32;
// Segments the scan uses for these shapes on a device with `cus` CUs (1 = none).
int prefill_segments(int N, int T_total, int H, int cus);
// Workspace bytes: the chunk records, then (when N * H <= SEG_MAX_PAIRS) the segment states.
inline int64_t prefill_record_bytes(int N, int T_total, int H) {
  return chunk_slots(N, T_total) * H * REC_BYTES;
}
inline int64_t prefill_segment_bytes(int N, int H) {
  const int64_t pairs = static_cast<int64_t>(N) * H;
  return pairs <= SEG_MAX_PAIRS ? pairs * SEG_SLOTS * D * D * 4 : 0;
}

// Fixed per-device scratch of the allocation-free prefill (kda_scratch.hip); equal to
// KDA_NOALLOC_SCRATCH_BYTES in include/kda.h.
constexpr int64_t NOALLOC_SCRATCH_BYTES = int64_t{128} << 20;
// Device address of this device's scratch array (looked up once per device).
hipError_t noalloc_scratch(void** out);

}  // namespace kda
