// Fused multi-step KDA verify for gfx950.
//
// Role: the one-launch verify of TensorRT-LLM PR #21179 ("GLM-5.3-Flash FP8
// performance fixes on Hopper", fused-verify commit message): every draft step
// of a row runs in one call, the state starts from the read-only pool and the
// state after each step is written to its own row of the intermediate buffer.
//
// Two forms of the same recurrence (the bounded-gate KDA step of vLLM PR #55737,
// opening commit message and "Purpose"), chosen by the number of (row, head) pairs:
//
// Step form (many pairs, bandwidth-bound; also the fused output norm).  A workgroup
// of 256 threads takes one item (row b, head h, value tile of BV = 32 or 128 columns)
// at a time (one workgroup per item, or with many 128-column items one per CU looping):
// the [128 x BV] fp32 state stays in registers for all T steps; thread (rg, cl) owns
// rows rg*R .. rg*R+R-1 and value columns 4cl .. 4cl+3, so every store of a state row
// segment is a contiguous BV*4-byte run and a wave writes whole 128-byte lines.
// Per step the two key-direction reductions r = S^T k^ and y = S^T q^ share one pass
// over the decayed state; the output then needs no second pass:
// o = scale * (y + (k^ . q^) u) with u = beta (v - r), because the update adds k^ u^T.
//
// Block form (few pairs, latency-bound).  The step form pays one reduction across
// the workgroup and one barrier per step.  Over a block of up to 8 steps the same
// results follow from the state at the block start, S_0 (the WY/UT form of the
// chunked algorithm on an 8-token chunk):
//   Gamma_t = prod_{s <= t} alpha_s (per key, within the block),
//   X_t = S_0^T (Gamma_t . k^_t),  Y_t = S_0^T (Gamma_t . q^_t),
//   A_ti = sum_j k^_t k^_i Gamma_t / Gamma_i (i < t),
//   QK_ti = sum_j q^_t k^_i Gamma_t / Gamma_i (i <= t),
//   u = (I + diag(beta) A)^-1 diag(beta) (v - X),
//   o_t = scale (Y_t + sum_{i <= t} QK_ti u_i),
// and then S_t = alpha_t . S_{t-1} + k^_t u_t^T is a purely per-row update.  So a
// block takes one batch of key-direction sums (all of its steps reduced together)
// and a tiny 8x8 solve, and the state rows stream out with no cross-lane work
// between steps.
//
// Both forms are bound by the fp32 state writes (T x 64 KiB per (b, h)), so they use
// non-temporal stores: nothing reads them back in this call.
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------------------
// Step form
//
// NORM: the output-gate sigmoid RMSNorm of each output row is applied before the store
// (SGLang PR #42489, "Modifications": the sigmoid RMSNorm tuned together with the
// recurrence).  It needs whole rows, so it runs with 128-column tiles only: each step
// leaves its fp32 output row in LDS (in the step's dead decay-table row), and after the
// last step groups of 32 threads normalise the rows and store y = o * rstd * weight *
// sigmoid(gate), with the gate rows staged in the prologue.
template <int BV, bool NORM, bool LOOP>
__global__ __launch_bounds__(256) void verify_step_kernel(VerifyParams p) {
  constexpr int NCG = BV / 4;      // column groups (float4) per state row
  constexpr int NRG = 256 / NCG;   // row groups
  constexpr int R = D / NRG;       // rows per thread
  constexpr int NVT = D / BV;      // value tiles per head
  static_assert(R >= 1 && D % NRG == 0, "bad tile");
  static_assert(!NORM || BV == D, "the fused norm needs whole rows");

  extern __shared__ float smem[];
  const int T = p.T;
  float* s_alpha = smem;              // [T][128]
  float* s_khat = s_alpha + T * D;    // [T][128]
  float* s_qhat = s_khat + T * D;     // [T][128]
  float* s_v = s_qhat + T * D;        // [T][BV]
  float* s_beta = s_v + T * BV;       // [T]
  float* s_kq = s_beta + T;           // [T]
  float* s_part = s_kq + T;           // [2 parity][4 waves][2 (r, y)][BV]
  int* s_orow = reinterpret_cast<int*>(s_part + 2 * 4 * 2 * BV);   // [T] output rows
  // NORM: the raw bf16 output-gate rows [T][128], 16-byte aligned after s_orow
  uint16_t* s_gate = reinterpret_cast<uint16_t*>(
      reinterpret_cast<uintptr_t>(s_orow + T + 3) & ~static_cast<uintptr_t>(15));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // LOOP: fewer workgroups than items (row, head, value tile); each workgroup takes items
  // gridDim.x apart and loads the next item's pool state into registers when the
  // current item's steps begin, so its pool reads overlap its own state writes instead
  // of all reads queueing at the start of the call.  Otherwise one item per workgroup,
  // its state gathered after the prologue.
  const int nitems = p.B * p.H * NVT;
  const int cl = tid % NCG;
  const int rg = tid / NCG;
  const int row0 = rg * R;
  const int64_t head_elems = static_cast<int64_t>(D) * D;
  auto state_src = [&](int it) -> const float* {   // this thread's rows, or null (padding)
    const int tile = it % NVT, rest = it / NVT, hh = rest % p.H, bb = rest / p.H;
    const int sl = p.idx[bb];
    if (sl < 0 || sl >= p.slots) return nullptr;
    return p.pool + (static_cast<int64_t>(sl) * p.H + hh) * head_elems +
           static_cast<int64_t>(row0) * D + tile * BV + 4 * cl;
  };
  auto load_state = [&](int it, float4 (&dst)[R]) {
    const float* src = it < nitems ? state_src(it) : nullptr;
    if (src) {
#pragma unroll
      for (int j = 0; j < R; ++j) dst[j] = *reinterpret_cast<const float4*>(src + j * D);
    }
  };
  float4 Sn[R];
  auto run_item = [&](const int item) {
    int blk = item;
    const int vt = blk % NVT;
    blk /= NVT;
    const int h = blk % p.H;
    const int b = blk / p.H;
    const int v0 = vt * BV;

    const int slot = p.idx[b];
    if (slot < 0 || slot >= p.slots) {
      // Padding row: zero outputs (normalised or not), no state rows written; the norm's
      // rstd of a zero row is 1/sqrt(eps).
      for (int e = tid; e < T * BV; e += 256) {
        const int t = e / BV, c = e % BV;
        int64_t orow = static_cast<int64_t>(b) * T + t;
        if (p.out_idx) orow = p.out_idx[orow];
        if (orow >= 0 && orow < p.out_rows) {
          p.out[orow * p.o_st + h * D + v0 + c] = 0;
          if (NORM && c == 0 && p.rstd) p.rstd[orow * p.H + h] = __builtin_amdgcn_rsqf(p.norm_eps);
        }
      }
      if (LOOP) load_state(item + gridDim.x, Sn);
      return;
    }

    // ---------------- prologue: per-token norms, gates and beta into LDS.
    const float eA = __builtin_amdgcn_exp2f(p.A_log[h] * LOG2E);
    const float2 dtb = *reinterpret_cast<const float2*>(p.dt_bias + h * D + 2 * lane);
    for (int t = wave; t < T; t += 4) {
      const int64_t tok = static_cast<int64_t>(b) * T + t;
      const uint32_t qw = *reinterpret_cast<const uint32_t*>(p.q + tok * p.q_st + h * D + 2 * lane);
      const uint32_t kw = *reinterpret_cast<const uint32_t*>(p.k + tok * p.k_st + h * D + 2 * lane);
      const uint32_t gw = *reinterpret_cast<const uint32_t*>(p.g + tok * p.g_st + h * D + 2 * lane);
      const float q0 = bf16lo_to_f32(qw), q1 = bf16hi_to_f32(qw);
      const float k0 = bf16lo_to_f32(kw), k1 = bf16hi_to_f32(kw);
      const float g0 = bf16lo_to_f32(gw), g1 = bf16hi_to_f32(gw);
      const float ssq = wave_sum(q0 * q0 + q1 * q1);
      const float ssk = wave_sum(k0 * k0 + k1 * k1);
      const float sqk = wave_sum(q0 * k0 + q1 * k1);
      const float rq = __builtin_amdgcn_rsqf(ssq + L2_EPS);
      const float rk = __builtin_amdgcn_rsqf(ssk + L2_EPS);
      const float a0 = __builtin_amdgcn_exp2f(p.lb_log2e * sigmoid_f32(eA * (g0 + dtb.x)));
      const float a1 = __builtin_amdgcn_exp2f(p.lb_log2e * sigmoid_f32(eA * (g1 + dtb.y)));
      *reinterpret_cast<float2*>(s_alpha + t * D + 2 * lane) = make_float2(a0, a1);
      *reinterpret_cast<float2*>(s_khat + t * D + 2 * lane) = make_float2(k0 * rk, k1 * rk);
      *reinterpret_cast<float2*>(s_qhat + t * D + 2 * lane) = make_float2(q0 * rq, q1 * rq);
      if (2 * lane < BV) {
        const uint32_t vw =
            *reinterpret_cast<const uint32_t*>(p.v + tok * p.v_st + h * D + v0 + 2 * lane);
        s_v[t * BV + 2 * lane] = bf16lo_to_f32(vw);
        s_v[t * BV + 2 * lane + 1] = bf16hi_to_f32(vw);
      }
      if (lane == 0) {
        s_beta[t] = sigmoid_f32(bf16_to_f32(p.beta[tok * p.b_st + h]));
        s_kq[t] = sqk * rq * rk;
      }
      if (NORM) {
        // the output gate of this token's output row (rows outside the output are never
        // stored; their gate is not read)
        const int64_t orow = p.out_idx ? static_cast<int64_t>(p.out_idx[tok]) : tok;
        uint32_t gw2 = 0;
        if (orow >= 0 && orow < p.out_rows)
          gw2 = *reinterpret_cast<const uint32_t*>(p.out_gate + orow * p.og_st + h * D + 2 * lane);
        *reinterpret_cast<uint32_t*>(s_gate + t * D + 2 * lane) = gw2;
      }
    }

    // Output row of each step (the scatter index, when given).
    for (int t = tid; t < T; t += 256) {
      const int bt = b * T + t;
      s_orow[t] = p.out_idx ? p.out_idx[bt] : bt;
    }

    // ---------------- the start state (gathered during the previous item when looping).
    float4 S[R];
    if (LOOP) {
#pragma unroll
      for (int j = 0; j < R; ++j) S[j] = Sn[j];
    } else {
      const float* src = p.pool + (static_cast<int64_t>(slot) * p.H + h) * head_elems +
                         static_cast<int64_t>(row0) * D + v0 + 4 * cl;
#pragma unroll
      for (int j = 0; j < R; ++j) S[j] = *reinterpret_cast<const float4*>(src + j * D);
    }
    __syncthreads();
    if (LOOP) load_state(item + gridDim.x, Sn);

    // ---------------- the T steps.
    for (int t = 0; t < T; ++t) {
      const float* al = s_alpha + t * D + row0;
      const float* kh = s_khat + t * D + row0;
      const float* qh = s_qhat + t * D + row0;
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f), y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float a = al[j], kk = kh[j], qq = qh[j];
        S[j].x *= a; S[j].y *= a; S[j].z *= a; S[j].w *= a;
        r.x += S[j].x * kk; r.y += S[j].y * kk; r.z += S[j].z * kk; r.w += S[j].w * kk;
        y.x += S[j].x * qq; y.y += S[j].y * qq; y.z += S[j].z * qq; y.w += S[j].w * qq;
      }
#pragma unroll
      for (int off = NCG; off < 64; off <<= 1) {
        r.x += __shfl_xor(r.x, off); r.y += __shfl_xor(r.y, off);
        r.z += __shfl_xor(r.z, off); r.w += __shfl_xor(r.w, off);
        y.x += __shfl_xor(y.x, off); y.y += __shfl_xor(y.y, off);
        y.z += __shfl_xor(y.z, off); y.w += __shfl_xor(y.w, off);
      }
      float* part = s_part + (t & 1) * (4 * 2 * BV);
      if (lane < NCG) {
        *reinterpret_cast<float4*>(part + (wave * 2 + 0) * BV + 4 * cl) = r;
        *reinterpret_cast<float4*>(part + (wave * 2 + 1) * BV + 4 * cl) = y;
      }
      __syncthreads();
      float4 rr = make_float4(0.f, 0.f, 0.f, 0.f), yy = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 a = *reinterpret_cast<const float4*>(part + (w * 2 + 0) * BV + 4 * cl);
        const float4 c = *reinterpret_cast<const float4*>(part + (w * 2 + 1) * BV + 4 * cl);
        rr.x += a.x; rr.y += a.y; rr.z += a.z; rr.w += a.w;
        yy.x += c.x; yy.y += c.y; yy.z += c.z; yy.w += c.w;
      }
      const float4 vv = *reinterpret_cast<const float4*>(s_v + t * BV + 4 * cl);
      const float be = s_beta[t], kq = s_kq[t];
      float4 u;
      u.x = be * (vv.x - rr.x); u.y = be * (vv.y - rr.y);
      u.z = be * (vv.z - rr.z); u.w = be * (vv.w - rr.w);

      float* dst = p.inter +
                   ((static_cast<int64_t>(b) * T + t) * p.H + h) * head_elems +
                   static_cast<int64_t>(row0) * D + v0 + 4 * cl;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float kk = kh[j];
        S[j].x += kk * u.x; S[j].y += kk * u.y; S[j].z += kk * u.z; S[j].w += kk * u.w;
        const f32x4 sv = {S[j].x, S[j].y, S[j].z, S[j].w};
        __builtin_nontemporal_store(sv, reinterpret_cast<f32x4*>(dst + j * D));
      }
      if (rg == 0) {
        const float s = p.scale;
        const float4 o = make_float4(s * (yy.x + kq * u.x), s * (yy.y + kq * u.y),
                                     s * (yy.z + kq * u.z), s * (yy.w + kq * u.w));
        if (NORM) {
          // Row t of the decay table is dead once this step's barrier has passed (every
          // thread read its entries before it): the fp32 output row waits there for the norm.
          *reinterpret_cast<float4*>(s_alpha + t * D + 4 * cl) = o;
        } else {
          const int64_t orow = s_orow[t];
          if (orow >= 0 && orow < p.out_rows)
            *reinterpret_cast<uint2*>(p.out + orow * p.o_st + h * D + v0 + 4 * cl) =
                make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
        }
      }
    }
    if (NORM) {
      // The norm of every output row after the last step, off the steps' critical path:
      // groups of 32 threads take one row each (4 channels per thread), reduce its squares
      // across the group and store y = o * rstd * weight * sigmoid(gate).
      __syncthreads();
      const int grp = tid >> 5, c4 = 4 * (tid & 31);
      const float4 w4 = *reinterpret_cast<const float4*>(p.norm_w + c4);
      for (int t = grp; t < T; t += 8) {
        const float4 o = *reinterpret_cast<const float4*>(s_alpha + t * D + c4);
        float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off);
        const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.norm_eps);
        const uint2 gr = *reinterpret_cast<const uint2*>(s_gate + t * D + c4);
        const float y0 = o.x * rs * w4.x * sigmoid_f32(bf16lo_to_f32(gr.x));
        const float y1 = o.y * rs * w4.y * sigmoid_f32(bf16hi_to_f32(gr.x));
        const float y2 = o.z * rs * w4.z * sigmoid_f32(bf16lo_to_f32(gr.y));
        const float y3 = o.w * rs * w4.w * sigmoid_f32(bf16hi_to_f32(gr.y));
        const int64_t orow = s_orow[t];
        if (orow >= 0 && orow < p.out_rows) {
          *reinterpret_cast<uint2*>(p.out + orow * p.o_st + h * D + c4) =
              make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
          if ((tid & 31) == 0 && p.rstd) p.rstd[orow * p.H + h] = rs;
        }
      }
    }
  };
  if (LOOP) {
    load_state(blockIdx.x, Sn);
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
      if (item != static_cast<int>(blockIdx.x))
        __syncthreads();   // the previous item's LDS tables are no longer read
      run_item(item);
    }
  } else {
    run_item(blockIdx.x);
  }
}

template <int BV, bool NORM>
size_t verify_lds_bytes(int T) {
  const size_t base = sizeof(float) * (static_cast<size_t>(T) * (3 * D + BV) + 3 * T + 2 * 4 * 2 * BV);
  // NORM: the gate rows as bf16 after 16-byte alignment (fits 160 KiB at 64 steps)
  return NORM ? ((base + 15) & ~size_t{15}) + static_cast<size_t>(T) * D * 2 : base;
}
static_assert(sizeof(float) * (64 * (3 * D + D) + 3 * 64 + 2 * 4 * 2 * D) + 16 + 64 * D * 2 <=
                  160 * 1024,
              "the fused-norm verify's LDS at the largest step count exceeds 160 KiB");

template <int BV, bool NORM>
hipError_t launch_verify_bv(const VerifyParams& p, hipStream_t s) {
  const size_t lds = verify_lds_bytes<BV, NORM>(p.T);
  // The LDS limit for the largest step count is set once per device, not per call.
  static PerDeviceOnce attr_once;
  hipError_t e = attr_once.run([](int, int*) {
    const int bytes = static_cast<int>(verify_lds_bytes<BV, NORM>(KDA_MAX_STEPS_INTERNAL));
    hipError_t r =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_step_kernel<BV, NORM, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (r == hipSuccess)
      r = hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_step_kernel<BV, NORM, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return r;
  });
  if (e != hipSuccess) return e;
  int cus = 0;
  if ((e = current_device_cus(&cus)) != hipSuccess) return e;
  // 128-column tiles with at least two items per CU: one looping workgroup per CU (64 x 8
  // x 16 heads, 1024 items: warm 108.6 -> 106.6 us, after a prefill 124.5 -> 118.1 us,
  // after a 1 GiB overwrite 143 -> 134 us, against one workgroup per item; 192, 320, 384
  // or 512 workgroups were slower; 512 and 768 items: 59.9 -> 59.2, 84.3 -> 82.6 us).
  // Otherwise one workgroup per item: with fewer items, or with 32-column tiles, whose
  // items are short and latency-bound, looping workgroups were slower (256, 384 items:
  // 33.7 -> 34.8, 45.6 -> 48.5 us; 32-column tiles at 448-960 items: 16.7 -> 24.6,
  // 31.3 -> 45.7 us).
  const int64_t items = static_cast<int64_t>(p.B) * p.H * (D / BV);
  if (BV == D && cus > 0 && items >= 2 * static_cast<int64_t>(cus))
    hipLaunchKernelGGL((verify_step_kernel<BV, NORM, true>), dim3(static_cast<unsigned>(cus)),
                       dim3(256), lds, s, p);
  else
    hipLaunchKernelGGL((verify_step_kernel<BV, NORM, false>), dim3(static_cast<unsigned>(items)),
                       dim3(256), lds, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Block form

constexpr int VB = 8;       // draft steps per block
constexpr int VCOLS = 32;   // value columns per wave

// ---------------------------------------------------------------- cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_XOR3 = 0x1B;          // quad_perm [3,2,1,0]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane ^ 7 within 8
constexpr int DPP_ROR8 = 0x128;         // lane ^ 8 within 16

__device__ __forceinline__ float xor4(float x) { return dpp<DPP_XOR3>(dpp<DPP_HALF_MIRROR>(x)); }

// Transposing butterfly levels: the first N values of v, halved across one lane bit.
// A lane with that bit clear keeps values [0, N/2), one with it set keeps [N/2, N), in
// v[0, N/2); each kept value becomes the sum of its own and the partner lane's copy.
// The two v_permlane*_swap levels need no selects: swapping v[i] (upper/odd half) with
// v[i + N/2] (lower/even half) leaves each lane the two copies of its kept value.
template <int N>
__device__ __forceinline__ void tlevel5(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + N / 2]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
template <int N>
__device__ __forceinline__ void tlevel4(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + N / 2]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
// Lane bits 3, 2, 1, 0 (DPP within 16-lane rows).
template <int BIT, int N>
__device__ __forceinline__ void tlevel_dpp(float* v, int lane) {
  const bool hi = (lane >> BIT) & 1;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = hi ? v[i + N / 2] : v[i];
    const float send = hi ? v[i] : v[i + N / 2];
    float got;
    if constexpr (BIT == 3) got = dpp<DPP_ROR8>(send);
    else if constexpr (BIT == 2) got = xor4(send);
    else if constexpr (BIT == 1) got = dpp<DPP_XOR2>(send);
    else got = dpp<DPP_XOR1>(send);
    v[i] = keep + got;
  }
}
__device__ __forceinline__ float sum_bit1(float x) { return x + dpp<DPP_XOR2>(x); }
__device__ __forceinline__ float sum_bit0(float x) { return x + dpp<DPP_XOR1>(x); }

__device__ __forceinline__ float rl(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ float comp(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One workgroup per (row b, head h) and TILES 32-column value tiles (TILES = 4: the
// whole head, as the fused output norm needs), four waves per tile.  Wave (tile, wq)
// owns key rows 32wq .. 32wq+31 of its tile: lane (m, cl) rows 32wq + 4m .. +3 and
// value columns 4cl .. 4cl+3 (16 fp32 registers), so each store instruction covers 8
// rows x 128 bytes.  In the block's solve thread (tile, t, c) owns step t of column c.
//
// NORM: the output-gate sigmoid RMSNorm of each output row is applied before the store
// (SGLang PR #42489, "Modifications"): the solve leaves the fp32 output rows in LDS,
// then groups of 32 threads normalise one row each.
template <int TILES, bool NORM>
__global__ __launch_bounds__(256 * TILES) void verify_block_kernel(VerifyParams p) {
  static_assert(TILES == 1 || TILES == 4, "one tile, or the whole head");
  static_assert(!NORM || TILES == 4, "the fused norm needs whole rows");
  // Per-token tables of the current block.
  __shared__ __attribute__((aligned(16))) float s_k[VB][D];    // k^
  __shared__ __attribute__((aligned(16))) float s_a[VB][D];    // alpha
  __shared__ __attribute__((aligned(16))) float s_kt[VB][D];   // Gamma_t . k^_t
  __shared__ __attribute__((aligned(16))) float s_qt[VB][D];   // Gamma_t . q^_t
  __shared__ __attribute__((aligned(16))) float s_kgi[VB][D];  // k^_t / Gamma_t
  // QK (c <= r) and A_cr (c > r) at 8r + c.
  __shared__ float s_aq[64];
  __shared__ float s_beta[VB];
  // Per-wave partial sums X (0) and Y (1) [tile][wq][x/y][step][col]; v and u
  // [step][column of the workgroup].
  __shared__ __attribute__((aligned(16))) float s_part[TILES][4][2][VB][VCOLS];
  __shared__ __attribute__((aligned(16))) float s_v[VB][VCOLS * TILES];
  __shared__ __attribute__((aligned(16))) float s_u[VB][VCOLS * TILES];
  __shared__ int s_orow[VB];
  // NORM: fp32 output rows and the raw bf16 gate rows of the block.
  __shared__ __attribute__((aligned(16))) float s_o[NORM ? VB : 1][D];
  __shared__ __attribute__((aligned(16))) uint16_t s_gate[NORM ? VB : 1][D];

  const int T = p.T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 3;     // row quarter of the tile
  const int tile = wave >> 2;  // tile within the workgroup
  const int vt0 = TILES == 1 ? static_cast<int>(blockIdx.x & 3) : 0;
  const int bh = TILES == 1 ? static_cast<int>(blockIdx.x >> 2) : static_cast<int>(blockIdx.x);
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int v0 = (vt0 + tile) * VCOLS;
  const int m = lane >> 3;
  const int cl = lane & 7;
  const int row0 = 32 * wq + 4 * m;   // this lane's 4 key rows
  // step and column of this thread's v, u and o: tile stile, column sc
  const int stile = tid >> 8, st = (tid >> 5) & 7, sc = tid & 31;
  const int sv0 = (vt0 + stile) * VCOLS, scol = VCOLS * stile + sc;

  const int64_t head_elems = static_cast<int64_t>(D) * D;
  const float scale = p.scale;

  // The block's inputs, loaded one block ahead.  Wave wq of tile 0: gates of every step
  // (the cumulative decay needs them all), q and k of steps wq and wq + 4; threads: v
  // of their (step, column), beta and the output row of step tid.  Steps past nt
  // repeat the last one (they are zeroed, and nothing of them is stored).
  uint32_t gw[VB], qw[2], kw[2];
  uint16_t vb = 0, bb = 0;
  int orow_l = 0;
  auto load_block = [&](int t0) {
    const int nt = min(VB, T - t0);
    const int64_t tok0 = static_cast<int64_t>(b) * T + t0;
    if (tile == 0) {
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        const int64_t tok = tok0 + min(i, nt - 1);
        gw[i] = *reinterpret_cast<const uint32_t*>(p.g + tok * p.g_st + h * D + 2 * lane);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t tok = tok0 + min(wq + 4 * e, nt - 1);
        qw[e] = *reinterpret_cast<const uint32_t*>(p.q + tok * p.q_st + h * D + 2 * lane);
        kw[e] = *reinterpret_cast<const uint32_t*>(p.k + tok * p.k_st + h * D + 2 * lane);
      }
    }
    vb = p.v[(tok0 + min(st, nt - 1)) * p.v_st + h * D + sv0 + sc];
    if (tid < nt) {
      bb = p.beta[(tok0 + tid) * p.b_st + h];
      orow_l = p.out_idx ? p.out_idx[tok0 + tid] : static_cast<int>(tok0 + tid);
    }
  };

  // The slot, the head's constants and the first block's inputs go out together.
  const int slot = p.idx[b];
  const float A_log = p.A_log[h];
  const float2 dtb = *reinterpret_cast<const float2*>(p.dt_bias + h * D + 2 * lane);
  load_block(0);
  if (slot < 0 || slot >= p.slots) {
    // Padding row: zero outputs (normalised or not), no state rows written; the norm's
    // rstd of a zero row is 1/sqrt(eps).
    for (int e = tid; e < T * VCOLS * TILES; e += 256 * TILES) {
      const int t = e / (VCOLS * TILES), c = e % (VCOLS * TILES);
      int64_t orow = static_cast<int64_t>(b) * T + t;
      if (p.out_idx) orow = p.out_idx[orow];
      if (orow >= 0 && orow < p.out_rows) {
        p.out[orow * p.o_st + h * D + vt0 * VCOLS + c] = 0;
        if (NORM && c == 0 && p.rstd) p.rstd[orow * p.H + h] = __builtin_amdgcn_rsqf(p.norm_eps);
      }
    }
    return;
  }
  // The start state, after the first block's loads so that their wait leaves it in
  // flight.
  float4 S[4];
  {
    const float* src = p.pool + (static_cast<int64_t>(slot) * p.H + h) * head_elems +
                       static_cast<int64_t>(row0) * D + v0 + 4 * cl;
#pragma unroll
    for (int j = 0; j < 4; ++j) S[j] = *reinterpret_cast<const float4*>(src + j * D);
  }
  const float eA = __builtin_amdgcn_exp2f(A_log * LOG2E);

  for (int t0 = 0; t0 < T; t0 += VB) {
    const int nt = min(VB, T - t0);
    const int64_t tok0 = static_cast<int64_t>(b) * T + t0;
    s_v[st][scol] = bf16_to_f32(vb);
    if (tid < nt) s_orow[tid] = orow_l;
    if (tid < VB) s_beta[tid] = tid < nt ? sigmoid_f32(bf16_to_f32(bb)) : 0.f;
    if (NORM && tid < 256) {
      // The output-gate rows of the block (rows outside the output are never stored;
      // their gate is not read).
      const int t = tid >> 5, c4 = 4 * (tid & 31);
      if (t < nt) {
        const int64_t orow = p.out_idx ? static_cast<int64_t>(p.out_idx[tok0 + t]) : tok0 + t;
        uint2 g2 = make_uint2(0, 0);
        if (orow >= 0 && orow < p.out_rows)
          g2 = *reinterpret_cast<const uint2*>(p.out_gate + orow * p.og_st + h * D + c4);
        *reinterpret_cast<uint2*>(&s_gate[t][c4]) = g2;
      }
    }

    if (tile == 0) {
      // ---------------- norms of steps wq, wq + 4 (lane: keys 2l, 2l+1): four sums, lane
      // l ends with sum (l >> 4) & 3
      {
        float nv[4];
  #pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float q0 = bf16lo_to_f32(qw[e]), q1 = bf16hi_to_f32(qw[e]);
          const float k0 = bf16lo_to_f32(kw[e]), k1 = bf16hi_to_f32(kw[e]);
          nv[e] = q0 * q0 + q1 * q1;
          nv[2 + e] = k0 * k0 + k1 * k1;
        }
        tlevel5<4>(nv);
        tlevel4<2>(nv);
        float nsum = nv[0] + dpp<DPP_ROR8>(nv[0]);
        nsum += xor4(nsum);
        nsum = sum_bit0(sum_bit1(nsum));

        // Gates and the in-block cumulative log2 decay b_t <= 0 of every step, then the
        // table rows of steps wq and wq + 4.  With G_t = 2^(b_t),
        //   QK_ti = sum_j (G_t q^_t)(k^_i / G_i),  A_ti = sum_j (G_t k^_t)(k^_i / G_i);
        // the lower bound keeps 1/G below 2^58 over 8 steps.  Uniform conditions are
        // taken as 0/1 factors and selects: no branches between the transcendentals.
        float la[VB][2], bc[VB][2];
        float run0 = 0.f, run1 = 0.f;
  #pragma unroll
        for (int i = 0; i < VB; ++i) {
          const float live = i < nt ? p.lb_log2e : 0.f;
          la[i][0] = live * sigmoid_f32(eA * (bf16lo_to_f32(gw[i]) + dtb.x));
          la[i][1] = live * sigmoid_f32(eA * (bf16hi_to_f32(gw[i]) + dtb.y));
          run0 += la[i][0];
          run1 += la[i][1];
          bc[i][0] = run0;
          bc[i][1] = run1;
        }
  #pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = wq + 4 * e;
          float l0 = la[4 * e][0], l1 = la[4 * e][1], r0 = bc[4 * e][0], r1 = bc[4 * e][1];
  #pragma unroll
          for (int j = 1; j < 4; ++j) {
            l0 = wq == j ? la[4 * e + j][0] : l0;
            l1 = wq == j ? la[4 * e + j][1] : l1;
            r0 = wq == j ? bc[4 * e + j][0] : r0;
            r1 = wq == j ? bc[4 * e + j][1] : r1;
          }
          const float live = i < nt ? 1.f : 0.f;
          const float rq = live * __builtin_amdgcn_rsqf(rl(nsum, 16 * e) + L2_EPS);
          const float rk = live * __builtin_amdgcn_rsqf(rl(nsum, 16 * (2 + e)) + L2_EPS);
          const float k0 = bf16lo_to_f32(kw[e]) * rk, k1 = bf16hi_to_f32(kw[e]) * rk;
          const float q0 = bf16lo_to_f32(qw[e]) * rq, q1 = bf16hi_to_f32(qw[e]) * rq;
          const float g0 = __builtin_amdgcn_exp2f(r0), g1 = __builtin_amdgcn_exp2f(r1);
          const float gi0 = __builtin_amdgcn_exp2f(-r0), gi1 = __builtin_amdgcn_exp2f(-r1);
          *reinterpret_cast<float2*>(&s_k[i][2 * lane]) = make_float2(k0, k1);
          *reinterpret_cast<float2*>(&s_a[i][2 * lane]) =
              make_float2(__builtin_amdgcn_exp2f(l0), __builtin_amdgcn_exp2f(l1));
          *reinterpret_cast<float2*>(&s_kt[i][2 * lane]) = make_float2(g0 * k0, g1 * k1);
          *reinterpret_cast<float2*>(&s_qt[i][2 * lane]) = make_float2(g0 * q0, g1 * q1);
          *reinterpret_cast<float2*>(&s_kgi[i][2 * lane]) = make_float2(gi0 * k0, gi1 * k1);
        }
      }
    }
    __syncthreads();   // the tables, beta and output rows complete
    if (tile == 0) {

      // ---------------- slots 8r + c of rows r = 2wq, 2wq + 1: QK_rc (c <= r) or A_cr
      // (c > r); lane l ends with slot 16wq + (l >> 2)
      {
        float aq[16];
  #pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = 2 * wq + rr;
          const float2 qgr = *reinterpret_cast<const float2*>(&s_qt[r][2 * lane]);
          const float2 kgir = *reinterpret_cast<const float2*>(&s_kgi[r][2 * lane]);
  #pragma unroll
          for (int c = 0; c < VB; ++c) {
            const float2 kgic = *reinterpret_cast<const float2*>(&s_kgi[c][2 * lane]);
            const float2 kgc = *reinterpret_cast<const float2*>(&s_kt[c][2 * lane]);
            // both candidates, chosen by a bit mask: no branch on the uniform r (the
            // candidate not taken can be as large as 2^58, so no arithmetic blend)
            const float vq = qgr.x * kgic.x + qgr.y * kgic.y;
            const float va = kgc.x * kgir.x + kgc.y * kgir.y;
            const uint32_t mq = c <= r ? 0xffffffffu : 0u;
            aq[8 * rr + c] = __uint_as_float((__float_as_uint(vq) & mq) | (__float_as_uint(va) & ~mq));
          }
        }
        tlevel5<16>(aq);
        tlevel4<8>(aq);
        tlevel_dpp<3, 4>(aq, lane);
        tlevel_dpp<2, 2>(aq, lane);
        const float av = sum_bit0(sum_bit1(aq[0]));
        if ((lane & 3) == 0) s_aq[16 * wq + (lane >> 2)] = av;
      }
    }
    // ---------------- X and Y: this wave's 32 rows, every step of the block; after the
    // butterfly lane (m, cl) holds step m, columns 4cl .. 4cl+3.
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const float(*tab)[D] = pass == 0 ? s_kt : s_qt;
      float acc[4 * VB];
#pragma unroll
      for (int t = 0; t < VB; ++t) {
        const float4 w4 = *reinterpret_cast<const float4*>(&tab[t][row0]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[4 * t + c] = w4.x * comp(S[0], c) + w4.y * comp(S[1], c) + w4.z * comp(S[2], c) +
                           w4.w * comp(S[3], c);
      }
      tlevel5<32>(acc);
      tlevel4<16>(acc);
      tlevel_dpp<3, 8>(acc, lane);
      *reinterpret_cast<float4*>(&s_part[tile][wq][pass][m][4 * cl]) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();   // QK / A and the partial sums complete

    // ---------------- the solve, in thread (t, c): d = v - X for every step of column c,
    // u by forward substitution of (I + diag(beta) A) u = diag(beta) d (every thread of
    // the column runs the whole chain and keeps u_t), o_t = scale (Y_t + sum QK_ti u_i).
    {
      float u[VB], r[VB];
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        float x = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) x += s_part[stile][q][0][i][sc];
        r[i] = s_v[i][scol] - x;
      }
      // beta and A are the same in every lane: held in scalar registers
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        u[i] = uniform(s_beta[i]) * r[i];
#pragma unroll
        for (int j = i + 1; j < VB; ++j) r[j] -= uniform(s_aq[8 * i + j]) * u[i];
      }
      float ut = u[0], o = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) o += s_part[stile][q][1][st][sc];
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        ut = st == i ? u[i] : ut;
        const float qa = s_aq[8 * st + i];      // QK_{st,i} for i <= st (A beyond)
        o += (i <= st ? qa : 0.f) * u[i];
      }
      s_u[st][scol] = ut;
      if (st < nt) {
        if (NORM) {
          s_o[st][sv0 + sc] = o * scale;
        } else {
          const int64_t orow = s_orow[st];
          if (orow >= 0 && orow < p.out_rows)
            p.out[orow * p.o_st + h * D + sv0 + sc] = static_cast<uint16_t>(pack_bf16x2(o * scale, 0.f));
        }
      }
    }
    __syncthreads();   // u complete; NORM: the output rows in LDS

    if (NORM && tid < 256) {
      // groups of 32 threads: one output row each (4 channels per thread)
      const int t = tid >> 5, c4 = 4 * (tid & 31);
      if (t < nt) {
        const float4 o = *reinterpret_cast<const float4*>(&s_o[t][c4]);
        float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off);
        const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.norm_eps);
        const float4 w4 = *reinterpret_cast<const float4*>(p.norm_w + c4);
        const uint2 gr = *reinterpret_cast<const uint2*>(&s_gate[t][c4]);
        const float y0 = o.x * rs * w4.x * sigmoid_f32(bf16lo_to_f32(gr.x));
        const float y1 = o.y * rs * w4.y * sigmoid_f32(bf16hi_to_f32(gr.x));
        const float y2 = o.z * rs * w4.z * sigmoid_f32(bf16lo_to_f32(gr.y));
        const float y3 = o.w * rs * w4.w * sigmoid_f32(bf16hi_to_f32(gr.y));
        const int64_t orow = s_orow[t];
        if (orow >= 0 && orow < p.out_rows) {
          *reinterpret_cast<uint2*>(p.out + orow * p.o_st + h * D + c4) =
              make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
          if ((tid & 31) == 0 && p.rstd) p.rstd[orow * p.H + h] = rs;
        }
      }
    }

    if (t0 + VB < T) load_block(t0 + VB);   // in flight during the state rows

    // ---------------- the state rows of every step: S_t = alpha_t . S_{t-1} + k^_t u_t^T
    // (the next step's LDS operands are read one step ahead)
    float4 u_n = *reinterpret_cast<const float4*>(&s_u[0][VCOLS * tile + 4 * cl]);
    float4 a_n = *reinterpret_cast<const float4*>(&s_a[0][row0]);
    float4 k_n = *reinterpret_cast<const float4*>(&s_k[0][row0]);
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
      const float4 u = u_n, a4 = a_n, k4 = k_n;
      if (t + 1 < VB) {
        u_n = *reinterpret_cast<const float4*>(&s_u[t + 1][VCOLS * tile + 4 * cl]);
        a_n = *reinterpret_cast<const float4*>(&s_a[t + 1][row0]);
        k_n = *reinterpret_cast<const float4*>(&s_k[t + 1][row0]);
      }
      float* dst = p.inter + ((tok0 + t) * p.H + h) * head_elems +
                   static_cast<int64_t>(row0) * D + v0 + 4 * cl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = comp(a4, j), kk = comp(k4, j);
        S[j].x = a * S[j].x + kk * u.x;
        S[j].y = a * S[j].y + kk * u.y;
        S[j].z = a * S[j].z + kk * u.z;
        S[j].w = a * S[j].w + kk * u.w;
        const f32x4 sv = {S[j].x, S[j].y, S[j].z, S[j].w};
        __builtin_nontemporal_store(sv, reinterpret_cast<f32x4*>(dst + j * D));
      }
    }
    // The block's tables and rows are read before the next block overwrites them.
    if (t0 + VB < T) __syncthreads();
  }
}

template <int TILES, bool NORM>
hipError_t launch_verify_block(const VerifyParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B) * p.H * (TILES == 1 ? D / VCOLS : 1));
  hipLaunchKernelGGL((verify_block_kernel<TILES, NORM>), grid, dim3(256 * TILES), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const int64_t pairs = static_cast<int64_t>(p.B) * p.H;
  if (p.out_gate) {
    // The fused output norm needs whole 128-column rows in one workgroup: the block
    // form with the head's four tiles in one workgroup for few pairs (15.2 against
    // 17.8 us per call at batch 1 of 16 heads, 14.9 against 17.4 at 64 pairs), else
    // the step form.
    if (pairs <= 64) return launch_verify_block<4, true>(p, s);
    return launch_verify_bv<128, true>(p, s);
  }
  // Few (row, head) pairs: the block form, a workgroup per 32-column tile (measured on
  // MI355X at 8 steps and 16 heads: 7.9 against 11.7 us of kernel time at batch 1).  As
  // the pairs grow the state writes bound the call, and the step form, which
  // interleaves them with each step's work, keeps the store path busier (per call,
  // 14.1 against 14.7 us at 96 pairs, 15.2 against 14.9 at 112): 32-column tiles while
  // there are fewer than 256 pairs, whole 512-byte rows after.
  if (pairs <= 96) return launch_verify_block<1, false>(p, s);
  if (pairs < 256) return launch_verify_bv<32, false>(p, s);
  return launch_verify_bv<128, false>(p, s);
}

}  // namespace kda
