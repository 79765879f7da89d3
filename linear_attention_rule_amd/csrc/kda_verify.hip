// Fused multi-step KDA verify for gfx950.
//
// Role: the one-launch verify of TensorRT-LLM PR #21179 ("GLM-5.3-Flash FP8
// performance fixes on Hopper", fused-verify commit message): every draft step
// of a row runs in one call, the state starts from the read-only pool and the
// state after each step is written to its own row of the intermediate buffer.
//
// Work split: one workgroup of 256 threads per (row b, head h, value tile).
// The [128 x BV] fp32 state tile stays in registers for all T steps; thread
// (rg, cl) owns rows rg*R .. rg*R+R-1 and value columns 4cl .. 4cl+3, so every
// store of a state row segment is a contiguous BV*4-byte run and a wave writes
// whole 128-byte lines.  Per step the two key-direction reductions
// r = S^T k^ and y = S^T q^ share one pass over the decayed state; the output
// then needs no second pass: o = scale * (y + (k^ . q^) u) with
// u = beta (v - r), because the update adds k^ u^T.
//
// The kernel is bound by the fp32 state writes (T x 64 KiB per (b, h)), so
// they use non-temporal stores: nothing reads them back in this call.
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// NORM: the output-gate sigmoid RMSNorm of each output row is applied before the store
// (SGLang PR #42489, "Modifications": the sigmoid RMSNorm tuned together with the
// recurrence).  It needs whole rows, so it runs with 128-column tiles only: each step
// leaves its fp32 output row in LDS (in the step's dead decay-table row), and after the
// last step groups of 32 threads normalise the rows and store y = o * rstd * weight *
// sigmoid(gate), with the gate rows staged in the prologue.
template <int BV, bool NORM>
__global__ __launch_bounds__(256) void verify_kernel(VerifyParams p) {
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
  int blk = blockIdx.x;
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

  // ---------------- gather the start state from the pool.
  const int cl = tid % NCG;
  const int rg = tid / NCG;
  const int row0 = rg * R;
  const int64_t head_elems = static_cast<int64_t>(D) * D;
  float4 S[R];
  {
    const float* src = p.pool + (static_cast<int64_t>(slot) * p.H + h) * head_elems +
                       static_cast<int64_t>(row0) * D + v0 + 4 * cl;
#pragma unroll
    for (int j = 0; j < R; ++j) S[j] = *reinterpret_cast<const float4*>(src + j * D);
  }
  __syncthreads();

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
  // The LDS limit for the largest step count is set once per device, not per call
  // (verify at batch 1 is latency-bound).
  static PerDeviceOnce attr_once;
  hipError_t e = attr_once.run([](int, int*) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_kernel<BV, NORM>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(verify_lds_bytes<BV, NORM>(KDA_MAX_STEPS_INTERNAL)));
  });
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(p.B) * p.H * (D / BV));
  hipLaunchKernelGGL((verify_kernel<BV, NORM>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  // The fused output norm needs whole 128-column rows in one workgroup.
  if (p.out_gate) return launch_verify_bv<128, true>(p, s);
  // Enough workgroups to cover the 256 compute units: split each head's value
  // columns four ways when there are few (row, head) pairs.
  if (static_cast<int64_t>(p.B) * p.H >= 256) return launch_verify_bv<128, false>(p, s);
  return launch_verify_bv<32, false>(p, s);
}

}  // namespace kda
