// Varlen chunked KDA prefill for gfx950 (CDNA4): two kernels on the caller's stream;
// this file holds the first.
//
// Role: the FlashKDA prefill of vLLM PR #55737 ("Use FlashKDA for KDA chunked
// prefill"): bounded gate, in-kernel q/k L2 norm and sigmoid of raw beta
// logits fused in, output written straight into the caller's layer buffer, final
// state returned.  The chunked form itself is derived from the token recurrence
// (no page writes it out): inside a chunk of C = 64 tokens with per-channel
// log-decays a_t, b_t = a_1 + ... + a_t and Gamma_t = 2^(b_t) (log2 units here),
//     G_ti = sum_c k_tc k_ic Gamma_tc / Gamma_ic   (i < t),  A = diag(beta) G
//     P_ti = sum_c q_tc k_ic Gamma_tc / Gamma_ic   (i <= t)
//     T'   = (I + A)^-1 diag(beta)
//     U    = T' (V - K_Gamma S)                       K_Gamma[t] = k_t * Gamma_t
//     O    = scale (Q_Gamma S + tril(P) U)            Q_Gamma[t] = q_t * Gamma_t
//     S'   = Diag(Gamma_C) S + K_C^T U                K_C[t]     = k_t * Gamma_C / Gamma_t
//

// Kernel 1 (prefill_intra): one workgroup per (chunk, head), fully parallel.
//   Computes everything that does not depend on the state: norms, gates, the
//   in-chunk cumulative decay, G and P on MFMA, the unit-lower-triangular
//   inverse, and writes a 61 KiB record of fp16 MFMA fragments (-K_Gamma, T',
//   scale*Q_Gamma, scale*tril(P), K_C^T) plus Gamma_C.  Fragments are stored
//   in exactly the per-lane order kernel 2 feeds to v_mfma_f32_16x16x32_f16,
//   so kernel 2 copies each record linearly into LDS.
//   Exponent range: Gamma_t itself underflows over a 64-token chunk, so G and P
//   are formed per 16-token row block m with the block's start as reference:
//   left factor 2^(b_t - base_m) <= 1 and right factor 2^(base_m - b_i), which
//   is <= 1 off the diagonal and <= 2^(16*5*log2 e) < 2^116 on it -- inside the
//   bf16/fp32 exponent range for lower_bound >= -5.  Off the diagonal both factors
//   are <= 1, so G and P take one fp16 product each (11-bit mantissa); on the
//   diagonal G uses bf16 operands and P a three-product bf16 split (hi*hi + hi*lo
//   + lo*hi), since its rounding reaches the output directly.
#include "kda_prefill_common.h"

namespace kda {

namespace {

using namespace prefill;

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  return x;
}

// bf16 split of a pair: hi = RNE(a, b), lo = RNE of what hi leaves, both packed with the
// low half holding a (the hardware pair conversion; a scalar bf16 cast is a multi-op
// software sequence).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16lo_to_f32(hi), b - bf16hi_to_f32(hi));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Record stores are non-temporal: the 61 KiB records of a call outgrow the caches, and the
// scan that reads them back ran 3-4% faster when they did not pass through as ordinary
// writes (4 x 8192 x 16 heads on MI355X: scan 266-271 us -> 255-260 us).
template <class T16>
__device__ __forceinline__ void rec_store(unsigned char* dst, const T16& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, not
// for its global stores (which nothing in the workgroup reads back).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float* dst) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  dst[0] = bf16lo_to_f32(w.x);
  dst[1] = bf16hi_to_f32(w.x);
  dst[2] = bf16lo_to_f32(w.y);
  dst[3] = bf16hi_to_f32(w.y);
}

// ============================================================================
// Intra-chunk work, one workgroup (4 waves) per (chunk slot, head).
// Thread (w, l): token t = 16w + l%16 of the chunk, key channels kperm(s, l/16, e)
// for s = 0..3, e = 0..7 (32 channels).
// ============================================================================

constexpr int ATS = 68;   // padded row stride (floats) of the 64x64 LDS matrices
constexpr int KCS = 72;   // padded row stride (halves) of the transposed K_C tile

struct IntraSmem {
  float AT[64 * ATS];          // A = diag(beta) strict(G), inverted in place into T
  float P[64 * ATS];           // scale * tril(P)
  union {
    // fp16 right factors of row blocks w = 0..2 re-referenced to each later row block m
    // (both factors of an off-diagonal block are <= 1), by (pair(m, w), k-step s, lane)
    half8 R16[6][4][64];
    struct {
      _Float16 KCt[128 * KCS]; // K_C transposed [channel][token]
      float tmp[3][256];       // 16x16 partial products of the block inverse
    } late;
  } u;
  float tot[4][128];           // per-block sums of log2 decay
  float Eb[5][128];            // 2^(base_m), m = 0..4 (base_4 = chunk total)
  float KCb[4][128];           // 2^(total - base_m)
  float Dsc[6][128];           // 2^(base_m - base_w), m > w, pair index m*(m-1)/2 + w
  float beta[64];
};

__device__ __forceinline__ int pair_idx(int m, int w) { return m * (m - 1) / 2 + w; }

// C = X * Y for 16x16 fp32 blocks in LDS (row strides ldx, ldy), accumulated into acc.
__device__ __forceinline__ f32x4 mm16_lds(const float* X, int ldx, const float* Y, int ldy,
                                          f32x4 acc, int lane) {
  const int r = lane & 15, k = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = mfma_f32(X[r * ldx + 4 * kk + k], Y[(4 * kk + k) * ldy + r], acc);
  return acc;
}

// Store a 16x16 accumulator tile (lane (n, g) holds rows 4g..4g+3 of column n).
__device__ __forceinline__ void store_tile(float* dst, int ld, f32x4 c, int lane, float mul) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(4 * g + r) * ld + n] = mul * c[r];
}

__global__ __launch_bounds__(256, 2) void prefill_intra_kernel(PrefillParams p) {
  __shared__ IntraSmem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  // Heads fastest: the H workgroups of one chunk slot run together, so their loads
  // cover whole token rows and their records are contiguous.
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;

  // ---- a0: chunk map.  Sequence n owns slots [cu[n]/64 + n, ... + nchunks); find the
  // last n whose first slot is <= this one (binary search on device, no host sync).
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] / CHUNK + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int cs = p.cu[n], ce = p.cu[n + 1];
  const int jc = slot - (cs / CHUNK + n);
  if (jc * CHUNK >= ce - cs) return;                     // surplus slot (uniform exit)
  const int t0 = cs + jc * CHUNK;
  const int L = min(CHUNK, ce - t0);
  unsigned char* rec = p.work + (static_cast<int64_t>(slot) * H + h) * REC_BYTES;

  // ---- a1: loads, norms, gate, beta.  Rows past the chunk end are read from the
  // last valid row (always in bounds) and zeroed arithmetically, so no per-lane
  // branches split the loads.
  const int t = 16 * w + m;
  const bool valid = t < L;
  const float vmask = valid ? 1.f : 0.f;
  const int64_t tok = static_cast<int64_t>(t0) + min(t, L - 1);
  float qv[32], kv[32], la[32];
  float beta_t;
  {
    // Every global load of the prologue is issued before the first is used (one
    // memory round trip instead of the compiler's staggered two or three).
    uint2 qr[8], kr[8], gr[8];
    float4 dr[8];
    const uint16_t* qp = p.q + tok * p.q_st + h * D;
    const uint16_t* kp = p.k + tok * p.k_st + h * D;
    const uint16_t* gp = p.g + tok * p.g_st + h * D;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int c0 = kperm(s, g, 4 * hh);
        qr[2 * s + hh] = *reinterpret_cast<const uint2*>(qp + c0);
        kr[2 * s + hh] = *reinterpret_cast<const uint2*>(kp + c0);
        gr[2 * s + hh] = *reinterpret_cast<const uint2*>(gp + c0);
        dr[2 * s + hh] = *reinterpret_cast<const float4*>(p.dt_bias + h * D + c0);
      }
    const uint16_t braw = p.beta[tok * p.b_st + h];
    const float alog = p.A_log[h];
    asm volatile("" ::: "memory");
    beta_t = vmask * sigmoid_f32(bf16_to_f32(braw));
    float gv[32], dt[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float* qq = qv + 4 * j;
      float* kk = kv + 4 * j;
      float* gg = gv + 4 * j;
      qq[0] = bf16lo_to_f32(qr[j].x); qq[1] = bf16hi_to_f32(qr[j].x);
      qq[2] = bf16lo_to_f32(qr[j].y); qq[3] = bf16hi_to_f32(qr[j].y);
      kk[0] = bf16lo_to_f32(kr[j].x); kk[1] = bf16hi_to_f32(kr[j].x);
      kk[2] = bf16lo_to_f32(kr[j].y); kk[3] = bf16hi_to_f32(kr[j].y);
      gg[0] = bf16lo_to_f32(gr[j].x); gg[1] = bf16hi_to_f32(gr[j].x);
      gg[2] = bf16lo_to_f32(gr[j].y); gg[3] = bf16hi_to_f32(gr[j].y);
      dt[4 * j] = dr[j].x; dt[4 * j + 1] = dr[j].y; dt[4 * j + 2] = dr[j].z; dt[4 * j + 3] = dr[j].w;
    }
    // log2 decay = lb log2(e) sigmoid(e^A_log (g + dt_bias)), with the exponent's
    // -e^A_log log2(e) folded into one factor.
    const float nEA = -__builtin_amdgcn_exp2f(alog * LOG2E) * LOG2E;
    const float lbm = p.lb_log2e * vmask;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      la[i] = lbm * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f((gv[i] + dt[i]) * nEA));
  }
  float ssq = 0.f, ssk = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    ssq += qv[i] * qv[i];
    ssk += kv[i] * kv[i];
  }
  ssq += __shfl_xor(ssq, 16);
  ssq += __shfl_xor(ssq, 32);
  ssk += __shfl_xor(ssk, 16);
  ssk += __shfl_xor(ssk, 32);
  // Rows past the chunk end hold a copy of the last row; zeroing the norm factors zeroes
  // every q and k product they feed.
  const float rq = __builtin_amdgcn_rsqf(ssq + L2_EPS) * vmask;
  const float rk = __builtin_amdgcn_rsqf(ssk + L2_EPS) * vmask;
  if (g == 0) sm.beta[t] = beta_t;

  // In-block inclusive cumulative log2 decay (lanes m = 0..15 of a row are 16 tokens).
#pragma unroll
  for (int i = 0; i < 32; ++i) la[i] = row_scan16(la[i]);
  if (m == 15) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.tot[w][kperm(s, g, e)] = la[8 * s + e];
  }
  lds_barrier();

  // Per-channel tables from the four block sums (2 threads per channel).
  {
    const int c = tid & 127, part = tid >> 7;
    float base[5];
    base[0] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) base[b + 1] = base[b] + sm.tot[b][c];
    if (part == 0) {
#pragma unroll
      for (int b = 0; b < 5; ++b) sm.Eb[b][c] = __builtin_amdgcn_exp2f(base[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b) sm.KCb[b][c] = __builtin_amdgcn_exp2f(base[4] - base[b]);
    } else {
#pragma unroll
      for (int mm = 1; mm < 4; ++mm)
#pragma unroll
        for (int ww = 0; ww < mm; ++ww)
          sm.Dsc[pair_idx(mm, ww)][c] = __builtin_amdgcn_exp2f(base[mm] - base[ww]);
    }
  }
  lds_barrier();
  if (tid < 128) __builtin_nontemporal_store(sm.Eb[4][tid], reinterpret_cast<float*>(rec + REC_GAMMA_OFF) + tid);

  // ---- operands.  b = la (in-block cumulative), Lf = 2^b <= 1, Rf = 2^-b >= 1.
  bf16x8 KL[4], QLh[4], QLl[4], Rh[4], Rl[4];
  half8 KL16[4], QL16[4];   // the left factors in fp16, for the off-diagonal blocks
  _Float16 kch[32];
  {
    const float rqs = rq * p.scale;
    // Table entries of this thread's 32 channels: 16-byte LDS reads, all issued first.
    float ebv[32], kcv[32];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.Eb[w][kperm(s, g, 4 * hh)]);
        const float4 c4 = *reinterpret_cast<const float4*>(&sm.KCb[w][kperm(s, g, 4 * hh)]);
        float* ee = ebv + 8 * s + 4 * hh;
        float* cc = kcv + 8 * s + 4 * hh;
        ee[0] = e4.x; ee[1] = e4.y; ee[2] = e4.z; ee[3] = e4.w;
        cc[0] = c4.x; cc[1] = c4.y; cc[2] = c4.z; cc[3] = c4.w;
      }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 kg, qg;
      float klv[8], qlv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * s + e;
        const float Lf = __builtin_amdgcn_exp2f(la[i]);
        const float Rf = __builtin_amdgcn_exp2f(-la[i]);
        const float kh = kv[i] * rk;
        const float kl = kh * Lf;             // k^ 2^(b_t - base_w)
        const float ql = qv[i] * rqs * Lf;    // scale q^ 2^(b_t - base_w)
        const float kr = kh * Rf;             // k^ 2^(base_w - b_t)
        kg[e] = static_cast<_Float16>(-kl * ebv[i]);
        qg[e] = static_cast<_Float16>(ql * ebv[i]);
        kch[i] = static_cast<_Float16>(kcv[i] * kr);
        klv[e] = kl;
        qlv[e] = ql;
        kv[i] = kr;  // the fp32 right factor (the diagonal split and the off-diagonal fp16)
      }
      u32x4 klp, qhp, qlp, rhp, rlp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        klp[j] = pack_bf16x2(klv[2 * j], klv[2 * j + 1]);
        uint32_t hi, lo;
        split_bf16x2(qlv[2 * j], qlv[2 * j + 1], hi, lo);
        qhp[j] = hi;
        qlp[j] = lo;
        split_bf16x2(kv[8 * s + 2 * j], kv[8 * s + 2 * j + 1], hi, lo);
        rhp[j] = hi;
        rlp[j] = lo;
      }
      KL[s] = as_bf16x8(klp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        KL16[s][e] = static_cast<_Float16>(klv[e]);
        QL16[s][e] = static_cast<_Float16>(qlv[e]);
      }
      // Off-diagonal right factors, made here by the wave that owns the column block: for
      // each later row block m, k^ 2^(base_w - b_i) * 2^(base_m - base_w) = k^ 2^(base_m - b_i)
      // <= 1, rounded to fp16 (its 11-bit mantissa beats bf16; the range is fine).  Wave w
      // makes 3 - w of them and consumes w, so the waves share the off-diagonal work evenly.
      for (int mm = w + 1; mm < 4; ++mm) {
        const float* dsc = sm.Dsc[pair_idx(mm, w)];
        const float4 d0 = *reinterpret_cast<const float4*>(dsc + kperm(s, g, 0));
        const float4 d1 = *reinterpret_cast<const float4*>(dsc + kperm(s, g, 4));
        const float* r = kv + 8 * s;
        const half8 hr = {static_cast<_Float16>(r[0] * d0.x), static_cast<_Float16>(r[1] * d0.y),
                          static_cast<_Float16>(r[2] * d0.z), static_cast<_Float16>(r[3] * d0.w),
                          static_cast<_Float16>(r[4] * d1.x), static_cast<_Float16>(r[5] * d1.y),
                          static_cast<_Float16>(r[6] * d1.z), static_cast<_Float16>(r[7] * d1.w)};
        sm.u.R16[pair_idx(mm, w)][s][lane] = hr;
      }
      QLh[s] = as_bf16x8(qhp);
      QLl[s] = as_bf16x8(qlp);
      Rh[s] = as_bf16x8(rhp);
      Rl[s] = as_bf16x8(rlp);
      rec_store(rec + (FR_KG + 4 * w + s) * 1024 + lane * 16, kg);
      rec_store(rec + (FR_QG + 4 * w + s) * 1024 + lane * 16, qg);
    }
  }
  lds_barrier();

  // ---- a2: G and P for row block w, column blocks 0..w (MFMA).  Off the diagonal one
  // fp16 product each (factors <= 1); on it bf16 (the right factor reaches 2^115): G one
  // product, P the three-product split.
  for (int wb = 0; wb <= w; ++wb) {
    f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
    if (wb == w) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        accG = mfma_bf16(KL[s], Rh[s], accG);
        accP = mfma_bf16(QLh[s], Rh[s], accP);
        accP = mfma_bf16(QLh[s], Rl[s], accP);
        accP = mfma_bf16(QLl[s], Rh[s], accP);
      }
    } else {
      half8 rf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) rf[s] = sm.u.R16[pair_idx(w, wb)][s][lane];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        accG = mfma_f16(KL16[s], rf[s], accG);
        accP = mfma_f16(QL16[s], rf[s], accP);
      }
    }
    // lane (n, g) holds rows t = 16w + 4g + r, column i = 16wb + n
    const int i = 16 * wb + m;
    const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + 16 * w + 4 * g);
    const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 16 * w + 4 * g + r;
      const float gval = bt[r] * accG[r];
      const float pval = accP[r];   // the left factors carry the scale
      sm.AT[tr * ATS + i] = (i < tr) ? gval : 0.f;
      sm.P[tr * ATS + i] = (i <= tr) ? pval : 0.f;
    }
  }
  // Above the diagonal only blocks (0, 1) and (2, 3) are ever read: the record's 32-deep
  // k-steps of row blocks 0 and 2 span them.  The inverse reads the lower blocks only.
  if ((w & 1) == 0) {
    const int i = 16 * (w + 1) + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 16 * w + 4 * g + r;
      sm.AT[tr * ATS + i] = 0.f;
      sm.P[tr * ATS + i] = 0.f;
    }
  }
  lds_barrier();   // R16 is dead from here on; the union's late view may be written

  // K_C transposed into LDS ([channel][token]) for the K_C^T fragments.
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.u.late.KCt[kperm(s, g, e) * KCS + t] = kch[8 * s + e];

  // ---- a3: T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution (one
  // column per lane, the four lane groups redundant), in place.
  {
    const int j = m;
    float x[16];
    const float* Ab = sm.AT + (16 * w) * ATS + 16 * w;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float a[16];
#pragma unroll
      for (int q4 = 0; q4 < (r + 3) / 4; ++q4) {
        const float4 v4 = *reinterpret_cast<const float4*>(Ab + r * ATS + 4 * q4);
        a[4 * q4] = v4.x; a[4 * q4 + 1] = v4.y; a[4 * q4 + 2] = v4.z; a[4 * q4 + 3] = v4.w;
      }
      float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int c = 0; c < r; ++c) acc -= a[c] * x[c];
      x[r] = acc;
    }
    // All lanes of this wave have read block (w, w) before any lane writes it.
    __builtin_amdgcn_wave_barrier();
    if (g == 0) {
      float* Tb = sm.AT + (16 * w) * ATS + 16 * w;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * ATS + j] = x[r];
    }
  }
  lds_barrier();
  // Off-diagonal blocks row by row: T_rc = -T_rr * sum_{j=c}^{r-1} A_rj T_jc, computed in
  // place (A_rc is last needed by T_rc itself; all reads of a row precede its writes).
  for (int rb = 1; rb < 4; ++rb) {
    const int cb = w;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (cb < rb) {
      for (int jb = cb; jb < rb; ++jb)
        acc = mm16_lds(sm.AT + (16 * rb) * ATS + 16 * jb, ATS, sm.AT + (16 * jb) * ATS + 16 * cb,
                       ATS, acc, lane);
      store_tile(sm.u.late.tmp[cb], 16, acc, lane, 1.f);
    }
    lds_barrier();
    if (cb < rb) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = mm16_lds(sm.AT + (16 * rb) * ATS + 16 * rb, ATS, sm.u.late.tmp[cb], 16, z, lane);
      store_tile(sm.AT + (16 * rb) * ATS + 16 * cb, ATS, z, lane, -1.f);
    }
    lds_barrier();
  }

  // ---- record fragments: T' = T diag(beta) and scale*tril(P) (row-major in LDS), K_C^T.
  // A/B fragment (row block rb, k-step s'): lane (r, g) holds row 16rb + r, columns
  // kperm(s', g, 0..7).
  {
    const int rb = w;
    for (int sp = 0; sp <= (rb >> 1); ++sp) {
      const int fi = (rb < 2) ? rb : 2 + 2 * (rb - 2) + sp;
      const int row = 16 * rb + m;
      const int c0 = kperm(sp, g, 0), c1 = kperm(sp, g, 4);
      const float4 ta = *reinterpret_cast<const float4*>(sm.AT + row * ATS + c0);
      const float4 tb = *reinterpret_cast<const float4*>(sm.AT + row * ATS + c1);
      const float4 ba = *reinterpret_cast<const float4*>(sm.beta + c0);
      const float4 bb = *reinterpret_cast<const float4*>(sm.beta + c1);
      half8 tf = {static_cast<_Float16>(ta.x * ba.x), static_cast<_Float16>(ta.y * ba.y),
                  static_cast<_Float16>(ta.z * ba.z), static_cast<_Float16>(ta.w * ba.w),
                  static_cast<_Float16>(tb.x * bb.x), static_cast<_Float16>(tb.y * bb.y),
                  static_cast<_Float16>(tb.z * bb.z), static_cast<_Float16>(tb.w * bb.w)};
      rec_store(rec + (FR_TP + fi) * 1024 + lane * 16, tf);
      const float4 pa = *reinterpret_cast<const float4*>(sm.P + row * ATS + c0);
      const float4 pb = *reinterpret_cast<const float4*>(sm.P + row * ATS + c1);
      half8 pf = {static_cast<_Float16>(pa.x), static_cast<_Float16>(pa.y),
                  static_cast<_Float16>(pa.z), static_cast<_Float16>(pa.w),
                  static_cast<_Float16>(pb.x), static_cast<_Float16>(pb.y),
                  static_cast<_Float16>(pb.z), static_cast<_Float16>(pb.w)};
      rec_store(rec + (FR_PM + fi) * 1024 + lane * 16, pf);
    }
    // K_C^T fragments (channel block cb, token k-step s'): lane (r, g) holds channel
    // 16cb + r, tokens kperm(s', g, 0..7).
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int cb = 2 * w + q2;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const _Float16* src = sm.u.late.KCt + (16 * cb + m) * KCS;
        const uint2 a = *reinterpret_cast<const uint2*>(src + kperm(sp, g, 0));
        const uint2 b = *reinterpret_cast<const uint2*>(src + kperm(sp, g, 4));
        rec_store(rec + (FR_KC + 2 * cb + sp) * 1024 + lane * 16, make_uint4(a.x, a.y, b.x, b.y));
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_intra(const PrefillParams& p, hipStream_t s) {
  if (p.num_slots_chunk <= 0 || p.T_total <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.num_slots_chunk) * p.H));
  hipLaunchKernelGGL(prefill_intra_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kda
