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

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// Sum of squares of the two bf16 values packed in x, added to acc.
__device__ __forceinline__ float sq2_bf16(uint32_t x, float acc) {
  const bf16x2v v = __builtin_bit_cast(bf16x2v, x);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const half2v h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

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
constexpr int TMS = 20;   // row stride (floats) of the inverse's 16x16 partial products

constexpr int PS = 68;    // row stride (halves) of the fp16 P matrix: conflict-free 8-byte row reads

// 50.25 KiB, so three workgroups share a CU's 160 KiB: the decay tables live in A's space
// (A is first written after the operands), P is kept in fp16 (the format the record holds),
// and the block sums sit in the union's tail, past the prologue's staging.
struct IntraSmem {
  union {
    float AT[64 * ATS];        // A = diag(beta) strict(G), inverted in place into T
    struct {                   // decay tables: written after the prologue, dead before A is written
      float Eb[5][128];        // 2^(base_m), m = 0..4 (base_4 = chunk total)
      float KCb[4][128];       // 2^(total - base_m)
      float Dsc[6][128];       // 2^(base_m - base_w), m > w, pair index m*(m-1)/2 + w
    } tab;
  } a;
  _Float16 P[64 * PS];         // scale * tril(P), fp16 (as the record holds it)
  union {
    // fp16 right factors of row blocks w = 0..2 re-referenced to each later row block m
    // (both factors of an off-diagonal block are <= 1), by (pair(m, w), k-step s, lane)
    half8 R16[6][4][64];
    struct {
      uint2 KCs[16 * 2 * 64];  // K_C^T record fragments by (fragment, 8-byte half, lane)
      float tmp[3][16 * TMS];  // 16x16 partial products of the block inverse, per wave
    } late;
    struct {
      unsigned char pad[3 * 64 * 256 - 64 * ATS * 4 - 64 * PS * 2];   // the staged q/k/g
      float tot[4][128];       // per-block sums of log2 decay (read before the union's other uses)
    } pre;
  } u;
  float beta[64];
};

// The prologue's q/k/g staging: 3 tensors x 64 rows x 256 bytes from the start of
// IntraSmem (A, P and the union are contiguous there and unused until the operands).
constexpr int STAGE_TENSOR = 64 * 256;
static_assert(offsetof(IntraSmem, u) + offsetof(decltype(IntraSmem::u), pre.tot) >= 3 * STAGE_TENSOR,
              "staging overlaps the block sums");
static_assert(sizeof(IntraSmem) <= 53 * 1024, "three workgroups per CU");

__device__ __forceinline__ int pair_idx(int m, int w) { return m * (m - 1) / 2 + w; }

// C = X * Y for 16x16 fp32 blocks in LDS (row strides ldx, ldy), accumulated into acc.
// Lane group k supplies contraction index 4k + kk to step kk, so X is read as one 16-byte
// row piece per lane.  With row strides of 4 (mod 32) words for X and of 4 (mod 8) words
// for Y, neither read has bank conflicts (32 banks of 4 bytes).
__device__ __forceinline__ f32x4 mm16_lds(const float* X, int ldx, const float* Y, int ldy,
                                          f32x4 acc, int lane) {
  const int r = lane & 15, k = lane >> 4;
  const float4 x4 = *reinterpret_cast<const float4*>(X + r * ldx + 4 * k);
  const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(xv[kk], Y[(4 * k + kk) * ldy + r], acc);
  return acc;
}

// Store a 16x16 accumulator tile (lane (n, g) holds rows 4g..4g+3 of column n).
__device__ __forceinline__ void store_tile(float* dst, int ld, f32x4 c, int lane, float mul) {
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(4 * g + r) * ld + n] = mul * c[r];
}

// Three workgroups (12 waves) per CU, 168 VGPRs at most: with two, the kernel was 13-15%
// slower (4x8192 and 8x2048 x16 heads on MI355X); its phases are latency-bound, and the
// third workgroup fills the issue slots the other two leave.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void prefill_intra_kernel(PrefillParams p) {
  __shared__ IntraSmem sm;
  const int tid = threadIdx.x;
  // The wave index is uniform; saying so keeps its loops and addressing on the scalar unit.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, m = lane & 15, g = lane >> 4;
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
  uint2 qr[8], kr[8];        // q and k stay packed bf16 until the operands
  float la[32];
  float beta_t;
  {
    // q, k and g rows go through LDS: wave w copies its own 16 token rows of each
    // (3 x 4 KiB) with 16-byte LDS-DMA loads, four whole rows per instruction, into
    // space the later phases use (A, P and the union are free until the operands).
    // Reading them back in the MFMA channel order from registers-sized 8-byte global
    // loads instead made every load instruction touch 16 rows at 32 bytes each, and
    // the kernel took 7-10% longer (4x8192 and 8x2048 x16 heads on MI355X).  Pieces
    // are XOR-swizzled by row (piece p of row r at p ^ (r & 15)) so the read-back of one
    // channel piece by 16 rows spreads over the banks.
    unsigned char* stage = reinterpret_cast<unsigned char*>(&sm);
    const uint32_t stage_lds = lds_addr(stage);
    const uint16_t* srcs[3] = {p.q, p.k, p.g};
    const int64_t sts[3] = {p.q_st, p.k_st, p.g_st};
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const uint64_t base = uniform_addr(srcs[x] + static_cast<int64_t>(t0) * sts[x] + h * D);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * j + (lane >> 4);            // chunk row of this slot
        const int piece = (lane & 15) ^ (r & 15);              // global piece held here
        const uint32_t off = static_cast<uint32_t>((min(r, L - 1) * sts[x] + 8 * piece) * 2);
        lds_dma16(base, off, stage_lds + static_cast<uint32_t>(x * STAGE_TENSOR + (16 * w + 4 * j) * 256));
      }
    }
    uint2 gr[8];
    float4 dr[8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        dr[2 * s + hh] = *reinterpret_cast<const float4*>(p.dt_bias + h * D + kperm(s, g, 4 * hh));
    const uint16_t braw = p.beta[tok * p.b_st + h];
    const float alog = p.A_log[h];
    // Only this wave's rows are read back, so its own copies are all it waits for.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // channels kperm(s, g, 4hh..4hh+3): bytes 64s + 32hh + 8g of the row
        const int piece = 4 * s + 2 * hh + (g >> 1);
        const int off = t * 256 + 16 * (piece ^ (t & 15)) + 8 * (g & 1);
        qr[2 * s + hh] = *reinterpret_cast<const uint2*>(stage + off);
        kr[2 * s + hh] = *reinterpret_cast<const uint2*>(stage + STAGE_TENSOR + off);
        gr[2 * s + hh] = *reinterpret_cast<const uint2*>(stage + 2 * STAGE_TENSOR + off);
      }
    beta_t = vmask * sigmoid_f32(bf16_to_f32(braw));
    // log2 decay = lb log2(e) sigmoid(e^A_log (g + dt_bias)), with the exponent's
    // -e^A_log log2(e) folded into one factor.
    const float nEA = -__builtin_amdgcn_exp2f(alog * LOG2E) * LOG2E;
    const float lbm = p.lb_log2e * vmask;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gg[4] = {bf16lo_to_f32(gr[j].x), bf16hi_to_f32(gr[j].x),
                           bf16lo_to_f32(gr[j].y), bf16hi_to_f32(gr[j].y)};
      const float dd[4] = {dr[j].x, dr[j].y, dr[j].z, dr[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        la[4 * j + e] = lbm * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f((gg[e] + dd[e]) * nEA));
    }
  }
  float ssq = 0.f, ssk = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ssq = sq2_bf16(qr[j].x, sq2_bf16(qr[j].y, ssq));
    ssk = sq2_bf16(kr[j].x, sq2_bf16(kr[j].y, ssk));
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
      for (int e = 0; e < 8; ++e) sm.u.pre.tot[w][kperm(s, g, e)] = la[8 * s + e];
  }
  lds_barrier();

  // Per-channel tables from the four block sums (2 threads per channel).
  {
    const int c = tid & 127, part = tid >> 7;
    float base[5];
    base[0] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) base[b + 1] = base[b] + sm.u.pre.tot[b][c];
    if (part == 0) {
#pragma unroll
      for (int b = 0; b < 5; ++b) sm.a.tab.Eb[b][c] = __builtin_amdgcn_exp2f(base[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b) sm.a.tab.KCb[b][c] = __builtin_amdgcn_exp2f(base[4] - base[b]);
    } else {
#pragma unroll
      for (int mm = 1; mm < 4; ++mm)
#pragma unroll
        for (int ww = 0; ww < mm; ++ww)
          sm.a.tab.Dsc[pair_idx(mm, ww)][c] = __builtin_amdgcn_exp2f(base[mm] - base[ww]);
    }
  }
  lds_barrier();
  if (tid < 128) __builtin_nontemporal_store(sm.a.tab.Eb[4][tid], reinterpret_cast<float*>(rec + REC_GAMMA_OFF) + tid);

  // ---- operands.  b = la (in-block cumulative), Lf = 2^b <= 1, Rf = 2^-b >= 1.  Per
  // k-step s this also accumulates the diagonal G/P block (bf16 MFMA), publishes the
  // off-diagonal right factors this wave owns, and turns K_C into K_C^T tiles.
  half8 KL16[4], QL16[4];   // the left factors in fp16, for the off-diagonal blocks
  uint2 kct[8];             // K_C^T tiles (channel block 2s + hf), packed fp16 (see below)
  f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
  {
    const float rqs = rq * p.scale;
    // Selector B operands that transpose a 16 x 32 fp16 A tile through the MFMA: column n
    // of tile hf picks key channel 16 hf + n of the k-step, which lane group n / 4 holds
    // as element 4 hf + n % 4.  The products are exact (x * 1 plus zeros).
    half8 sel[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sel[hf][e] = static_cast<_Float16>(((m >> 2) == g && e == 4 * hf + (m & 3)) ? 1.f : 0.f);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // This k-step's table entries and q, k channels (unpacked here to keep registers
      // for the third workgroup).
      float ebv[8], kcv[8], qs[8], ks[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.a.tab.Eb[w][kperm(s, g, 4 * hh)]);
        const float4 c4 = *reinterpret_cast<const float4*>(&sm.a.tab.KCb[w][kperm(s, g, 4 * hh)]);
        ebv[4 * hh] = e4.x; ebv[4 * hh + 1] = e4.y; ebv[4 * hh + 2] = e4.z; ebv[4 * hh + 3] = e4.w;
        kcv[4 * hh] = c4.x; kcv[4 * hh + 1] = c4.y; kcv[4 * hh + 2] = c4.z; kcv[4 * hh + 3] = c4.w;
        const uint2 qw = qr[2 * s + hh], kw = kr[2 * s + hh];
        qs[4 * hh] = bf16lo_to_f32(qw.x); qs[4 * hh + 1] = bf16hi_to_f32(qw.x);
        qs[4 * hh + 2] = bf16lo_to_f32(qw.y); qs[4 * hh + 3] = bf16hi_to_f32(qw.y);
        ks[4 * hh] = bf16lo_to_f32(kw.x); ks[4 * hh + 1] = bf16hi_to_f32(kw.x);
        ks[4 * hh + 2] = bf16lo_to_f32(kw.y); ks[4 * hh + 3] = bf16hi_to_f32(kw.y);
      }
      half8 kg, qg, kc;
      float klv[8], qlv[8], krv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * s + e;
        const float Lf = __builtin_amdgcn_exp2f(la[i]);
        const float Rf = __builtin_amdgcn_exp2f(-la[i]);
        const float kh = ks[e] * rk;
        const float kl = kh * Lf;             // k^ 2^(b_t - base_w)
        const float ql = qs[e] * rqs * Lf;    // scale q^ 2^(b_t - base_w)
        const float kr = kh * Rf;             // k^ 2^(base_w - b_t)
        kg[e] = static_cast<_Float16>(-kl * ebv[e]);
        qg[e] = static_cast<_Float16>(ql * ebv[e]);
        kc[e] = static_cast<_Float16>(kcv[e] * kr);
        klv[e] = kl;
        qlv[e] = ql;
        krv[e] = kr;
      }
      rec_store(rec + (FR_KG + 4 * w + s) * 1024 + lane * 16, kg);
      rec_store(rec + (FR_QG + 4 * w + s) * 1024 + lane * 16, qg);
      // K_C^T: lane (n, g) of tile hf receives channel 32 s + 16 hf + n of tokens
      // 16 w + 4 g + r, i.e. half (w & 1) of its slot in record fragment (2 s + hf, w / 2).
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 t4 = mfma_f16(kc, sel[hf], zero4);
        kct[2 * s + hf] = make_uint2(pack_f16x2(t4[0], t4[1]), pack_f16x2(t4[2], t4[3]));
      }
      // Diagonal block: the right factor reaches 2^115, so bf16 operands; G one product,
      // P the three-product split.
      u32x4 klp, qhp, qlp, rhp, rlp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        klp[j] = pack_bf16x2(klv[2 * j], klv[2 * j + 1]);
        uint32_t hi, lo;
        split_bf16x2(qlv[2 * j], qlv[2 * j + 1], hi, lo);
        qhp[j] = hi;
        qlp[j] = lo;
        split_bf16x2(krv[2 * j], krv[2 * j + 1], hi, lo);
        rhp[j] = hi;
        rlp[j] = lo;
      }
      accG = mfma_bf16(as_bf16x8(klp), as_bf16x8(rhp), accG);
      accP = mfma_bf16(as_bf16x8(qhp), as_bf16x8(rhp), accP);
      accP = mfma_bf16(as_bf16x8(qhp), as_bf16x8(rlp), accP);
      accP = mfma_bf16(as_bf16x8(qlp), as_bf16x8(rhp), accP);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        KL16[s][e] = static_cast<_Float16>(klv[e]);
        QL16[s][e] = static_cast<_Float16>(qlv[e]);
      }
      // Off-diagonal right factors, made by the wave that owns the column block: for each
      // later row block mm, k^ 2^(base_w - b_i) * 2^(base_mm - base_w) = k^ 2^(base_mm - b_i)
      // <= 1, rounded to fp16 (its 11-bit mantissa beats bf16; the range is fine).  Wave w
      // makes 3 - w of them and consumes w.
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j < 3 - w) {
          const float* dsc = sm.a.tab.Dsc[pair_idx(w + 1 + j, w)];
          const float4 d0 = *reinterpret_cast<const float4*>(dsc + kperm(s, g, 0));
          const float4 d1 = *reinterpret_cast<const float4*>(dsc + kperm(s, g, 4));
          const half8 hr = {static_cast<_Float16>(krv[0] * d0.x), static_cast<_Float16>(krv[1] * d0.y),
                            static_cast<_Float16>(krv[2] * d0.z), static_cast<_Float16>(krv[3] * d0.w),
                            static_cast<_Float16>(krv[4] * d1.x), static_cast<_Float16>(krv[5] * d1.y),
                            static_cast<_Float16>(krv[6] * d1.z), static_cast<_Float16>(krv[7] * d1.w)};
          sm.u.R16[pair_idx(w + 1 + j, w)][s][lane] = hr;
        }
      }
    }
  }
  // lane (n, g) of a G/P tile holds rows t = 16w + 4g + r, column 16wb + n
  const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + 16 * w + 4 * g);
  const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
  lds_barrier();   // the decay tables are dead from here on; A may be written
  {
    const int i = 16 * w + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 16 * w + 4 * g + r;
      sm.a.AT[tr * ATS + i] = (i < tr) ? bt[r] * accG[r] : 0.f;
      sm.P[tr * PS + i] = static_cast<_Float16>((i <= tr) ? accP[r] : 0.f);   // the left factors carry the scale
    }
  }

  // ---- a2, off the diagonal: row block w against column blocks wb < w, one fp16 product
  // each for G and P (both factors <= 1).  Every right operand is read before any product.
  {
    half8 rf[3][4];
#pragma unroll
    for (int wb = 0; wb < 3; ++wb)
      if (wb < w) {
#pragma unroll
        for (int s = 0; s < 4; ++s) rf[wb][s] = sm.u.R16[pair_idx(w, wb)][s][lane];
      }
#pragma unroll
    for (int wb = 0; wb < 3; ++wb)
      if (wb < w) {
        f32x4 oG = {0.f, 0.f, 0.f, 0.f}, oP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          oG = mfma_f16(KL16[s], rf[wb][s], oG);
          oP = mfma_f16(QL16[s], rf[wb][s], oP);
        }
        const int i = 16 * wb + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 16 * w + 4 * g + r;
          sm.a.AT[tr * ATS + i] = bt[r] * oG[r];
          sm.P[tr * PS + i] = static_cast<_Float16>(oP[r]);
        }
      }
  }
  lds_barrier();   // R16 is dead from here on; the union's late view may be written

  // K_C^T halves to their record slots in LDS: [fragment][half][lane], 8 bytes each.
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
    sm.u.late.KCs[((2 * cb + (w >> 1)) * 2 + (w & 1)) * 64 + lane] = kct[cb];

  // ---- a3: T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution (one
  // column per lane, the four lane groups redundant), in place.
  {
    const int j = m;
    float x[16];
    const float* Ab = sm.a.AT + (16 * w) * ATS + 16 * w;
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
      float* Tb = sm.a.AT + (16 * w) * ATS + 16 * w;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * ATS + j] = x[r];
    }
  }
  lds_barrier();
  // Off-diagonal blocks by column: wave w makes T_rw = -T_rr sum_{j=w}^{r-1} A_rj T_jw for
  // r = w+1..3 from the diagonal inverses, the A blocks and its own earlier results.  Each
  // T_rw goes to the unused upper block (w, r) of the same array, so no A block is
  // overwritten and no other wave's result is needed: no workgroup barrier until the end.
  {
    float* tmp = sm.u.late.tmp[min(w, 2)];
#pragma unroll
    for (int rb = 1; rb < 4; ++rb)
      if (rb > w) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < 3; ++jb)
          if (jb >= w && jb < rb) {
            const float* Tjw = (jb == w) ? sm.a.AT + (16 * w) * ATS + 16 * w
                                         : sm.a.AT + (16 * w) * ATS + 16 * jb;
            acc = mm16_lds(sm.a.AT + (16 * rb) * ATS + 16 * jb, ATS, Tjw, ATS, acc, lane);
          }
        store_tile(tmp, TMS, acc, lane, 1.f);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mm16_lds(sm.a.AT + (16 * rb) * ATS + 16 * rb, ATS, tmp, TMS, z, lane);
        store_tile(sm.a.AT + (16 * w) * ATS + 16 * rb, ATS, z, lane, -1.f);
      }
  }
  lds_barrier();

  // ---- record fragments: T' = T diag(beta) and scale*tril(P), K_C^T.
  // A/B fragment (row block rb, k-step s'): lane (r, g) holds row 16rb + r, columns
  // kperm(s', g, 0..7); the two 4-column halves lie in column blocks 2s' and 2s' + 1.
  // T_{rb,c} sits at block (rb, rb) on the diagonal and at block (c, rb) below it; blocks
  // above the diagonal are zero in both matrices.
  {
    const int rb = w;
    for (int sp = 0; sp <= (rb >> 1); ++sp) {
      const int fi = (rb < 2) ? rb : 2 + 2 * (rb - 2) + sp;
      float tv[8];
      uint32_t pw[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int cblk = 2 * sp + hf;
        const int col = kperm(sp, g, 4 * hf);          // 16 cblk + 4 g
        float4 t4 = make_float4(0.f, 0.f, 0.f, 0.f);
        uint2 p2 = make_uint2(0u, 0u);
        if (cblk <= rb) {
          const float* src = (cblk == rb) ? sm.a.AT + (16 * rb + m) * ATS + col
                                          : sm.a.AT + (16 * cblk + m) * ATS + 16 * rb + 4 * g;
          t4 = *reinterpret_cast<const float4*>(src);
          p2 = *reinterpret_cast<const uint2*>(sm.P + (16 * rb + m) * PS + col);
        }
        const float4 bb = *reinterpret_cast<const float4*>(sm.beta + col);
        tv[4 * hf] = t4.x * bb.x; tv[4 * hf + 1] = t4.y * bb.y;
        tv[4 * hf + 2] = t4.z * bb.z; tv[4 * hf + 3] = t4.w * bb.w;
        pw[2 * hf] = p2.x; pw[2 * hf + 1] = p2.y;
      }
      half8 tf;
#pragma unroll
      for (int e = 0; e < 8; ++e) tf[e] = static_cast<_Float16>(tv[e]);
      const u32x4 pwv = {pw[0], pw[1], pw[2], pw[3]};
      const half8 pf = __builtin_bit_cast(half8, pwv);
      rec_store(rec + (FR_TP + fi) * 1024 + lane * 16, tf);
      rec_store(rec + (FR_PM + fi) * 1024 + lane * 16, pf);
    }
    // K_C^T fragments 4w..4w+3 from the two halves staged by the wave pairs.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = 4 * w + q;
      const uint2 a = sm.u.late.KCs[(2 * f) * 64 + lane];
      const uint2 b = sm.u.late.KCs[(2 * f + 1) * 64 + lane];
      rec_store(rec + (FR_KC + f) * 1024 + lane * 16, make_uint4(a.x, a.y, b.x, b.y));
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
