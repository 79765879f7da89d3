// Varlen chunked KDA prefill for gfx950 (CDNA4), second kernel: the state scan over
// each sequence's chunks, reading the per-(chunk, head) records that the intra kernel
// (kda_prefill_intra.hip, which also states the chunked form) leaves in the workspace.
//
// Kernel 2 (prefill_scan): one workgroup per (sequence, head, value slice),
//   sequential over the sequence's chunks.  Each compute wave owns 16 value
//   columns; the [128 x 16] fp32 state lives in registers in the MFMA
//   accumulator layout.  That layout is reused as the next product's operand by
//   pairing 16-row blocks (2s, 2s+1) into one 32-deep k-step, so no shuffles are
//   needed; the record fragments carry the matching k order.  Copy waves, one
//   per compute wave, double-buffer the records in LDS with
//   global_load_lds_dwordx4, pull the chunk after next into L2, and store the
//   output tiles the compute waves leave in LDS, so the compute waves run only
//   LDS reads and MFMAs while the next chunk is in flight.
#include "kda_prefill_common.h"

namespace kda {

namespace {

using namespace prefill;

// 16-column value blocks per scan compute wave.  One copy wave per compute wave:
// more copy waves do not raise a CU's copy rate (measured on MI355X: 2 compute
// waves with 4 or 6 copy waves took 292 and 328 us at 4x8192 x16 heads, vs 283).
constexpr int SCAN_NB = 1;

// 16 bytes per lane from global memory straight into LDS (no VGPR staging):
// lane l's bytes land at LDS address lds + 16 l.  The global address is a
// wave-uniform base (SGPR pair) plus a per-lane 32-bit byte offset.  Issued as
// inline asm so the compiler does not track it: the scan loop orders these copies
// itself with an explicit s_waitcnt vmcnt and a barrier before any wave reads
// the buffer.
__device__ __forceinline__ void lds_dma16(uint64_t gbase, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(lane_off), "s"(gbase)
               : "memory", "m0");
}

// 4 bytes per lane, same addressing (lane l writes lds + 4 l).
__device__ __forceinline__ void lds_dma4(uint64_t gbase, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(lane_off), "s"(gbase)
               : "memory", "m0");
}

__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// LDS byte address of a __shared__ object (computed once; no per-use cast).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)p)));
}

__device__ __forceinline__ half8 frag(const unsigned char* r, int f, int lane) {
  return *reinterpret_cast<const half8*>(r + f * 1024 + lane * 16);
}

__device__ __forceinline__ half8 pack_f16(f32x4 a, f32x4 b) {
  half8 h = {static_cast<_Float16>(a[0]), static_cast<_Float16>(a[1]),
             static_cast<_Float16>(a[2]), static_cast<_Float16>(a[3]),
             static_cast<_Float16>(b[0]), static_cast<_Float16>(b[1]),
             static_cast<_Float16>(b[2]), static_cast<_Float16>(b[3])};
  return h;
}

// Each LDS buffer holds one chunk record followed by NW per-wave value tiles
// (64 tokens x 16*NB value columns, bf16, row-major).
template <int NB>
struct VTile {
  static constexpr int COLS = 16 * NB;
  static constexpr int BYTES = 64 * COLS * 2;
  static constexpr int LANES_PER_ROW = COLS * 2 / 16;       // 16 bytes per lane
  static constexpr int ROWS_PER_COPY = 64 / LANES_PER_ROW;
  static constexpr int COPIES = 64 / ROWS_PER_COPY;
};

// The copies copy wave c of NC issues to bring chunk jj into an LDS buffer: its share
// of the chunk record (the contiguous 1 KiB fragments [c*PER, (c+1)*PER); all issue the
// same compile-time count, surplus copies repeating the last fragment with identical
// bytes) and, when it serves a compute wave (has_vt), that wave's value tile (16 bytes
// per lane per copy, rows in order; rows past the chunk end re-read the last valid
// row, in bounds, whose values only ever meet zero columns of T' and are never stored).
template <int NC, int NB>
struct ChunkCopy {
  using VTl = VTile<NB>;
  static constexpr int NF = REC_BYTES / 1024;
  static constexpr int PER = (NF + NC - 1) / NC;
  static constexpr int NDMA = VTl::COPIES + PER;
  uint64_t rec;    // chunk record base (wave-uniform)
  uint64_t vt;     // value tile base (wave-uniform)
  uint32_t lds;    // destination buffer (LDS byte address)
  uint32_t vlds;   // this wave's value tile inside it
  uint32_t lane_off;
  uint32_t voff[VTl::COPIES];
  int f0;
  bool has_vt;

  __device__ __forceinline__ ChunkCopy(const PrefillParams& p, const unsigned char* recbase,
                                       int cs, int ce, int jj, int h, int v0, int c, bool vt_,
                                       int lane, uint32_t lds_, int vt_off) {
    has_vt = vt_;
    rec = uniform_addr(recbase + static_cast<int64_t>(jj) * p.H * REC_BYTES);
    const int tbj = cs + jj * CHUNK;
    const int Lc = min(CHUNK, ce - tbj);
    vt = uniform_addr(p.v + static_cast<int64_t>(tbj) * p.v_st + h * D + v0);
    lds = lds_;
    vlds = lds_ + static_cast<uint32_t>(vt_off);
    lane_off = static_cast<uint32_t>(lane * 16);
#pragma unroll
    for (int i = 0; i < VTl::COPIES; ++i) {
      const int row = min(lane / VTl::LANES_PER_ROW + VTl::ROWS_PER_COPY * i, Lc - 1);
      voff[i] = static_cast<uint32_t>((row * p.v_st + 8 * (lane % VTl::LANES_PER_ROW)) * 2);
    }
    f0 = c * PER;
    vrow_lane = static_cast<uint32_t>(min(lane, Lc - 1) * p.v_st * 2);
  }
  __device__ __forceinline__ void all() const {
    if (has_vt) {
#pragma unroll
      for (int i = 0; i < VTl::COPIES; ++i) lds_dma16(vt, voff[i], vlds + i * 1024u);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t f = static_cast<uint32_t>(min(f0 + i, NF - 1));
      lds_dma16(rec + f * 1024u, lane_off, lds + f * 1024u);
    }
  }
  // Pulls this wave's share of the chunk into L2 ahead of its copy: one dword per
  // 128-byte line of the record share (lines past the record clamp to its last
  // dword) and one per value-tile row (a wave without a value tile re-touches the
  // record's last dword, so every wave issues NTOUCH), dropped into a 256-byte LDS
  // sink that nothing reads.
  static constexpr int NTOUCH = (PER * 8 + 63) / 64 + 1;
  __device__ __forceinline__ void touch(int lane, uint32_t sink) const {
#pragma unroll
    for (int i = 0; i < NTOUCH - 1; ++i) {
      const uint32_t off = min(static_cast<uint32_t>(f0 * 1024 + (64 * i + lane) * 128),
                               static_cast<uint32_t>(REC_BYTES - 4));
      lds_dma4(rec, off, sink);
    }
    if (has_vt)
      lds_dma4(vt, vrow_lane, sink);
    else
      lds_dma4(rec, static_cast<uint32_t>(REC_BYTES - 4), sink);
  }
  uint32_t vrow_lane;
};

// The scatter indices of chunk jj's tokens (one per lane, rows past the chunk end
// re-reading the last, in bounds) into the 64-entry LDS array at `lds`.  The copy
// waves read them from there: a vector load the compiler tracks would make it wait
// for the in-flight record copies it cannot see.
__device__ __forceinline__ void copy_out_index(const PrefillParams& p, int cs, int ce, int jj,
                                               int lane, uint32_t lds) {
  const int tbj = cs + jj * CHUNK;
  const int Lc = min(CHUNK, ce - tbj);
  lds_dma4(uniform_addr(p.out_idx + tbj), static_cast<uint32_t>(min(lane, Lc - 1) * 4), lds);
}

// Stores the output tile of compute wave w for chunk jj (rows < chunk length) from LDS
// to out: 16 bytes per lane, LANES_PER_ROW lanes per row.  With a scatter index (sidx:
// the chunk's indices in LDS), token t goes to row out_idx[t] when that lies in
// [0, out_rows).
template <int NB>
__device__ __forceinline__ void store_out_tile(const PrefillParams& p, const uint16_t* so,
                                               const int* sidx, int cs, int ce, int jj, int h,
                                               int v0, int lane) {
  using VTl = VTile<NB>;
  const int tbj = cs + jj * CHUNK;
  const int Lc = min(CHUNK, ce - tbj);
#pragma unroll
  for (int i = 0; i < VTl::COPIES; ++i) {
    const int row = lane / VTl::LANES_PER_ROW + VTl::ROWS_PER_COPY * i;
    const int col = 8 * (lane % VTl::LANES_PER_ROW);
    const uint4 val = *reinterpret_cast<const uint4*>(so + row * VTl::COLS + col);
    const int64_t orow = p.out_idx ? static_cast<int64_t>(sidx[row]) : tbj + row;
    if (row < Lc && orow >= 0 && orow < p.out_rows)
      *reinterpret_cast<uint4*>(p.out + orow * p.o_st + h * D + v0 + col) = val;
  }
}

// One chunk of the state scan for NB 16-column blocks of this wave, reading the record
// from LDS buffer R and writing the chunk's output rows (bf16, 64 x 16 NB, row-major,
// rows past the chunk end included) to the LDS tile SO.  Every fragment read from LDS
// feeds NB MFMAs.
template <int NB>
__device__ __forceinline__ void scan_chunk(const unsigned char* __restrict__ R,
                                           const unsigned char* __restrict__ VT,
                                           uint16_t* __restrict__ SO, int Lc, int lane,
                                           f32x4 (&S)[NB][8]) {
  const int nl = lane & 15, g = lane >> 4;
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(VT);
  half8 Sf[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < 4; ++s) Sf[nb][s] = pack_f16(S[nb][2 * s], S[nb][2 * s + 1]);

  // X = V - K_Gamma S   (rows = tokens, lane column = value channel)
  f32x4 X[NB][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 16 * tb + 4 * g + r;
        const float vv = bf16_to_f32(vt[tt * (16 * NB) + 16 * nb + nl]);
        X[nb][tb][r] = (tt < Lc) ? vv : 0.f;
      }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half8 a = frag(R, FR_KG + 4 * tb + s, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) X[nb][tb] = mfma_f16(a, Sf[nb][s], X[nb][tb]);
    }
  }
  // U = T' X
  half8 Xf[NB][2];
  f32x4 U[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    Xf[nb][0] = pack_f16(X[nb][0], X[nb][1]);
    Xf[nb][1] = pack_f16(X[nb][2], X[nb][3]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) U[nb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    const half8 t0 = frag(R, FR_TP + 0, lane), t1 = frag(R, FR_TP + 1, lane);
    const half8 t2 = frag(R, FR_TP + 2, lane), t3 = frag(R, FR_TP + 3, lane);
    const half8 t4 = frag(R, FR_TP + 4, lane), t5 = frag(R, FR_TP + 5, lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      U[nb][0] = mfma_f16(t0, Xf[nb][0], U[nb][0]);
      U[nb][1] = mfma_f16(t1, Xf[nb][0], U[nb][1]);
      U[nb][2] = mfma_f16(t2, Xf[nb][0], U[nb][2]);
      U[nb][2] = mfma_f16(t3, Xf[nb][1], U[nb][2]);
      U[nb][3] = mfma_f16(t4, Xf[nb][0], U[nb][3]);
      U[nb][3] = mfma_f16(t5, Xf[nb][1], U[nb][3]);
    }
  }
  half8 Uf[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    Uf[nb][0] = pack_f16(U[nb][0], U[nb][1]);
    Uf[nb][1] = pack_f16(U[nb][2], U[nb][3]);
  }

  // O^T = S^T (scale Q_Gamma)^T + U^T (scale tril P)^T; lane (token, g) holds 4 value columns.
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    f32x4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half8 bq = frag(R, FR_QG + 4 * tb + s, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Sf[nb][s], bq, o[nb]);
    }
    const int fi = (tb < 2) ? tb : 2 + 2 * (tb - 2);
    {
      const half8 bp = frag(R, FR_PM + fi, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Uf[nb][0], bp, o[nb]);
    }
    if (tb >= 2) {
      const half8 bp = frag(R, FR_PM + fi + 1, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Uf[nb][1], bp, o[nb]);
    }
    uint16_t* orow = SO + (16 * tb + nl) * (16 * NB) + 4 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<uint2*>(orow + 16 * nb) =
          make_uint2(pack_bf16x2(o[nb][0], o[nb][1]), pack_bf16x2(o[nb][2], o[nb][3]));
  }
  // S <- Diag(Gamma_C) S + K_C^T U
  const float* gam = reinterpret_cast<const float*>(R + REC_GAMMA_OFF);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const float4 gc = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
    const half8 k0 = frag(R, FR_KC + 2 * cb + 0, lane), k1 = frag(R, FR_KC + 2 * cb + 1, lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      S[nb][cb][0] *= gc.x;
      S[nb][cb][1] *= gc.y;
      S[nb][cb][2] *= gc.z;
      S[nb][cb][3] *= gc.w;
      S[nb][cb] = mfma_f16(k0, Uf[nb][0], S[nb][cb]);
      S[nb][cb] = mfma_f16(k1, Uf[nb][1], S[nb][cb]);
    }
  }
}

// Workgroup: NW compute waves (wave w owns value columns v0 .. v0 + 16 NB) and NC >= NW
// copy waves (copy wave c < NW serves compute wave c's value and output tiles).  A wave that issues a whole chunk's copies stalls at issue until the copy
// engine has drained most of them, and copies issued piecemeal during the compute land
// too late; so all vector-memory work goes to waves of their own: they issue a chunk's
// copies at once at the start of the previous chunk and wait for them, and store the
// output tiles the compute waves leave in LDS.  The compute waves only read LDS and
// run MFMAs.  One barrier per chunk plus a final one: when every wave has reached
// barrier j, chunk j has landed in buffer j%2, chunk j-1's buffer is free and chunk
// j-1's output tiles are complete.
template <int NW, int NC, int NB>
__global__ __launch_bounds__(64 * (NW + NC))
__attribute__((amdgpu_waves_per_eu((NW + NC + 3) / 4, (NW + NC + 3) / 4)))
void prefill_scan_kernel(PrefillParams p) {
  using VTl = VTile<NB>;
  constexpr int BUF_BYTES = REC_BYTES + NW * VTl::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char srec0[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char srec1[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t touch_sink[NC][64];
  __shared__ __attribute__((aligned(16))) uint16_t sout[2][NW][64 * VTl::COLS];
  __shared__ __attribute__((aligned(16))) int sidx[2][64];   // scatter indices of a chunk
  constexpr int BV = 16 * NB * NW;
  constexpr int NVS = D / BV;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = wave >= NW;
  const int cw = wave - NW;                  // copy wave index
  const bool has_vt = cw < NW;               // copy wave serves compute wave cw
  const int w = copier ? (has_vt ? cw : 0) : wave;   // compute wave served / owned
  const int lane = tid & 63, nl = lane & 15, g = lane >> 4;
  // XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs (id % 8),
  // so the NVS value slices of one (sequence, head) pair get ids congruent mod 8
  // and share one L2 for the record they all read.
  const int H = p.H;
  const int pairs = p.N * H;
  const int blk = blockIdx.x;
  const int grp = blk / (8 * NVS), rr = blk % (8 * NVS);
  const int vs = rr / 8;
  const int pair = grp * 8 + (rr & 7);
  if (pair >= pairs) return;
  const int n = pair / H;
  const int h = pair % H;
  const int v0 = vs * BV + 16 * NB * w;   // first value column of compute wave w
  const int cs = p.cu[n], ce = p.cu[n + 1];
  const int len = ce - cs;
  const int nch = (len + CHUNK - 1) / CHUNK;
  const int64_t slot0 = cs / CHUNK + n;
  const int64_t HDD = static_cast<int64_t>(D) * D;
  const unsigned char* recbase = p.work + (slot0 * H + h) * REC_BYTES;
  const int vt_off = REC_BYTES + w * VTl::BYTES;

  if (copier) {
    // Each chunk: copy chunk j+1 into LDS, pull chunk j+2 into L2 (the copies then hit
    // L2 instead of paying the full memory latency), wait for the copies only: vmcnt
    // counts in issue order, so NTOUCH outstanding operations left means exactly the
    // touches are still in flight.
    using CC = ChunkCopy<NC, NB>;
    const uint32_t lds0 = lds_addr(srec0), lds1 = lds_addr(srec1);
    const uint32_t sink = lds_addr(touch_sink[cw]);
    for (int j = 0; j < nch; ++j) {
      if (j == 0) {
        CC(p, recbase, cs, ce, 0, h, v0, cw, has_vt, lane, lds0, vt_off).all();
        CC(p, recbase, cs, ce, min(1, nch - 1), h, v0, cw, has_vt, lane, lds1, vt_off).touch(lane, sink);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CC::NTOUCH) : "memory");
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (j + 1 < nch)
        CC(p, recbase, cs, ce, j + 1, h, v0, cw, has_vt, lane, (j & 1) ? lds0 : lds1, vt_off).all();
      // Chunk j's scatter indices, read when its outputs are stored at the next chunk.
      if (p.out_idx && cw == 0) copy_out_index(p, cs, ce, j, lane, lds_addr(sidx[j & 1]));
      if (j > 0 && has_vt)
        store_out_tile<NB>(p, sout[(j - 1) & 1][w], sidx[(j - 1) & 1], cs, ce, j - 1, h, v0,
                           lane);
      if (j + 1 < nch) {
        CC(p, recbase, cs, ce, min(j + 2, nch - 1), h, v0, cw, has_vt, lane, lds0, vt_off).touch(lane, sink);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CC::NTOUCH) : "memory");
      }
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nch > 0 && has_vt)
      store_out_tile<NB>(p, sout[(nch - 1) & 1][w], sidx[(nch - 1) & 1], cs, ce, nch - 1, h, v0,
                         lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // Start state: S[nb][cb][r] = S[16cb + 4g + r][v0 + 16nb + nl].
  f32x4 S[NB][8];
  {
    int row = -1;
    if (p.init) {
      if (p.init_idx) {
        const int ri = p.init_idx[n];
        row = (ri >= 0 && ri < p.init_rows) ? ri : -1;
      } else {
        row = n;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (row >= 0) {
        const float* src = p.init + (static_cast<int64_t>(row) * H + h) * HDD + v0 + 16 * nb + nl;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nb][cb][r] = src[(16 * cb + 4 * g + r) * D];
      } else {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) S[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // Two chunks per trip so each half reads one fixed LDS buffer.
  for (int j = 0; j < nch; j += 2) {
    // Reads of the buffer about to be refilled are complete once lgkmcnt is zero.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    scan_chunk<NB>(srec0, srec0 + vt_off, sout[0][w], min(CHUNK, len - j * CHUNK), lane, S);
    if (j + 1 >= nch) break;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    scan_chunk<NB>(srec1, srec1 + vt_off, sout[1][w], min(CHUNK, len - (j + 1) * CHUNK), lane,
                   S);
  }
  // Output tiles of the last chunk complete before the copy waves store them.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if (p.final_state) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float* dst = p.final_state + (static_cast<int64_t>(n) * H + h) * HDD + v0 + 16 * nb + nl;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g + r) * D] = S[nb][cb][r];
    }
  }
  // Drain the final-state stores where the compiler sees it: its wait analysis joins
  // this path with the copy waves' code, and stores it thinks pending there would make
  // it wait inside the copy loop, on record copies it cannot see.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unchanged
}

template <int NW, int NC, int NB>
hipError_t launch_scan(const PrefillParams& p, hipStream_t s) {
  const int64_t pairs = static_cast<int64_t>(p.N) * p.H;
  const int64_t groups = (pairs + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / (16 * NB * NW))));
  hipLaunchKernelGGL((prefill_scan_kernel<NW, NC, NB>), grid, dim3(64 * (NW + NC)), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int phases, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  if (phases & PHASE_INTRA) {
    const hipError_t e = launch_prefill_intra(p, s);
    if (e != hipSuccess) return e;
  }
  if (!(phases & PHASE_SCAN)) return hipSuccess;
  // Two compute waves (32 value columns) per workgroup when the four workgroups of every
  // (sequence, head) pair fit on the chip at once, else four (64 columns): each CU then
  // takes in half as much record per column, which costs a second wave of
  // workgroups when the pairs outnumber a quarter of the CUs (measured on MI355X:
  // 279 vs 320 us at 4x8192 x16 heads, 145 vs 102 us at 8x2048 x16 heads).
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t pairs = static_cast<int64_t>(p.N) * p.H;
  if (pairs * 4 <= cus) return launch_scan<2, 2, SCAN_NB>(p, s);
  return launch_scan<4, 4, SCAN_NB>(p, s);
}

}  // namespace kda
