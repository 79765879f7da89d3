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
//   global_load_lds_dwordx4 and pull this workgroup's share of the chunk after
//   next into L2; the output tiles the compute waves leave in LDS are stored by a
//   store wave (two compute waves) or by the copy waves (four), so the compute
//   waves run only LDS reads and MFMAs while the next chunk is in flight.
#include <algorithm>

#include "kda_prefill_common.h"

namespace kda {

namespace {

using namespace prefill;

// 16-column value blocks per scan compute wave.  One copy wave per compute wave:
// more copy waves do not raise a CU's copy rate (measured on MI355X at 4x8192 x16
// heads: 2 compute waves with 4 or 6 copy waves took 292 and 328 us against 283
// before the shared touch-ahead, and 4 took 206-209 against 201-204 us after it).
constexpr int SCAN_NB = 1;

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

// Bank-conflict-free LDS layouts (32 banks of 4 bytes).  Value tile: in rows 4..7 of
// every 8 the 16-byte pieces are stored with piece bit 1 flipped, so the compute waves'
// column reads of rows 4g + r (lane groups g = 0, 1 read together) fall in different
// banks.  Output tile: the 8-byte piece g of row r is stored at piece g ^ ((r >> 2) & 3),
// so the 16 rows of one 8-byte write land in all 32 banks.
__device__ __forceinline__ int vswz(int row) { return 2 * ((row >> 2) & 1); }
__device__ __forceinline__ int oswz(int row) { return (row >> 2) & 3; }
// Output tiles are padded by 64 bytes so tiles read side by side by the store wave start
// 16 banks apart.
constexpr int OUT_PAD = 32;

// The copies copy wave c of NC issues to bring chunk jj into an LDS buffer: its share
// of the chunk record (the contiguous 1 KiB fragments [c*PER, (c+1)*PER); all issue the
// same compile-time count, surplus copies repeating the last fragment with identical
// bytes) and, when has_vt, its share of the workgroup's value tile (16 bytes per lane
// per copy, rows in order; rows past the chunk end re-read the last valid row, in
// bounds, whose values only ever meet zero columns of T' and are never stored).
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
    vlds = lds_ + static_cast<uint32_t>(vt_off + c * VTl::COPIES * 1024);
    lane_off = static_cast<uint32_t>(lane * 16);
    // The value tiles of all compute waves form one [64][16 NB NC] tile (rows of
    // 32 NB NC bytes, pieces swizzled by vswz); copy wave c issues its instructions
    // c*COPIES .. c*COPIES+COPIES-1, each 16 bytes per lane, so rows go out as runs of
    // that length.
    constexpr int LPR = 2 * NB * NC, RPI = 64 / LPR;
    static_assert(LPR >= 4, "the value-tile swizzle needs four 16-byte pieces per row");
#pragma unroll
    for (int i = 0; i < VTl::COPIES; ++i) {
      const int lrow = lane / LPR + RPI * (c * VTl::COPIES + i);   // row in the LDS tile
      const int row = min(lrow, Lc - 1);
      voff[i] = static_cast<uint32_t>((row * p.v_st + 8 * ((lane % LPR) ^ vswz(lrow))) * 2);
    }
    f0 = c * PER;
    vrow_lane = static_cast<uint32_t>(min(lane, Lc - 1) * p.v_st * 2);
  }
  // A scan without outputs (a segment's state map or offset) reads neither scale * Q_Gamma
  // nor scale * tril(P): it copies the other 39 fragments, spread over its copy waves.
  static constexpr int NF_NO_OUT = NF - (FR_KC - FR_QG);
  static constexpr int PER_NO_OUT = (NF_NO_OUT + NC - 1) / NC;
  __device__ __forceinline__ void all(bool outputs) const {
    if (has_vt) {
#pragma unroll
      for (int i = 0; i < VTl::COPIES; ++i) lds_dma16(vt, voff[i], vlds + i * 1024u);
    }
    if (outputs) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t f = static_cast<uint32_t>(min(f0 + i, NF - 1));
        lds_dma16(rec + f * 1024u, lane_off, lds + f * 1024u);
      }
    } else {
      const int k0 = (f0 / PER) * PER_NO_OUT;   // this copy wave's share
#pragma unroll
      for (int i = 0; i < PER_NO_OUT; ++i) {
        const int k = min(k0 + i, NF_NO_OUT - 1);
        const uint32_t f = static_cast<uint32_t>(k < FR_QG ? k : k + (FR_KC - FR_QG));
        lds_dma16(rec + f * 1024u, lane_off, lds + f * 1024u);
      }
    }
  }
  // Pulls this workgroup's share of chunk jj's record into L2 ahead of its copy: the
  // workgroups that read the same records (nshare of them) each touch one dword per
  // 128-byte line of their own part of it, split over the NC copy waves, plus one dword
  // per value-tile row of their own slice (a wave without a value tile re-touches a
  // line of its part), dropped into a 256-byte LDS sink that nothing reads.  Every
  // workgroup touching the whole record instead ran slower than no touch at all (copy
  // probe on MI355X, 64 records per step shared four ways: 3430 cycles per step without
  // touches, 4680 touching the whole record, 2150 touching a quarter each).
  static constexpr int REC_LINES = (REC_BYTES + 127) / 128;
  static constexpr int MIN_SHARE = D / (16 * NB * NC);   // value slices: fewest sharers
  static constexpr int NTOUCH_REC = ((REC_LINES + MIN_SHARE - 1) / MIN_SHARE + NC - 1) / NC;
  static_assert(NTOUCH_REC <= 64, "one touch instruction per copy wave");
  static constexpr int NTOUCH = 2;
  __device__ __forceinline__ void touch(int lane, uint32_t sink, int c, int share,
                                        int nshare, bool touch_v) const {
    const int per_wg = (REC_LINES + nshare - 1) / nshare;
    const int per_wave = (per_wg + NC - 1) / NC;
    const int first = min(share * per_wg + c * per_wave, REC_LINES - 1);
    const int last = min(min(share * per_wg + (c + 1) * per_wave, (share + 1) * per_wg),
                         REC_LINES) - 1;
    const int line = min(first + lane, max(last, first));
    const uint32_t off = min(static_cast<uint32_t>(line * 128), static_cast<uint32_t>(REC_BYTES - 4));
    lds_dma4(rec, off, sink);
    if (touch_v)
      lds_dma4(vt, vrow_lane, sink);
    else
      lds_dma4(rec, off, sink);
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
    const int f = oswz(row);
    uint4 val = *reinterpret_cast<const uint4*>(so + row * VTl::COLS + (col ^ (8 * (f >> 1))));
    if (f & 1) val = make_uint4(val.z, val.w, val.x, val.y);
    const int64_t orow = p.out_idx ? static_cast<int64_t>(sidx[row]) : tbj + row;
    if (row < Lc && orow >= 0 && orow < p.out_rows)
      *reinterpret_cast<uint4*>(p.out + orow * p.o_st + h * D + v0 + col) = val;
  }
}

// The store wave's variant: the NW output tiles of a chunk (one per compute wave, 16 NB
// columns each, side by side in the output row) stored together, so each lane's 16 bytes
// and its row neighbours form one contiguous 32 NB NW-byte run per row (fewer, longer
// row segments per store instruction than one tile at a time).
template <int NB, int NW>
__device__ __forceinline__ void store_out_tiles(const PrefillParams& p,
                                                const uint16_t (*so)[64 * 16 * NB + OUT_PAD],
                                                const int* sidx, int cs, int ce, int jj, int h,
                                                int vbase, int lane) {
  constexpr int TCOLS = 16 * NB;                 // columns of one tile
  constexpr int LPR = NW * TCOLS * 2 / 16;        // lanes per output row
  constexpr int RPI = 64 / LPR;                   // rows per store instruction
  const int tbj = cs + jj * CHUNK;
  const int Lc = min(CHUNK, ce - tbj);
  const int q = lane % LPR;                       // 16-byte piece of the row
  const int tile = q / (TCOLS / 8), tc = 8 * (q % (TCOLS / 8));
#pragma unroll
  for (int i = 0; i < 64 / RPI; ++i) {
    const int row = lane / LPR + RPI * i;
    const int f = oswz(row);
    uint4 val = *reinterpret_cast<const uint4*>(so[tile] + row * TCOLS + (tc ^ (8 * (f >> 1))));
    if (f & 1) val = make_uint4(val.z, val.w, val.x, val.y);
    const int64_t orow = p.out_idx ? static_cast<int64_t>(sidx[row]) : tbj + row;
    if (row < Lc && orow >= 0 && orow < p.out_rows)
      *reinterpret_cast<uint4*>(p.out + orow * p.o_st + h * D + vbase + 8 * q) = val;
  }
}

// One chunk of the state scan for NB 16-column blocks of this wave, reading the record
// from LDS buffer R and writing the chunk's output rows (bf16, 64 x 16 NB, row-major,
// rows past the chunk end included) to the LDS tile SO.  Every fragment read from LDS
// feeds NB MFMAs.
template <int NB, int NW>
__device__ __forceinline__ void scan_chunk(const unsigned char* __restrict__ R,
                                           const unsigned char* __restrict__ VT, int vcol,
                                           uint16_t* __restrict__ SO, int Lc, bool zero_v,
                                           bool write_out, int lane, f32x4 (&S)[NB][8]) {
  const int nl = lane & 15, g = lane >> 4;
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(VT);
  // Stage 1: every LDS read of the X and U products goes out before the first MFMA.
  uint16_t vraw[NB][4][4];
  half8 kgf[16], tpf[6];
  // Rows 16 tb + 4 g + r have vswz = 2 (g & 1): the swizzled column is one per lane.
  int vcl[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) vcl[nb] = ((vcol + 16 * nb) ^ (16 * (g & 1))) + nl;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vraw[nb][tb][r] = vt[(16 * tb + 4 * g + r) * (16 * NB * NW) + vcl[nb]];
#pragma unroll
  for (int f = 0; f < 16; ++f) kgf[f] = frag(R, FR_KG + f, lane);
#pragma unroll
  for (int f = 0; f < 6; ++f) tpf[f] = frag(R, FR_TP + f, lane);
  __builtin_amdgcn_sched_barrier(0);

  half8 Sf[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < 4; ++s) Sf[nb][s] = pack_f16(S[nb][2 * s], S[nb][2 * s + 1]);
  f32x4 X[NB][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 16 * tb + 4 * g + r;
        X[nb][tb][r] = (tt < Lc && !zero_v) ? bf16_to_f32(vraw[nb][tb][r]) : 0.f;
      }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) X[nb][tb] = mfma_f16(kgf[4 * tb + s], Sf[nb][s], X[nb][tb]);

  // Stage 2 reads (the output products' operands) go out behind the X products.
  half8 qgf[16], pmf[6];
  if (write_out) {
#pragma unroll
    for (int f = 0; f < 16; ++f) qgf[f] = frag(R, FR_QG + f, lane);
#pragma unroll
    for (int f = 0; f < 6; ++f) pmf[f] = frag(R, FR_PM + f, lane);
  }
  __builtin_amdgcn_sched_barrier(0);

  half8 Xf[NB][2];
  f32x4 U[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    Xf[nb][0] = pack_f16(X[nb][0], X[nb][1]);
    Xf[nb][1] = pack_f16(X[nb][2], X[nb][3]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) U[nb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    U[nb][0] = mfma_f16(tpf[0], Xf[nb][0], U[nb][0]);
    U[nb][1] = mfma_f16(tpf[1], Xf[nb][0], U[nb][1]);
    U[nb][2] = mfma_f16(tpf[2], Xf[nb][0], U[nb][2]);
    U[nb][2] = mfma_f16(tpf[3], Xf[nb][1], U[nb][2]);
    U[nb][3] = mfma_f16(tpf[4], Xf[nb][0], U[nb][3]);
    U[nb][3] = mfma_f16(tpf[5], Xf[nb][1], U[nb][3]);
  }
  half8 Uf[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    Uf[nb][0] = pack_f16(U[nb][0], U[nb][1]);
    Uf[nb][1] = pack_f16(U[nb][2], U[nb][3]);
  }

  // O^T = S^T (scale Q_Gamma)^T + U^T (scale tril P)^T; lane (token, g) holds 4 value columns.
  if (write_out) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x4 o[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Sf[nb][s], qgf[4 * tb + s], o[nb]);
      const int fi = (tb < 2) ? tb : 2 + 2 * (tb - 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Uf[nb][0], pmf[fi], o[nb]);
      if (tb >= 2) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f16(Uf[nb][1], pmf[fi + 1], o[nb]);
      }
      // row 16 tb + nl: oswz = (nl >> 2) & 3
      uint16_t* orow = SO + (16 * tb + nl) * (16 * NB) + 4 * (g ^ ((nl >> 2) & 3));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<uint2*>(orow + 16 * nb) =
            make_uint2(pack_bf16x2(o[nb][0], o[nb][1]), pack_bf16x2(o[nb][2], o[nb][3]));
    }
  }
  // Stage 3 reads (the state update's operands) go out behind the output products.
  half8 kcf[16];
  float4 gcv[8];
  const float* gam = reinterpret_cast<const float*>(R + REC_GAMMA_OFF);
#pragma unroll
  for (int f = 0; f < 16; ++f) kcf[f] = frag(R, FR_KC + f, lane);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) gcv[cb] = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
  __builtin_amdgcn_sched_barrier(0);

  // S <- Diag(Gamma_C) S + K_C^T U
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      S[nb][cb][0] *= gcv[cb].x;
      S[nb][cb][1] *= gcv[cb].y;
      S[nb][cb][2] *= gcv[cb].z;
      S[nb][cb][3] *= gcv[cb].w;
      S[nb][cb] = mfma_f16(kcf[2 * cb], Uf[nb][0], S[nb][cb]);
      S[nb][cb] = mfma_f16(kcf[2 * cb + 1], Uf[nb][1], S[nb][cb]);
    }
  }
}

// What one scan workgroup does: a chunk range of one (sequence, head) pair for one
// slice of value columns, from a start state, optionally writing outputs and a final
// state.
constexpr int START_INIT = 0;    // the caller's initial state (direct, gathered, or zero)
constexpr int START_ZERO = 1;
constexpr int START_IDENT = 2;   // identity columns: the segment's state map
constexpr int START_WS = 3;      // a state in the segment workspace

struct ScanWork {
  int n, h, vs, jb, je;          // sequence, head, value slice, chunks [jb, je)
  int share, nshare;             // this workgroup's index among those reading the same records
  int start;
  const float* start_blk;        // START_WS: the [128][128] start state
  float* fin_blk;                // [128][128] destination of the end state, or null
  bool zero_v, write_out;
  int active;                    // bit w set: compute wave w scans its value columns
};

// Workspace of the segment-parallel scan: per (sequence, head), SEG_SLOTS states of
// [128][128] fp32.  Slot s-1 holds the start state S_in(s) of segment s (1 <= s < G);
// slot (G-1) + (s-1) the map M_s and slot 2(G-1) - 1 + (s-1) the offset B_s of middle
// segment s (1 <= s <= G-2), where S_out(s) = M_s S_in(s) + B_s.
__device__ __forceinline__ float* seg_slot(const PrefillParams& p, int n, int h, int slot) {
  return p.seg_ws + ((static_cast<int64_t>(n) * p.H + h) * SEG_SLOTS + slot) * (D * D);
}
__device__ __forceinline__ int seg_m_slot(int G, int s) { return (G - 1) + (s - 1); }
__device__ __forceinline__ int seg_b_slot(int G, int s) { return (G - 1) + (G - 2) + (s - 1); }

// Chunks [jb, je) of segment s of G over a sequence of nch chunks.  Segment 0 gets
// SEG0_WEIGHT / SEG_WEIGHT of a later segment's share: phase A runs it with its outputs,
// whose chunk steps take longer than those of the middle segments' state maps beside it
// (no output products or stores, 39 of the 61 record fragments), so a shorter segment 0
// ends with them.  Measured at 1 x 16384 x 16 heads (G = 5, segment 0 on half-active
// workgroups): prefill call 264, 262, 267, 278, 287 us for weights 4, 5, 6, 7, 8 of 8;
// with segment 0 on full four-wave workgroups, 287, 284, 279, 288, 299 us.
constexpr int SEG0_WEIGHT = 5;
constexpr int SEG_WEIGHT = 8;
__device__ __forceinline__ int seg_begin(int nch, int G, int s) {
  if (s == 0) return 0;
  return static_cast<int>(static_cast<int64_t>(nch) * (SEG0_WEIGHT + SEG_WEIGHT * (s - 1)) /
                          (SEG0_WEIGHT + SEG_WEIGHT * (G - 1)));
}

// MODE_SEQ: whole sequences.  MODE_SEG_A: segment 0 with outputs, and the state maps
// (M_s, B_s) of the middle segments.  MODE_SEG_C: segments 1..G-1 from their start
// states, with outputs.
constexpr int MODE_SEQ = 0;
constexpr int MODE_SEG_A = 1;
constexpr int MODE_SEG_C = 2;

// Workgroups per unit of work (a pair, or a pair's segment) and the workgroup -> unit
// order: ids are dealt round-robin to the 8 XCDs (id % 8), so the workgroups of one
// unit get ids congruent mod 8 and share one L2 for the records they all read.
template <int MODE, int NVS, int NW>
__device__ __forceinline__ bool decode_work(const PrefillParams& p, ScanWork& wk) {
  constexpr int PER_UNIT = (MODE == MODE_SEG_A) ? 2 * NVS : NVS;
  const int H = p.H;
  const int pairs = p.N * H;
  const int G = p.seg_G;
  const int units = (MODE == MODE_SEQ) ? pairs : pairs * (G - 1);
  const int blk = blockIdx.x;
  const int grp = blk / (8 * PER_UNIT), rr = blk % (8 * PER_UNIT);
  const int cg = rr / 8;
  const int unit = grp * 8 + (rr & 7);
  if (unit >= units) return false;
  const int pair = (MODE == MODE_SEQ) ? unit : unit / (G - 1);
  wk.n = pair / H;
  wk.h = pair % H;
  const int len = p.cu[wk.n + 1] - p.cu[wk.n];
  const int nch = (len + CHUNK - 1) / CHUNK;
  wk.start_blk = nullptr;
  wk.zero_v = false;
  wk.write_out = true;
  wk.active = (1 << NW) - 1;
  wk.share = cg;
  wk.nshare = NVS;
  if (MODE == MODE_SEQ) {
    wk.vs = cg;
    wk.jb = 0;
    wk.je = nch;
    wk.start = START_INIT;
    wk.fin_blk = p.final_state ? p.final_state + (static_cast<int64_t>(wk.n) * H + wk.h) * (D * D)
                               : nullptr;
    return true;
  }
  if (MODE == MODE_SEG_A) {
    const int s = unit % (G - 1);        // segments 0 .. G-2
    wk.jb = seg_begin(nch, G, s);
    wk.je = seg_begin(nch, G, s + 1);
    if (s == 0) {
      // Segment 0 carries the outputs: its 2 NVS workgroups each run half of their
      // compute waves, so each CU reads the record once per 32 value columns, as the
      // two-compute-wave scans do (the chunk step of a full four-wave scan with outputs
      // is longer than that of the maps beside it).
      wk.vs = cg >> 1;
      wk.active = ((1 << (NW / 2)) - 1) << ((cg & 1) * (NW / 2));
      wk.start = START_INIT;
      wk.fin_blk = seg_slot(p, wk.n, wk.h, 0);          // S_in(1)
      return true;
    }
    wk.write_out = false;
    wk.nshare = 2 * NVS;                 // the map and offset workgroups read the same records
    if (cg < NVS) {                      // the map M_s: identity columns, no values
      wk.vs = cg;
      wk.start = START_IDENT;
      wk.zero_v = true;
      wk.fin_blk = seg_slot(p, wk.n, wk.h, seg_m_slot(G, s));
    } else {                             // the offset B_s: zero start, the values
      wk.vs = cg - NVS;
      wk.start = START_ZERO;
      wk.fin_blk = seg_slot(p, wk.n, wk.h, seg_b_slot(G, s));
    }
    return true;
  }
  const int s = 1 + unit % (G - 1);      // MODE_SEG_C: segments 1 .. G-1
  wk.vs = cg;
  wk.jb = seg_begin(nch, G, s);
  wk.je = seg_begin(nch, G, s + 1);
  wk.start = START_WS;
  wk.start_blk = seg_slot(p, wk.n, wk.h, s - 1);
  wk.fin_blk = (s == G - 1 && p.final_state)
                   ? p.final_state + (static_cast<int64_t>(wk.n) * H + wk.h) * (D * D)
                   : nullptr;
  return true;
}

// Workgroup: NW compute waves (wave w owns value columns v0 .. v0 + 16 NB), NC = NW copy
// waves (each copies its share of the record and of the combined value tile; without a
// store wave, copy wave c stores compute wave c's output tile) and, with two compute
// waves, a store wave.  A wave that issues a whole chunk's copies stalls at issue until
// the copy engine has drained most of them, and copies issued piecemeal during the
// compute land too late; so all vector-memory work goes to waves of their own: they
// issue a chunk's copies at once at the start of the previous chunk and wait for them,
// and store the output tiles the compute waves leave in LDS.  The compute waves only
// read LDS and run MFMAs.  One barrier per chunk plus a final one: when every wave has
// reached the barrier of chunk j, chunk j has landed in buffer (j - jb) % 2, chunk j-1's
// buffer is free and chunk j-1's output tiles are complete.
// With two compute waves the copy waves bound the chunk step, and a separate store wave
// takes the output stores off them; with four the compute does, and the copy waves store.
template <int NW>
constexpr int store_waves() { return NW == 2 ? 1 : 0; }

template <int NW, int NC, int NB, int MODE>
__global__ __launch_bounds__(64 * (NW + NC + store_waves<NW>()))
__attribute__((amdgpu_waves_per_eu((NW + NC + store_waves<NW>() + 3) / 4,
                                   (NW + NC + store_waves<NW>() + 3) / 4)))
void prefill_scan_kernel(PrefillParams p) {
  using VTl = VTile<NB>;
  static_assert(NC == NW, "each copy wave fills its share of the combined value tile");
  static_assert(MODE != MODE_SEG_A || store_waves<NW>() == 0,
                "segment 0's half-active workgroups have their copy waves store the outputs");
  constexpr int BUF_BYTES = REC_BYTES + NW * VTl::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char srec0[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char srec1[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t touch_sink[NC][64];
  __shared__ __attribute__((aligned(16))) uint16_t sout[2][NW][64 * VTl::COLS + OUT_PAD];
  __shared__ __attribute__((aligned(16))) int sidx[2][64];   // scatter indices of a chunk
  constexpr int BV = 16 * NB * NW;
  constexpr int NVS = D / BV;
  ScanWork wk;
  if (!decode_work<MODE, NVS, NW>(p, wk)) return;   // uniform: the whole workgroup exits
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool STORE_WAVE = store_waves<NW>() == 1;
  const bool storer = STORE_WAVE && wave == NW + NC;
  const bool copier = wave >= NW && !storer;
  const int cw = wave - NW;                  // copy wave index
  const bool has_vt = cw < NW;               // every copy wave (NC = NW) copies value rows
  const int w = copier ? (has_vt ? cw : 0) : wave;   // compute wave served / owned
  const int lane = tid & 63, nl = lane & 15, g = lane >> 4;
  const int H = p.H;
  const int n = wk.n, h = wk.h, jb = wk.jb, je = wk.je;
  const int v0 = wk.vs * BV + 16 * NB * w;   // first value column of compute wave w
  const int cs = p.cu[n], ce = p.cu[n + 1];
  const int len = ce - cs;
  const int64_t slot0 = cs / CHUNK + n;
  const unsigned char* recbase = p.work + (slot0 * H + h) * REC_BYTES;
  const int vt_off = REC_BYTES;                // the combined value tile

  if (STORE_WAVE && storer) {
    // The store wave: after each chunk's barrier, the previous chunk's output tiles
    // (left in LDS by the compute waves) go to out.  Its stores have their own vmcnt,
    // so neither their issue nor their acknowledgements delay the copy waves' waits.
    for (int j = jb; j < je; ++j) {
      const int par = (j - jb) & 1;
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (j > jb && wk.write_out)
        store_out_tiles<NB, NW>(p, sout[par ^ 1], sidx[par ^ 1], cs, ce, j - 1, h, wk.vs * BV,
                                lane);
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (je > jb && wk.write_out) {
      const int par = (je - 1 - jb) & 1;
      store_out_tiles<NB, NW>(p, sout[par], sidx[par], cs, ce, je - 1, h, wk.vs * BV, lane);
    }
    return;
  }

  if (copier) {
    // Each chunk: copy chunk j+1 into LDS, pull chunk j+2 into L2 (the copies then hit
    // L2 instead of paying the full memory latency; see TOUCH), wait for the copies only:
    // vmcnt counts in issue order, so NTOUCH outstanding operations left means exactly the
    // touches are still in flight.  Without a store wave the previous chunk's output
    // stores are issued after that wait, so their write acknowledgements stay off this
    // chunk's critical path (their issue does not: 4 x 8192 x 16 heads, 201 -> 190 us
    // with the store wave).
    using CC = ChunkCopy<NC, NB>;
    // The touch-ahead pays off with four workgroups per pair (two compute waves each:
    // 4 x 8192 x 16 heads, 259 -> 194 us; 1 x 16384 segmented, 238 -> 210 us), where the
    // copies bound the chunk step.  With two (four compute waves: 8 x 2048 x 16 heads,
    // 90 us either way) the compute does, so it is left out there.
    constexpr bool TOUCH = (NW == 2);
    const bool copy_vt = has_vt && !wk.zero_v;
    // One wave touches each 128-byte line of value rows: the two 64-byte halves of a
    // line belong to value slices 2k and 2k+1, and a workgroup's copy waves share it.
    const bool touch_v = copy_vt && cw == 0 && (wk.vs & 1) == 0;
    // Only phase A has inactive compute waves and scans without outputs; elsewhere these
    // conditions fold away at compile time.
    constexpr bool SEG_A = MODE == MODE_SEG_A;
    const bool store = has_vt && (!SEG_A || (wk.write_out && ((wk.active >> w) & 1)));
    const bool full_rec = !SEG_A || wk.write_out;
    const uint32_t lds0 = lds_addr(srec0), lds1 = lds_addr(srec1);
    const uint32_t sink = lds_addr(touch_sink[cw]);
    for (int j = jb; j < je; ++j) {
      const int par = (j - jb) & 1;
      if (j == jb) {
        CC(p, recbase, cs, ce, jb, h, wk.vs * BV, cw, copy_vt, lane, lds0, vt_off).all(full_rec);
        if (TOUCH) {
          CC(p, recbase, cs, ce, min(jb + 1, je - 1), h, wk.vs * BV, cw, copy_vt, lane, lds1, vt_off)
              .touch(lane, sink, cw, wk.share, wk.nshare, touch_v);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CC::NTOUCH) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // Chunk j's scatter indices (read when its outputs are stored at the next chunk)
      // go first, so the wait below covers them before the next barrier.
      if (wk.write_out && p.out_idx && cw == 0)
        copy_out_index(p, cs, ce, j, lane, lds_addr(sidx[par]));
      if (j + 1 < je) {
        CC(p, recbase, cs, ce, j + 1, h, wk.vs * BV, cw, copy_vt, lane, par ? lds0 : lds1, vt_off)
            .all(full_rec);
        if (TOUCH) {
          CC(p, recbase, cs, ce, min(j + 2, je - 1), h, wk.vs * BV, cw, copy_vt, lane, lds0, vt_off)
              .touch(lane, sink, cw, wk.share, wk.nshare, touch_v);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CC::NTOUCH) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      if (!STORE_WAVE && j > jb && store)
        store_out_tile<NB>(p, sout[par ^ 1][w], sidx[par ^ 1], cs, ce, j - 1, h, v0, lane);
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (!STORE_WAVE && je > jb && store) {
      const int par = (je - 1 - jb) & 1;
      store_out_tile<NB>(p, sout[par][w], sidx[par], cs, ce, je - 1, h, v0, lane);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // Start state: S[nb][cb][r] = S[16cb + 4g + r][v0 + 16nb + nl].  An inactive compute
  // wave keeps the workgroup's barrier count and does nothing else.
  const bool act = MODE != MODE_SEG_A || ((wk.active >> w) & 1);
  f32x4 S[NB][8];
  if (act) {
    const float* src_blk = nullptr;
    if (wk.start == START_INIT && p.init) {
      int row = n;
      if (p.init_idx) {
        const int ri = p.init_idx[n];
        row = (ri >= 0 && ri < p.init_rows) ? ri : -1;
      }
      if (row >= 0) src_blk = p.init + (static_cast<int64_t>(row) * H + h) * (D * D);
    } else if (wk.start == START_WS) {
      src_blk = wk.start_blk;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = v0 + 16 * nb + nl;
      if (src_blk) {
        const float* src = src_blk + col;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nb][cb][r] = src[(16 * cb + 4 * g + r) * D];
      } else {
        const float one = (wk.start == START_IDENT) ? 1.f : 0.f;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nb][cb][r] = (16 * cb + 4 * g + r == col) ? one : 0.f;
      }
    }
  }

  // Two chunks per trip so each half reads one fixed LDS buffer.
  for (int j = jb; j < je; j += 2) {
    // Reads of the buffer about to be refilled are complete once lgkmcnt is zero.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (act)
      scan_chunk<NB, NW>(srec0, srec0 + vt_off, 16 * NB * w, sout[0][w], min(CHUNK, len - j * CHUNK),
                         wk.zero_v, wk.write_out, lane, S);
    if (j + 1 >= je) break;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (act)
      scan_chunk<NB, NW>(srec1, srec1 + vt_off, 16 * NB * w, sout[1][w], min(CHUNK, len - (j + 1) * CHUNK),
                         wk.zero_v, wk.write_out, lane, S);
  }
  // Output tiles of the last chunk complete before the copy waves store them.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if (wk.fin_blk && act) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float* dst = wk.fin_blk + v0 + 16 * nb + nl;
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

// Segment start states: S_in(1) comes from segment 0; then, for each middle segment s in
// order, S_in(s+1) = M_s S_in(s) + B_s, as fp32 MFMA products (v_mfma_f32_16x16x4_f32:
// fp32 operands, fp32 accumulation).  One workgroup of 8 waves per (sequence, head,
// 16-column slice); wave w computes the 16x16 output tile of rows 16w.. over the 128-deep
// contraction in 32 k-steps, so every row of M is loaded by one wave of the workgroup.
// The contraction is taken in the order in which lane group g's k-step (j, e) is column
// 16j + 4g + e of M: the four lane groups read each row of M as one 64-byte run.  The
// eight slices of a pair get workgroup ids congruent mod 8 (one XCD), so they share M in
// one L2.  Only S_in is a chain: it stays in LDS from one step to the next (double-
// buffered, rows padded to 20 words so that the two lane groups of a half-wave, four rows
// apart, read disjoint banks), and each step's M and B tiles are loaded into registers
// during the step before.  Each step is 1 MFLOP of fp32 MFMA per pair, about 2K cycles
// on each of its eight CUs.  Measured at 1 x 16384 x 16 heads (three steps, 128
// workgroups): 10.2 us, against 15-16 us with 32-column slices of 16 waves (64
// workgroups; 4.4 us per step with the next step's loads, 2.5 us without, bound by the
// fp32 MFMA rate of one CU), 18.3 us for a VALU loop and 19.4 us for MFMA tiles without
// the prefetch.
constexpr int COMB_COLS = 16;
constexpr int COMB_PAD = 4;
constexpr int COMB_THREADS = 64 * (D / 16);
__global__ __launch_bounds__(COMB_THREADS) void seg_combine_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) float sbuf[2][D][COMB_COLS + COMB_PAD];
  const int G = p.seg_G;
  constexpr int slices = D / COMB_COLS;
  const int grp = blockIdx.x / (8 * slices), rr8 = blockIdx.x % (8 * slices);
  const int pair = grp * 8 + (rr8 & 7);
  if (pair >= p.N * p.H) return;       // the grid is rounded up to whole groups of 8 pairs
  const int c0 = (rr8 >> 3) * COMB_COLS;
  const int n = pair / p.H, h = pair % p.H;
  const int tid = threadIdx.x, rt = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  // lane (r, g) of the tile holds rows 16 rt + 4g + i, column r of the slice
  auto load_mb = [&](int s, float4 (&m)[8], f32x4& bt) {
    const float* M = seg_slot(p, n, h, seg_m_slot(G, s)) + (16 * rt + r) * D + 4 * g;
    const float* B = seg_slot(p, n, h, seg_b_slot(G, s));
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = *reinterpret_cast<const float4*>(M + 16 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) bt[i] = B[(16 * rt + 4 * g + i) * D + c0 + r];
  };
  float4 mcur[8];
  f32x4 bcur;
  if (G >= 3) load_mb(1, mcur, bcur);
  {
    const float* sin = seg_slot(p, n, h, 0);       // S_in(1), from segment 0
    const int rr = tid >> 2, cc = 4 * (tid & 3);   // 128 rows x 4 float4
    *reinterpret_cast<float4*>(&sbuf[0][rr][cc]) =
        *reinterpret_cast<const float4*>(sin + rr * D + c0 + cc);
  }
  __syncthreads();
  for (int s = 1; s <= G - 2; ++s) {
    float4 mnext[8];
    f32x4 bnext = bcur;
    if (s + 1 <= G - 2) load_mb(s + 1, mnext, bnext);
    const float (*sin)[COMB_COLS + COMB_PAD] = sbuf[(s - 1) & 1];
    f32x4 acc = bcur;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a[4] = {mcur[j].x, mcur[j].y, mcur[j].z, mcur[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], sin[16 * j + 4 * g + e][r], acc);
    }
    float* sout = seg_slot(p, n, h, s);
    float (*snext)[COMB_COLS + COMB_PAD] = sbuf[s & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sout[(16 * rt + 4 * g + i) * D + c0 + r] = acc[i];
      snext[16 * rt + 4 * g + i][r] = acc[i];
    }
    __syncthreads();   // S_in(s+1) complete in LDS; S_in(s)'s buffer may be reused
    if (s + 1 <= G - 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mcur[j] = mnext[j];
      bcur = bnext;
    }
  }
}

template <int NW, int NC, int NB, int MODE>
hipError_t launch_scan(const PrefillParams& p, hipStream_t s) {
  constexpr int NVS = D / (16 * NB * NW);
  constexpr int PER_UNIT = (MODE == MODE_SEG_A) ? 2 * NVS : NVS;
  const int64_t pairs = static_cast<int64_t>(p.N) * p.H;
  const int64_t units = (MODE == MODE_SEQ) ? pairs : pairs * (p.seg_G - 1);
  const int64_t groups = (units + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * PER_UNIT));
  hipLaunchKernelGGL((prefill_scan_kernel<NW, NC, NB, MODE>), grid,
                     dim3(64 * (NW + NC + store_waves<NW>())), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int prefill_segments(int N, int T_total, int H, int cus) {
  // Segments pay off when the pairs leave most CUs idle and sequences are long: the
  // critical path goes from G segment lengths to about two, for about three times the
  // scan work spread over otherwise idle CUs.  G is the largest count whose phase A
  // (4 workgroups per segment of G - 1: segment 0 on half-active four-wave scans, the
  // middle segments' maps and offsets on full ones) and phase C (4 two-wave workgroups
  // per segment of G - 1) fit the CUs at once, with at least SEG_MIN_CHUNKS chunks per
  // segment on average.
  const int64_t pairs = static_cast<int64_t>(N) * H;
  if (N <= 0 || pairs > SEG_MAX_PAIRS || pairs * 8 > cus) return 1;
  const int64_t avg_chunks = static_cast<int64_t>(T_total) / CHUNK / N;
  int64_t G = cus / pairs / 4 + 1;
  G = std::min<int64_t>(G, SEG_MAX);
  G = std::min<int64_t>(G, avg_chunks / SEG_MIN_CHUNKS);
  return G >= 3 ? static_cast<int>(G) : 1;
}

hipError_t launch_prefill(const PrefillParams& p_in, int phases, hipStream_t s) {
  if (p_in.N == 0) return hipSuccess;
  if (phases & PHASE_INTRA) {
    const hipError_t e = launch_prefill_intra(p_in, s);
    if (e != hipSuccess) return e;
  }
  if (!(phases & PHASE_SCAN)) return hipSuccess;
  int cus = 0;
  hipError_t e = current_device_cus(&cus);
  if (e != hipSuccess) return e;
  PrefillParams p = p_in;
  const int64_t pairs = static_cast<int64_t>(p.N) * p.H;
  p.seg_G = p.seg_ws ? prefill_segments(p.N, p.T_total, p.H, cus) : 1;
  if (p.seg_G >= 3) {
    // Segment-parallel scan (phase A: segment 0 and the middle segments' state maps;
    // combine; phase C: the later segments from their start states).
    if ((e = launch_scan<4, 4, SCAN_NB, MODE_SEG_A>(p, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel,
                       dim3(static_cast<unsigned>(((pairs + 7) / 8) * 8 * (D / COMB_COLS))),
                       dim3(COMB_THREADS), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_scan<2, 2, SCAN_NB, MODE_SEG_C>(p, s);
  }
  // Two compute waves (32 value columns) per workgroup when the four workgroups of every
  // (sequence, head) pair fit on the chip at once, else four (64 columns): each CU then
  // takes in half as much record per column, which costs a second wave of
  // workgroups when the pairs outnumber a quarter of the CUs (measured on MI355X:
  // 279 vs 320 us at 4x8192 x16 heads, 145 vs 102 us at 8x2048 x16 heads).
  if (pairs * 4 <= cus) return launch_scan<2, 2, SCAN_NB, MODE_SEQ>(p, s);
  return launch_scan<4, 4, SCAN_NB, MODE_SEQ>(p, s);
}

}  // namespace kda
