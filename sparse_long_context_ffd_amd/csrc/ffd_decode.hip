// Fused FFD decode: split-K scan -> Top-δ select -> exact attention, plus the
// log-sum-exp split combine.
//
// Method: "Faster Than Flash: Exploiting Attention Sparsity for Efficient
// Long-Context Decoding" ([TS] = its technical-summary page, Methodology 1-3).
// The selector (low-bit scan + Top-δ) and the computer (exact attention over
// the kept blocks) run in ONE kernel per (sequence, kv head, split), so the
// kept set never leaves the workgroup ([TS] Methodology 3, "Fused Kernel").
//
// One workgroup = 4 wave64s (8 on grids one round long) owns `split_blocks`
// consecutive 64-token blocks of one (sequence b, kv head j) and serves all
// G = Hq/Hkv query heads of the group -- for Q query tokens per sequence,
// G x Q query rows -- so every K/V byte it reads is shared by all of them. When the grid is too small to fill
// the chip, P workgroups share a split (each scans and selects all of it; the
// P x 8 waves of the split take its kept blocks round-robin).
//
//  prologue  the query rows -> LDS (one 16-byte load per thread): the bf16
//            rows and the int8 copy + per-row scale (the scan query), reduced
//            within the lanes holding a row.
//  scan      each wave takes whole blocks, 16-token tiles; lane (g, n) holds
//            D/8 bytes of int4 codes of token n (16 tokens x D/2 B = one
//            contiguous wave load). Nibbles are moved to offset binary (x ^ 8
//            = code + 8, 0..15) and all query rows' dots are one
//            v_mfma_i32_16x16x64_i8 per 64 dims, tokens as rows, so a lane
//            ends with 4 tokens of one query row; the accumulator starts at
//            the -8*sum(q) excess. Block score = max over valid tokens -> LDS.
//            (2-bit thumbnails: the codes spread to bytes, same MFMA.)
//  select    the waves share the rows: per row split max m~ (or the
//            sink/local estimate), threshold fl32(m~ - δ), forced sink/local
//            blocks; then wave 0 compacts the blocks kept by at least one row
//            into a list (with a per-row bit mask) by ballot. The mask is
//            stored in the epilogue.
//  attend    waves take kept blocks round-robin (last-scanned first), one
//            64-token block at a time, on the matrix cores (v_mfma_f32_16x16x32_bf16, the query
//            rows padded to 16 columns):
//              QK  A = K rows straight from HBM into registers (16 tokens x
//                  32 dims per MFMA; each lane reads D/2 contiguous bytes of a
//                  row), B = the bf16 query, 4*(D/32) MFMAs per block;
//              softmax in the MFMA output layout (lane = row, 4 tokens per
//                  tile); the running max of every row starts at the scan's
//                  split max (the scan result reused to seed the softmax) so
//                  rescaling is rare; rows skip blocks they did not keep;
//              PV  A = P as bf16 hi + lo parts (~fp32 precision), B = V, staged
//                  through a per-wave XOR-swizzled LDS tile and read with the
//                  transposing ds_read_b64_tr_b16, 2*2*(D/16) MFMAs per block.
//  epilogue  wave partials merged through LDS; the split's normalised output
//            and natural-log LSE go to workspace; a second, small kernel
//            merges the splits (a merge inside this kernel needs device-scope
//            publication of the partials, which measured slower on gfx950).
#include <math.h>

#include <type_traits>

#include "ffd_device.h"
#include "ffd_internal.h"

namespace ffd {

namespace {


// R query rows per workgroup: R = G heads of the kv group for one query token,
// or G x Q for Q query tokens (row r = token r / G, head r % G).
template <int D, int R, int NW>
struct DecodeSmem {
  // The V tiles are live only during attend: the bf16 query rows (read into
  // registers at its start) and the epilogue's per-wave partial outputs reuse
  // their space.
  union alignas(16) {
    uint16_t vt[NW][kBlockSize * D];      // per-wave V tile (bf16, swizzled rows)
    uint16_t qb[R][D];                    // bf16 query rows
    float wo[NW][R][D];                   // per-wave partial outputs (epilogue)
  };
  alignas(16) int8_t qc[R][D];  // int8 scan query
  static_assert(sizeof(float) * R <= sizeof(uint16_t) * kBlockSize, "wave partials must fit the V tiles");
  static_assert(R <= kMaxRows, "at most 16 query rows per workgroup");
  float cq[R];              // fl32(sq * sm_scale)
  int sumq[R];              // sum of qc (offset-binary correction)
  float qsumf[R];           // sum of the bf16 query (thumbnail refinement correction)
  float blk[kMaxSplit][R];  // block scores of the split
  int xidx[kMaxPseudoMax];  // sink/local blocks outside the split (sink/local pseudo-max)
  int nx;
  float xblk[kMaxPseudoMax][R];
  float seed[R];            // split max of the block scores (natural-log units)
  int rowp[kMaxSplit];      // paged cache: first cache row of each block of the split
  uint8_t kidx[kMaxSplit];  // kept blocks (split-local index)
  uint16_t khm[kMaxSplit];  // per-row keep bits of each kept block
  uint16_t hmb[kMaxSplit];  // per-row keep bits of every block of the split (mask)
  uint16_t hmw[NW][kMaxSplit];  // the same, for the rows of each wave
  int nkept;
  float wm[NW][R];
  float wl[NW][R];
  float wa[NW][R];          // epilogue: each wave's weight in the row's merge
  float rlse[R];            // epilogue: the row's natural-log LSE
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Query-head row of row r of the workgroup of (sequence b, kv head j): query
// token r / G, head j * G + r % G. Rows index q, out, lse, mask and partials.
template <int G>
__device__ __forceinline__ size_t row_index(const DecodeParams& p, int b, int j, int r) {
  return ((size_t)b * p.Q + r / G) * p.Hq + (size_t)j * G + r % G;
}

// Tokens row r may see: its query token i = r / G sits at position sl - Q + i
// of a sequence of length sl, so it sees sl - Q + 1 + i tokens (capped by
// max_seq_len). Rows past the Q tokens (padding) see none.
template <int G>
__device__ __forceinline__ int row_len(const DecodeParams& p, int sl, int r) {
  const int i = r / G;
  if (i >= p.Q) return 0;
  const int L = sl - p.Q + 1 + i;
  return L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
}

// First cache row of block jb of (sequence b, kv head j). For a paged cache
// the split's rows were looked up once into LDS (rowp); blocks outside the
// split (sink/local pseudo-max) read the block table directly.
template <int D, int R, int NW>
__device__ __forceinline__ size_t block_row(const DecodeParams& p, const DecodeSmem<D, R, NW>& sm, int b, int j, int j0,
                                            int nblk, int jb) {
  if (p.block_table != nullptr && jb >= j0 && jb < j0 + nblk) return (size_t)(unsigned)sm.rowp[jb - j0] * kBlockSize;
  return cache_block_row(p.block_table, p.table_stride, p.num_pages, p.cap, p.Hkv, b, j, jb);
}

__device__ __forceinline__ int pack4_i8(int8_t a, int8_t b, int8_t c, int8_t d) {
  return (int)((uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
               ((uint32_t)(uint8_t)d << 24));
}

// ---------------------------------------------------------------------------
// scan: tentative block scores ([TS] Methodology 3, "Top-δ Selection": stream
// the low-bit keys, compute tentative scores per block)
// ---------------------------------------------------------------------------
// int4 scan: the R query rows' scores (the G heads, or G x Q for Q query
// tokens) are one small integer matrix product per 16-token tile, done on the
// matrix cores (v_mfma_i32_16x16x64_i8; exact int32): A = the tile's codes
// moved to offset binary (code + 8, token row n = lane % 16), B = the int8
// queries (row column n = lane % 16); lane group g = lane / 16 holds dims
// g*D/4 .. +D/4 of both, in the order the nibbles are unpacked. Output lane
// (g, n) holds tokens 4g..4g+3 of row n, so a block's max per row is a max
// over the lane's 16 scores and then over its 4 lane groups. The accumulator
// starts at -8*sum(q), the offset-binary excess, so it ends at the dot product;
// s^ = fl32(float(dot) * fl32(scale * cq)). Each row only counts the tokens
// its query token sees (a mask needed only in a block that reaches past the
// shortest row). (A v_dot4_i32_i8 scan, a quad of lanes per token, measured
// slower: 371 vs 365 us at 128K x4, 45 vs 41 us at 32K.)
// THUMB: the 2-bit thumbnail codes u instead ([TS] Methodology 1: the
// thumbnails are what the scan streams): operand word e of MFMA s is
// (codes >> 2e) & 0x03030303, whose byte m is the code of dim 16s + 4m + e;
// dot = 2 * sum qc*u - 3 * sum qc, s^ = fl32(float(dot) * fl32(t * cq)).
// First block (within the split) of the scan's pass over a paged cache: the
// split index mod its block count. In a page-major pool filled in order, the
// same block of every split lies at one offset of a large power-of-two
// stride, and workgroups that start together would all read it at once;
// rotating the start spreads them. The order of the scan changes no result.
// A contiguous cache keeps the plain order (rotated, it measured ~0.3%
// slower).
__device__ __forceinline__ int scan_rotation(const DecodeParams& p, int j0, int nblk) {
  return (p.block_table != nullptr && nblk > 0) ? (j0 / p.split_blocks) % nblk : 0;
}

// Per-lane constants of the scan: the B operand (the int8 query rows in the
// order the codes unpack), the offset-binary correction, cq and the row's
// visible length. Lane (g, n) serves row n (rows past R: no tokens).
template <int D, bool THUMB>
struct ScanQuery {
  i32x4_t qa[D / 64];
  i32x4_t acc0;
  int corr;
  float cq;
  int Lr;     // tokens row n sees
  int Lmin;   // tokens the first query token's rows see (the fewest)
};

template <int D, int G, int QT, bool THUMB, int NW>
__device__ __forceinline__ ScanQuery<D, THUMB> scan_query(const DecodeParams& p, const DecodeSmem<D, G * QT, NW>& sm,
                                                          int sl, int lane) {
  constexpr int R = G * QT;
  constexpr int NM = D / 64;   // MFMAs per tile (k = 64 each)
  const int n = lane & 15;
  const int g = lane >> 4;
  ScanQuery<D, THUMB> sq;
  // B operand: word e of MFMA s holds dims g*D/4 + 8*(2s + e/2) + 2*i + (e & 1)
  // (int4) or g*D/4 + 16s + 4i + e (thumbnail), i = 0..3, of row n
#pragma unroll
  for (int s = 0; s < NM; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int8_t* qrow = &sm.qc[n < R ? n : 0][g * (D / 4)];
      if constexpr (THUMB) {
        const int8_t* q8 = qrow + 16 * s + e;
        sq.qa[s][e] = n < R ? pack4_i8(q8[0], q8[4], q8[8], q8[12]) : 0;
      } else {
        const int8_t* q8 = qrow + 8 * (2 * s + e / 2) + (e & 1);
        sq.qa[s][e] = n < R ? pack4_i8(q8[0], q8[2], q8[4], q8[6]) : 0;
      }
    }
  // row n's correction, scale and length (rows past R: no tokens)
  sq.corr = n < R ? (THUMB ? 3 : 8) * sm.sumq[n] : 0;
  sq.cq = n < R ? sm.cq[n] : 0.f;
  sq.Lr = n < R ? row_len<G>(p, sl, n) : 0;
  sq.Lmin = row_len<G>(p, sl, 0);
  sq.acc0 = THUMB ? i32x4_t{0, 0, 0, 0} : i32x4_t{-sq.corr, -sq.corr, -sq.corr, -sq.corr};
  return sq;
}

// Code bytes per token in the scan's sketch: D/2 (int4) or D/4 (thumbnail).
template <int D, bool THUMB>
constexpr int sketch_row_bytes() { return THUMB ? D / 4 : D / 2; }

// Issue the loads of one block's sketch for one wave: lane (g, n) gets the
// code bytes g*RB/4 .. +RB/4 of token t0 + 16T + n of each tile T, and the
// scale of token t0 + 16*(n/4) + 4g + n%4; tokens at or past L are not read
// (zero). The int4 sketch is read once (streaming loads); thumbnail codes and
// scales use ordinary loads, since a kept block's are used again.
template <int D, bool THUMB>
__device__ __forceinline__ void load_sketch(const DecodeParams& p, size_t r0, int t0, int L, int lane, u32x4_t (&cw)[4],
                                            float& scl) {
  constexpr int RB = sketch_row_bytes<D, THUMB>();
  const int n = lane & 15;
  const int g = lane >> 4;
  const uint8_t* kq = (THUMB ? p.k2 : p.kq) + r0 * RB;
  const float* ks = (THUMB ? p.k2scale : p.kscale) + r0;
  // (Loading every row from a clamped address and zeroing the ones past the
  // sequence afterwards, with no branch around a load, measured 1-4% slower.)
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int t = t0 + 16 * T + n;
    const bool ok = t < L;
    const uint8_t* src = kq + (size_t)(ok ? t - t0 : 0) * RB + g * (RB / 4);
    if constexpr (RB / 4 == 16) {
      cw[T] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src)) : u32x4_t{0u, 0u, 0u, 0u};
    } else if constexpr (RB / 4 == 8) {
      const u32x2_t* s2 = reinterpret_cast<const u32x2_t*>(src);
      const u32x2_t u = ok ? (THUMB ? *s2 : __builtin_nontemporal_load(s2)) : u32x2_t{0u, 0u};
      cw[T] = u32x4_t{u.x, u.y, 0u, 0u};
    } else {
      const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
      const uint32_t u = ok ? (THUMB ? *s1 : __builtin_nontemporal_load(s1)) : 0u;
      cw[T] = u32x4_t{u, 0u, 0u, 0u};
    }
  }
  // the 16 scales lane (g, n) needs (tokens 16T + 4g + r) are held by
  // lanes 4T + r of its own 16-lane row: one load per lane, then row
  // broadcasts; tokens past the sequence are not read
  const int tl = 16 * (n >> 2) + 4 * g + (n & 3);
  scl = t0 + tl < L ? (THUMB ? ks[tl] : __builtin_nontemporal_load(ks + tl)) : 0.f;
}

// The block's score for row n = lane % 16 from its sketch registers, in every
// lane of the row: the max over the tokens the row sees of
// fl32(float(dot) * fl32(scale * cq)).
template <int D, bool THUMB>
__device__ __forceinline__ float score_block(const ScanQuery<D, THUMB>& sq, const u32x4_t (&cw)[4], float scl, int t0,
                                             int lane) {
  constexpr int NM = D / 64;
  const int g = lane >> 4;
  float bm = -INFINITY;
  // scores of the block's 4 tiles; MASKED: drop the tokens row n cannot see
  auto tiles = [&](auto masked) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      i32x4_t acc = sq.acc0;
#pragma unroll
      for (int s = 0; s < NM; ++s) {
        i32x4_t kb;
        if constexpr (THUMB) {
          const uint32_t x = cw[T][s];
          kb = i32x4_t{(int)(x & 0x03030303u), (int)((x >> 2) & 0x03030303u), (int)((x >> 4) & 0x03030303u),
                       (int)((x >> 6) & 0x03030303u)};
        } else {
          // two's complement -> code + 8, low and high nibbles
          const uint32_t x0 = cw[T][2 * s], x1 = cw[T][2 * s + 1];
          kb = i32x4_t{(int)((x0 ^ 0x88888888u) & 0x0f0f0f0fu), (int)(((x0 >> 4) ^ 0x08080808u) & 0x0f0f0f0fu),
                       (int)((x1 ^ 0x88888888u) & 0x0f0f0f0fu), (int)(((x1 >> 4) ^ 0x08080808u) & 0x0f0f0f0fu)};
        }
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb, sq.qa[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float wgt = row_bcast_f(scl, 4 * T + r) * sq.cq;
        const int dot = THUMB ? 2 * acc[r] - sq.corr : acc[r];
        const float sv = (float)dot * wgt;
        if constexpr (decltype(masked)::value)
          bm = fmaxf(bm, t0 + 16 * T + 4 * g + r < sq.Lr ? sv : -INFINITY);
        else
          bm = fmaxf(bm, sv);
      }
    }
  };
  if (t0 + kBlockSize <= sq.Lmin) tiles(std::false_type{});
  else tiles(std::true_type{});
  // max over the 4 lane groups (tokens 4g..4g+3 of each tile)
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  return bm;
}

template <int D, int G, int QT, bool THUMB, int NW>
__device__ __forceinline__ void scan_blocks_mq(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, int b, int j,
                                               int j0, int nblk_split, int nx, int L, int sl, int lane, int w) {
  constexpr int R = G * QT;
  const int nblk = nblk_split + nx;
  const int n = lane & 15;
  const int g = lane >> 4;
  const ScanQuery<D, THUMB> sq = scan_query<D, G, QT, THUMB, NW>(p, sm, sl, lane);

  constexpr int kChunk = 4;
  const int rot = scan_rotation(p, j0, nblk_split);
  for (int jc = w; jc < nblk; jc += NW * kChunk) {
    u32x4_t cw[kChunk][4];
    float scl[kChunk];   // lane (g, n): scale of token 16 * (n / 4) + 4g + n % 4 of the block
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int jl = jc + c * NW;
      if (jl < nblk) {
        int jp = jl + rot;   // the split's blocks in rotated order
        if (jp >= nblk_split) jp -= nblk_split;
        const int jb = jl < nblk_split ? j0 + jp : sm.xidx[jl - nblk_split];
        load_sketch<D, THUMB>(p, block_row(p, sm, b, j, j0, nblk_split, jb), jb * kBlockSize, L, lane, cw[c], scl[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int jl = jc + c * NW;
      if (jl >= nblk) continue;
      int jp = jl + rot;
      if (jp >= nblk_split) jp -= nblk_split;
      const int t0 = (jl < nblk_split ? j0 + jp : sm.xidx[jl - nblk_split]) * kBlockSize;
      const float bm = score_block<D, THUMB>(sq, cw[c], scl[c], t0, lane);
      if (g == 0 && n < R) {
        if (jl < nblk_split) sm.blk[jp][n] = bm;
        else sm.xblk[jl - nblk_split][n] = bm;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// select: split-local Top-δ ([TS] Methodology 2, "Mechanism" and
// "Pseudo-Max Approximation"; sink and local blocks always kept)
// ---------------------------------------------------------------------------
// Row r (query token r / G, head r % G) sees NB_r blocks; a block it cannot see
// is never kept for it, and its sink/local blocks are those of its own range.
// Wave w takes rows w, w + NW, ...; lane = block of the split. Per row: the
// split max m~ (the seed of its softmax, and the pseudo-max in split mode),
// the sink/local estimate (max over the row's own sink and local blocks, the
// extra ones scanned outside the split first), or the larger of the two; the
// threshold fl32(pm - δ), the forced blocks; the row's keep bits go to LDS
// per wave.
template <int D, int G, int QT, int NW>
__device__ __forceinline__ void select_rows(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, int j0, int nblk,
                                            int nx, int sl, int lane, int w) {
  constexpr int R = G * QT;
  const int jl = lane;
  const int jb = j0 + jl;
  const bool in_split = jl < nblk;
  unsigned hm = 0;
  for (int r = w; r < R; r += NW) {
    const int NBr = (row_len<G>(p, sl, r) + kBlockSize - 1) / kBlockSize;
    float pm = 0.f;
    if (p.pm_sink_local) {
      float m = -INFINITY;
      for (int i = lane; i < nx + nblk; i += kWave) {
        const int jx = i < nx ? sm.xidx[i] : j0 + (i - nx);
        const float sc = i < nx ? sm.xblk[i][r] : sm.blk[i - nx][r];
        if (jx < NBr && (jx < p.sink || jx >= NBr - p.local)) m = fmaxf(m, sc);
      }
      pm = wave_max_f(m);
    }
    const bool vis = in_split && jb < NBr;
    const float s = vis ? sm.blk[jl][r] : -INFINITY;
    const bool forced = jb < p.sink || jb >= NBr - p.local;
    const float mt = wave_max_f(s);
    if (!p.pm_sink_local) pm = mt;
    else if (p.pm_with_split) pm = fmaxf(pm, mt);
    const float thr = pm - p.delta;
    if (vis && (s >= thr || forced)) hm |= 1u << r;
    if (lane == 0) sm.seed[r] = mt;
  }
  sm.hmw[w][jl] = (uint16_t)hm;
}

// The kept list (one wave, lane = block): blocks kept by at least one row,
// compacted by ballot, each with its per-row keep bits; hm also goes to LDS
// for the mask, which is written in the epilogue.
template <int D, int R, int NW>
__device__ __forceinline__ void compact_kept(DecodeSmem<D, R, NW>& sm, unsigned hm, int lane) {
  sm.hmb[lane] = (uint16_t)hm;
  const unsigned long long bal = __ballot(hm != 0u);
  const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (hm != 0u) {
    sm.kidx[pos] = (uint8_t)lane;
    sm.khm[pos] = (uint16_t)hm;
  }
  if (lane == 0) sm.nkept = __popcll(bal);
}

// ---------------------------------------------------------------------------
// attend: exact attention over the kept blocks ([TS] Methodology 3,
// "Fine-Grained Refinement") on the matrix cores.
// ---------------------------------------------------------------------------

// LDS byte offset of 16-byte chunk `q` of V row `r` in a wave's tile. Rows are
// 2*D bytes; pairs of chunks are XOR-swizzled by row so that the 16 rows x
// 32 bytes one transposing read touches fall on distinct banks.
template <int D>
__device__ __forceinline__ int vt_swz(int r) {
  return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1;
}
template <int D>
__device__ __forceinline__ int vt_off(int r, int q) {
  return r * (2 * D) + ((q ^ vt_swz<D>(r)) << 4);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// 2^x for x <= 0 with the hardware exp (v_exp_f32). exp2f adds a rescaling
// path so that results below 2^-126 come out denormal; a softmax weight that
// small relative to the running max contributes nothing, so it is not needed.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 bit patterns of the thumbnail codes u = 0..3 (0, 1, 2, 3), as byte
// tables for v_perm_b32: selector u picks the low byte, 4 + u the high byte.
constexpr uint32_t kCodeBf16Lo = 0x40008000u;   // low bytes of 0x0000, 0x3F80, 0x4000, 0x4040
constexpr uint32_t kCodeBf16Hi = 0x40403F00u;   // high bytes
// Two bf16 values from the code bytes b0, b1 (each 0..3) of y: (u(b0), u(b1)).
// sel01 / sel23 pick bytes 0,1 / 2,3 of y.
template <uint32_t SEL>
__device__ __forceinline__ uint32_t code_pair_bf16(uint32_t y) {
  const uint32_t sel = __builtin_amdgcn_perm(y | 0x04040404u, y, SEL);   // (b, b + 4, b', b' + 4)
  return __builtin_amdgcn_perm(kCodeBf16Hi, kCodeBf16Lo, sel);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each aligned group of 16
// lanes, lane i receives element i%4 of the 8-byte rows addressed by lanes
// i/4, 4+i/4, 8+i/4 and 12+i/4 of its group.
__device__ __forceinline__ bf16x4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<bf16x4_t __attribute__((address_space(3)))*>((__attribute__((address_space(3))) char*)p));
}

// Per-wave online-softmax state of the attend phase. Lane l serves query row
// h = l % 16 (rows h >= R are padding) for the tokens 4*(l/16)..+3 of every
// 16-token tile; o[nt][r] holds output row 4*(l/16)+r, column 16*nt + l%16.
template <int D>
struct AttendState {
  f32x4_t o[D / 16];
  float m;      // running max (base-2 logits), same in the 4 lanes of a head
  float l;      // this lane's share of the normaliser
  bool fresh;   // the row has met no exact logit yet (o and l are still 0)
};

// How far (base-2 logit units) the scan's seed may sit above the first exact
// block maximum of a row before it is replaced by that maximum. The low-bit
// score of a token can overshoot its exact logit by far more than the
// exponent range of fp32 (a coarse sketch, large logits, an outlier key
// channel); a seed kept that high would flush every weight exp2(z - m) to 0.
// While a row is fresh nothing has been accumulated relative to m, so moving
// m down is exact; afterwards m stays within this slack of the largest exact
// logit the row has met, so its largest weight is >= 2^-64 and the smallest
// nonzero weights it drops are below 2^-62 of the row's sum.
constexpr float kSeedSlack = 64.f;

// Per-wave constants of the attend phase.
template <int D>
struct AttendCtx {
  bf16x8_t qop[D / 32];   // B operand of QK: the bf16 query of row h = lane % 16
  int wbase[2];           // LDS addresses of this lane's V-tile stores
  int rbase, rx;          // LDS address parts of this lane's transposed V reads
  float zscale;           // sm_scale * log2(e)
  float qs;               // thumbnail path: sum of the row's bf16 query
  bool hv;                // lane's row is a row of a real query token
  char* vt;               // this wave's V tile
};

// Set up wave w's attend: the query rows as the QK B operand, the V tile's
// addresses, and the softmax state, its running max seeded with seed[h]
// (natural-log units) unless DENSE. Reads the bf16 query rows from LDS, which
// share their space with the V tiles: the caller must place a workgroup
// barrier between every wave's set-up and any wave's first block.
template <int D, int G, int QT, bool DENSE, bool THUMB, int NW>
__device__ __forceinline__ void attend_setup(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, int lane, int w,
                                             AttendCtx<D>& c, AttendState<D>& st) {
  constexpr int R = G * QT;
  constexpr int KS = D / 32;    // MFMA k-steps over the head dimension
  constexpr int NT = D / 16;    // MFMA n-tiles of the output
  constexpr int VC = D / 8;     // 16-byte chunks per V row
  const int h = lane & 15;
  const int g = lane >> 4;

  c.hv = h < R && h / G < p.Q;   // a row of a real query token
  // B operand of QK: the bf16 query of row h, dims g*D/4 + 8s .. +8 for k-step s
  {
    const uint16_t* qh = &sm.qb[c.hv ? h : 0][g * (D / 4)];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t u = u32x4_t{0u, 0u, 0u, 0u};
      if constexpr (!THUMB) {
        if (c.hv) u = *reinterpret_cast<const u32x4_t*>(qh + 8 * s);
      } else {
        // thumbnail order (see the QK below): slot 4*kk + m of k-step s is
        // dim 16*(s/2) + 4m + k0 + kk, k0 = 2*(s%2); dword m of that row part
        // holds dims (4m + k0, 4m + k0 + 1)
        if (c.hv) {
          uint32_t dw[4];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            dw[m] = *reinterpret_cast<const uint32_t*>(qh + 16 * (s >> 1) + 4 * m + 2 * (s & 1));
          u = u32x4_t{(dw[0] & 0xffffu) | (dw[1] << 16), (dw[2] & 0xffffu) | (dw[3] << 16),
                      (dw[0] >> 16) | (dw[1] & 0xffff0000u), (dw[2] >> 16) | (dw[3] & 0xffff0000u)};
        }
      }
      c.qop[s] = as_bf16x8(u);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) st.o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = c.hv ? (DENSE ? -INFINITY : sm.seed[h] * kLog2e) : 0.f;
  st.l = 0.f;
  st.fresh = true;

  c.vt = reinterpret_cast<char*>(sm.vt[w]);
  // LDS addresses of the V tile. Store: 16-byte chunk n*64 + lane of the tile
  // goes to wbase[n & 1] + (n >> 1) * 2048 (the row swizzle repeats every 8
  // rows for D=128, and every 2 stores for D=64). Transposed read for k-step
  // ks, half hf, n-tile nt: rbase + 32 rows*ks + 16 rows*hf + ((nt ^ rx) << 5).
  constexpr int ROWB = 2 * D;
  constexpr int RPS = kWave / VC;   // rows per 1 KiB store
#pragma unroll
  for (int par = 0; par < 2; ++par) c.wbase[par] = vt_off<D>(par * RPS + lane / VC, lane % VC);
  const int rr = 4 * g + (h >> 2);
  c.rx = (D == 128) ? (rr & 7) : ((rr >> 1) & 3);
  c.rbase = rr * ROWB + ((h & 3) >> 1) * 16 + (h & 1) * 8;
  c.zscale = p.sm_scale * kLog2e;
  c.qs = (THUMB && c.hv) ? sm.qsumf[h] : 0.f;
}

// The registers a block's attend loads into.
template <int D, bool THUMB>
struct BlockLoads {
  u32x4_t kr[4][D / 32];                        // bf16 K rows (int4 path)
  uint32_t kc[4][(D / 64) > 0 ? D / 64 : 1];    // thumbnail codes (16 per word)
  u32x2_t kres[4][D / 32];                      // residual bytes, 8 per k-step
  float tsl, s8l;                               // thumbnail and residual scales of row `lane`
  u32x4_t vr[64 * (D / 8) / kWave];             // V chunks
};

// Attend one block (first cache row r0, first token t0) for the rows whose
// bit is set in hm: its K (or thumbnail codes + residuals) and V, QK on the
// matrix cores, the online softmax, PV. Lrow: tokens this lane's row (lane %
// 16) may see; L: tokens of the sequence (the longest row), which bounds
// every load.
template <int D, int G, int QT, bool THUMB>
__device__ __forceinline__ void attend_issue(const DecodeParams& p, const AttendCtx<D>& c, size_t r0, int t0, int L,
                                             int lane, BlockLoads<D, THUMB>& ld) {
  constexpr int KS = D / 32;    // MFMA k-steps over the head dimension
  constexpr int VC = D / 8;     // 16-byte chunks per V row
  constexpr int VL = 64 * VC / kWave;  // 16-byte V loads per lane per block
  const int h = lane & 15;
  const int g = lane >> 4;
  const int tlast = L - 1;   // rows past the sequence are read from its last row and masked
  const uint16_t* kb = p.k + r0 * D;   // token t of this block is row t - t0
  const uint16_t* vb = p.v + r0 * D;

  // ---- issue the block's loads: K (or its thumbnail + residual) and V ----
  auto& kr = ld.kr;
  auto& kc = ld.kc;
  auto& kres = ld.kres;
  float& tsl = ld.tsl;
  float& s8l = ld.s8l;
  tsl = 0.f;
  s8l = 0.f;
  if constexpr (!THUMB) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int t = min(t0 + 16 * T + h, tlast);
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(kb + (size_t)(t - t0) * D + g * (D / 4));
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[T][s] = src[s];
    }
  } else {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int t = min(t0 + 16 * T + h, tlast);
      const uint8_t* cs = p.k2 + (r0 + (size_t)(t - t0)) * (D / 4) + g * (D / 16);
      if constexpr (D == 128) {
        const u32x2_t u = *reinterpret_cast<const u32x2_t*>(cs);
        kc[T][0] = u.x;
        kc[T][1] = u.y;
      } else {
        kc[T][0] = *reinterpret_cast<const uint32_t*>(cs);
      }
      const u32x2_t* rs = reinterpret_cast<const u32x2_t*>(p.kr + (r0 + (size_t)(t - t0)) * D + g * (D / 4));
#pragma unroll
      for (int s = 0; s < KS; ++s) kres[T][s] = __builtin_nontemporal_load(rs + s);   // read once
    }
    // per-token scales: lane l holds those of row l of the block
    const int tl = min(t0 + lane, tlast) - t0;
    tsl = p.k2scale[r0 + tl];
    s8l = __builtin_nontemporal_load(p.krscale + r0 + tl);
  }
  // The whole V tile is in flight across QK, on the thumbnail path too.
  // (Loading V straight into LDS with global_load_lds_dwordx4 frees its
  // registers, but the compiler then waits for every outstanding load, the
  // V DMA included, before the first use of the codes, which serialises V
  // behind QK: slower.)
  auto& vr = ld.vr;
#pragma unroll
  for (int n = 0; n < VL; ++n) {
    const int f = n * kWave + lane;        // chunk id within the tile
    const int r = f / VC, q = f % VC;
    const int t = min(t0 + r, tlast);
    vr[n] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + (size_t)(t - t0) * D + q * 8));
  }

}

// The compute half: QK, V tile, online softmax, PV of a block whose loads
// attend_issue put in flight (waiting for them here).
template <int D, int G, int QT, bool THUMB>
__device__ __forceinline__ void attend_compute(const AttendCtx<D>& c, AttendState<D>& st, int t0, int Lrow,
                                               unsigned hm, int lane, const BlockLoads<D, THUMB>& ld) {
  constexpr int KS = D / 32;    // MFMA k-steps over the head dimension
  constexpr int NT = D / 16;    // MFMA n-tiles of the output
  constexpr int VC = D / 8;     // 16-byte chunks per V row
  constexpr int VL = 64 * VC / kWave;  // 16-byte V loads per lane per block
  constexpr int ROWB = 2 * D;
  const int h = lane & 15;
  const int g = lane >> 4;
  const auto& kr = ld.kr;
  const auto& kc = ld.kc;
  const auto& kres = ld.kres;
  const float tsl = ld.tsl, s8l = ld.s8l;
  const auto& vr = ld.vr;
  // ---- QK on the matrix cores ----
  const auto& qop = c.qop;
  f32x4_t sacc[4];
  if constexpr (!THUMB) {
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      sacc[T] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[T][s]), qop[s], sacc[T], 0, 0, 0);
    }
  } else {
    // q.K^ = t * (2 q.u - 3 sum q) + s8 * q.r8: u and r8 are small integers,
    // exact in bf16, so both dot products run on the matrix cores exactly up
    // to fp32 accumulation and K^ is never formed.
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      f32x4_t au = f32x4_t{0.f, 0.f, 0.f, 0.f};
      f32x4_t ar = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // k-step s covers the lane's dims 16*(s/2) + 4m + k0 + kk (m = 0..3,
      // kk = 0..1, k0 = 2*(s%2)) in slot 4*kk + m: byte m of
      // (codes >> 2(k0 + kk)) & 0x03030303 is exactly the code of that dim,
      // so each pair of bf16 codes is two byte permutes from a table; the
      // residual byte of dim d is byte d%4 of word d/4, read by the convert.
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k0 = 2 * (s & 1);
        const uint32_t w = kc[T][s >> 1];
        const uint32_t y0 = (w >> (2 * k0)) & 0x03030303u;
        const uint32_t y1 = (w >> (2 * k0 + 2)) & 0x03030303u;
        const u32x4_t ub = u32x4_t{code_pair_bf16<0x05010400u>(y0), code_pair_bf16<0x07030602u>(y0),
                                   code_pair_bf16<0x05010400u>(y1), code_pair_bf16<0x07030602u>(y1)};
        bf16x8_t a_r;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x2_t rw = kres[T][2 * (s >> 1) + (m >> 1)];
            const uint32_t word = (m & 1) ? rw.y : rw.x;
            a_r[4 * kk + m] = (__bf16)(float)(int8_t)(word >> (8 * (k0 + kk)));
          }
        au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ub), qop[s], au, 0, 0, 0);
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_r, qop[s], ar, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int src = 16 * T + 4 * g + r;   // the lane holding this row's scales
        const float ts = __shfl(tsl, src);
        const float s8 = __shfl(s8l, src);
        sacc[T][r] = ts * (2.f * au[r] - 3.f * c.qs) + s8 * ar[r];
      }
      __builtin_amdgcn_sched_barrier(0);   // convert tile by tile: bounds live registers
    }
  }

  // ---- V tile to LDS (this wave's region) ----
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int n = 0; n < VL; ++n)
    *reinterpret_cast<u32x4_t*>(c.vt + c.wbase[n & 1] + (n >> 1) * 2048) = vr[n];

  // ---- online softmax in the MFMA output layout ----
  const bool head_keeps = c.hv && ((hm >> h) & 1u);
  float sv[4][4];
  float mx = -INFINITY;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * T + 4 * g + r;
      const float z = sacc[T][r] * c.zscale;
      sv[T][r] = (head_keeps && t < Lrow) ? z : -INFINITY;
      mx = fmaxf(mx, sv[T][r]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // a fresh row takes the block's exact max when the seed lies too far
  // above it (nothing to rescale: o and l are 0); afterwards m only rises
  const bool fresh = st.fresh;
  const bool up = mx > st.m || (fresh && mx != -INFINITY && mx < st.m - kSeedSlack);   // (unseeded: m = -inf)
  if (mx != -INFINITY) st.fresh = false;
  if (__ballot(up)) {
    const float mn = up ? mx : st.m;
    const float alpha = (st.m == -INFINITY || fresh) ? 0.f : fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st.o[nt][r] *= ar;
    }
  }
  bf16x8_t phi[2], plo[2];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = (sv[T][r] == -INFINITY) ? 0.f : fast_exp2(sv[T][r] - st.m);
      st.l += pr;
      const __bf16 hi = (__bf16)pr;
      const __bf16 lo = (__bf16)(pr - (float)hi);
      phi[T >> 1][(T & 1) * 4 + r] = hi;
      plo[T >> 1][(T & 1) * 4 + r] = lo;
    }

  // ---- PV on the matrix cores: B = V read transposed from LDS ----
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // providing lane (g, h): row 32ks + 16hf + 4g + h/4, dims 16nt + 4(h%4) .. +4
      const char* a = c.vt + c.rbase + ks * 32 * ROWB + ((nt ^ c.rx) << 5);
      const bf16x4_t v0 = lds_read_tr(a);
      const bf16x4_t v1 = lds_read_tr(a + 16 * ROWB);
      const bf16x8_t vb8 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      st.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[ks], vb8, st.o[nt], 0, 0, 0);
      st.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], vb8, st.o[nt], 0, 0, 0);
    }
  }
}

template <int D, int G, int QT, bool THUMB>
__device__ __forceinline__ void attend_block(const DecodeParams& p, const AttendCtx<D>& c, AttendState<D>& st,
                                             size_t r0, int t0, int L, int Lrow, unsigned hm, int lane) {
  BlockLoads<D, THUMB> ld;
  attend_issue<D, G, QT, THUMB>(p, c, r0, t0, L, lane, ld);
  attend_compute<D, G, QT, THUMB>(c, st, t0, Lrow, hm, lane, ld);
}

// Lrow: tokens this lane's row (lane % 16) may see; L: tokens of the sequence
// (the longest row), which bounds every load.
// Kept blocks first, first + stride, ... are this wave's; its V tile is the
// one of wave w of the workgroup.
template <int D, int G, int QT, bool DENSE, bool THUMB, int NW>
__device__ __forceinline__ void attend_blocks(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, int b, int j,
                                              int j0, int L, int Lrow, int lane, int first, int stride,
                                              AttendState<D>& st) {
  AttendCtx<D> c;
  attend_setup<D, G, QT, DENSE, THUMB, NW>(p, sm, lane, first % NW, c, st);
  const int nkept = sm.nkept;
  __syncthreads();   // the query rows share their space with the V tiles

  // Kept blocks are taken last-scanned first: on the thumbnail path their
  // codes, read again here, are then the likeliest to be still in L2. (The
  // order is the same for every cache layout, so a paged cache gives the bits
  // of a contiguous one.)
  for (int e0 = first; e0 < nkept; e0 += stride) {
    const int e = nkept - 1 - e0;
    const int jb = j0 + sm.kidx[e];
    const size_t r0 = block_row(p, sm, b, j, j0, kMaxSplit, jb);   // kept blocks lie in the split
    attend_block<D, G, QT, THUMB>(p, c, st, r0, jb * kBlockSize, L, Lrow, sm.khm[e], lane);
  }
}

// ---------------------------------------------------------------------------
// split combine: lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) o_s
// ---------------------------------------------------------------------------

__device__ __forceinline__ void store_out(const DecodeParams& p, size_t idx, float v) {
  if (p.out_f32) static_cast<float*>(p.out)[idx] = v;
  else static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(v);
}

// The query rows of the workgroup to LDS (thread (qr, qk) holds the 16-byte
// chunk qk of row qr in qw): the bf16 rows, the int8 scan query with its
// scale cq and code sum, and (thumbnail path) the bf16 row sums.
template <int D, int G, int QT, bool DENSE, bool THUMB, int NW>
__device__ __forceinline__ void query_to_lds(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, u32x4_t qw, int qr,
                                             int qk) {
  constexpr int R = G * QT;
  constexpr int QC = D / 8;   // 16-byte chunks per query row
  if (qr < R) {
    // row qr's chunks sit in QC consecutive lanes: its reductions stay there
    *reinterpret_cast<u32x4_t*>(&sm.qb[qr][qk * 8]) = qw;
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(qw[e]);
      x[2 * e + 1] = bf16_hi(qw[e]);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = group_max_f<QC>(amax);
    if constexpr (THUMB) {
      float fs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) fs += x[e];
      fs = group_sum_f<QC>(fs);
      if (qk == 0) sm.qsumf[qr] = fs;
    }
    if constexpr (!DENSE) {
      // amax < 2^-120 counts as a zero query: 127/amax would overflow to +inf
      const bool nz = amax >= 0x1p-120f;
      int qsum = 0;
      uint32_t cw[2] = {0u, 0u};
      if (nz) {
        const float inv = 127.0f / amax;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c = rintf(x[e] * inv);
          c = fminf(fmaxf(c, -127.f), 127.f);
          const int ci = (int)c;
          qsum += ci;
          cw[e >> 2] |= (uint32_t)(uint8_t)(int8_t)ci << (8 * (e & 3));
        }
      }
      *reinterpret_cast<u32x2_t*>(&sm.qc[qr][qk * 8]) = u32x2_t{cw[0], cw[1]};
      qsum = group_sum_i<QC>(qsum);
      if (qk == 0) {
        sm.sumq[qr] = qsum;
        sm.cq[qr] = nz ? (amax / 127.0f) * p.sm_scale : 0.f;
      }
    }
  }
}

// This wave's softmax state to LDS for the workgroup's merge: the
// normaliser of row h summed over its 4 lane groups, the running max and the
// unnormalised outputs (which overwrite the V tiles: every wave must be done
// attending before any wave calls this).
template <int D, int R, int NW>
__device__ __forceinline__ void wave_state_to_lds(DecodeSmem<D, R, NW>& sm, const AttendState<D>& st, int lane,
                                                  int w) {
  float lw = st.l;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  {
    const int g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * g + r;
      if (hh < R) {
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) sm.wo[w][hh][16 * nt + (lane & 15)] = st.o[nt][r];
      }
    }
    if (lane < R) {
      sm.wm[w][lane] = st.m;
      sm.wl[w][lane] = lw;
    }
  }
}

// Merge the waves' states (after wave_state_to_lds and a barrier) and write
// the part's normalised output and natural-log LSE for every row.
template <int D, int G, int QT, int NW>
__device__ __forceinline__ void write_partial(const DecodeParams& p, DecodeSmem<D, G * QT, NW>& sm, int b, int j,
                                              int split, int part, int tid) {
  constexpr int R = G * QT;
  constexpr int kThreads = 64 * NW;
  // ---- epilogue: merge waves, write the split partial -------------------
  // per row, once: the waves' weights exp2(m_w - m) / den and the LSE
  if (tid < R) {
    const int h = tid;
    // a wave that accumulated nothing for the row (its m may still be the
    // seed, above every exact logit) takes no part in the merge
    float wmv[NW];
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      wmv[ww] = sm.wl[ww][h] > 0.f ? sm.wm[ww][h] : -INFINITY;
      mx = fmaxf(mx, wmv[ww]);
    }
    float a[NW], den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      a[ww] = (wmv[ww] == -INFINITY) ? 0.f : exp2f(wmv[ww] - mx);
      den += sm.wl[ww][h] * a[ww];
    }
    // a row can keep no block of a split (sink/local pseudo-max, or a query
    // token that does not see the split): empty partial, weight 0
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) sm.wa[ww][h] = den > 0.f ? a[ww] / den : 0.f;
    sm.rlse[h] = den > 0.f ? (mx + log2f(den)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int i = tid; i < R * D4; i += kThreads) {
    const int h = i / D4, cc = (i % D4) * 4;
    if (h / G >= p.Q) continue;
    f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&sm.wo[ww][h][cc]);
      const float a = sm.wa[ww][h];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += x[e] * a;
    }
    const size_t row = (row_index<G>(p, b, j, h) * p.n_splits + split) * p.split_parts + part;
    *reinterpret_cast<f32x4_t*>(p.o_part + row * D + cc) = o;
    if (cc == 0) p.lse_part[row] = sm.rlse[h];
  }
}

// The split's mask entries from the per-block row bits in sm.hmb (blocks past
// the sequence are 0), four per thread.
template <int D, int G, int QT, int NW>
__device__ __forceinline__ void write_mask(const DecodeParams& p, const DecodeSmem<D, G * QT, NW>& sm, int b, int j,
                                           int j0, int nmask, int tid) {
  constexpr int R = G * QT;
  constexpr int kThreads = 64 * NW;
  const int n4 = (nmask + 3) / 4;
  for (int i = tid; i < R * n4; i += kThreads) {
    const int r = i / n4, c = 4 * (i % n4);
    if (r / G >= p.Q) continue;
    uint8_t* dst = p.mask + row_index<G>(p, b, j, r) * p.nb_max + j0 + c;
    uint32_t m4 = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) m4 |= (uint32_t)((sm.hmb[min(c + e, kMaxSplit - 1)] >> r) & 1u) << (8 * e);
    if (c + 4 <= nmask && ((uintptr_t)dst & 3u) == 0) {
      *reinterpret_cast<uint32_t*>(dst) = m4;
    } else {
      for (int e = 0; e < 4 && c + e < nmask; ++e) dst[e] = (uint8_t)(m4 >> (8 * e));
    }
  }
}

// One workgroup per (split, kv head j, sequence b) serving R = G x QT query
// rows: the G heads of the group for each of the (up to QT) query tokens.
// NW waves per workgroup: 4 (two workgroups per CU), or 8 on small grids (one
// per CU, each wave scanning and attending half as many blocks).
template <int D, int G, int QT, bool DENSE, bool THUMB, int NW>
// Two waves per SIMD: the LDS of the workgroups that fit a CU allows no more,
// and the registers must not allow fewer.
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void fused_decode_kernel(
    const DecodeParams p) {
  constexpr int R = G * QT;
  constexpr int kThreads = 64 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  static_assert(QT == 1 || !THUMB, "several query tokens only with the int4 sketch");
  __shared__ DecodeSmem<D, R, NW> sm;
  const int j = blockIdx.y, b = blockIdx.z;
  int split = blockIdx.x, part = 0;
  // The dispatcher deals workgroups to the 8 XCDs by linear id mod 8, i.e. by
  // blockIdx.x mod 8 here. Splits past a sequence's end exit at once, so with
  // ragged lengths a fixed split -> x map loads the XCDs that get the low
  // splits more; rotating each (sequence, kv head)'s splits by a different
  // amount spreads every split index over all XCDs.
  if (p.split_parts == 1) split = (int)(((long)split + (long)b * p.Hkv + j) % p.n_splits);
  if (p.split_parts > 1) {
    // The P workgroups of a split get linear ids 8 apart (the x extent is a
    // multiple of 8), which the dispatcher, dealing workgroups round-robin
    // over the 8 XCDs, places on one XCD: their repeated scan reads share its L2.
    const int x = blockIdx.x;
    split = (x / (8 * p.split_parts)) * 8 + x % 8;
    part = (x / 8) % p.split_parts;
    if (split >= p.n_splits) return;
  }
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  // the query rows, one 16-byte chunk per thread, in flight from the start
  constexpr int QC = D / 8;   // 16-byte chunks per query row
  static_assert(R * QC <= kThreads, "one query chunk per thread");
  const int qr = tid / QC, qk = tid % QC;
  u32x4_t qw = u32x4_t{0u, 0u, 0u, 0u};
  if (qr < R && qr / G < p.Q) qw = *reinterpret_cast<const u32x4_t*>(p.q + row_index<G>(p, b, j, qr) * D + qk * 8);
  const int sl = max(p.seq_lens[b], 0);   // a device value: negative means empty (and must not wrap below)
  // the last query token sees the whole sequence: every load is bounded by it
  const int L = row_len<G>(p, sl, G * (p.Q - 1));
  const int NB = (L + kBlockSize - 1) / kBlockSize;
  const int j0 = split * p.split_blocks;
  const int nmask = min(p.split_blocks, p.nb_max - j0);
  if (j0 >= NB) {
    // no valid block in this split: only the mask entries are owned here
    if (p.mask != nullptr && part == 0) {
      for (int i = tid; i < nmask * R; i += kThreads) {
        const int r = i / nmask, jl = i % nmask;
        if (r / G < p.Q) p.mask[row_index<G>(p, b, j, r) * p.nb_max + j0 + jl] = 0;
      }
    }
    return;
  }
  const int nblk = min(p.split_blocks, NB - j0);

  // ---- prologue: query rows to LDS, int8 scan query -----------------------
  if (p.block_table != nullptr && tid < nblk)
    sm.rowp[tid] = (int)(cache_block_row(p.block_table, p.table_stride, p.num_pages, p.cap, p.Hkv, b, j, j0 + tid) /
                         kBlockSize);
  if (!DENSE && p.pm_sink_local && tid == 0) {
    // sink and local blocks of every row that lie outside the split: the rows'
    // local windows end at NB_0 .. NB (first to last query token)
    const int NB0 = (row_len<G>(p, sl, 0) + kBlockSize - 1) / kBlockSize;
    int nx = 0;
    const int s_end = min(p.sink, NB);
    const int l_beg = max(s_end, NB0 - p.local);
    for (int jb = 0; jb < s_end; ++jb)
      if (jb < j0 || jb >= j0 + nblk) sm.xidx[nx++] = jb;
    for (int jb = l_beg; jb < NB; ++jb)
      if (jb < j0 || jb >= j0 + nblk) sm.xidx[nx++] = jb;
    sm.nx = nx;
  }
  query_to_lds<D, G, QT, DENSE, THUMB, NW>(p, sm, qw, qr, qk);
  __syncthreads();

  // ---- scan + select ------------------------------------------------------
  if constexpr (!DENSE) {
    // sink/local pseudo-max: the sink and local blocks outside this split are
    // listed in the prologue and scanned in the same pass as the split
    const int nx = p.pm_sink_local ? sm.nx : 0;
    scan_blocks_mq<D, G, QT, THUMB, NW>(p, sm, b, j, j0, nblk, nx, L, sl, lane, w);
    __syncthreads();
    select_rows<D, G, QT, NW>(p, sm, j0, nblk, nx, sl, lane, w);
    __syncthreads();
    if (w == 0) {
      unsigned hm = 0;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) hm |= sm.hmw[ww][lane];
      compact_kept(sm, hm, lane);
    }
  } else {
    // every block the row sees
    if (w == 0) {
      unsigned hm = 0;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane < nblk && j0 + lane < (row_len<G>(p, sl, r) + kBlockSize - 1) / kBlockSize) hm |= 1u << r;
      compact_kept(sm, hm, lane);
    }
  }
  __syncthreads();

  // ---- attend -------------------------------------------------------------
  AttendState<D> st;
  attend_blocks<D, G, QT, DENSE, THUMB, NW>(p, sm, b, j, j0, L, row_len<G>(p, sl, lane & 15), lane,
                                        part * NW + w, NW * p.split_parts, st);

  // this wave's partial: normaliser of row h summed over its 4 lane groups;
  // the partial outputs overwrite the V tiles, so every wave must be done
  __syncthreads();
  wave_state_to_lds<D, R, NW>(sm, st, lane, w);
  __syncthreads();
  write_partial<D, G, QT, NW>(p, sm, b, j, split, part, tid);
  if (p.mask != nullptr && part == 0) write_mask<D, G, QT, NW>(p, sm, b, j, j0, nmask, tid);
}

// ---------------------------------------------------------------------------
// split combine: lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) o_s
// ---------------------------------------------------------------------------
// One workgroup per (query-head row, 32 output dims), one pass: 8 groups of 32
// threads each merge an interleaved eighth of the row's partials online (a
// running max m and sum l of exp(lse_s - m), the outputs weighted alike), with
// the loads of up to 8 partials per thread issued before the sequence length
// arrives (reads past the sequence's partials stay inside the row's slots and
// are dropped); the 8 groups are then merged in a fixed order (deterministic).
// Spreading a row over D/32 workgroups keeps the latency chain short.
constexpr int kCombineDims = 32;
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const DecodeParams p) {
  constexpr int PARTS = kCombineThreads / kCombineDims;
  constexpr int U = 8;   // partials per thread per step
  __shared__ float gm[PARTS], gl[PARTS];
  __shared__ float red[PARTS][kCombineDims];
  const int h = blockIdx.x, b = blockIdx.y, c0 = blockIdx.z * kCombineDims, tid = threadIdx.x;
  const int c = tid % kCombineDims, part = tid / kCombineDims;
  const size_t bh = (size_t)b * p.Q * p.Hq + h;   // row (b, query token h / Hq, head h % Hq)
  const int per_row = p.n_splits * p.split_parts;
  const float* lp = p.lse_part + bh * per_row;
  const float* op = p.o_part + bh * per_row * D + c0 + c;
  int L = p.seq_lens[b];
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int s0 = part; s0 < per_row; s0 += U * PARTS) {
    float lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * PARTS;
      lv[u] = s < per_row ? lp[s] : -INFINITY;
      ov[u] = s < per_row ? op[(size_t)s * D] : 0.f;
    }
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int NB = (L + kBlockSize - 1) / kBlockSize;
    const int ns = (NB + p.split_blocks - 1) / p.split_blocks * p.split_parts;   // partials of this sequence
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u * PARTS >= ns) lv[u] = -INFINITY;   // slots past the sequence's partials
      mx = fmaxf(mx, lv[u]);
    }
    if (mx == -INFINITY) continue;   // nothing seen yet
    const float a = (m == -INFINITY) ? 0.f : expf(m - mx);
    l *= a;
    acc *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // an empty partial (or an unwritten slot) adds nothing, whatever it holds
      if (lv[u] != -INFINITY) {
        const float wt = expf(lv[u] - mx);
        l += wt;
        acc += wt * ov[u];
      }
    }
    m = mx;
  }
  red[part][c] = acc;
  if (c == 0) {
    gm[part] = m;
    gl[part] = l;
  }
  __syncthreads();
  if (part == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) M = fmaxf(M, gm[q]);
    float den = 0.f, res = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < PARTS; ++q) {
        const float a = (gm[q] == -INFINITY) ? 0.f : expf(gm[q] - M);
        den += gl[q] * a;
        res += red[q][c] * a;
      }
    }
    const bool any = den > 0.f;
    store_out(p, bh * D + c0 + c, any ? res / den : 0.f);
    if (c0 == 0 && c == 0) p.lse[bh] = any ? M + logf(den) : -INFINITY;
  }
}

template <int D, int G, int QT, bool DENSE, bool THUMB>
hipError_t launch_fused(const DecodeParams& p, Stage stage, hipStream_t stream) {
  if ((static_cast<int>(stage) & static_cast<int>(Stage::kPartials)) && p.n_splits > 0) {
    const int gx = p.split_parts == 1 ? p.n_splits : (p.n_splits + 7) / 8 * 8 * p.split_parts;
    dim3 grid(gx, p.Hkv, p.B);
    if (p.waves == 8) {
      fused_decode_kernel<D, G, QT, DENSE, THUMB, 8><<<grid, 512, 0, stream>>>(p);
    } else {
      fused_decode_kernel<D, G, QT, DENSE, THUMB, 4><<<grid, 256, 0, stream>>>(p);
    }
  }
  if (static_cast<int>(stage) & static_cast<int>(Stage::kCombine)) {
    combine_kernel<D><<<dim3(p.Q * p.Hq, p.B, D / kCombineDims), kCombineThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

// Query tokens per workgroup: the smallest power of two >= Q (rows of the
// missing tokens are padding); G * QT <= 16.
template <int D, int G, bool DENSE, bool THUMB>
hipError_t launch_q(const DecodeParams& p, Stage stage, hipStream_t stream) {
  if (p.Q == 1) return launch_fused<D, G, 1, DENSE, THUMB>(p, stage, stream);
  if constexpr (THUMB) {
    return hipErrorInvalidValue;
  } else {
    if (p.Q <= 2) return launch_fused<D, G, 2, DENSE, false>(p, stage, stream);
    if constexpr (G <= 4) {
      if (p.Q <= 4) return launch_fused<D, G, 4, DENSE, false>(p, stage, stream);
    }
    if constexpr (G <= 2) {
      if (p.Q <= 8) return launch_fused<D, G, 8, DENSE, false>(p, stage, stream);
    }
    if constexpr (G == 1) {
      if (p.Q <= 16) return launch_fused<D, G, 16, DENSE, false>(p, stage, stream);
    }
    return hipErrorInvalidValue;
  }
}

template <int D, bool DENSE, bool THUMB>
hipError_t launch_g(const DecodeParams& p, int G, Stage stage, hipStream_t stream) {
  switch (G) {
    case 1: return launch_q<D, 1, DENSE, THUMB>(p, stage, stream);
    case 2: return launch_q<D, 2, DENSE, THUMB>(p, stage, stream);
    case 4: return launch_q<D, 4, DENSE, THUMB>(p, stage, stream);
    case 8: return launch_q<D, 8, DENSE, THUMB>(p, stage, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// One family of kernels (head dim D, dense or sparse, key storage) per
// compilation of this file: the build compiles it once per family with
// FFD_VARIANT_D, FFD_VARIANT_DENSE and FFD_VARIANT_THUMB defined, so the
// families compile in parallel; with none defined every family is
// instantiated here.
template <int D, bool DENSE, bool THUMB>
hipError_t launch_variant(const DecodeParams& p, int G, Stage stage, hipStream_t stream) {
  return launch_g<D, DENSE, THUMB>(p, G, stage, stream);
}

#if defined(FFD_VARIANT_D)
template hipError_t launch_variant<FFD_VARIANT_D, FFD_VARIANT_DENSE, FFD_VARIANT_THUMB>(const DecodeParams&, int, Stage,
                                                                                      hipStream_t);
#else
template hipError_t launch_variant<128, false, false>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<128, true, false>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<128, false, true>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<128, true, true>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<64, false, false>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<64, true, false>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<64, false, true>(const DecodeParams&, int, Stage, hipStream_t);
template hipError_t launch_variant<64, true, true>(const DecodeParams&, int, Stage, hipStream_t);
#endif

}  // namespace ffd
