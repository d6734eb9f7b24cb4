// Fused FFD decode: split-K scan -> Top-δ select -> exact attention, plus the
// log-sum-exp split combine.
//
// Method: "Faster Than Flash: Exploiting Attention Sparsity for Efficient
// Long-Context Decoding" ([TS] = its technical-summary page, Methodology 1-3).
// The selector (low-bit scan + Top-δ) and the computer (exact attention over
// the kept blocks) run in ONE kernel per (sequence, kv head, split), so the
// kept set never leaves the workgroup ([TS] Methodology 3, "Fused Kernel").
//
// One workgroup = 4 wave64s owns `split_blocks` consecutive 64-token blocks of
// one (sequence b, kv head j) and serves all G = Hq/Hkv query heads of the
// group, so every K/V byte it reads is shared by the G heads.
//
//  prologue  q[b, jG..jG+G) -> LDS: fp32 copy (pre-scaled by sm_scale*log2 e)
//            and int8 copy + per-head scale (the scan query).
//  scan      each wave takes whole blocks; a quad of lanes owns one token (each
//            lane 16 B of int4 codes for D=128), 16 tokens per wave load =
//            1 KiB contiguous. Nibbles are moved to offset binary (x ^ 8 =
//            code + 8, 0..15) so v_dot4_i32_i8 can take them; the 8*sum(q)
//            excess is subtracted after the quad reduction. Block score =
//            max over valid tokens -> LDS.
//  select    wave 0: per head split max m~, threshold fl32(m~ - δ), forced
//            sink/local blocks, mask store, and a ballot-compacted list of the
//            blocks kept by at least one head of the group (with a per-head
//            bit mask).
//  attend    waves take kept blocks round-robin; D/8 lanes own one token row
//            (16 B of K and of V each). The running max of every head starts
//            at the scan's split max (the scan result reused to seed the
//            softmax), so rescaling is rare; a head skips the blocks it did
//            not keep.
//  epilogue  wave and token-group partials merged in registers/LDS; the
//            split's normalised output and natural-log LSE go to workspace.
#include <math.h>

#include "ffd_device.h"
#include "ffd_internal.h"

namespace ffd {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int D, int G>
struct DecodeSmem {
  float q[G][D];            // bf16 query, fp32, times sm_scale * log2(e)
  int8_t qc[G][D];          // int8 scan query
  float cq[G];              // fl32(sq * sm_scale)
  int sumq[G];              // sum of qc (offset-binary correction)
  float blk[kMaxSplit][G];  // block scores
  float seed[G];            // split max m~ (natural-log units)
  uint8_t kidx[kMaxSplit];  // kept blocks (split-local index)
  uint8_t khm[kMaxSplit];   // per-head keep bits of each kept block
  int nkept;
  float wm[kWaves][G];
  float wl[kWaves][G];
  float wo[kWaves][G][D];
};

__device__ __forceinline__ int pack4_i8(int8_t a, int8_t b, int8_t c, int8_t d) {
  return (int)((uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
               ((uint32_t)(uint8_t)d << 24));
}

// ---------------------------------------------------------------------------
// scan: tentative block scores for the G heads ([TS] Methodology 3, "Top-δ
// Selection": stream the low-bit keys, compute tentative scores per block)
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ __forceinline__ void scan_blocks(const DecodeParams& p, DecodeSmem<D, G>& sm, size_t bh, int j0,
                                            int nblk, int L, int lane, int w) {
  constexpr int NCW = D / 32;  // 32-bit code words per lane (8 codes each)
  const int quad = lane >> 2;
  const int ql = lane & 3;
  // this lane's slice of the int8 query: elements [ql*D/4, ql*D/4 + D/4)
  int qe[G][NCW], qo[G][NCW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const int8_t* s = &sm.qc[h][ql * (D / 4) + 8 * i];
      qe[h][i] = pack4_i8(s[0], s[2], s[4], s[6]);
      qo[h][i] = pack4_i8(s[1], s[3], s[5], s[7]);
    }
  }
  int corr[G];
  float cq[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    corr[h] = 8 * sm.sumq[h];
    cq[h] = sm.cq[h];
  }
  const uint8_t* kq = p.kq + bh * (size_t)p.cap * (D / 2);
  const float* ks = p.kscale + bh * (size_t)p.cap;

  for (int jl = w; jl < nblk; jl += kWaves) {
    const int t0 = (j0 + jl) * kBlockSize;
    uint32_t cw[4][NCW];
    float sc[4];
    bool valid[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = t0 + it * 16 + quad;
      valid[it] = t < L;
      if (valid[it]) {
        const uint8_t* src = kq + (size_t)t * (D / 2) + ql * (D / 8);
        if constexpr (NCW == 4) {
          uint4 u = *reinterpret_cast<const uint4*>(src);
          cw[it][0] = u.x; cw[it][1] = u.y; cw[it][2] = u.z; cw[it][3] = u.w;
        } else {
          uint2 u = *reinterpret_cast<const uint2*>(src);
          cw[it][0] = u.x; cw[it][1] = u.y;
        }
        sc[it] = ks[t];
      } else {
#pragma unroll
        for (int i = 0; i < NCW; ++i) cw[it][i] = 0u;
        sc[it] = 0.f;
      }
    }
    float bm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) bm[h] = -INFINITY;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0;
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        const uint32_t x = cw[it][i] ^ 0x88888888u;   // two's complement -> code + 8
        const int lo = (int)(x & 0x0f0f0f0fu);
        const int hi = (int)((x >> 4) & 0x0f0f0f0fu);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h] = __builtin_amdgcn_sdot4(lo, qe[h][i], acc[h], false);
          acc[h] = __builtin_amdgcn_sdot4(hi, qo[h][i], acc[h], false);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int dot = quad_sum_i(acc[h]) - corr[h];
        const float wgt = sc[it] * cq[h];
        const float s = (float)dot * wgt;
        if (valid[it]) bm[h] = fmaxf(bm[h], s);
      }
    }
    // max over the 16 quads (each quad's lanes hold identical values)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m = bm[h];
      m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
      m = fmaxf(m, dpp_f<kDppMirror>(m));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      bm[h] = m;
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) sm.blk[jl][h] = bm[h];
    }
  }
}

// ---------------------------------------------------------------------------
// select: split-local Top-δ ([TS] Methodology 2, "Mechanism" and
// "Pseudo-Max Approximation"; sink and local blocks always kept)
// ---------------------------------------------------------------------------
template <int D, int G, bool DENSE>
__device__ __forceinline__ void select_blocks(const DecodeParams& p, DecodeSmem<D, G>& sm, int b, int j,
                                              int j0, int nblk, int nmask, int NB, int lane) {
  const int jl = lane;
  const int jb = j0 + jl;
  const bool in_split = jl < nblk;
  unsigned hm = 0;
  if constexpr (DENSE) {
    hm = in_split ? ((1u << G) - 1u) : 0u;
  } else {
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = in_split ? sm.blk[jl][h] : -INFINITY;
    const bool forced = jb < p.sink || jb >= NB - p.local;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = wave_max_f(s[h]);
      const float thr = mt - p.delta;
      if (in_split && (s[h] >= thr || forced)) hm |= 1u << h;
      if (lane == 0) sm.seed[h] = mt;
    }
  }
  if (p.mask != nullptr && jl < nmask) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      p.mask[((size_t)b * p.Hq + (size_t)j * G + h) * p.nb_max + jb] = (uint8_t)((hm >> h) & 1u);
  }
  const unsigned long long bal = __ballot(hm != 0u);
  const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (hm != 0u) {
    sm.kidx[pos] = (uint8_t)jl;
    sm.khm[pos] = (uint8_t)hm;
  }
  if (lane == 0) sm.nkept = __popcll(bal);
}

// ---------------------------------------------------------------------------
// attend: exact attention over the kept blocks ([TS] Methodology 3,
// "Fine-Grained Refinement"), VALU version.
// ---------------------------------------------------------------------------
template <int D, int G, bool DENSE>
__device__ __forceinline__ void attend_blocks(const DecodeParams& p, DecodeSmem<D, G>& sm, size_t bh, int j0,
                                              int L, int lane, int w, float (&m)[G], float (&l)[G],
                                              float (&o)[G][8]) {
  constexpr int LPT = D / 8;      // lanes per token row
  constexpr int TPI = kWave / LPT;  // token rows per wave load
  const int tg = lane / LPT;
  const int c = lane % LPT;
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = sm.q[h][c * 8 + e];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = DENSE ? -INFINITY : sm.seed[h] * kLog2e;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const uint16_t* kb = p.k + bh * (size_t)p.cap * D;
  const uint16_t* vb = p.v + bh * (size_t)p.cap * D;
  const int nkept = sm.nkept;
  for (int e = w; e < nkept; e += kWaves) {
    const int jb = j0 + sm.kidx[e];
    const unsigned hm = sm.khm[e];
    for (int it = 0; it < kBlockSize / TPI; ++it) {
      const int t = jb * kBlockSize + it * TPI + tg;
      const bool valid = t < L;
      uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (valid) {
        kw = *reinterpret_cast<const uint4*>(kb + (size_t)t * D + c * 8);
        vw = *reinterpret_cast<const uint4*>(vb + (size_t)t * D + c * 8);
      }
      const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                           bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
      const float vf[8] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y),
                           bf16_lo(vw.z), bf16_hi(vw.z), bf16_lo(vw.w), bf16_hi(vw.w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += qr[h][i] * kf[i];
        s = group_sum_f<LPT>(s);
        if (!valid || !((hm >> h) & 1u)) s = -INFINITY;
        if (s > m[h]) {
          const float a = exp2f(m[h] - s);
          l[h] *= a;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[h][i] *= a;
          m[h] = s;
        }
        const float pr = (s == -INFINITY) ? 0.f : exp2f(s - m[h]);
        l[h] += pr;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] += pr * vf[i];
      }
    }
  }
}

// Merge two online-softmax states (base-2 logits).
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, int n, float m2, float l2, const float* o2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == -INFINITY) ? 0.f : exp2f(m - mn);
  const float b = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mn);
  l = l * a + l2 * b;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a + o2[i] * b;
  m = mn;
}

template <int D, int G, bool DENSE>
__global__ __launch_bounds__(kThreads) void fused_decode_kernel(const DecodeParams p) {
  __shared__ DecodeSmem<D, G> sm;
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int NB = (L + kBlockSize - 1) / kBlockSize;
  const int j0 = split * p.split_blocks;
  const int nmask = min(p.split_blocks, p.nb_max - j0);
  if (j0 >= NB) {
    // no valid block in this split: only the mask entries are owned here
    if (p.mask != nullptr) {
      for (int i = tid; i < nmask * G; i += kThreads) {
        const int h = i / nmask, jl = i % nmask;
        p.mask[((size_t)b * p.Hq + (size_t)j * G + h) * p.nb_max + j0 + jl] = 0;
      }
    }
    return;
  }
  const int nblk = min(p.split_blocks, NB - j0);
  const size_t bh = (size_t)b * p.Hkv + j;

  // ---- prologue: query to LDS, int8 scan query --------------------------
  const uint16_t* qg = p.q + ((size_t)b * p.Hq + (size_t)j * G) * D;
  for (int i = tid; i < G * D; i += kThreads) sm.q[i / D][i % D] = bf16_to_f32(qg[i]);
  __syncthreads();
  const float qscale = p.sm_scale * kLog2e;
  for (int h = w; h < G; h += kWaves) {
    constexpr int PER = D / kWave;
    float x[PER];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      x[r] = sm.q[h][lane + r * kWave];
      amax = fmaxf(amax, fabsf(x[r]));
    }
    amax = wave_max_f(amax);
    int qsum = 0;
    if constexpr (!DENSE) {
      // amax < 2^-120 counts as a zero query: 127/amax would overflow to +inf
      const bool nz = amax >= 0x1p-120f;
      if (nz) {
        const float inv = 127.0f / amax;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          float c = rintf(x[r] * inv);
          c = fminf(fmaxf(c, -127.f), 127.f);
          sm.qc[h][lane + r * kWave] = (int8_t)(int)c;
          qsum += (int)c;
        }
      } else {
#pragma unroll
        for (int r = 0; r < PER; ++r) sm.qc[h][lane + r * kWave] = 0;
      }
      qsum = wave_sum_i(qsum);
      if (lane == 0) {
        sm.sumq[h] = qsum;
        sm.cq[h] = nz ? (amax / 127.0f) * p.sm_scale : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) sm.q[h][lane + r * kWave] = x[r] * qscale;
  }
  __syncthreads();

  // ---- scan + select ------------------------------------------------------
  if constexpr (!DENSE) {
    scan_blocks<D, G>(p, sm, bh, j0, nblk, L, lane, w);
    __syncthreads();
  }
  if (w == 0) select_blocks<D, G, DENSE>(p, sm, b, j, j0, nblk, nmask, NB, lane);
  __syncthreads();

  // ---- attend -------------------------------------------------------------
  float m[G], l[G], o[G][8];
  attend_blocks<D, G, DENSE>(p, sm, bh, j0, L, lane, w, m, l, o);

  // merge the token groups of this wave (lanes that differ by multiples of D/8)
  constexpr int LPT = D / 8;
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off);
      const float l2 = __shfl_xor(l[h], off);
      float o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o2[i] = __shfl_xor(o[h][i], off);
      merge_state(m[h], l[h], o[h], 8, m2, l2, o2);
    }
  }
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.wo[w][h][lane * 8 + i] = o[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm.wm[w][h] = m[h];
      sm.wl[w][h] = l[h];
    }
  }
  __syncthreads();

  // ---- epilogue: merge waves, write the split partial -------------------
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, cc = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mx = fmaxf(mx, sm.wm[ww][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float a = (sm.wm[ww][h] == -INFINITY) ? 0.f : exp2f(sm.wm[ww][h] - mx);
      den += sm.wl[ww][h] * a;
      num += sm.wo[ww][h][cc] * a;
    }
    const size_t row = ((size_t)b * p.Hq + (size_t)j * G + h) * p.n_splits + split;
    p.o_part[row * D + cc] = num / den;
    if (cc == 0) p.lse_part[row] = (mx + log2f(den)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// split combine: lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) o_s
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int NB = (L + kBlockSize - 1) / kBlockSize;
  const int ns = (NB + p.split_blocks - 1) / p.split_blocks;
  const size_t bh = (size_t)b * p.Hq + h;
  const float* lp = p.lse_part + bh * p.n_splits;
  const float* op = p.o_part + bh * p.n_splits * D;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, lp[s]);
  float den = 0.f, num = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float a = (lp[s] == -INFINITY) ? 0.f : expf(lp[s] - mx);
    den += a;
    num += a * op[(size_t)s * D + c];
  }
  float res = 0.f, lse = -INFINITY;
  if (ns > 0 && den > 0.f) {
    res = num / den;
    lse = mx + logf(den);
  }
  if (p.out_f32) {
    static_cast<float*>(p.out)[bh * D + c] = res;
  } else {
    static_cast<uint16_t*>(p.out)[bh * D + c] = f32_to_bf16(res);
  }
  if (c == 0) p.lse[bh] = lse;
}

template <int D, int G, bool DENSE>
hipError_t launch_fused(const DecodeParams& p, hipStream_t stream) {
  if (p.n_splits > 0) {
    dim3 grid(p.n_splits, p.Hkv, p.B);
    fused_decode_kernel<D, G, DENSE><<<grid, kThreads, 0, stream>>>(p);
  }
  combine_kernel<D><<<dim3(p.Hq, p.B), D, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, bool DENSE>
hipError_t launch_g(const DecodeParams& p, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_fused<D, 1, DENSE>(p, stream);
    case 2: return launch_fused<D, 2, DENSE>(p, stream);
    case 4: return launch_fused<D, 4, DENSE>(p, stream);
    case 8: return launch_fused<D, 8, DENSE>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int D, int G, bool dense, hipStream_t stream) {
  if (D == 128) return dense ? launch_g<128, true>(p, G, stream) : launch_g<128, false>(p, G, stream);
  if (D == 64) return dense ? launch_g<64, true>(p, G, stream) : launch_g<64, false>(p, G, stream);
  return hipErrorInvalidValue;
}

}  // namespace ffd
