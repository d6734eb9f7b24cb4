// Device helpers shared by the FFD kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffd {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round half to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- DPP lane exchanges (all 64 lanes must be active) ----------------------
// quad_perm [1,0,3,2] and [2,3,0,1]; row_half_mirror (lane i <-> 7-i within
// each 8-lane half row); row_mirror (lane i <-> 15-i within each 16-lane row);
// row_newbcast:k (lane k of each 16-lane row to the whole row).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;
constexpr int kDppQuadXor2 = 0x4e;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowBcast0 = 0x150;   // row_newbcast:k = 0x150 + k (gfx90a and later)

// Lane k (0..15) of each 16-lane row, to every lane of that row. k must fold
// to a constant (an unrolled loop index): the switch then leaves one DPP move.
__device__ __forceinline__ float row_bcast_f(float x, int k) {
  switch (k) {
    case 0: return dpp_f<kDppRowBcast0 + 0>(x);
    case 1: return dpp_f<kDppRowBcast0 + 1>(x);
    case 2: return dpp_f<kDppRowBcast0 + 2>(x);
    case 3: return dpp_f<kDppRowBcast0 + 3>(x);
    case 4: return dpp_f<kDppRowBcast0 + 4>(x);
    case 5: return dpp_f<kDppRowBcast0 + 5>(x);
    case 6: return dpp_f<kDppRowBcast0 + 6>(x);
    case 7: return dpp_f<kDppRowBcast0 + 7>(x);
    case 8: return dpp_f<kDppRowBcast0 + 8>(x);
    case 9: return dpp_f<kDppRowBcast0 + 9>(x);
    case 10: return dpp_f<kDppRowBcast0 + 10>(x);
    case 11: return dpp_f<kDppRowBcast0 + 11>(x);
    case 12: return dpp_f<kDppRowBcast0 + 12>(x);
    case 13: return dpp_f<kDppRowBcast0 + 13>(x);
    case 14: return dpp_f<kDppRowBcast0 + 14>(x);
    default: return dpp_f<kDppRowBcast0 + 15>(x);
  }
}

// Max over the wave; every lane gets it. The steps inside each 16-lane row are
// DPP moves (VALU latency), only the two steps across rows go through LDS.
__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Reductions over aligned groups of N = 8 or 16 consecutive lanes, DPP moves
// only; every lane of a group gets its group's result (the partners of each
// step hold equal partial results, so a float sum is the same on every lane).
// All lanes of a group must be active.
template <int N>
__device__ __forceinline__ float group_max_f(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  if constexpr (N == 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float group_sum_f(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_f<kDppMirror>(x);
  return x;
}
template <int N>
__device__ __forceinline__ int group_sum_i(int x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor1, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor2, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppHalfMirror, 0xf, 0xf, false);
  if constexpr (N == 16) x += __builtin_amdgcn_update_dpp(0, x, kDppMirror, 0xf, 0xf, false);
  return x;
}

// Row index (in a [rows, D] view of the cache) of token 0 of block jb of
// sequence b, kv head j. Contiguous cache: [B, Hkv, cap, D]. Paged cache: the
// block lives in page block_table[b, jb] of a [num_pages, Hkv, 64, D] pool;
// out-of-range page numbers are clamped so a bad table cannot fault.
__device__ __forceinline__ size_t cache_block_row(const int32_t* block_table, int table_stride, int num_pages,
                                                  int cap, int Hkv, int b, int j, int jb) {
  if (block_table != nullptr) {
    int pg = block_table[(size_t)b * table_stride + jb];
    pg = pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : pg);
    return ((size_t)pg * Hkv + j) * 64;
  }
  return ((size_t)b * Hkv + j) * cap + (size_t)jb * 64;
}

}  // namespace ffd
