// KV quantise/append kernel: bf16 K rows -> int4 codes + fp32 per-token scale.
//
// The low-bit key sketch that the scan reads ([TS] "Faster Than Flash", technical
// summary, Methodology 1: keys kept in a low-bit form for content-aware
// scanning). This library's sketch is symmetric int4 in [-7, 7] with one fp32
// scale per (token, kv head):
//   amax = max|k_i|, scale = fl32(amax/7), code_i = clamp(rne(fl32(k_i*fl32(7/amax))), -7, 7)
// (a row with amax < 2^-125 gets scale 0 and zero codes), packed as
// two's-complement nibbles, element 2i in the low nibble of byte i.
//
// Layout: one token row is D bf16 = D*2 bytes; D/8 lanes each own 8 elements
// (one 16-byte load) and produce one 32-bit word of codes, so a wave reads
// 1 KiB of K and writes 256 B of codes + 16 B of scales per instruction.
#include "ffd_device.h"
#include "ffd_internal.h"

namespace ffd {

template <int D>
__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ k,
                                                          uint8_t* __restrict__ kq,
                                                          float* __restrict__ kscale,
                                                          const int32_t* __restrict__ pos_begin,
                                                          const int32_t* __restrict__ pos_end,
                                                          const int32_t* __restrict__ block_table, int table_stride,
                                                          int num_pages, int Hkv, int cap) {
  constexpr int LPT = D / 8;         // lanes per token
  constexpr int TPB = 256 / LPT;     // tokens per workgroup
  const int b = blockIdx.z, j = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid % LPT;
  int begin = pos_begin[b];
  int end = pos_end[b];
  begin = begin < 0 ? 0 : begin;
  const int limit = block_table ? table_stride * 64 : cap;
  end = end > limit ? limit : end;
  const int t = begin + blockIdx.x * TPB + tid / LPT;
  const bool valid = t < end;
  const int tv = valid ? t : 0;
  const size_t row = cache_block_row(block_table, table_stride, num_pages, cap, Hkv, b, j, tv / 64) + tv % 64;

  uint4 w = make_uint4(0, 0, 0, 0);
  if (valid) w = *reinterpret_cast<const uint4*>(k + row * D + sub * 8);
  float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // max over the LPT lanes of this token (aligned groups of 8 or 16 lanes)
  amax = fmaxf(amax, dpp_f<kDppQuadXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppQuadXor2>(amax));
  amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
  if constexpr (LPT == 16) amax = fmaxf(amax, dpp_f<kDppMirror>(amax));

  uint32_t packed = 0;
  float scale = 0.f;
  // amax < 2^-125 counts as a zero row: 7/amax would overflow to +inf
  if (amax >= 0x1p-125f) {
    const float inv = 7.0f / amax;   // correctly rounded division
    scale = amax / 7.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = rintf(x[i] * inv);
      c = fminf(fmaxf(c, -7.f), 7.f);
      packed |= ((uint32_t)(int)c & 0xfu) << (4 * i);
    }
  }
  if (valid) {
    *reinterpret_cast<uint32_t*>(kq + row * (D / 2) + sub * 4) = packed;
    if (sub == 0) kscale[row] = scale;
  }
}

hipError_t launch_quantize_kv(const uint16_t* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                              const int32_t* pos_end, const int32_t* block_table, int table_stride, int num_pages,
                              int B, int Hkv, int cap, int D, int max_span, hipStream_t stream) {
  const int lpt = D / 8;
  const int tpb = 256 / lpt;
  dim3 grid((max_span + tpb - 1) / tpb, Hkv, B);
  if (D == 128) {
    quantize_kv_kernel<128><<<grid, 256, 0, stream>>>(k, kq, kscale, pos_begin, pos_end, block_table, table_stride,
                                                      num_pages, Hkv, cap);
  } else if (D == 64) {
    quantize_kv_kernel<64><<<grid, 256, 0, stream>>>(k, kq, kscale, pos_begin, pos_end, block_table, table_stride,
                                                     num_pages, Hkv, cap);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ffd

// ---------------------------------------------------------------------------
// Thumbnail + residual keys ([TS] Methodology 1: 2-bit thumbnails for the scan,
// 8-bit residuals to reconstruct the keys for refinement). Per token row:
//   t = fl32(amax/3); x = fl32(k * fl32(3/amax)); u = clamp(rne(fl32(x+3)*0.5), 0, 3)
//   r = fl32(k - fl32((2u-3) * t)); s8 = fl32(amax_r/127);
//   r8 = clamp(rne(fl32(r * fl32(127/amax_r))), -127, 127)
// (amax < 2^-125: t = 0 and u, r8, s8 all 0; amax_r < 2^-120: s8 = 0, r8 = 0).
// Codes are packed four per byte, element 4i + c in bits 2c of byte i.
// ---------------------------------------------------------------------------
namespace ffd {

template <int D>
__global__ __launch_bounds__(256) void quantize_thumb_kernel(const uint16_t* __restrict__ k,
                                                             uint8_t* __restrict__ k2, float* __restrict__ k2scale,
                                                             int8_t* __restrict__ kr, float* __restrict__ krscale,
                                                             const int32_t* __restrict__ pos_begin,
                                                             const int32_t* __restrict__ pos_end, int Hkv, int cap) {
  constexpr int LPT = D / 8;
  constexpr int TPB = 256 / LPT;
  const int b = blockIdx.z, j = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid % LPT;
  int begin = pos_begin[b];
  int end = pos_end[b];
  begin = begin < 0 ? 0 : begin;
  end = end > cap ? cap : end;
  const int t = begin + blockIdx.x * TPB + tid / LPT;
  const bool valid = t < end;
  const size_t row = ((size_t)b * Hkv + j) * cap + (valid ? t : 0);

  uint4 w = make_uint4(0, 0, 0, 0);
  if (valid) w = *reinterpret_cast<const uint4*>(k + row * D + sub * 8);
  const float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                      bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, dpp_f<kDppQuadXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppQuadXor2>(amax));
  amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
  if constexpr (LPT == 16) amax = fmaxf(amax, dpp_f<kDppMirror>(amax));

  const bool nz = amax >= 0x1p-125f;
  const float inv3 = nz ? 3.0f / amax : 0.f;
  const float ts = nz ? amax / 3.0f : 0.f;
  uint32_t codes = 0;
  float r[8];
  float ramax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int u = 0;
    if (nz) {
      const float xs = x[i] * inv3;
      const float y = (xs + 3.0f) * 0.5f;
      u = (int)fminf(fmaxf(rintf(y), 0.f), 3.f);
    }
    codes |= (uint32_t)u << (2 * i);
    const float lev = (float)(2 * u - 3) * ts;
    r[i] = nz ? x[i] - lev : 0.f;
    ramax = fmaxf(ramax, fabsf(r[i]));
  }
  ramax = fmaxf(ramax, dpp_f<kDppQuadXor1>(ramax));
  ramax = fmaxf(ramax, dpp_f<kDppQuadXor2>(ramax));
  ramax = fmaxf(ramax, dpp_f<kDppHalfMirror>(ramax));
  if constexpr (LPT == 16) ramax = fmaxf(ramax, dpp_f<kDppMirror>(ramax));
  const bool nzr = ramax >= 0x1p-120f;
  const float invr = nzr ? 127.0f / ramax : 0.f;
  const float s8 = nzr ? ramax / 127.0f : 0.f;
  uint32_t rp[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int q = 0;
    if (nzr) q = (int)fminf(fmaxf(rintf(r[i] * invr), -127.f), 127.f);
    rp[i >> 2] |= ((uint32_t)q & 0xffu) << (8 * (i & 3));
  }
  if (valid) {
    *reinterpret_cast<uint16_t*>(k2 + row * (D / 4) + sub * 2) = (uint16_t)codes;
    *reinterpret_cast<uint2*>(kr + row * D + sub * 8) = make_uint2(rp[0], rp[1]);
    if (sub == 0) {
      k2scale[row] = ts;
      krscale[row] = s8;
    }
  }
}

hipError_t launch_quantize_thumb(const uint16_t* k, uint8_t* k2, float* k2scale, int8_t* kr, float* krscale,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int cap, int D,
                                 int max_span, hipStream_t stream) {
  const int tpb = 256 / (D / 8);
  dim3 grid((max_span + tpb - 1) / tpb, Hkv, B);
  if (D == 128) {
    quantize_thumb_kernel<128><<<grid, 256, 0, stream>>>(k, k2, k2scale, kr, krscale, pos_begin, pos_end, Hkv, cap);
  } else if (D == 64) {
    quantize_thumb_kernel<64><<<grid, 256, 0, stream>>>(k, k2, k2scale, kr, krscale, pos_begin, pos_end, Hkv, cap);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ffd
