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
// (one 16-byte load) and produce one 32-bit word of codes. A thread handles
// kRowsPerThread rows, 256 / (D/8) rows apart, with all their loads issued
// before any is used (a workgroup covers 16·kRowsPerThread consecutive rows
// for D = 128), so that the build streams instead of paying one load's
// latency per workgroup.
#include "ffd_device.h"
#include "ffd_internal.h"

namespace ffd {

constexpr int kRowsPerThread = 8;

typedef uint32_t u32x4q_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack_bf16x8(u32x4q_t w, float x[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// max over the LPT lanes of a token row (aligned groups of 8 or 16 lanes)
template <int LPT>
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (LPT == 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ k,
                                                          uint8_t* __restrict__ kq,
                                                          float* __restrict__ kscale,
                                                          const int32_t* __restrict__ pos_begin,
                                                          const int32_t* __restrict__ pos_end,
                                                          const int32_t* __restrict__ block_table, int table_stride,
                                                          int num_pages, int Hkv, int cap) {
  constexpr int LPT = D / 8;         // lanes per token
  constexpr int TPB = 256 / LPT;     // tokens per workgroup pass
  const int b = blockIdx.z, j = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid % LPT;
  int begin = pos_begin[b];
  int end = pos_end[b];
  begin = begin < 0 ? 0 : begin;
  const int limit = block_table ? table_stride * 64 : cap;   // <= 2^30 (checked on the host)
  end = end > limit ? limit : end;
  // 64-bit: begin is a device value (unchecked), and may sit near INT_MAX
  const long long t_base = (long long)begin + (long long)blockIdx.x * TPB * kRowsPerThread + tid / LPT;

  u32x4q_t w[kRowsPerThread];
  size_t row[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const long long t = t_base + u * TPB;
    const int tv = t < end ? (int)t : 0;
    row[u] = cache_block_row(block_table, table_stride, num_pages, cap, Hkv, b, j, tv / 64) + tv % 64;
    w[u] = t < end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4q_t*>(k + row[u] * D + sub * 8))
                   : u32x4q_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    float x[8];
    unpack_bf16x8(w[u], x);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = row_max<LPT>(amax);
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
    if (t_base + u * TPB < (long long)end) {
      *reinterpret_cast<uint32_t*>(kq + row[u] * (D / 2) + sub * 4) = packed;
      if (sub == 0) kscale[row[u]] = scale;
    }
  }
}

hipError_t launch_quantize_kv(const uint16_t* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                              const int32_t* pos_end, const int32_t* block_table, int table_stride, int num_pages,
                              int B, int Hkv, int cap, int D, int max_span, hipStream_t stream) {
  const int rows = 256 / (D / 8) * kRowsPerThread;   // token rows per workgroup
  dim3 grid((unsigned)(((long)max_span + rows - 1) / rows), Hkv, B);
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
  // 64-bit: begin is a device value (unchecked), and may sit near INT_MAX
  const long long t_base = (long long)begin + (long long)blockIdx.x * TPB * kRowsPerThread + tid / LPT;

  u32x4q_t w[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const long long t = t_base + u * TPB;
    const size_t row = ((size_t)b * Hkv + j) * cap + (t < end ? (int)t : 0);
    w[u] = t < end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4q_t*>(k + row * D + sub * 8))
                   : u32x4q_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const long long t = t_base + u * TPB;
    const size_t row = ((size_t)b * Hkv + j) * cap + (t < end ? (int)t : 0);
    float x[8];
    unpack_bf16x8(w[u], x);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = row_max<LPT>(amax);

    const bool nz = amax >= 0x1p-125f;
    const float inv3 = nz ? 3.0f / amax : 0.f;
    const float ts = nz ? amax / 3.0f : 0.f;
    uint32_t codes = 0;
    float r[8];
    float ramax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int uc = 0;
      if (nz) {
        const float xs = x[i] * inv3;
        const float y = (xs + 3.0f) * 0.5f;
        uc = (int)fminf(fmaxf(rintf(y), 0.f), 3.f);
      }
      codes |= (uint32_t)uc << (2 * i);
      const float lev = (float)(2 * uc - 3) * ts;
      r[i] = nz ? x[i] - lev : 0.f;
      ramax = fmaxf(ramax, fabsf(r[i]));
    }
    ramax = row_max<LPT>(ramax);
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
    if (t < end) {
      *reinterpret_cast<uint16_t*>(k2 + row * (D / 4) + sub * 2) = (uint16_t)codes;
      *reinterpret_cast<uint2*>(kr + row * D + sub * 8) = make_uint2(rp[0], rp[1]);
      if (sub == 0) {
        k2scale[row] = ts;
        krscale[row] = s8;
      }
    }
  }
}

hipError_t launch_quantize_thumb(const uint16_t* k, uint8_t* k2, float* k2scale, int8_t* kr, float* krscale,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int cap, int D,
                                 int max_span, hipStream_t stream) {
  const int rows = 256 / (D / 8) * kRowsPerThread;   // token rows per workgroup
  dim3 grid((unsigned)(((long)max_span + rows - 1) / rows), Hkv, B);
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
