// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ffd {

constexpr int kBlockSize = 64;   // tokens per selection block
constexpr int kMaxSplit = 64;    // max blocks per split (one workgroup)
constexpr int kMaxPseudoMax = 64; // max sink + local blocks with the sink/local pseudo-max
constexpr int kMaxRows = 16;     // query rows (query tokens x heads of a kv group) per workgroup
constexpr size_t kWsAlign = 256;
constexpr int kMaxParts = 4;     // workgroups sharing one split's attend work

// Waves per workgroup. On a grid of at most 1024 (sequence, query head,
// split) units -- at most one 4-wave workgroup per CU at G = 4 -- the kernel
// runs 8 waves per workgroup, one workgroup per CU: each wave then has half
// the scan and attend blocks, which halves the latency chain of a grid that
// is one round long.
inline int waves_for(int B, int Hq, int n_splits) {
  const long units = (long)B * Hq * n_splits;
  return units > 0 && units <= 1024 ? 8 : 4;
}

// Workgroups per split. When (sequence, kv head, split) units are too few to
// fill the chip, P workgroups share a split: each scans and selects the whole
// split (same kept set) and attends a disjoint share of its kept blocks (the
// P * waves waves of the split take them round-robin), leaving one partial
// each. A function of (B, Hq, n_splits) alone, so the workspace size
// and a separate combine call agree with the decode.
inline int split_parts_for(int B, int Hq, int n_splits) {
  const long units = (long)B * Hq * n_splits;
  if (units <= 0 || waves_for(B, Hq, n_splits) == 4) return 1;
  const long P = 1024 / units;   // about one round of resident 8-wave workgroups at G = 4
  return P < 1 ? 1 : (P > kMaxParts ? kMaxParts : (int)P);
}

// Q query tokens per sequence (Q = 1: ordinary decode). Query-head rows are
// indexed (b * Q + i) * Hq + h throughout: q, out, lse, mask and partials.
struct DecodeParams {
  const uint16_t* q;       // bf16 [B, Q, Hq, D]
  const uint16_t* k;       // bf16 [B, Hkv, cap, D]
  const uint16_t* v;       // bf16 [B, Hkv, cap, D]
  const uint8_t* kq;       // u8   [B, Hkv, cap, D/2]
  const float* kscale;     // f32  [B, Hkv, cap]
  const uint8_t* k2;       // thumbnail storage: 2-bit codes u8 [B, Hkv, cap, D/4]
  const float* k2scale;    //   f32 [B, Hkv, cap]  (t)
  const int8_t* kr;        //   int8 residual [B, Hkv, cap, D]
  const float* krscale;    //   f32 [B, Hkv, cap]  (s8)
  const int32_t* seq_lens; // [B]
  const int32_t* block_table;  // [B, table_stride] page of each block, or null (contiguous cache)
  int table_stride, num_pages; // paged cache: K/V [num_pages, Hkv, 64, D], kq/kscale alike
  float* o_part;           // f32  [B, Q, Hq, n_splits * split_parts, D]   (normalised per part)
  float* lse_part;         // f32  [B, Q, Hq, n_splits * split_parts]      (natural log)
  uint8_t* mask;           // u8   [B, Q, Hq, nb_max] or null
  void* out;               // bf16 / f32 [B, Q, Hq, D]
  float* lse;              // f32 [B, Q, Hq]
  int out_f32;
  int max_seq_len, B, Q, Hq, Hkv, cap;
  int nb_max;              // ceil(max_seq_len / kBlockSize)
  int n_splits;            // ceil(nb_max / split_blocks)
  int split_parts;         // workgroups per split (split_parts_for); partials per row = n_splits * split_parts
  int waves;               // waves per workgroup (waves_for): 4 or 8
  int split_blocks;
  int sink, local;
  int pm_sink_local;       // 1: pseudo-max over the sink/local blocks; 0: split max
  int pm_with_split;       // with pm_sink_local: the larger of that estimate and the split max
  float delta, sm_scale;
};

// Workspace carving shared by sizing and launch.
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t ws_opart_bytes(int B, int Hq, int n_splits, int D) {
  return align_up((size_t)B * Hq * n_splits * D * sizeof(float), kWsAlign);
}
inline size_t ws_lse_bytes(int B, int Hq, int n_splits) {
  return align_up((size_t)B * Hq * n_splits * sizeof(float), kWsAlign);
}


// block_table == null: contiguous [B, Hkv, cap, D]; else paged [num_pages, Hkv, 64, D]
hipError_t launch_quantize_kv(const uint16_t* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                              const int32_t* pos_end, const int32_t* block_table, int table_stride, int num_pages,
                              int B, int Hkv, int cap, int D, int max_span, hipStream_t stream);

hipError_t launch_quantize_thumb(const uint16_t* k, uint8_t* k2, float* k2scale, int8_t* kr, float* krscale,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int cap, int D,
                                 int max_span, hipStream_t stream);

enum class Stage { kPartials = 1, kCombine = 2, kBoth = 3 };

// The kernels of one (D, dense, thumb) family (defined in ffd_decode.hip).
// Returns hipErrorInvalidValue for an unsupported (G, p.Q) combination
// (G * Q <= 16; Q > 1 only with the int4 storage). THUMB: K comes from the
// thumbnail + residual storage instead of bf16 K and the int4 sketch.
template <int D, bool DENSE, bool THUMB>
hipError_t launch_variant(const DecodeParams& p, int G, Stage stage, hipStream_t stream);

// Dispatch on the runtime (D, dense, thumb) (defined in ffd_api.hip, outside
// the translation units that define the kernel families);
// hipErrorInvalidValue for an unsupported combination.
hipError_t launch_decode(const DecodeParams& p, int D, int G, bool dense, Stage stage, hipStream_t stream,
                         bool thumb = false);

}  // namespace ffd
