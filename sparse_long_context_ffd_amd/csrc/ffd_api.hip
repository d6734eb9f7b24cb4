// C-ABI layer: argument validation, dispatch, workspace carving, launch.
// Allocates nothing and never synchronises (safe inside stream capture).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "ffd.h"
#include "ffd_internal.h"

namespace ffd {

hipError_t launch_decode(const DecodeParams& p, int D, int G, bool dense, Stage stage, hipStream_t stream, bool thumb) {
  if (D == 128) {
    if (thumb) return dense ? launch_variant<128, true, true>(p, G, stage, stream)
                            : launch_variant<128, false, true>(p, G, stage, stream);
    return dense ? launch_variant<128, true, false>(p, G, stage, stream)
                 : launch_variant<128, false, false>(p, G, stage, stream);
  }
  if (D == 64) {
    if (thumb) return dense ? launch_variant<64, true, true>(p, G, stage, stream)
                            : launch_variant<64, false, true>(p, G, stage, stream);
    return dense ? launch_variant<64, true, false>(p, G, stage, stream)
                 : launch_variant<64, false, false>(p, G, stage, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ffd

namespace {

thread_local std::string g_err;

ffd_status fail(ffd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ffd_status ok() {
  g_err.clear();
  return FFD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Longest max_seq_len, cap or max_span accepted: token positions and block
// counts (plus a block or a workgroup's rows) then stay inside int everywhere.
constexpr int kMaxTokens = 1 << 30;

int nb_max_for(int max_seq_len) { return (int)(((long)max_seq_len + ffd::kBlockSize - 1) / ffd::kBlockSize); }

int n_splits_for(int max_seq_len, int split_blocks) {
  return (int)(((long)nb_max_for(max_seq_len) + split_blocks - 1) / split_blocks);
}

// Workspace of a decode over B sequences with `rows` query-head rows each
// (Hq, or Q * Hq), Hq query heads per token: one partial per row, split and part.
size_t decode_ws_bytes(int B, int rows, int Hq, int max_seq_len, int split_blocks, int d) {
  const int ns = n_splits_for(max_seq_len, split_blocks);
  const int np = ns * ffd::split_parts_for(B, Hq, ns);
  return ffd::ws_opart_bytes(B, rows, np, d) + ffd::ws_lse_bytes(B, rows, np);
}

}  // namespace

extern "C" {

int ffd_abi_version(void) { return FFD_ABI_VERSION; }

const char* ffd_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

ffd_status quantize_common(const char* fn, const void* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                           const int32_t* pos_end, const int32_t* block_table, int table_stride, int num_pages,
                           int B, int Hkv, int cap, int d, int max_span, void* stream) {
  if (B < 0 || Hkv < 0 || cap < 0 || max_span < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: negative size (B=%d Hkv=%d cap=%d max_span=%d)", fn, B, Hkv, cap, max_span);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "%s: d must be positive and even (d=%d)", fn, d);
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "%s: d=%d not supported (64, 128)", fn, d);
  if (B == 0 || Hkv == 0 || cap == 0 || max_span == 0) return ok();
  if (!k || !kq || !kscale || !pos_begin || !pos_end) return fail(FFD_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(k) || !aligned16(kq)) return fail(FFD_ERR_INVALID_ARG, "%s: k and kq must be 16-byte aligned", fn);
  if (B > 65535 || Hkv > 65535) return fail(FFD_ERR_UNSUPPORTED, "%s: B and Hkv must be <= 65535", fn);
  if (max_span > kMaxTokens || cap > kMaxTokens)
    return fail(FFD_ERR_UNSUPPORTED, "%s: cap and max_span must be <= 2^30 tokens", fn);
  hipError_t e = ffd::launch_quantize_kv(static_cast<const uint16_t*>(k), kq, kscale, pos_begin, pos_end, block_table,
                                         table_stride, num_pages, B, Hkv, cap, d, max_span,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ffd_status ffd_quantize_kv(const void* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                           const int32_t* pos_end, int B, int Hkv, int cap, int d, int max_span,
                           void* stream) {
  return quantize_common("ffd_quantize_kv", k, kq, kscale, pos_begin, pos_end, nullptr, 0, 0, B, Hkv, cap, d,
                         max_span, stream);
}

ffd_status ffd_quantize_kv_thumb(const void* k, uint8_t* k2, float* k2scale, int8_t* kr, float* krscale,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int cap, int d,
                                 int max_span, void* stream) {
  const char* fn = "ffd_quantize_kv_thumb";
  if (B < 0 || Hkv < 0 || cap < 0 || max_span < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: negative size (B=%d Hkv=%d cap=%d max_span=%d)", fn, B, Hkv, cap, max_span);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "%s: d must be positive and even (d=%d)", fn, d);
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "%s: d=%d not supported (64, 128)", fn, d);
  if (B == 0 || Hkv == 0 || cap == 0 || max_span == 0) return ok();
  if (!k || !k2 || !k2scale || !kr || !krscale || !pos_begin || !pos_end)
    return fail(FFD_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(k) || !aligned16(k2) || !aligned16(kr))
    return fail(FFD_ERR_INVALID_ARG, "%s: k, k2, kr must be 16-byte aligned", fn);
  if (B > 65535 || Hkv > 65535) return fail(FFD_ERR_UNSUPPORTED, "%s: B and Hkv must be <= 65535", fn);
  if (max_span > kMaxTokens || cap > kMaxTokens)
    return fail(FFD_ERR_UNSUPPORTED, "%s: cap and max_span must be <= 2^30 tokens", fn);
  hipError_t e = ffd::launch_quantize_thumb(static_cast<const uint16_t*>(k), k2, k2scale, kr, krscale, pos_begin,
                                            pos_end, B, Hkv, cap, d, max_span, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

ffd_status ffd_quantize_kv_paged(const void* k_pages, uint8_t* kq_pages, float* kscale_pages,
                                 const int32_t* block_table, int table_stride, int num_pages,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int d,
                                 int max_span, void* stream) {
  const char* fn = "ffd_quantize_kv_paged";
  if (table_stride < 0 || num_pages < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: negative table_stride/num_pages (%d, %d)", fn, table_stride, num_pages);
  if (B > 0 && Hkv > 0 && max_span > 0 && table_stride > 0 && num_pages > 0 && !block_table)
    return fail(FFD_ERR_INVALID_ARG, "%s: null block_table", fn);
  if (table_stride > kMaxTokens / ffd::kBlockSize)
    return fail(FFD_ERR_UNSUPPORTED, "%s: table_stride=%d above 2^24 pages per sequence", fn, table_stride);
  if (table_stride == 0 || num_pages == 0) {   // nothing addressable
    if (B < 0 || Hkv < 0 || max_span < 0) return fail(FFD_ERR_INVALID_ARG, "%s: negative size", fn);
    return ok();
  }
  return quantize_common(fn, k_pages, kq_pages, kscale_pages, pos_begin, pos_end, block_table, table_stride,
                         num_pages, B, Hkv, table_stride * ffd::kBlockSize, d, max_span, stream);
}

size_t ffd_decode_multi_workspace_bytes(int B, int Q, int Hq, int d, int max_seq_len, int block_size,
                                        int split_blocks) {
  if (Q <= 0 || Hq <= 0 || (long)Q * Hq > 65535) return 0;
  if (B <= 0 || d <= 0 || max_seq_len <= 0 || block_size != ffd::kBlockSize || split_blocks < 1) return 0;
  if (max_seq_len > kMaxTokens) return 0;
  return decode_ws_bytes(B, Q * Hq, Hq, max_seq_len, split_blocks, d);
}

size_t ffd_decode_workspace_bytes(int B, int Hq, int d, int max_seq_len, int block_size, int split_blocks) {
  if (B <= 0 || Hq <= 0 || d <= 0 || max_seq_len <= 0 || block_size != ffd::kBlockSize || split_blocks < 1) return 0;
  if (max_seq_len > kMaxTokens) return 0;
  return decode_ws_bytes(B, Hq, Hq, max_seq_len, split_blocks, d);
}

}  // extern "C"

namespace {

// Validates the decode arguments shared by ffd_decode and ffd_decode_partials
// and fills `p` (except the output fields). `need_bytes` gets the workspace
// size the call requires.
ffd_status prepare_decode(const char* fn, const void* q, const void* k, const void* v, const uint8_t* kq,
                          const float* kscale, const int32_t* seq_lens, int max_seq_len, int B, int Q, int Hq, int Hkv,
                          int d, int cap, int block_size, float delta, int sink_blocks, int local_blocks,
                          int pseudo_max, int split_blocks, float sm_scale, uint8_t* kept_mask, void* workspace,
                          size_t workspace_bytes, const int32_t* block_table, int table_stride, int num_pages,
                          ffd::DecodeParams& p, int& G, bool& dense) {
  if (B < 0 || Q < 1 || Hq <= 0 || Hkv <= 0 || cap < 0 || max_seq_len < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: bad sizes (B=%d Q=%d Hq=%d Hkv=%d cap=%d max_seq_len=%d)", fn, B, Q, Hq, Hkv,
                cap, max_seq_len);
  if (Hq % Hkv) return fail(FFD_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "%s: d must be positive and even (d=%d)", fn, d);
  if (max_seq_len > kMaxTokens)
    return fail(FFD_ERR_UNSUPPORTED, "%s: max_seq_len=%d above 2^30 tokens", fn, max_seq_len);
  if (block_table == nullptr && cap < max_seq_len)
    return fail(FFD_ERR_INVALID_ARG, "%s: cap=%d < max_seq_len=%d", fn, cap, max_seq_len);
  if (block_table != nullptr) {
    const long nbm = ((long)max_seq_len + ffd::kBlockSize - 1) / ffd::kBlockSize;
    if (table_stride < nbm)
      return fail(FFD_ERR_INVALID_ARG, "%s: table_stride=%d < ceil(max_seq_len/64)=%ld", fn, table_stride, nbm);
    if (num_pages < 1) return fail(FFD_ERR_INVALID_ARG, "%s: num_pages must be >= 1 (got %d)", fn, num_pages);
    // the kernel keeps a split's (page, kv head) slot numbers as 32-bit ints
    if ((long)num_pages * Hkv > 0x7fffffffL)
      return fail(FFD_ERR_UNSUPPORTED, "%s: num_pages * Hkv = %ld above 2^31 - 1", fn, (long)num_pages * Hkv);
  }
  if (isnan(delta) || delta < 0.f) return fail(FFD_ERR_INVALID_ARG, "%s: delta must be >= 0 (got %g)", fn, (double)delta);
  if (sink_blocks < 0 || local_blocks < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: sink/local must be >= 0 (%d, %d)", fn, sink_blocks, local_blocks);
  if (split_blocks < 1) return fail(FFD_ERR_INVALID_ARG, "%s: split_blocks must be >= 1 (got %d)", fn, split_blocks);
  if (!(sm_scale > 0.f) || isinf(sm_scale))
    return fail(FFD_ERR_INVALID_ARG, "%s: sm_scale must be positive and finite (got %g)", fn, (double)sm_scale);
  if (block_size <= 0) return fail(FFD_ERR_INVALID_ARG, "%s: block_size must be positive (got %d)", fn, block_size);
  if (pseudo_max != FFD_PSEUDO_MAX_SPLIT && pseudo_max != FFD_PSEUDO_MAX_SINK_LOCAL &&
      pseudo_max != FFD_PSEUDO_MAX_BOTH)
    return fail(FFD_ERR_INVALID_ARG, "%s: unknown pseudo_max mode %d", fn, pseudo_max);
  if (pseudo_max != FFD_PSEUDO_MAX_SPLIT && (long)sink_blocks + local_blocks < 1)
    return fail(FFD_ERR_INVALID_ARG, "%s: the sink/local pseudo-max needs sink_blocks + local_blocks >= 1", fn);
  G = Hq / Hkv;
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "%s: d=%d not supported (64, 128)", fn, d);
  if (block_size != ffd::kBlockSize) return fail(FFD_ERR_UNSUPPORTED, "%s: block_size=%d not supported (64)", fn, block_size);
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(FFD_ERR_UNSUPPORTED, "%s: group size %d not supported (1, 2, 4, 8)", fn, G);
  if ((long)G * Q > ffd::kMaxRows)
    return fail(FFD_ERR_UNSUPPORTED, "%s: %d query tokens x group size %d exceeds %d rows per workgroup", fn, Q, G,
                ffd::kMaxRows);
  if (split_blocks > ffd::kMaxSplit)
    return fail(FFD_ERR_UNSUPPORTED, "%s: split_blocks=%d not supported (<= %d)", fn, split_blocks, ffd::kMaxSplit);
  // the query tokens' local windows together span local + ceil((Q - 1) / 64) + 1 blocks at most
  if (pseudo_max != FFD_PSEUDO_MAX_SPLIT &&
      (long)sink_blocks + local_blocks + (Q > 1 ? (Q - 1 + ffd::kBlockSize - 1) / ffd::kBlockSize : 0) >
          ffd::kMaxPseudoMax)
    return fail(FFD_ERR_UNSUPPORTED, "%s: sink_blocks + local_blocks = %ld exceeds %d with the sink/local pseudo-max",
                fn, (long)sink_blocks + local_blocks, ffd::kMaxPseudoMax);
  if (B > 65535 || Hkv > 65535 || (long)Q * Hq > 65535)
    return fail(FFD_ERR_UNSUPPORTED, "%s: B, Q * Hq, Hkv must be <= 65535", fn);
  dense = isinf(delta);
  if (B > 0) {
    if (!q || !seq_lens) return fail(FFD_ERR_INVALID_ARG, "%s: null q/seq_lens", fn);
    if (max_seq_len > 0 && (!k || !v)) return fail(FFD_ERR_INVALID_ARG, "%s: null k/v", fn);
    if (max_seq_len > 0 && !dense && (!kq || !kscale))
      return fail(FFD_ERR_INVALID_ARG, "%s: kq/kscale required unless delta is +inf", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kq))
      return fail(FFD_ERR_INVALID_ARG, "%s: q, k, v, kq must be 16-byte aligned", fn);
  }
  const int nb_max = nb_max_for(max_seq_len);
  const int ns = max_seq_len > 0 ? n_splits_for(max_seq_len, split_blocks) : 0;
  const int rows = Q * Hq;   // query-head rows per sequence
  const int parts = ns > 0 ? ffd::split_parts_for(B, Hq, ns) : 1;
  const size_t need = (B > 0 && max_seq_len > 0)
                          ? ffd::ws_opart_bytes(B, rows, ns * parts, d) + ffd::ws_lse_bytes(B, rows, ns * parts)
                          : 0;
  if (need > 0) {
    if (!workspace) return fail(FFD_ERR_INVALID_ARG, "%s: null workspace", fn);
    if (workspace_bytes < need)
      return fail(FFD_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % ffd::kWsAlign)
      return fail(FFD_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  }
  p = ffd::DecodeParams{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kq = kq;
  p.kscale = kscale;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.table_stride = table_stride;
  p.num_pages = num_pages;
  char* ws = static_cast<char*>(workspace);
  p.o_part = need ? reinterpret_cast<float*>(ws) : nullptr;
  p.lse_part = need ? reinterpret_cast<float*>(ws + ffd::ws_opart_bytes(B, rows, ns * parts, d)) : nullptr;
  p.mask = kept_mask;
  p.max_seq_len = max_seq_len;
  p.B = B;
  p.Q = Q;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.cap = cap;
  p.nb_max = nb_max;
  p.n_splits = ns;
  p.split_parts = parts;
  p.waves = ns > 0 ? ffd::waves_for(B, Hq, ns) : 4;
  p.split_blocks = split_blocks;
  p.sink = sink_blocks;
  p.local = local_blocks;
  p.pm_sink_local = pseudo_max != FFD_PSEUDO_MAX_SPLIT;
  p.pm_with_split = pseudo_max == FFD_PSEUDO_MAX_BOTH;
  p.delta = delta;
  p.sm_scale = sm_scale;
  return FFD_OK;
}

ffd_status check_out_dtype(const char* fn, int out_dtype) {
  if (out_dtype != FFD_OUT_BF16 && out_dtype != FFD_OUT_F32)
    return fail(FFD_ERR_INVALID_ARG, "%s: unknown out_dtype %d", fn, out_dtype);
  return FFD_OK;
}

ffd_status check_out_ptrs(const char* fn, int B, void* out, float* lse) {
  if (B > 0 && (!out || !lse)) return fail(FFD_ERR_INVALID_ARG, "%s: null out/lse", fn);
  return FFD_OK;
}

ffd_status launch(const char* fn, const ffd::DecodeParams& p, int d, int G, bool dense, ffd::Stage stage,
                  void* stream) {
  if (p.B == 0) return ok();
  hipError_t e = ffd::launch_decode(p, d, G, dense, stage, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ffd_status ffd_decode(const void* q, const void* k, const void* v, const uint8_t* kq, const float* kscale,
                      const int32_t* seq_lens, int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                      int block_size, float delta, int sink_blocks, int local_blocks, int pseudo_max,
                      int split_blocks, float sm_scale, void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                      void* workspace, size_t workspace_bytes, void* stream) {
  ffd::DecodeParams p;
  int G;
  bool dense;
  ffd_status st = check_out_dtype("ffd_decode", out_dtype);
  if (st != FFD_OK) return st;
  st = prepare_decode("ffd_decode", q, k, v, kq, kscale, seq_lens, max_seq_len, B, 1, Hq, Hkv, d, cap, block_size,
                      delta, sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale, kept_mask, workspace,
                      workspace_bytes, nullptr, 0, 0, p, G, dense);
  if (st != FFD_OK) return st;
  st = check_out_ptrs("ffd_decode", B, out, lse);
  if (st != FFD_OK) return st;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  return launch("ffd_decode", p, d, G, dense, ffd::Stage::kBoth, stream);
}

ffd_status ffd_decode_multi(const void* q, const void* k, const void* v, const uint8_t* kq, const float* kscale,
                            const int32_t* seq_lens, int max_seq_len, int B, int Q, int Hq, int Hkv, int d, int cap,
                            int block_size, float delta, int sink_blocks, int local_blocks, int pseudo_max,
                            int split_blocks, float sm_scale, void* out, int out_dtype, float* lse,
                            uint8_t* kept_mask, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "ffd_decode_multi";
  ffd::DecodeParams p;
  int G;
  bool dense;
  ffd_status st = check_out_dtype(fn, out_dtype);
  if (st != FFD_OK) return st;
  st = prepare_decode(fn, q, k, v, kq, kscale, seq_lens, max_seq_len, B, Q, Hq, Hkv, d, cap, block_size, delta,
                      sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale, kept_mask, workspace,
                      workspace_bytes, nullptr, 0, 0, p, G, dense);
  if (st != FFD_OK) return st;
  st = check_out_ptrs(fn, B, out, lse);
  if (st != FFD_OK) return st;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  return launch(fn, p, d, G, dense, ffd::Stage::kBoth, stream);
}

}  // extern "C"

namespace {

// ffd_decode_paged and ffd_decode_paged_multi: the block-table path for Q
// query tokens per sequence (Q = 1: single-token decode).
ffd_status decode_paged(const char* fn, const void* q, const void* k_pages, const void* v_pages,
                        const uint8_t* kq_pages, const float* kscale_pages, const int32_t* block_table,
                        int table_stride, int num_pages, const int32_t* seq_lens, int max_seq_len, int B, int Q,
                        int Hq, int Hkv, int d, int block_size, float delta, int sink_blocks, int local_blocks,
                        int pseudo_max, int split_blocks, float sm_scale, void* out, int out_dtype, float* lse,
                        uint8_t* kept_mask, void* workspace, size_t workspace_bytes, void* stream) {
  if (max_seq_len > 0 && B > 0 && !block_table) return fail(FFD_ERR_INVALID_ARG, "%s: null block_table", fn);
  ffd::DecodeParams p;
  int G;
  bool dense;
  ffd_status st = check_out_dtype(fn, out_dtype);
  if (st != FFD_OK) return st;
  const int32_t* table = (max_seq_len > 0 && B > 0) ? block_table : nullptr;
  st = prepare_decode(fn, q, k_pages, v_pages, kq_pages, kscale_pages, seq_lens, max_seq_len, B, Q, Hq, Hkv, d,
                      max_seq_len, block_size, delta, sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale,
                      kept_mask, workspace, workspace_bytes, table, table_stride, num_pages, p, G, dense);
  if (st != FFD_OK) return st;
  st = check_out_ptrs(fn, B, out, lse);
  if (st != FFD_OK) return st;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  return launch(fn, p, d, G, dense, ffd::Stage::kBoth, stream);
}

}  // namespace

extern "C" {

ffd_status ffd_decode_paged(const void* q, const void* k_pages, const void* v_pages, const uint8_t* kq_pages,
                            const float* kscale_pages, const int32_t* block_table, int table_stride, int num_pages,
                            const int32_t* seq_lens, int max_seq_len, int B, int Hq, int Hkv, int d,
                            int block_size, float delta, int sink_blocks, int local_blocks, int pseudo_max,
                            int split_blocks, float sm_scale, void* out, int out_dtype, float* lse,
                            uint8_t* kept_mask, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged("ffd_decode_paged", q, k_pages, v_pages, kq_pages, kscale_pages, block_table, table_stride,
                      num_pages, seq_lens, max_seq_len, B, 1, Hq, Hkv, d, block_size, delta, sink_blocks,
                      local_blocks, pseudo_max, split_blocks, sm_scale, out, out_dtype, lse, kept_mask, workspace,
                      workspace_bytes, stream);
}

ffd_status ffd_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages, const uint8_t* kq_pages,
                                  const float* kscale_pages, const int32_t* block_table, int table_stride,
                                  int num_pages, const int32_t* seq_lens, int max_seq_len, int B, int Q, int Hq,
                                  int Hkv, int d, int block_size, float delta, int sink_blocks, int local_blocks,
                                  int pseudo_max, int split_blocks, float sm_scale, void* out, int out_dtype,
                                  float* lse, uint8_t* kept_mask, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return decode_paged("ffd_decode_paged_multi", q, k_pages, v_pages, kq_pages, kscale_pages, block_table,
                      table_stride, num_pages, seq_lens, max_seq_len, B, Q, Hq, Hkv, d, block_size, delta,
                      sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale, out, out_dtype, lse, kept_mask,
                      workspace, workspace_bytes, stream);
}

ffd_status ffd_decode_thumb(const void* q, const uint8_t* k2, const float* k2scale, const int8_t* kr,
                            const float* krscale, const void* v, const int32_t* seq_lens, int max_seq_len, int B,
                            int Hq, int Hkv, int d, int cap, int block_size, float delta, int sink_blocks,
                            int local_blocks, int pseudo_max, int split_blocks, float sm_scale, void* out,
                            int out_dtype, float* lse, uint8_t* kept_mask, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const char* fn = "ffd_decode_thumb";
  ffd::DecodeParams p;
  int G;
  bool dense;
  ffd_status st = check_out_dtype(fn, out_dtype);
  if (st != FFD_OK) return st;
  if (B > 0 && max_seq_len > 0 && (!k2 || !k2scale || !kr || !krscale))
    return fail(FFD_ERR_INVALID_ARG, "%s: null thumbnail/residual pointer", fn);
  if (!aligned16(k2) || !aligned16(kr)) return fail(FFD_ERR_INVALID_ARG, "%s: k2 and kr must be 16-byte aligned", fn);
  // the thumbnail codes stand in for the int4 sketch and K in the shared checks
  st = prepare_decode(fn, q, v, v, k2, k2scale, seq_lens, max_seq_len, B, 1, Hq, Hkv, d, cap, block_size, delta,
                      sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale, kept_mask, workspace,
                      workspace_bytes, nullptr, 0, 0, p, G, dense);
  if (st != FFD_OK) return st;
  st = check_out_ptrs(fn, B, out, lse);
  if (st != FFD_OK) return st;
  p.k = nullptr;
  p.kq = nullptr;
  p.kscale = nullptr;
  p.k2 = k2;
  p.k2scale = k2scale;
  p.kr = kr;
  p.krscale = krscale;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  if (p.B == 0) return ok();
  hipError_t e = ffd::launch_decode(p, d, G, dense, ffd::Stage::kBoth, static_cast<hipStream_t>(stream), true);
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

ffd_status ffd_decode_partials(const void* q, const void* k, const void* v, const uint8_t* kq,
                               const float* kscale, const int32_t* seq_lens, int max_seq_len, int B, int Hq,
                               int Hkv, int d, int cap, int block_size, float delta, int sink_blocks,
                               int local_blocks, int pseudo_max, int split_blocks, float sm_scale,
                               uint8_t* kept_mask, void* workspace, size_t workspace_bytes, void* stream) {
  ffd::DecodeParams p;
  int G;
  bool dense;
  ffd_status st = prepare_decode("ffd_decode_partials", q, k, v, kq, kscale, seq_lens, max_seq_len, B, 1, Hq, Hkv, d,
                                 cap, block_size, delta, sink_blocks, local_blocks, pseudo_max, split_blocks,
                                 sm_scale, kept_mask, workspace, workspace_bytes, nullptr, 0, 0, p, G, dense);
  if (st != FFD_OK) return st;
  return launch("ffd_decode_partials", p, d, G, dense, ffd::Stage::kPartials, stream);
}

ffd_status ffd_combine(const int32_t* seq_lens, int max_seq_len, int B, int Hq, int d, int block_size,
                       int split_blocks, const void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                       float* lse, void* stream) {
  const char* fn = "ffd_combine";
  if (B < 0 || Hq <= 0 || max_seq_len < 0)
    return fail(FFD_ERR_INVALID_ARG, "%s: bad sizes (B=%d Hq=%d max_seq_len=%d)", fn, B, Hq, max_seq_len);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "%s: d must be positive and even (d=%d)", fn, d);
  if (split_blocks < 1) return fail(FFD_ERR_INVALID_ARG, "%s: split_blocks must be >= 1 (got %d)", fn, split_blocks);
  if (block_size <= 0) return fail(FFD_ERR_INVALID_ARG, "%s: block_size must be positive (got %d)", fn, block_size);
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "%s: d=%d not supported (64, 128)", fn, d);
  if (block_size != ffd::kBlockSize) return fail(FFD_ERR_UNSUPPORTED, "%s: block_size=%d not supported (64)", fn, block_size);
  if (split_blocks > ffd::kMaxSplit)
    return fail(FFD_ERR_UNSUPPORTED, "%s: split_blocks=%d not supported (<= %d)", fn, split_blocks, ffd::kMaxSplit);
  if (B > 65535 || Hq > 65535) return fail(FFD_ERR_UNSUPPORTED, "%s: B, Hq must be <= 65535", fn);
  if (max_seq_len > kMaxTokens)
    return fail(FFD_ERR_UNSUPPORTED, "%s: max_seq_len=%d above 2^30 tokens", fn, max_seq_len);
  ffd_status st = check_out_dtype(fn, out_dtype);
  if (st != FFD_OK) return st;
  st = check_out_ptrs(fn, B, out, lse);
  if (st != FFD_OK) return st;
  if (B > 0 && !seq_lens) return fail(FFD_ERR_INVALID_ARG, "%s: null seq_lens", fn);
  const int ns = max_seq_len > 0 ? n_splits_for(max_seq_len, split_blocks) : 0;
  const int parts = ns > 0 ? ffd::split_parts_for(B, Hq, ns) : 1;
  const size_t need = (B > 0 && max_seq_len > 0)
                          ? ffd::ws_opart_bytes(B, Hq, ns * parts, d) + ffd::ws_lse_bytes(B, Hq, ns * parts)
                          : 0;
  if (need > 0) {
    if (!workspace) return fail(FFD_ERR_INVALID_ARG, "%s: null workspace", fn);
    if (workspace_bytes < need)
      return fail(FFD_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % ffd::kWsAlign)
      return fail(FFD_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  }
  ffd::DecodeParams p{};
  const char* ws = static_cast<const char*>(workspace);
  p.o_part = need ? reinterpret_cast<float*>(const_cast<char*>(ws)) : nullptr;
  p.lse_part =
      need ? reinterpret_cast<float*>(const_cast<char*>(ws) + ffd::ws_opart_bytes(B, Hq, ns * parts, d)) : nullptr;
  p.seq_lens = seq_lens;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  p.max_seq_len = max_seq_len;
  p.B = B;
  p.Q = 1;
  p.Hq = Hq;
  p.Hkv = 1;
  p.nb_max = nb_max_for(max_seq_len);
  p.n_splits = ns;
  p.split_parts = parts;
  p.waves = ns > 0 ? ffd::waves_for(B, Hq, ns) : 4;
  p.split_blocks = split_blocks;
  return launch(fn, p, d, 1, false, ffd::Stage::kCombine, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// ffd_decode_noalloc: ffd_decode with the split partials in a static device
// array instead of a caller workspace.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = FFD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The partials of ffd_decode_noalloc. Every device the library's code object
// is loaded on holds its own copy until the process ends. In host code this
// name is a host-side stand-in, not a device address: kernels get the address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, looked up on its first call

ffd_status scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FFD_ERR_UNSUPPORTED, "%s: device %d outside the %d devices the scratch table holds", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(FFD_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FFD_OK;
}

}  // namespace

extern "C" {

ffd_status ffd_decode_noalloc(const void* q, const void* k, const void* v, const uint8_t* kq, const float* kscale,
                              const int32_t* seq_lens, int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                              int block_size, float delta, int sink_blocks, int local_blocks, int pseudo_max,
                              int split_blocks, float sm_scale, void* out, int out_dtype, float* lse,
                              uint8_t* kept_mask, void* stream) {
  const char* fn = "ffd_decode_noalloc";
  ffd_status st = check_out_dtype(fn, out_dtype);
  if (st != FFD_OK) return st;
  const size_t need = ffd_decode_workspace_bytes(B, Hq, d, max_seq_len, block_size, split_blocks);
  if (need > kScratchBytes)
    return fail(FFD_ERR_WORKSPACE,
                "%s: these sizes need %zu bytes of partials, above the %zu bytes of the static scratch array "
                "(use ffd_decode with a workspace)",
                fn, need, kScratchBytes);
  // Validate everything on the host first, against a stand-in workspace
  // address (aligned, never dereferenced), then carve the real array.
  char* const stand_in = reinterpret_cast<char*>(ffd::kWsAlign);
  ffd::DecodeParams p;
  int G;
  bool dense;
  st = prepare_decode(fn, q, k, v, kq, kscale, seq_lens, max_seq_len, B, 1, Hq, Hkv, d, cap, block_size, delta,
                      sink_blocks, local_blocks, pseudo_max, split_blocks, sm_scale, kept_mask, stand_in,
                      kScratchBytes, nullptr, 0, 0, p, G, dense);
  if (st != FFD_OK) return st;
  st = check_out_ptrs(fn, B, out, lse);
  if (st != FFD_OK) return st;
  if (p.o_part != nullptr) {
    void* base = nullptr;
    st = scratch_for_current_device(fn, &base);
    if (st != FFD_OK) return st;
    char* ws = static_cast<char*>(base);
    p.lse_part = reinterpret_cast<float*>(ws + (reinterpret_cast<char*>(p.lse_part) - stand_in));
    p.o_part = reinterpret_cast<float*>(ws);
  }
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  return launch(fn, p, d, G, dense, ffd::Stage::kBoth, stream);
}

}  // extern "C"
