// C-ABI layer: argument validation, dispatch, workspace carving, launch.
// Allocates nothing and never synchronises (safe inside stream capture).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "ffd.h"
#include "ffd_internal.h"

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

int n_splits_for(int max_seq_len, int split_blocks) {
  const int nb_max = (max_seq_len + ffd::kBlockSize - 1) / ffd::kBlockSize;
  return (nb_max + split_blocks - 1) / split_blocks;
}

}  // namespace

extern "C" {

int ffd_abi_version(void) { return FFD_ABI_VERSION; }

const char* ffd_last_error(void) { return g_err.c_str(); }

ffd_status ffd_quantize_kv(const void* k, uint8_t* kq, float* kscale, const int32_t* pos_begin,
                           const int32_t* pos_end, int B, int Hkv, int cap, int d, int max_span,
                           void* stream) {
  if (B < 0 || Hkv < 0 || cap < 0 || max_span < 0)
    return fail(FFD_ERR_INVALID_ARG, "ffd_quantize_kv: negative size (B=%d Hkv=%d cap=%d max_span=%d)", B, Hkv,
                cap, max_span);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "ffd_quantize_kv: d must be positive and even (d=%d)", d);
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "ffd_quantize_kv: d=%d not supported (64, 128)", d);
  if (B == 0 || Hkv == 0 || cap == 0 || max_span == 0) return ok();
  if (!k || !kq || !kscale || !pos_begin || !pos_end)
    return fail(FFD_ERR_INVALID_ARG, "ffd_quantize_kv: null pointer argument");
  if (!aligned16(k) || !aligned16(kq)) return fail(FFD_ERR_INVALID_ARG, "ffd_quantize_kv: k and kq must be 16-byte aligned");
  if (B > 65535 || Hkv > 65535) return fail(FFD_ERR_UNSUPPORTED, "ffd_quantize_kv: B and Hkv must be <= 65535");
  hipError_t e = ffd::launch_quantize_kv(static_cast<const uint16_t*>(k), kq, kscale, pos_begin, pos_end, B, Hkv,
                                         cap, d, max_span, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "ffd_quantize_kv: launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t ffd_decode_workspace_bytes(int B, int Hq, int d, int max_seq_len, int block_size, int split_blocks) {
  if (B <= 0 || Hq <= 0 || d <= 0 || max_seq_len <= 0 || block_size != ffd::kBlockSize || split_blocks < 1) return 0;
  const int ns = n_splits_for(max_seq_len, split_blocks);
  return ffd::ws_opart_bytes(B, Hq, ns, d) + ffd::ws_lse_bytes(B, Hq, ns);
}

ffd_status ffd_decode(const void* q, const void* k, const void* v, const uint8_t* kq, const float* kscale,
                      const int32_t* seq_lens, int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                      int block_size, float delta, int sink_blocks, int local_blocks, int split_blocks,
                      float sm_scale, void* out, int out_dtype, float* lse, uint8_t* kept_mask, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || cap < 0 || max_seq_len < 0)
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: bad sizes (B=%d Hq=%d Hkv=%d cap=%d max_seq_len=%d)", B, Hq, Hkv,
                cap, max_seq_len);
  if (Hq % Hkv) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d <= 0 || (d & 1)) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: d must be positive and even (d=%d)", d);
  if (cap < max_seq_len) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: cap=%d < max_seq_len=%d", cap, max_seq_len);
  if (isnan(delta) || delta < 0.f) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: delta must be >= 0 (got %g)", (double)delta);
  if (sink_blocks < 0 || local_blocks < 0)
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: sink/local must be >= 0 (%d, %d)", sink_blocks, local_blocks);
  if (split_blocks < 1) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: split_blocks must be >= 1 (got %d)", split_blocks);
  if (!(sm_scale > 0.f) || isinf(sm_scale))
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: sm_scale must be positive and finite (got %g)", (double)sm_scale);
  if (out_dtype != FFD_OUT_BF16 && out_dtype != FFD_OUT_F32)
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: unknown out_dtype %d", out_dtype);
  if (block_size <= 0) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: block_size must be positive (got %d)", block_size);
  const int G = Hq / Hkv;
  if (d != 64 && d != 128) return fail(FFD_ERR_UNSUPPORTED, "ffd_decode: d=%d not supported (64, 128)", d);
  if (block_size != ffd::kBlockSize) return fail(FFD_ERR_UNSUPPORTED, "ffd_decode: block_size=%d not supported (64)", block_size);
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(FFD_ERR_UNSUPPORTED, "ffd_decode: group size %d not supported (1, 2, 4, 8)", G);
  if (split_blocks > ffd::kMaxSplit)
    return fail(FFD_ERR_UNSUPPORTED, "ffd_decode: split_blocks=%d not supported (<= %d)", split_blocks, ffd::kMaxSplit);
  if (B == 0) return ok();
  if (B > 65535 || Hkv > 65535 || Hq > 65535) return fail(FFD_ERR_UNSUPPORTED, "ffd_decode: B, Hq, Hkv must be <= 65535");
  const bool dense = isinf(delta);
  if (!q || !seq_lens || !out || !lse) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: null q/seq_lens/out/lse");
  if (max_seq_len > 0 && (!k || !v)) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: null k/v");
  if (max_seq_len > 0 && !dense && (!kq || !kscale))
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: kq/kscale required unless delta is +inf");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kq))
    return fail(FFD_ERR_INVALID_ARG, "ffd_decode: q, k, v, kq must be 16-byte aligned");

  const int nb_max = (max_seq_len + ffd::kBlockSize - 1) / ffd::kBlockSize;
  const int ns = max_seq_len > 0 ? n_splits_for(max_seq_len, split_blocks) : 0;
  const size_t need = max_seq_len > 0 ? ffd::ws_opart_bytes(B, Hq, ns, d) + ffd::ws_lse_bytes(B, Hq, ns) : 0;
  if (need > 0) {
    if (!workspace) return fail(FFD_ERR_INVALID_ARG, "ffd_decode: null workspace");
    if (workspace_bytes < need)
      return fail(FFD_ERR_WORKSPACE, "ffd_decode: workspace %zu bytes < required %zu", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % ffd::kWsAlign)
      return fail(FFD_ERR_INVALID_ARG, "ffd_decode: workspace must be 256-byte aligned");
  }
  ffd::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kq = kq;
  p.kscale = kscale;
  p.seq_lens = seq_lens;
  char* ws = static_cast<char*>(workspace);
  p.o_part = need ? reinterpret_cast<float*>(ws) : nullptr;
  p.lse_part = need ? reinterpret_cast<float*>(ws + ffd::ws_opart_bytes(B, Hq, ns, d)) : nullptr;
  p.mask = kept_mask;
  p.out = out;
  p.lse = lse;
  p.out_f32 = out_dtype == FFD_OUT_F32;
  p.max_seq_len = max_seq_len;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.cap = cap;
  p.nb_max = nb_max;
  p.n_splits = ns;
  p.split_blocks = split_blocks;
  p.sink = sink_blocks;
  p.local = local_blocks;
  p.delta = delta;
  p.sm_scale = sm_scale;
  hipError_t e = ffd::launch_decode(p, d, G, dense, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FFD_ERR_HIP, "ffd_decode: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
