/*
 * ffd.h -- C ABI of the FFD sparse decode-attention library (MI355X, gfx950).
 *
 * The method: "Faster Than Flash: Exploiting Attention Sparsity for Efficient
 * Long-Context Decoding" (FFD). Cited below as
 *   [TS]  the technical-summary page (gist.science) of that paper, by its
 *         Methodology sections 1-3;
 *   [AB]  the English abstract / "Key Innovations of FFD" on the
 *         insight.aitobox.com blog page about the same paper.
 *
 * Conventions shared by every entry point:
 *   - Every tensor argument is a DEVICE pointer to contiguous row-major
 *     memory that the caller allocated and owns. The library allocates
 *     nothing, keeps no state except a per-thread error string (and the
 *     static scratch array of ffd_decode_noalloc, one per device), and never
 *     synchronises: work is enqueued on `stream` (a hipStream_t; NULL means
 *     the default stream) and the call returns at once.
 *   - bf16 tensors hold IEEE bfloat16 values (raw 16-bit patterns).
 *   - A non-zero ffd_status means nothing was enqueued (argument errors) or
 *     a launch failed (FFD_ERR_HIP); ffd_last_error() then describes it.
 *   - Device-side values (sequence lengths, positions) are not validated;
 *     out-of-range ones are clamped as documented per call.
 *   - Outputs must not alias inputs.
 */
#ifndef FFD_H
#define FFD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: the first release; 2: adds ffd_decode_noalloc (every version-1 call is
 * unchanged). */
#define FFD_ABI_VERSION 2

typedef enum {
  FFD_OK = 0,
  FFD_ERR_INVALID_ARG = 1, /* null pointer, inconsistent shape, bad scalar, misaligned pointer */
  FFD_ERR_UNSUPPORTED = 2, /* valid request the kernels do not implement (d, block size, G, G*Q, S, sink+local,
                              more than 2^30 tokens in max_seq_len, cap or max_span) */
  FFD_ERR_WORKSPACE = 3,   /* workspace smaller than ffd_decode_workspace_bytes() */
  FFD_ERR_HIP = 4          /* a HIP launch error */
} ffd_status;

typedef enum { FFD_OUT_BF16 = 0, FFD_OUT_F32 = 1 } ffd_out_dtype;
/* The same values under the names a plain "dtype" enum would use. */
typedef enum { FFD_BF16 = FFD_OUT_BF16, FFD_F32 = FFD_OUT_F32 } ffd_dtype;

/* How the pseudo-max m~ of the Top-δ rule is estimated ([TS] Methodology 2). */
typedef enum {
  FFD_PSEUDO_MAX_SPLIT = 0,      /* max block score within the block's split (one workgroup) */
  FFD_PSEUDO_MAX_SINK_LOCAL = 1, /* max block score over the sink and local blocks ([TS]
                                    Methodology 2 "Pseudo-Max Approximation", 3 "Pseudo-max
                                    Estimation"); the kept set does not depend on split_blocks */
  FFD_PSEUDO_MAX_BOTH = 2        /* per split, the larger of the two above: a block is kept iff
                                    both other modes keep it (a low sink/local estimate cannot
                                    widen a split's kept set beyond its own maximum) */
} ffd_pseudo_max;

/* Version of this ABI (FFD_ABI_VERSION). */
int ffd_abi_version(void);

/* Message of the last failed call on this thread ("" if none). Host memory
 * owned by the library, valid until the next library call on the thread. */
const char* ffd_last_error(void);

/*
 * ffd_quantize_kv -- build or append the low-bit key sketch that the scan
 * reads ([TS] Methodology 1: keys are kept in a low-bit form next to the
 * full-precision cache and scanned instead of metadata indices; [AB]
 * "content-aware scanning via low-bit quantization").
 *
 * For every sequence b, kv head j and token t in [pos_begin[b], pos_end[b])
 * (clamped to [0, cap)), with k = K[b, j, t, :]:
 *   amax = max_i |k_i|;  scale = fl32(amax / 7);  inv = fl32(7 / amax)
 *   code_i = clamp(round_half_even(fl32(k_i * inv)), -7, 7)
 *   (amax < 2^-125, zero included: scale = 0 and every code 0, since 7/amax
 *   would overflow)
 * and stores kscale[b, j, t] = scale and the codes as two's-complement
 * nibbles, element 2i in the low nibble of byte i of kq[b, j, t, :].
 * Tokens outside the ranges are not touched.
 *
 *   k         bf16  [B, Hkv, cap, d]      input
 *   kq        uint8 [B, Hkv, cap, d/2]    output (written for the range only)
 *   kscale    f32   [B, Hkv, cap]         output (written for the range only)
 *   pos_begin int32 [B]                   device; first token to (re)quantise
 *   pos_end   int32 [B]                   device; one past the last
 *   max_span  host int >= max_b (pos_end[b] - pos_begin[b]); sizes the grid,
 *             tokens beyond pos_begin[b] + max_span are not processed
 * Build a prefix with begin = 0, end = len; append one decoded token with
 * begin = len - 1, end = len (after writing its bf16 K/V row). Both give the
 * same bytes for the same token.
 * Supported: d in {64, 128}; cap, max_span <= 2^30. kq and k must be 16-byte
 * aligned.
 */
ffd_status ffd_quantize_kv(const void* k, uint8_t* kq, float* kscale,
                           const int32_t* pos_begin, const int32_t* pos_end,
                           int B, int Hkv, int cap, int d, int max_span, void* stream);

/*
 * ffd_quantize_kv_paged -- ffd_quantize_kv for a paged cache. A page holds one
 * 64-token block of every kv head: K pages bf16 [num_pages, Hkv, 64, d], kq
 * pages uint8 [num_pages, Hkv, 64, d/2], kscale pages f32 [num_pages, Hkv,
 * 64]. Token t of sequence b lives in page block_table[b * table_stride + t/64]
 * (int32, device), row t % 64. Tokens at or past table_stride * 64 are not
 * processed; page numbers outside [0, num_pages) are clamped (never fault).
 * table_stride <= 2^24.
 * Same arithmetic and output bytes as ffd_quantize_kv.
 */
ffd_status ffd_quantize_kv_paged(const void* k_pages, uint8_t* kq_pages, float* kscale_pages,
                                 const int32_t* block_table, int table_stride, int num_pages,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int d,
                                 int max_span, void* stream);

/*
 * ffd_quantize_kv_thumb -- the pages' own key storage ([TS] Methodology 1: a
 * 2-bit "thumbnail" of every key for the scan plus an 8-bit residual that
 * reconstructs the key for the refinement). The formats are this library's:
 * per token and kv head, with k = K[b, j, t, :] and amax = max|k_i|:
 *   t = fl32(amax / 3); x_i = fl32(k_i * fl32(3 / amax));
 *   u_i = clamp(round_half_even(fl32(fl32(x_i + 3) * 0.5)), 0, 3)
 *     (2-bit code; the level is (2u - 3) * t, one of -3t, -t, t, 3t)
 *   r_i = fl32(k_i - fl32((2u_i - 3) * t)); s8 = fl32(amax_r / 127);
 *   r8_i = clamp(round_half_even(fl32(r_i * fl32(127 / amax_r))), -127, 127)
 *   (amax < 2^-125: t = 0, u = r8 = 0, s8 = 0; amax_r < 2^-120: s8 = 0, r8 = 0)
 * and the reconstructed key is K^ = (2u - 3) t + s8 r8.
 *   k        bf16 [B, Hkv, cap, d]     input
 *   k2       uint8 [B, Hkv, cap, d/4]  codes, element 4i + c in bits 2c of byte i
 *   k2scale  f32 [B, Hkv, cap]         t
 *   kr       int8 [B, Hkv, cap, d]     r8
 *   krscale  f32 [B, Hkv, cap]         s8
 * Other arguments and conventions as ffd_quantize_kv. d in {64, 128}.
 */
ffd_status ffd_quantize_kv_thumb(const void* k, uint8_t* k2, float* k2scale, int8_t* kr, float* krscale,
                                 const int32_t* pos_begin, const int32_t* pos_end, int B, int Hkv, int cap, int d,
                                 int max_span, void* stream);

/* Bytes of scratch that ffd_decode, ffd_decode_partials and ffd_combine need
 * for these sizes: per-split partial outputs and log-sum-exps (fp32). 0 for
 * unsupported sizes. */
size_t ffd_decode_workspace_bytes(int B, int Hq, int d, int max_seq_len, int block_size,
                                  int split_blocks);

/*
 * ffd_decode -- one FFD decode step: single-token attention of every query
 * head over its sequence's KV cache, with the block selector and the
 * attention computer fused ([TS] Methodology 3, "Fused Kernel": pseudo-max,
 * Top-δ selection and fine-grained refinement in one kernel; [AB] "fully
 * fused kernel").
 *
 * Query head h reads kv head h / (Hq / Hkv). For sequence b let
 * L = clamp(seq_lens[b], 0, max_seq_len), NB = ceil(L / block_size). The
 * blocks of a sequence are cut into splits of `split_blocks` consecutive
 * blocks, one workgroup each. Per query head:
 *   1. The query is quantised to int8 (scale sq = fl32(amax/127), codes
 *      clamp(rne(fl32(q_i * fl32(127/amax))), +-127)), cq = fl32(sq * sm_scale);
 *      amax < 2^-120 (zero included) gives all-zero codes and cq = 0.
 *   2. Scan ([TS] Methodology 3, "Top-δ Selection"): each valid token's
 *      tentative score is fl32(float(dot) * fl32(kscale_t * cq)), dot being
 *      the exact integer dot of the int8 query with the int4 codes; a block's
 *      score is the max over its valid tokens.
 *   3. Top-δ ([TS] Methodology 2, "Mechanism"): block j is kept iff
 *      score_j >= fl32(m~ - delta), or j < sink_blocks, or j >= NB -
 *      local_blocks. m~ is the max block score in j's split
 *      (FFD_PSEUDO_MAX_SPLIT), over the sink and local blocks
 *      (FFD_PSEUDO_MAX_SINK_LOCAL), or the larger of the two
 *      (FFD_PSEUDO_MAX_BOTH). δ is in natural-log logit units ([TS]
 *      Methodology 2, "Adaptivity").
 *   4. Refinement ([TS] Methodology 3, "Fine-Grained Refinement"): exact
 *      softmax attention (logit = sm_scale * q.k on the bf16 values, fp32
 *      accumulation) over the valid tokens of the kept blocks; per-split
 *      partials are merged by a log-sum-exp combine.
 * delta = +INFINITY selects the dense flash-decoding path: no scan, every
 * valid block kept; kq and kscale may then be NULL.
 *
 *   q          bf16 [B, Hq, d]
 *   k, v       bf16 [B, Hkv, cap, d]            rows >= L are never read
 *   kq, kscale from ffd_quantize_kv over every valid token
 *   seq_lens   int32 [B], device
 *   max_seq_len host; bounds every L and sizes the grid and the mask
 *   delta      >= 0 (fp32), +INFINITY allowed
 *   sink_blocks, local_blocks >= 0
 *   pseudo_max FFD_PSEUDO_MAX_SPLIT, FFD_PSEUDO_MAX_SINK_LOCAL or
 *              FFD_PSEUDO_MAX_BOTH (the last two need
 *              1 <= sink_blocks + local_blocks <= 64)
 *   split_blocks in [1, 64]; with FFD_PSEUDO_MAX_SPLIT part of the semantics
 *              (the kept set depends on it); otherwise only a work partition
 *   sm_scale   > 0 and finite (commonly fl32(1/sqrt(d)))
 *   out        [B, Hq, d], bf16 (round half to even) or f32 per out_dtype
 *   lse        f32 [B, Hq], natural log of the softmax normaliser over the
 *              kept tokens of that head
 *   kept_mask  uint8 [B, Hq, ceil(max_seq_len / block_size)] or NULL;
 *              1 = kept, 0 = dropped or past NB
 *   workspace  >= ffd_decode_workspace_bytes(B, Hq, d, max_seq_len,
 *              block_size, split_blocks) bytes, 256-byte aligned, no
 *              initialisation needed. Calls that share a workspace must not
 *              overlap (calls on one stream never do).
 * A sequence with L == 0 gives out = 0, lse = -INFINITY and a zero mask row.
 * With FFD_PSEUDO_MAX_SINK_LOCAL a split may keep no block of a head; its
 * partial then has lse = -INFINITY and weight 0 in the combine.
 * Supported: d in {64, 128}, block_size == 64, Hq / Hkv in {1, 2, 4, 8},
 * max_seq_len <= 2^30. q, k, v, kq must be 16-byte aligned. Equivalent to
 * ffd_decode_partials
 * followed by ffd_combine on the same stream.
 */
ffd_status ffd_decode(const void* q, const void* k, const void* v,
                      const uint8_t* kq, const float* kscale, const int32_t* seq_lens,
                      int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                      int block_size, float delta, int sink_blocks, int local_blocks,
                      int pseudo_max, int split_blocks, float sm_scale,
                      void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffd_decode_multi -- Q query tokens per sequence in one call (a speculative
 * verify step, or several new tokens at once). The pages describe one query
 * token per decode step ([TS] Problem Statement; Methodology 3); this call
 * applies the same step to each of Q tokens whose keys and values are already
 * in the cache: token i of sequence b sits at position seq_lens[b] - Q + i and
 * sees the rows before and at its own position, so its result is exactly that
 * of ffd_decode with seq_lens[b] - Q + 1 + i in place of seq_lens[b] (own
 * scores, pseudo-max, Top-δ set, sink/local range and attention; a length
 * <= 0 gives out 0, lse -INFINITY and a zero mask row). The Q tokens share
 * one pass over the int4 sketch (their scores are one small integer matrix
 * product per tile, [TS] Significance: scanning is cheap compute) and one
 * read of the blocks any of them keeps.
 *   q          bf16 [B, Q, Hq, d]
 *   out        [B, Q, Hq, d];  lse f32 [B, Q, Hq]
 *   kept_mask  uint8 [B, Q, Hq, ceil(max_seq_len / block_size)] or NULL
 *   workspace  >= ffd_decode_multi_workspace_bytes(B, Q, Hq, d, max_seq_len,
 *              block_size, split_blocks) bytes, 256-byte aligned
 * Everything else as ffd_decode. Supported: Q >= 1 with (Hq / Hkv) * Q <= 16;
 * with FFD_PSEUDO_MAX_SINK_LOCAL or FFD_PSEUDO_MAX_BOTH, sink_blocks + local_blocks +
 * ceil((Q - 1) / 64) <= 64. FFD_ERR_UNSUPPORTED otherwise. Q == 1 is ffd_decode.
 */
ffd_status ffd_decode_multi(const void* q, const void* k, const void* v,
                            const uint8_t* kq, const float* kscale, const int32_t* seq_lens,
                            int max_seq_len, int B, int Q, int Hq, int Hkv, int d, int cap,
                            int block_size, float delta, int sink_blocks, int local_blocks,
                            int pseudo_max, int split_blocks, float sm_scale,
                            void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for ffd_decode_multi (the partials of Q * Hq query rows);
 * 0 for unsupported sizes. */
size_t ffd_decode_multi_workspace_bytes(int B, int Q, int Hq, int d, int max_seq_len,
                                        int block_size, int split_blocks);

/*
 * ffd_decode_paged -- ffd_decode on a paged KV cache (a block table instead of
 * one contiguous cache per sequence, as serving engines keep it). Pages are laid
 * out as for ffd_quantize_kv_paged (K and V pages bf16 [num_pages, Hkv, 64, d]);
 * block j of sequence b is page block_table[b * table_stride + j], for
 * j < ceil(L / 64); table_stride >= ceil(max_seq_len / 64). num_pages is the
 * pool's page count (num_pages * Hkv <= 2^31 - 1, else FFD_ERR_UNSUPPORTED);
 * page numbers outside [0, num_pages) are clamped. Same semantics, results and
 * workspace as ffd_decode: a paged cache holding the same rows gives
 * bit-identical outputs.
 */
ffd_status ffd_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const uint8_t* kq_pages, const float* kscale_pages,
                            const int32_t* block_table, int table_stride, int num_pages,
                            const int32_t* seq_lens, int max_seq_len, int B, int Hq, int Hkv, int d,
                            int block_size, float delta, int sink_blocks, int local_blocks,
                            int pseudo_max, int split_blocks, float sm_scale,
                            void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffd_decode_paged_multi -- ffd_decode_multi on a paged KV cache: Q query
 * tokens per sequence (q [B, Q, Hq, d], outputs [B, Q, Hq, ...]) with the
 * semantics of ffd_decode_multi, over pages laid out and addressed as for
 * ffd_decode_paged. Workspace: ffd_decode_multi_workspace_bytes. A paged
 * cache holding the same rows gives outputs bit-identical to
 * ffd_decode_multi. Supported as ffd_decode_multi.
 */
ffd_status ffd_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages,
                                  const uint8_t* kq_pages, const float* kscale_pages,
                                  const int32_t* block_table, int table_stride, int num_pages,
                                  const int32_t* seq_lens, int max_seq_len, int B, int Q, int Hq, int Hkv,
                                  int d, int block_size, float delta, int sink_blocks, int local_blocks,
                                  int pseudo_max, int split_blocks, float sm_scale,
                                  void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffd_decode_thumb -- ffd_decode over the thumbnail + residual key storage of
 * ffd_quantize_kv_thumb (no bf16 K is read). The scan uses the thumbnail:
 * dot = sum qc_i (2u_i - 3) (exact integer), score fl32(float(dot) *
 * fl32(t * cq)); selection as in ffd_decode; the refinement is exact softmax
 * attention over the reconstructed keys, logit sm_scale * q.K^ with K^ =
 * (2u - 3) t + s8 r8, and the bf16 V. Same outputs, workspace and errors as
 * ffd_decode (kq/kscale/k replaced by k2, k2scale, kr, krscale).
 */
ffd_status ffd_decode_thumb(const void* q, const uint8_t* k2, const float* k2scale, const int8_t* kr,
                            const float* krscale, const void* v, const int32_t* seq_lens, int max_seq_len,
                            int B, int Hq, int Hkv, int d, int cap, int block_size, float delta,
                            int sink_blocks, int local_blocks, int pseudo_max, int split_blocks,
                            float sm_scale, void* out, int out_dtype, float* lse, uint8_t* kept_mask,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffd_decode_partials -- the first half of ffd_decode: the fused scan ->
 * Top-δ select -> attend kernel, one workgroup per (sequence, kv head,
 * split) ([TS] Methodology 3, "Fused Kernel"). Same arguments and semantics
 * as ffd_decode (the kept_mask is written here); instead of the final output
 * it leaves every split's partial results in the workspace:
 *   n_splits = ceil(ceil(max_seq_len / block_size) / split_blocks)
 *   units    = B * Hq * n_splits
 *   P        = clamp(floor(1024 / units), 1, 4) if units <= 1024, else 1:
 *              workgroups per split when the grid alone would leave the
 *              chip idle; each scans and selects the whole split (one kept
 *              set) and attends a disjoint share of its kept blocks (the
 *              P * waves waves of the split take them round-robin)
 *   o_part   f32 [B, Hq, n_splits, P, d] at byte offset 0: each part's
 *            attention output, normalised over the kept tokens it attended
 *   lse_part f32 [B, Hq, n_splits, P] at byte offset
 *            round_up(B*Hq*n_splits*P*d*4, 256): natural-log normaliser
 *            (-INFINITY for a part that attended nothing)
 * Only splits s < ceil(NB_b / split_blocks) of sequence b are written.
 * Combining the partials of disjoint token sets by log-sum-exp is exact,
 * which is what lets a sequence be split across workgroups (and, by the
 * same merge, across devices) without any global maximum.
 */
ffd_status ffd_decode_partials(const void* q, const void* k, const void* v,
                               const uint8_t* kq, const float* kscale, const int32_t* seq_lens,
                               int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                               int block_size, float delta, int sink_blocks, int local_blocks,
                               int pseudo_max, int split_blocks, float sm_scale, uint8_t* kept_mask,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffd_combine -- the second half of ffd_decode: per (sequence, query head),
 *   lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s
 * over the splits written by ffd_decode_partials (same seq_lens,
 * max_seq_len, block_size and split_blocks; workspace laid out as described
 * there). A sequence with L == 0 gives out = 0 and lse = -INFINITY.
 * Supported: d in {64, 128}, block_size == 64, split_blocks in [1, 64],
 * max_seq_len <= 2^30.
 */
ffd_status ffd_combine(const int32_t* seq_lens, int max_seq_len, int B, int Hq, int d,
                       int block_size, int split_blocks, const void* workspace,
                       size_t workspace_bytes, void* out, int out_dtype, float* lse,
                       void* stream);

/*
 * ffd_decode_noalloc -- ffd_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments as ffd_decode minus the workspace; same
 * kernels, semantics and results. The per-split partials go to a static
 * device array of FFD_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it is loaded on until the process ends; the call allocates nothing.
 *   - Sizes whose partials need more (ffd_decode_workspace_bytes above
 *     FFD_NOALLOC_SCRATCH_BYTES) give FFD_ERR_WORKSPACE and enqueue nothing.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's partials (nothing in it needs clearing). Calls that overlap
 *     on one device -- on different streams with no ordering between them --
 *     race on it and give wrong results; calls on one stream never overlap.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress, no allocation); make that first call outside
 *     stream capture.
 */
#define FFD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

ffd_status ffd_decode_noalloc(const void* q, const void* k, const void* v,
                              const uint8_t* kq, const float* kscale, const int32_t* seq_lens,
                              int max_seq_len, int B, int Hq, int Hkv, int d, int cap,
                              int block_size, float delta, int sink_blocks, int local_blocks,
                              int pseudo_max, int split_blocks, float sm_scale,
                              void* out, int out_dtype, float* lse, uint8_t* kept_mask, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FFD_H */
