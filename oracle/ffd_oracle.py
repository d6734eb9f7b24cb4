"""CPU oracle for FFD sparse decode attention.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The library's product
path (HIP kernels behind the C ABI) never calls it, and it shares no code,
table or helper with that path.

What it computes, step by step, in the order of the method as the pages
describe it. Citations name the page and section:

* [TS] "Faster Than Flash: Exploiting Attention Sparsity for Efficient
  Long-Context Decoding" -- the technical-summary page (gist.science), its
  Methodology sections: 1 "Content-Aware Scanning via Low-Bit Quantization";
  2 "The Top-δ Selection Strategy" (Mechanism, Pseudo-Max Approximation,
  Adaptivity); 3 "Fused Kernel and System Optimization" (Top-δ Selection,
  Fine-Grained Refinement); and "Significance and Claims".
* [AB] the English abstract and "Key Innovations of FFD" list on the
  insight.aitobox.com blog page about the same paper.

Readings where the pages leave a step open (each one is a fixed design
choice of this library, applied identically by the HIP path):

* The scan sketch is int4 per key element, symmetric range [-7, 7], with one
  fp32 scale per token and kv head (the pages use 2-bit thumbnails plus 8-bit
  residuals, [TS] Methodology 1). The query is quantised to int8 in [-127, 127]
  with one fp32 scale per head, so a token's dot product is an exact integer.
* Rounding is round-half-to-even; clamping follows rounding. A zero row gets
  scale 0 and all-zero codes.
* A block's score is the maximum tentative score over its valid tokens
  ([TS] Methodology 3, "Top-δ Selection": blocks are filtered).
* The pseudo-max m~ of [TS] Methodology 2 has two modes. "split" (default):
  per query head, the maximum block score inside the split of
  ``split_blocks`` consecutive blocks that one workgroup owns; this needs no
  global reduction. "sink_local": per query head, the maximum block score over
  the sink and local blocks, the estimate [TS] Methodology 2 (Pseudo-Max
  Approximation) and 3 (Pseudo-max Estimation) describe; the kept set then
  does not depend on the split size. "max": per query head and split, the
  larger of the two (so a low sink/local estimate cannot keep more of a split
  than its own maximum would). In every mode the sink blocks (first ``sink``)
  and local blocks (last ``local``) are always kept.
* δ is in natural-log logit units ([TS] Methodology 2, "Adaptivity"), the
  comparison is ``>=`` ([TS] Methodology 2, "Mechanism"), and the logit is
  ``sm_scale * q.k``.
* The kept blocks are attended exactly ([TS] Methodology 3, "Fine-Grained
  Refinement"); here that is done in fp64.

Second storage scheme ("thumb"), closer to the pages' own ([TS] Methodology
1: 2-bit key thumbnails for the scan, 8-bit residuals that reconstruct the keys
for refinement). The formats are not given there; this library fixes them:

* thumbnail: t = fl32(amax/3); x = fl32(k * fl32(3/amax));
  u = clamp(rne(fl32(fl32(x + 3) * 0.5)), 0, 3); level (2u - 3) * t, i.e. one
  of {-3t, -t, t, 3t};
* residual: r = fl32(k - fl32((2u - 3) * t)), quantised to int8 with its own
  per-token scale exactly like the int8 query (amax/127, clamp to +-127);
* reconstructed key K^ = (2u - 3) * t + s8 * r8 in exact arithmetic; the
  refinement attends over K^ (fp64 here), V stays bf16;
* the scan uses the thumbnail: dot = sum qc * (2u - 3) (exact integer),
  s^ = fl32(float(dot) * fl32(t * cq)).

Several query tokens per step (multi-query decode, :func:`decode_multi`): the
pages describe one query token per decode step. This library's reading for Q
tokens (a speculative-decoding verify step, or a chunk of new tokens): their
keys and values are already in the cache, token i of a sequence of length L
sits at position L - Q + i and sees rows 0 .. L - Q + i, so it is one decode
step of length L - Q + 1 + i with its own selection. A GPU kernel may share
the scan and the kept blocks between the Q tokens; the result is defined per
token.

Floating point: every selection step is done in explicit np.float32 scalars
and arrays (no Python floats, which would promote to fp64), so the kept-block
mask is reproducible bit for bit. Attention is done in fp64.
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32
KEY_QMAX = 7      # int4 symmetric range
QUERY_QMAX = 127  # int8 symmetric range
# Rows whose amax is below these powers of two are treated as all-zero: for
# smaller amax, fl32(QMAX / amax) would overflow to +inf (and 0 * inf = NaN).
KEY_TINY = np.float32(2.0 ** -125)
QUERY_TINY = np.float32(2.0 ** -120)
THUMB_QMAX = 3   # thumbnail levels (2u - 3) in {-3, -1, 1, 3}
RESID_QMAX = 127


# --------------------------------------------------------------------------
# bf16 decoding (inputs arrive as raw bf16 bit patterns in uint16 arrays)
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an fp32 word; widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# O1: key quantisation (int4 + per-token fp32 scale)   [TS] Methodology 1
# --------------------------------------------------------------------------

def quantize_keys(k32: np.ndarray):
    """Quantise fp32 key rows ``[..., d]`` to int4 codes and one scale per row.

    amax = max_i |k_i|; scale = fl32(amax / 7); inv = fl32(7 / amax);
    code_i = clamp(rne(fl32(k_i * inv)), -7, 7). A row with amax < 2^-125
    (including an all-zero row) gives scale 0 and zero codes. Returns ``(codes int8 [..., d], scale float32 [...])``.
    """
    k32 = np.asarray(k32, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=-1)
    nz = amax >= KEY_TINY
    safe = np.where(nz, amax, F32(1)).astype(np.float32)
    inv = (F32(KEY_QMAX) / safe).astype(np.float32)
    scale = np.where(nz, (safe / F32(KEY_QMAX)).astype(np.float32), F32(0)).astype(np.float32)
    prod = (k32 * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -KEY_QMAX, KEY_QMAX).astype(np.int8)
    codes[~nz] = 0
    return codes, scale


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, two per byte: element 2i in the low nibble,
    element 2i+1 in the high nibble. ``[..., d] int8 -> [..., d/2] uint8``."""
    c = np.asarray(codes, dtype=np.int8).astype(np.uint8) & np.uint8(0x0F)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4` (sign-extends each nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & np.uint8(0x0F)).astype(np.int16)
    hi = (p >> np.uint8(4)).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------------------------
# O1': thumbnail + residual keys ("thumb" storage)    [TS] Methodology 1, 3
# --------------------------------------------------------------------------

def quantize_keys_thumb(k32: np.ndarray):
    """2-bit thumbnail codes and an int8 residual per key row ``[..., d]``.

    Returns ``(u uint8 [..., d] in 0..3, t float32 [...], r8 int8 [..., d],
    s8 float32 [...])``. A row with amax < 2^-125 gives t = 0, u = 0, r8 = 0,
    s8 = 0 (reconstructs to zero); a residual with amax < 2^-120 gives s8 = 0,
    r8 = 0."""
    k32 = np.asarray(k32, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=-1)
    nz = amax >= KEY_TINY
    safe = np.where(nz, amax, F32(1)).astype(np.float32)
    inv = (F32(THUMB_QMAX) / safe).astype(np.float32)
    t = np.where(nz, (safe / F32(THUMB_QMAX)).astype(np.float32), F32(0)).astype(np.float32)
    x = (k32 * inv[..., None]).astype(np.float32)
    y = ((x + F32(3)).astype(np.float32) * F32(0.5)).astype(np.float32)
    u = np.clip(np.rint(y), 0, 3).astype(np.int64)
    u[~nz] = 0
    lev = ((2 * u - 3).astype(np.float32) * t[..., None]).astype(np.float32)
    r = (k32 - lev).astype(np.float32)
    r[~nz] = 0
    ar = np.max(np.abs(r), axis=-1)
    nzr = ar >= QUERY_TINY
    safe_r = np.where(nzr, ar, F32(1)).astype(np.float32)
    inv_r = (F32(RESID_QMAX) / safe_r).astype(np.float32)
    s8 = np.where(nzr, (safe_r / F32(RESID_QMAX)).astype(np.float32), F32(0)).astype(np.float32)
    r8 = np.clip(np.rint((r * inv_r[..., None]).astype(np.float32)), -RESID_QMAX, RESID_QMAX).astype(np.int8)
    r8[~nzr] = 0
    return u.astype(np.uint8), t, r8, s8


def reconstruct_thumb(u: np.ndarray, t: np.ndarray, r8: np.ndarray, s8: np.ndarray) -> np.ndarray:
    """K^ = (2u - 3) * t + s8 * r8, exact in fp64."""
    return ((2 * u.astype(np.float64) - 3) * t.astype(np.float64)[..., None]
            + s8.astype(np.float64)[..., None] * r8.astype(np.float64))


def pack_2bit(u: np.ndarray) -> np.ndarray:
    """Four 2-bit codes per byte: element 4i + c in bits 2c..2c+1 of byte i."""
    u = np.asarray(u, dtype=np.uint8) & np.uint8(3)
    return (u[..., 0::4] | (u[..., 1::4] << np.uint8(2)) | (u[..., 2::4] << np.uint8(4))
            | (u[..., 3::4] << np.uint8(6))).astype(np.uint8)


def unpack_2bit(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (4 * p.shape[-1],), dtype=np.uint8)
    for c in range(4):
        out[..., c::4] = (p >> np.uint8(2 * c)) & np.uint8(3)
    return out


def thumb_token_scores(qc: np.ndarray, cq, u: np.ndarray, t: np.ndarray) -> np.ndarray:
    """s^_t = fl32(float32(dot_t) * fl32(t_t * cq)), dot_t = sum qc * (2u - 3)."""
    dot = (2 * u.astype(np.int64) - 3) @ np.asarray(qc, dtype=np.int64)
    w = (np.asarray(t, dtype=np.float32) * F32(cq)).astype(np.float32)
    return (dot.astype(np.float32) * w).astype(np.float32)


def quantize_cache_thumb(k, seq_lens):
    """Thumbnail cache of a bf16 K cache ``[B, Hkv, cap, d]``: ``(k2 uint8
    [B,Hkv,cap,d/4], t f32 [B,Hkv,cap], kr int8 [B,Hkv,cap,d], s8 f32
    [B,Hkv,cap])``; rows at or past a sequence's length are left 0."""
    B, Hkv, cap, d = k.shape
    k2 = np.zeros((B, Hkv, cap, d // 4), dtype=np.uint8)
    t = np.zeros((B, Hkv, cap), dtype=np.float32)
    kr = np.zeros((B, Hkv, cap, d), dtype=np.int8)
    s8 = np.zeros((B, Hkv, cap), dtype=np.float32)
    for b in range(B):
        L = max(0, min(int(seq_lens[b]), cap))
        for j in range(Hkv):
            u, tt, r8, ss = quantize_keys_thumb(bf16_bits_to_f32(k[b, j, :L]))
            k2[b, j, :L] = pack_2bit(u)
            t[b, j, :L] = tt
            kr[b, j, :L] = r8
            s8[b, j, :L] = ss
    return k2, t, kr, s8


# --------------------------------------------------------------------------
# O2: query quantisation (int8 + per-head scale, folded with sm_scale)
# --------------------------------------------------------------------------

def quantize_query(q32: np.ndarray, sm_scale) -> tuple:
    """int8 query for the scan. amax = max |q_i|; sq = fl32(amax/127);
    inv = fl32(127/amax); qc_i = clamp(rne(fl32(q_i*inv)), -127, 127);
    cq = fl32(sq * sm_scale). A query with amax < 2^-120 (including zero)
    gives qc = 0 and cq = 0."""
    q32 = np.asarray(q32, dtype=np.float32)
    sm = F32(sm_scale)
    amax = F32(np.max(np.abs(q32)))
    if not amax >= QUERY_TINY:
        return np.zeros(q32.shape, dtype=np.int8), F32(0)
    inv = F32(F32(QUERY_QMAX) / amax)
    sq = F32(amax / F32(QUERY_QMAX))
    qc = np.clip(np.rint((q32 * inv).astype(np.float32)), -QUERY_QMAX, QUERY_QMAX).astype(np.int8)
    return qc, F32(sq * sm)


# --------------------------------------------------------------------------
# O3: tentative token scores from the low-bit scan   [TS] Methodology 1, 3
# --------------------------------------------------------------------------

def token_scores(qc: np.ndarray, cq, codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """s^_t = fl32(float32(dot_t) * fl32(scale_t * cq)) with dot_t the exact
    integer dot product of the int8 query and the int4 key codes of token t."""
    dot = codes.astype(np.int64) @ np.asarray(qc, dtype=np.int64)
    w = (np.asarray(scale, dtype=np.float32) * F32(cq)).astype(np.float32)
    return (dot.astype(np.float32) * w).astype(np.float32)


# --------------------------------------------------------------------------
# O4: block scores                              [TS] Methodology 3 (Top-δ)
# --------------------------------------------------------------------------

def block_scores(tok: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Max tentative score over the valid tokens (t < L) of each block."""
    nb = -(-L // block_size)
    out = np.empty(nb, dtype=tok.dtype)
    for j in range(nb):
        out[j] = np.max(tok[j * block_size:min((j + 1) * block_size, L)])
    return out


# --------------------------------------------------------------------------
# O5 + O6: split-local Top-δ with sink and local blocks   [TS] Methodology 2
# --------------------------------------------------------------------------

PSEUDO_MAX_MODES = ("split", "sink_local", "max")


def select_blocks(scores: np.ndarray, split_blocks: int, delta, sink: int, local: int,
                  pseudo_max: str = "split") -> np.ndarray:
    """Keep block j iff score_j >= m~ - δ, or j is one of the first ``sink`` or
    last ``local`` blocks. m~ is the maximum block score in j's split (blocks
    [s*S, s*S+S)) for ``pseudo_max="split"``, the maximum over the sink and
    local blocks for ``pseudo_max="sink_local"``, and the larger of the two
    for ``pseudo_max="max"``. The subtraction and comparison run in the dtype
    of ``scores`` (fp32 for the quantised scan)."""
    if pseudo_max not in PSEUDO_MAX_MODES:
        raise ValueError(f"pseudo_max must be one of {PSEUDO_MAX_MODES}")
    dt = scores.dtype.type
    nb = scores.shape[0]
    keep = np.zeros(nb, dtype=bool)
    d = dt(delta)
    forced = np.zeros(nb, dtype=bool)
    forced[:min(sink, nb)] = True
    if local > 0:
        forced[max(0, nb - local):] = True
    m_sl = None
    if pseudo_max != "split":
        if sink + local < 1:
            raise ValueError("the sink/local pseudo-max needs sink + local >= 1")
        m_sl = dt(np.max(scores[forced]))
    if pseudo_max == "sink_local":
        thr = dt(m_sl - d)
        keep = scores >= thr
    else:
        for s0 in range(0, nb, split_blocks):
            seg = scores[s0:s0 + split_blocks]
            m_tilde = dt(np.max(seg))
            if pseudo_max == "max":
                m_tilde = max(m_tilde, m_sl)
            thr = dt(m_tilde - d)
            keep[s0:s0 + split_blocks] = seg >= thr
    return keep | forced


# --------------------------------------------------------------------------
# O7: exact attention over the kept tokens   [TS] Methodology 3 (Refinement)
# --------------------------------------------------------------------------

def attend(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, sm_scale) -> tuple:
    """Softmax attention of one query over the given key/value rows, fp64.
    Returns ``(out [d], lse)``; lse is the natural log of the normaliser."""
    if k64.shape[0] == 0:
        return np.zeros(q64.shape[0]), -math.inf
    z = float(sm_scale) * (k64 @ q64)
    m = np.max(z)
    p = np.exp(z - m)
    l = np.sum(p)
    return (p @ v64) / l, float(m + math.log(l))


# --------------------------------------------------------------------------
# One decode step
# --------------------------------------------------------------------------

def select_head(q32: np.ndarray, codes: np.ndarray, scale: np.ndarray, k64: np.ndarray, L: int,
                block_size: int, delta, sink: int, local: int, split_blocks: int, sm_scale,
                quantize: bool = True, pseudo_max: str = "split", thumb=None) -> np.ndarray:
    """Kept-block mask of one query head over one sequence (O2-O6).

    With ``quantize=False`` the tentative scores are replaced by the exact fp64
    logits and the threshold is taken in fp64 (used to check the dense limit)."""
    if thumb is not None:
        qc, cq = quantize_query(q32, sm_scale)
        tok = thumb_token_scores(qc, cq, thumb[0][:L], thumb[1][:L])
    elif quantize:
        qc, cq = quantize_query(q32, sm_scale)
        tok = token_scores(qc, cq, codes[:L], scale[:L])
    else:
        tok = float(sm_scale) * (k64[:L] @ q32.astype(np.float64))
    blk = block_scores(tok, L, block_size)
    return select_blocks(blk, split_blocks, delta, sink, local, pseudo_max)


def decode(q, k, v, seq_lens, *, max_seq_len: int, block_size: int, delta, sink: int, local: int,
           split_blocks: int, sm_scale=None, quantize: bool = True, heads=None, mask_only: bool = False,
           pseudo_max: str = "split", storage: str = "int4"):
    """One FFD decode step.

    ``q`` bf16 bits ``[B, Hq, d]``; ``k``, ``v`` bf16 bits ``[B, Hkv, cap, d]``;
    ``seq_lens`` int ``[B]`` (each used as ``min(seq_lens[b], max_seq_len)``).
    Query head h reads kv head ``h // (Hq // Hkv)``.

    Returns ``(out fp64 [B,Hq,d], lse fp64 [B,Hq], mask uint8 [B,Hq,NB_max])``
    with ``NB_max = ceil(max_seq_len / block_size)``. A sequence with no valid
    token gives out 0, lse -inf and an all-zero mask row. ``heads`` restricts
    the work to a list of ``(b, h)`` pairs (other rows are left NaN / 0);
    ``mask_only`` skips the attention step (out and lse stay NaN).
    ``pseudo_max`` picks how m~ is estimated (see :func:`select_blocks`).
    ``storage="thumb"`` scans 2-bit thumbnails and attends over the
    reconstructed keys K^ (see :func:`quantize_keys_thumb`) instead of the int4
    sketch and the bf16 keys.
    """
    if storage not in ("int4", "thumb"):
        raise ValueError("storage must be 'int4' or 'thumb'")
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = F32(1.0 / math.sqrt(d))
    sm_scale = F32(sm_scale)
    nb_max = -(-max_seq_len // block_size)
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    mask = np.zeros((B, Hq, nb_max), dtype=np.uint8)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)

    for b in range(B):
        L = int(min(int(seq_lens[b]), max_seq_len))
        for j in range(Hkv):
            hs = [h for h in range(j * G, (j + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            if L <= 0:
                for h in hs:
                    out[b, h] = 0.0
                    lse[b, h] = -math.inf
                continue
            k32 = bf16_bits_to_f32(k[b, j, :L])
            thumb = None
            if storage == "thumb":
                thumb = quantize_keys_thumb(k32)
                k64 = None if mask_only else reconstruct_thumb(*thumb)
            else:
                k64 = k32.astype(np.float64) if (not mask_only or not quantize) else None
            v64 = None if mask_only else bf16_bits_to_f32(v[b, j, :L]).astype(np.float64)
            codes, scale = quantize_keys(k32) if (quantize and storage == "int4") else (None, None)
            for h in hs:
                q32 = bf16_bits_to_f32(q[b, h])
                keep = select_head(q32, codes, scale, k64, L, block_size, delta, sink, local,
                                   split_blocks, sm_scale, quantize, pseudo_max, thumb)
                mask[b, h, :keep.shape[0]] = keep
                if mask_only:
                    continue
                tok_keep = np.repeat(keep, block_size)[:L]
                o, s = attend(q32.astype(np.float64), k64[tok_keep], v64[tok_keep], sm_scale)
                out[b, h] = o
                lse[b, h] = s
    return out, lse, mask


def decode_multi(q, k, v, seq_lens, *, max_seq_len: int, block_size: int, delta, sink: int, local: int,
                 split_blocks: int, sm_scale=None, quantize: bool = True, heads=None, mask_only: bool = False,
                 pseudo_max: str = "split"):
    """Several query tokens per sequence in one step (multi-query decode).

    The pages describe one query token per step. This library's reading for Q
    query tokens: the cache already holds the keys and values of all Q new
    tokens, query token i of sequence b sits at position ``seq_lens[b] - Q + i``
    and sees the rows up to and including its own position. Each query token
    is therefore exactly one decode step of :func:`decode` with sequence length
    ``seq_lens[b] - Q + 1 + i`` (then capped by ``max_seq_len``; a length <= 0
    is an empty step): its own scores, pseudo-max, Top-δ set and attention.

    ``q`` bf16 bits ``[B, Q, Hq, d]``. Returns ``(out [B,Q,Hq,d], lse [B,Q,Hq],
    mask uint8 [B,Q,Hq,NB_max])``. ``heads`` restricts the work to ``(b, i, h)``
    triples.
    """
    q = np.asarray(q)
    B, Q, Hq, d = q.shape
    lens = np.asarray(seq_lens, dtype=np.int64)
    nb_max = -(-max_seq_len // block_size)
    out = np.full((B, Q, Hq, d), np.nan)
    lse = np.full((B, Q, Hq), np.nan)
    mask = np.zeros((B, Q, Hq, nb_max), dtype=np.uint8)
    for i in range(Q):
        hs = None
        if heads is not None:
            hs = [(b, h) for (b, qi, h) in heads if qi == i]
            if not hs:
                continue
        o, s, m = decode(q[:, i], k, v, lens - Q + 1 + i, max_seq_len=max_seq_len, block_size=block_size,
                         delta=delta, sink=sink, local=local, split_blocks=split_blocks, sm_scale=sm_scale,
                         quantize=quantize, heads=hs, mask_only=mask_only, pseudo_max=pseudo_max)
        out[:, i] = o
        lse[:, i] = s
        mask[:, i] = m
    return out, lse, mask


def quantize_cache(k, seq_lens, *, max_seq_len=None):
    """Quantised key cache of a whole bf16 K cache ``[B, Hkv, cap, d]``.

    Returns ``(kq uint8 [B,Hkv,cap,d/2], kscale float32 [B,Hkv,cap])``; rows at
    or past a sequence's length are left 0 (the library does not write them)."""
    B, Hkv, cap, d = k.shape
    kq = np.zeros((B, Hkv, cap, d // 2), dtype=np.uint8)
    ks = np.zeros((B, Hkv, cap), dtype=np.float32)
    for b in range(B):
        L = int(seq_lens[b]) if max_seq_len is None else int(min(int(seq_lens[b]), max_seq_len))
        L = max(0, min(L, cap))
        for j in range(Hkv):
            c, s = quantize_keys(bf16_bits_to_f32(k[b, j, :L]))
            kq[b, j, :L] = pack_int4(c)
            ks[b, j, :L] = s
    return kq, ks
