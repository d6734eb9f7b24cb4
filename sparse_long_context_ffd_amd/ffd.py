"""Python binding of ``libffd.so`` (ctypes).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/ffd.h``. PyTorch supplies device
memory and the current HIP stream. If the library has not been built this
module raises on first use; there is no fallback.

Low-level entry points keep the C names (every name in ``EXPORTED_SYMBOLS``:
the int4 sketch ``ffd_quantize_kv`` / ``ffd_decode`` and its halves
``ffd_decode_partials`` / ``ffd_combine``, the thumbnail storage
``ffd_quantize_kv_thumb`` / ``ffd_decode_thumb``, the paged cache
``ffd_quantize_kv_paged`` / ``ffd_decode_paged``, several query tokens
``ffd_decode_multi`` / ``ffd_decode_paged_multi``, ``ffd_decode_noalloc``
(no workspace: a static device array), the workspace sizes, ``ffd_last_error`` and
``ffd_abi_version``) and take preallocated tensors. ``quantize_kv``,
``quantize_kv_thumb``, ``decode`` and ``decode_multi`` are conveniences that
allocate the outputs and the workspace with torch and then call them.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

# FFD_LIBRARY selects another build of the same library (the sanitizer build
# of the host layer, for the CPU tests); it must exist like the default one.
LIB_PATH = os.environ.get("FFD_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libffd.so")

FFD_OK = 0
FFD_ERR_INVALID_ARG = 1
FFD_ERR_UNSUPPORTED = 2
FFD_ERR_WORKSPACE = 3
FFD_ERR_HIP = 4
FFD_OUT_BF16 = 0
FFD_OUT_F32 = 1
PSEUDO_MAX = {"split": 0, "sink_local": 1, "max": 2}

EXPORTED_SYMBOLS = ("ffd_abi_version", "ffd_last_error", "ffd_quantize_kv", "ffd_quantize_kv_paged",
                    "ffd_quantize_kv_thumb", "ffd_decode_workspace_bytes", "ffd_decode", "ffd_decode_paged",
                    "ffd_decode_thumb", "ffd_decode_partials", "ffd_combine", "ffd_decode_multi",
                    "ffd_decode_multi_workspace_bytes", "ffd_decode_paged_multi", "ffd_decode_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20   # FFD_NOALLOC_SCRATCH_BYTES


class FFDError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ffd status {status}: {message}")
        self.status = status
        self.message = message


_lib: Optional[ctypes.CDLL] = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load ``libffd.so`` once; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FFDError(-1, f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python sparse_long_context_ffd_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    L.ffd_abi_version.restype = _i
    L.ffd_abi_version.argtypes = []
    L.ffd_last_error.restype = ctypes.c_char_p
    L.ffd_last_error.argtypes = []
    L.ffd_quantize_kv.restype = _i
    L.ffd_quantize_kv.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    L.ffd_decode_workspace_bytes.restype = ctypes.c_size_t
    L.ffd_decode_workspace_bytes.argtypes = [_i] * 6
    L.ffd_decode.restype = _i
    L.ffd_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp,          # q k v kq kscale seq_lens
                             _i, _i, _i, _i, _i, _i,                # max_seq_len B Hq Hkv d cap
                             _i, ctypes.c_float, _i, _i, _i, _i,    # block_size delta sink local pm split
                             ctypes.c_float,                        # sm_scale
                             _vp, _i, _vp, _vp,                     # out out_dtype lse mask
                             _vp, ctypes.c_size_t, _vp]             # workspace bytes stream
    L.ffd_decode_multi.restype = _i
    L.ffd_decode_multi.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp,        # q k v kq kscale seq_lens
                                   _i, _i, _i, _i, _i, _i, _i,          # max_seq_len B Q Hq Hkv d cap
                                   _i, ctypes.c_float, _i, _i, _i, _i,  # block_size delta sink local pm split
                                   ctypes.c_float,                      # sm_scale
                                   _vp, _i, _vp, _vp,                   # out out_dtype lse mask
                                   _vp, ctypes.c_size_t, _vp]           # workspace bytes stream
    L.ffd_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    L.ffd_decode_multi_workspace_bytes.argtypes = [_i] * 7
    L.ffd_decode_partials.restype = _i
    L.ffd_decode_partials.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                      _i, ctypes.c_float, _i, _i, _i, _i, ctypes.c_float,
                                      _vp, _vp, ctypes.c_size_t, _vp]
    L.ffd_quantize_kv_paged.restype = _i
    L.ffd_quantize_kv_paged.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _vp]
    L.ffd_decode_paged.restype = _i
    L.ffd_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i,      # q kp vp kqp ksp table stride pages
                                   _vp, _i, _i, _i, _i, _i,                   # seq_lens max_seq_len B Hq Hkv d
                                   _i, ctypes.c_float, _i, _i, _i, _i,        # block_size delta sink local pm split
                                   ctypes.c_float, _vp, _i, _vp, _vp,         # sm_scale out out_dtype lse mask
                                   _vp, ctypes.c_size_t, _vp]                 # workspace bytes stream
    L.ffd_decode_paged_multi.restype = _i
    L.ffd_decode_paged_multi.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i,  # q kp vp kqp ksp table stride pages
                                         _vp, _i, _i, _i, _i, _i, _i,        # seq_lens max_seq_len B Q Hq Hkv d
                                         _i, ctypes.c_float, _i, _i, _i, _i,  # block_size delta sink local pm split
                                         ctypes.c_float, _vp, _i, _vp, _vp,   # sm_scale out out_dtype lse mask
                                         _vp, ctypes.c_size_t, _vp]           # workspace bytes stream
    L.ffd_quantize_kv_thumb.restype = _i
    L.ffd_quantize_kv_thumb.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    L.ffd_decode_thumb.restype = _i
    L.ffd_decode_thumb.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp,          # q k2 k2s kr krs v seq_lens
                                   _i, _i, _i, _i, _i, _i,                     # max_seq_len B Hq Hkv d cap
                                   _i, ctypes.c_float, _i, _i, _i, _i,         # block_size delta sink local pm split
                                   ctypes.c_float, _vp, _i, _vp, _vp,          # sm_scale out out_dtype lse mask
                                   _vp, ctypes.c_size_t, _vp]                  # workspace bytes stream
    L.ffd_decode_noalloc.restype = _i
    L.ffd_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp,          # q k v kq kscale seq_lens
                                     _i, _i, _i, _i, _i, _i,                # max_seq_len B Hq Hkv d cap
                                     _i, ctypes.c_float, _i, _i, _i, _i,    # block_size delta sink local pm split
                                     ctypes.c_float,                        # sm_scale
                                     _vp, _i, _vp, _vp, _vp]                # out out_dtype lse mask stream
    L.ffd_combine.restype = _i
    L.ffd_combine.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _vp, ctypes.c_size_t, _vp, _i, _vp, _vp]
    _lib = L
    return L


def ffd_abi_version() -> int:
    return lib().ffd_abi_version()


def ffd_last_error() -> str:
    return lib().ffd_last_error().decode()


def _check(status: int) -> None:
    if status != FFD_OK:
        raise FFDError(status, ffd_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {ndim}-d {dtype} CUDA tensor, got "
                         f"{tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()} device={t.device}")


def _need_per_seq(t: torch.Tensor, name: str, B: int) -> None:
    """An int32 vector with one entry per sequence."""
    _need(t, name, torch.int32, 1)
    if t.shape[0] != B:
        raise ValueError(f"{name} needs one entry per sequence ({B}), got {t.shape[0]}")


def ffd_decode_workspace_bytes(B: int, Hq: int, d: int, max_seq_len: int, block_size: int = 64,
                               split_blocks: int = 32) -> int:
    return int(lib().ffd_decode_workspace_bytes(B, Hq, d, max_seq_len, block_size, split_blocks))


def ffd_quantize_kv(k: torch.Tensor, kq: torch.Tensor, kscale: torch.Tensor, pos_begin: torch.Tensor,
                    pos_end: torch.Tensor, max_span: int, stream=None) -> None:
    """Quantise bf16 K rows ``[pos_begin[b], pos_end[b])`` into ``kq``/``kscale`` (in place)."""
    _need(k, "k", torch.bfloat16, 4)
    B, Hkv, cap, d = k.shape
    _need(kq, "kq", torch.uint8, 4)
    _need(kscale, "kscale", torch.float32, 3)
    _need(pos_begin, "pos_begin", torch.int32, 1)
    _need(pos_end, "pos_end", torch.int32, 1)
    if tuple(kq.shape) != (B, Hkv, cap, d // 2) or tuple(kscale.shape) != (B, Hkv, cap):
        raise ValueError("kq/kscale shapes do not match k")
    if pos_begin.shape[0] != B or pos_end.shape[0] != B:
        raise ValueError("pos_begin/pos_end need one entry per sequence")
    _check(lib().ffd_quantize_kv(_ptr(k), _ptr(kq), _ptr(kscale), _ptr(pos_begin), _ptr(pos_end),
                                 B, Hkv, cap, d, int(max_span), _stream(stream)))


def _check_decode_inputs(q, k, v, kq, kscale, seq_lens, max_seq_len, block_size, kept_mask):
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    if tuple(k.shape) != (B, Hkv, cap, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v shapes do not match q")
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens needs one entry per sequence")
    if kq is not None:
        _need(kq, "kq", torch.uint8, 4)
        _need(kscale, "kscale", torch.float32, 3)
        if tuple(kq.shape) != (B, Hkv, cap, d // 2) or tuple(kscale.shape) != (B, Hkv, cap):
            raise ValueError("kq/kscale shapes do not match k")
    if kept_mask is not None:
        _need(kept_mask, "kept_mask", torch.uint8, 3)
        if tuple(kept_mask.shape) != (B, Hq, -(-max_seq_len // block_size)):
            raise ValueError("kept_mask shape")
    return B, Hq, Hkv, d, cap


def _check_outputs(out, lse, B, Hq, d):
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bf16 or f32")
    _need(out, "out", out.dtype, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out/lse shapes")
    return FFD_OUT_F32 if out.dtype == torch.float32 else FFD_OUT_BF16


def _pm(pseudo_max) -> int:
    if pseudo_max not in PSEUDO_MAX:
        raise ValueError(f"pseudo_max must be one of {tuple(PSEUDO_MAX)}")
    return PSEUDO_MAX[pseudo_max]


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def ffd_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kq: Optional[torch.Tensor],
               kscale: Optional[torch.Tensor], seq_lens: torch.Tensor, *, max_seq_len: int, block_size: int,
               delta: float, sink: int, local: int, split_blocks: int, sm_scale: float, out: torch.Tensor,
               lse: torch.Tensor, kept_mask: Optional[torch.Tensor], workspace: Optional[torch.Tensor],
               pseudo_max: str = "split", stream=None) -> None:
    """One decode step into preallocated ``out`` / ``lse`` / ``kept_mask``."""
    B, Hq, Hkv, d, cap = _check_decode_inputs(q, k, v, kq, kscale, seq_lens, max_seq_len, block_size, kept_mask)
    odt = _check_outputs(out, lse, B, Hq, d)
    _check(lib().ffd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(kq), _ptr(kscale), _ptr(seq_lens),
                            int(max_seq_len), B, Hq, Hkv, d, cap, int(block_size), float(delta), int(sink),
                            int(local), _pm(pseudo_max), int(split_blocks), float(sm_scale), _ptr(out), odt,
                            _ptr(lse),
                            _ptr(kept_mask), _ptr(workspace), _ws(workspace), _stream(stream)))


def ffd_decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kq: Optional[torch.Tensor],
                       kscale: Optional[torch.Tensor], seq_lens: torch.Tensor, *, max_seq_len: int,
                       block_size: int, delta: float, sink: int, local: int, split_blocks: int, sm_scale: float,
                       out: torch.Tensor, lse: torch.Tensor, kept_mask: Optional[torch.Tensor],
                       pseudo_max: str = "split", stream=None) -> None:
    """``ffd_decode`` with the partials in the library's static scratch array
    (no workspace argument, no allocation)."""
    B, Hq, Hkv, d, cap = _check_decode_inputs(q, k, v, kq, kscale, seq_lens, max_seq_len, block_size, kept_mask)
    odt = _check_outputs(out, lse, B, Hq, d)
    _check(lib().ffd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(kq), _ptr(kscale), _ptr(seq_lens),
                                    int(max_seq_len), B, Hq, Hkv, d, cap, int(block_size), float(delta), int(sink),
                                    int(local), _pm(pseudo_max), int(split_blocks), float(sm_scale), _ptr(out),
                                    odt, _ptr(lse), _ptr(kept_mask), _stream(stream)))


def ffd_decode_multi_workspace_bytes(B: int, Q: int, Hq: int, d: int, max_seq_len: int, block_size: int = 64,
                                     split_blocks: int = 32) -> int:
    return int(lib().ffd_decode_multi_workspace_bytes(B, Q, Hq, d, max_seq_len, block_size, split_blocks))


def ffd_decode_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kq: Optional[torch.Tensor],
                     kscale: Optional[torch.Tensor], seq_lens: torch.Tensor, *, max_seq_len: int, block_size: int,
                     delta: float, sink: int, local: int, split_blocks: int, sm_scale: float, out: torch.Tensor,
                     lse: torch.Tensor, kept_mask: Optional[torch.Tensor], workspace: Optional[torch.Tensor],
                     pseudo_max: str = "split", stream=None) -> None:
    """Q query tokens per sequence (``q`` ``[B, Q, Hq, d]``; token i sees the
    cache up to position ``seq_lens[b] - Q + i``) into preallocated ``out``
    ``[B, Q, Hq, d]`` / ``lse`` ``[B, Q, Hq]`` / ``kept_mask`` ``[B, Q, Hq, NB]``."""
    _need(q, "q", torch.bfloat16, 4)
    B, Q, Hq, d = q.shape
    flat = q.view(B, Q * Hq, d)
    mflat = None if kept_mask is None else kept_mask.view(B, Q * Hq, kept_mask.shape[-1])
    _, _, Hkv, _, cap = _check_decode_inputs(flat, k, v, kq, kscale, seq_lens, max_seq_len, block_size, mflat)
    if tuple(out.shape[:3]) != (B, Q, Hq) or tuple(lse.shape) != (B, Q, Hq):
        raise ValueError("out/lse shapes")
    if kept_mask is not None and tuple(kept_mask.shape[:3]) != (B, Q, Hq):
        raise ValueError("kept_mask shape")
    odt = _check_outputs(out.view(B, Q * Hq, out.shape[-1]), lse.view(B, Q * Hq), B, Q * Hq, d)
    _check(lib().ffd_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(kq), _ptr(kscale), _ptr(seq_lens),
                                  int(max_seq_len), B, Q, Hq, Hkv, d, cap, int(block_size), float(delta), int(sink),
                                  int(local), _pm(pseudo_max), int(split_blocks), float(sm_scale), _ptr(out), odt,
                                  _ptr(lse), _ptr(kept_mask), _ptr(workspace), _ws(workspace), _stream(stream)))


def ffd_decode_partials(q, k, v, kq, kscale, seq_lens, *, max_seq_len: int, block_size: int, delta: float,
                        sink: int, local: int, split_blocks: int, sm_scale: float,
                        kept_mask: Optional[torch.Tensor], workspace: torch.Tensor, pseudo_max: str = "split",
                        stream=None) -> None:
    """The fused scan -> select -> attend kernel alone; partials stay in ``workspace``."""
    B, Hq, Hkv, d, cap = _check_decode_inputs(q, k, v, kq, kscale, seq_lens, max_seq_len, block_size, kept_mask)
    _check(lib().ffd_decode_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(kq), _ptr(kscale), _ptr(seq_lens),
                                     int(max_seq_len), B, Hq, Hkv, d, cap, int(block_size), float(delta),
                                     int(sink), int(local), _pm(pseudo_max), int(split_blocks), float(sm_scale),
                                     _ptr(kept_mask),
                                     _ptr(workspace), _ws(workspace), _stream(stream)))


def ffd_combine(seq_lens, *, max_seq_len: int, block_size: int, split_blocks: int, workspace: torch.Tensor,
                out: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    """Log-sum-exp merge of the per-split partials in ``workspace`` into ``out`` / ``lse``."""
    B, Hq, d = out.shape
    _need_per_seq(seq_lens, "seq_lens", B)
    odt = _check_outputs(out, lse, B, Hq, d)
    _check(lib().ffd_combine(_ptr(seq_lens), int(max_seq_len), B, Hq, d, int(block_size), int(split_blocks),
                             _ptr(workspace), _ws(workspace), _ptr(out), odt, _ptr(lse), _stream(stream)))


def ffd_quantize_kv_paged(k_pages: torch.Tensor, kq_pages: torch.Tensor, kscale_pages: torch.Tensor,
                          block_table: torch.Tensor, pos_begin: torch.Tensor, pos_end: torch.Tensor, max_span: int,
                          stream=None) -> None:
    """Quantise tokens ``[pos_begin[b], pos_end[b])`` of a paged K cache in place."""
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    P, Hkv, bs, d = k_pages.shape
    if bs != 64:
        raise ValueError("pages hold 64 tokens")
    _need(kq_pages, "kq_pages", torch.uint8, 4)
    _need(kscale_pages, "kscale_pages", torch.float32, 3)
    _need(block_table, "block_table", torch.int32, 2)
    if tuple(kq_pages.shape) != (P, Hkv, 64, d // 2) or tuple(kscale_pages.shape) != (P, Hkv, 64):
        raise ValueError("kq/kscale page shapes do not match k_pages")
    B, stride = block_table.shape
    _need_per_seq(pos_begin, "pos_begin", B)
    _need_per_seq(pos_end, "pos_end", B)
    _check(lib().ffd_quantize_kv_paged(_ptr(k_pages), _ptr(kq_pages), _ptr(kscale_pages), _ptr(block_table), stride,
                                       P, _ptr(pos_begin), _ptr(pos_end), B, Hkv, d, int(max_span), _stream(stream)))


def _check_pages(k_pages, v_pages, kq_pages, kscale_pages, block_table, seq_lens, B: int, d: int):
    """Shapes of a page pool and its block table; returns (num_pages, Hkv)."""
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    P, Hkv, bs, _ = k_pages.shape
    if bs != 64 or tuple(k_pages.shape) != (P, Hkv, 64, d) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k/v pages must be [num_pages, Hkv, 64, d]")
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] != B:
        raise ValueError("block_table needs one row per sequence")
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens needs one entry per sequence")
    if kq_pages is not None:
        _need(kq_pages, "kq_pages", torch.uint8, 4)
        _need(kscale_pages, "kscale_pages", torch.float32, 3)
        if tuple(kq_pages.shape) != (P, Hkv, 64, d // 2) or tuple(kscale_pages.shape) != (P, Hkv, 64):
            raise ValueError("kq/kscale pages must be [num_pages, Hkv, 64, d/2] and [num_pages, Hkv, 64]")
    return P, Hkv


def ffd_decode_paged(q, k_pages, v_pages, kq_pages, kscale_pages, block_table, seq_lens, *, max_seq_len: int,
                     block_size: int, delta: float, sink: int, local: int, split_blocks: int, sm_scale: float,
                     out: torch.Tensor, lse: torch.Tensor, kept_mask: Optional[torch.Tensor],
                     workspace: Optional[torch.Tensor], pseudo_max: str = "split", stream=None) -> None:
    """One decode step over a paged cache into preallocated outputs."""
    _need(q, "q", torch.bfloat16, 3)
    B, Hq, d = q.shape
    P, Hkv = _check_pages(k_pages, v_pages, kq_pages, kscale_pages, block_table, seq_lens, B, d)
    if kept_mask is not None:
        _need(kept_mask, "kept_mask", torch.uint8, 3)
        if tuple(kept_mask.shape) != (B, Hq, -(-max_seq_len // block_size)):
            raise ValueError("kept_mask shape")
    odt = _check_outputs(out, lse, B, Hq, d)
    _check(lib().ffd_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kq_pages), _ptr(kscale_pages),
                                  _ptr(block_table), block_table.shape[1], P, _ptr(seq_lens), int(max_seq_len), B, Hq,
                                  Hkv, d, int(block_size), float(delta), int(sink), int(local), _pm(pseudo_max),
                                  int(split_blocks), float(sm_scale), _ptr(out), odt, _ptr(lse), _ptr(kept_mask),
                                  _ptr(workspace), _ws(workspace), _stream(stream)))


def ffd_decode_paged_multi(q, k_pages, v_pages, kq_pages, kscale_pages, block_table, seq_lens, *,
                           max_seq_len: int, block_size: int, delta: float, sink: int, local: int,
                           split_blocks: int, sm_scale: float, out: torch.Tensor, lse: torch.Tensor,
                           kept_mask: Optional[torch.Tensor], workspace: Optional[torch.Tensor],
                           pseudo_max: str = "split", stream=None) -> None:
    """Q query tokens per sequence (``q`` ``[B, Q, Hq, d]``, as
    :func:`ffd_decode_multi`) over a paged cache (as :func:`ffd_decode_paged`)
    into preallocated ``out`` ``[B, Q, Hq, d]`` / ``lse`` ``[B, Q, Hq]`` /
    ``kept_mask`` ``[B, Q, Hq, NB]``."""
    _need(q, "q", torch.bfloat16, 4)
    B, Q, Hq, d = q.shape
    P, Hkv = _check_pages(k_pages, v_pages, kq_pages, kscale_pages, block_table, seq_lens, B, d)
    if kept_mask is not None:
        _need(kept_mask, "kept_mask", torch.uint8, 4)
        if tuple(kept_mask.shape) != (B, Q, Hq, -(-max_seq_len // block_size)):
            raise ValueError("kept_mask shape")
    if tuple(out.shape[:3]) != (B, Q, Hq) or tuple(lse.shape) != (B, Q, Hq):
        raise ValueError("out/lse shapes")
    odt = _check_outputs(out.view(B, Q * Hq, out.shape[-1]), lse.view(B, Q * Hq), B, Q * Hq, d)
    _check(lib().ffd_decode_paged_multi(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kq_pages), _ptr(kscale_pages),
                                        _ptr(block_table), block_table.shape[1], P, _ptr(seq_lens), int(max_seq_len),
                                        B, Q, Hq, Hkv, d, int(block_size), float(delta), int(sink), int(local),
                                        _pm(pseudo_max), int(split_blocks), float(sm_scale), _ptr(out), odt,
                                        _ptr(lse), _ptr(kept_mask), _ptr(workspace), _ws(workspace),
                                        _stream(stream)))


def ffd_quantize_kv_thumb(k, k2, k2scale, kr, krscale, pos_begin, pos_end, max_span: int, stream=None) -> None:
    """Thumbnail + residual storage of bf16 K rows ``[pos_begin[b], pos_end[b])`` (in place)."""
    _need(k, "k", torch.bfloat16, 4)
    B, Hkv, cap, d = k.shape
    _need(k2, "k2", torch.uint8, 4)
    _need(k2scale, "k2scale", torch.float32, 3)
    _need(kr, "kr", torch.int8, 4)
    _need(krscale, "krscale", torch.float32, 3)
    if (tuple(k2.shape) != (B, Hkv, cap, d // 4) or tuple(kr.shape) != (B, Hkv, cap, d)
            or tuple(k2scale.shape) != (B, Hkv, cap) or tuple(krscale.shape) != (B, Hkv, cap)):
        raise ValueError("thumbnail/residual shapes do not match k")
    _need_per_seq(pos_begin, "pos_begin", B)
    _need_per_seq(pos_end, "pos_end", B)
    _check(lib().ffd_quantize_kv_thumb(_ptr(k), _ptr(k2), _ptr(k2scale), _ptr(kr), _ptr(krscale), _ptr(pos_begin),
                                       _ptr(pos_end), B, Hkv, cap, d, int(max_span), _stream(stream)))


def ffd_decode_thumb(q, k2, k2scale, kr, krscale, v, seq_lens, *, max_seq_len: int, block_size: int, delta: float,
                     sink: int, local: int, split_blocks: int, sm_scale: float, out: torch.Tensor,
                     lse: torch.Tensor, kept_mask: Optional[torch.Tensor], workspace: Optional[torch.Tensor],
                     pseudo_max: str = "split", stream=None) -> None:
    """One decode step over the thumbnail + residual key storage."""
    _need(q, "q", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = v.shape
    _need(k2, "k2", torch.uint8, 4)
    _need(k2scale, "k2scale", torch.float32, 3)
    _need(kr, "kr", torch.int8, 4)
    _need(krscale, "krscale", torch.float32, 3)
    if (tuple(k2.shape) != (B, Hkv, cap, d // 4) or tuple(kr.shape) != (B, Hkv, cap, d)
            or tuple(v.shape) != (B, Hkv, cap, d) or tuple(k2scale.shape) != (B, Hkv, cap)
            or tuple(krscale.shape) != (B, Hkv, cap)):
        raise ValueError("thumbnail/residual/v shapes do not match q")
    _need_per_seq(seq_lens, "seq_lens", B)
    if kept_mask is not None:
        _need(kept_mask, "kept_mask", torch.uint8, 3)
        if tuple(kept_mask.shape) != (B, Hq, -(-max_seq_len // block_size)):
            raise ValueError("kept_mask shape")
    odt = _check_outputs(out, lse, B, Hq, d)
    _check(lib().ffd_decode_thumb(_ptr(q), _ptr(k2), _ptr(k2scale), _ptr(kr), _ptr(krscale), _ptr(v), _ptr(seq_lens),
                                  int(max_seq_len), B, Hq, Hkv, d, cap, int(block_size), float(delta), int(sink),
                                  int(local), _pm(pseudo_max), int(split_blocks), float(sm_scale), _ptr(out), odt,
                                  _ptr(lse), _ptr(kept_mask), _ptr(workspace), _ws(workspace), _stream(stream)))


def quantize_kv_thumb(k: torch.Tensor, seq_lens: torch.Tensor, stream=None):
    """Allocate and build the thumbnail + residual storage of ``k`` for tokens ``[0, seq_lens[b])``."""
    B, Hkv, cap, d = k.shape
    dev = k.device
    k2 = torch.zeros((B, Hkv, cap, d // 4), dtype=torch.uint8, device=dev)
    k2s = torch.zeros((B, Hkv, cap), dtype=torch.float32, device=dev)
    kr = torch.zeros((B, Hkv, cap, d), dtype=torch.int8, device=dev)
    krs = torch.zeros((B, Hkv, cap), dtype=torch.float32, device=dev)
    begin = torch.zeros(B, dtype=torch.int32, device=dev)
    ffd_quantize_kv_thumb(k, k2, k2s, kr, krs, begin, seq_lens.to(device=dev, dtype=torch.int32).contiguous(), cap,
                          stream)
    return k2, k2s, kr, krs


# ---------------------------------------------------------------------------
# conveniences (allocate with torch, then call the C ABI)
# ---------------------------------------------------------------------------

def quantize_kv(k: torch.Tensor, seq_lens: torch.Tensor, kq: Optional[torch.Tensor] = None,
                kscale: Optional[torch.Tensor] = None, max_span: Optional[int] = None, stream=None):
    """Build the int4 sketch of ``k`` for tokens ``[0, seq_lens[b])``; returns ``(kq, kscale)``."""
    B, Hkv, cap, d = k.shape
    if kq is None:
        kq = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device=k.device)
    if kscale is None:
        kscale = torch.zeros((B, Hkv, cap), dtype=torch.float32, device=k.device)
    begin = torch.zeros(B, dtype=torch.int32, device=k.device)
    end = seq_lens.to(device=k.device, dtype=torch.int32).contiguous()
    span = cap if max_span is None else max_span
    ffd_quantize_kv(k, kq, kscale, begin, end, span, stream)
    return kq, kscale


def alloc_workspace(B: int, Hq: int, d: int, max_seq_len: int, block_size: int = 64, split_blocks: int = 32,
                    device="cuda") -> Optional[torch.Tensor]:
    n = ffd_decode_workspace_bytes(B, Hq, d, max_seq_len, block_size, split_blocks)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(q, k, v, kq, kscale, seq_lens, *, max_seq_len: Optional[int] = None, block_size: int = 64,
           delta: float = 6.0, sink: int = 1, local: int = 4, split_blocks: int = 32,
           sm_scale: Optional[float] = None, out_dtype=torch.bfloat16, with_mask: bool = True,
           workspace: Optional[torch.Tensor] = None, pseudo_max: str = "split", stream=None):
    """Allocate outputs and run one decode step; returns ``(out, lse, kept_mask)``."""
    B, Hq, d = q.shape
    if max_seq_len is None:
        max_seq_len = k.shape[2]
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    nb_max = -(-max_seq_len // block_size)
    mask = torch.empty((B, Hq, nb_max), dtype=torch.uint8, device=q.device) if with_mask else None
    if workspace is None:
        workspace = alloc_workspace(B, Hq, d, max_seq_len, block_size, split_blocks, q.device)
    ffd_decode(q, k, v, kq, kscale, seq_lens, max_seq_len=max_seq_len, block_size=block_size, delta=delta,
               sink=sink, local=local, split_blocks=split_blocks, sm_scale=sm_scale, out=out, lse=lse,
               kept_mask=mask, workspace=workspace, pseudo_max=pseudo_max, stream=stream)
    return out, lse, mask


def decode_multi(q, k, v, kq, kscale, seq_lens, *, max_seq_len: Optional[int] = None, block_size: int = 64,
                 delta: float = 6.0, sink: int = 1, local: int = 4, split_blocks: int = 32,
                 sm_scale: Optional[float] = None, out_dtype=torch.bfloat16, with_mask: bool = True,
                 workspace: Optional[torch.Tensor] = None, pseudo_max: str = "split", stream=None):
    """Allocate outputs and run one multi-query step (``q`` ``[B, Q, Hq, d]``);
    returns ``(out, lse, kept_mask)``."""
    B, Q, Hq, d = q.shape
    if max_seq_len is None:
        max_seq_len = k.shape[2]
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    out = torch.empty((B, Q, Hq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=q.device)
    nb_max = -(-max_seq_len // block_size)
    mask = torch.empty((B, Q, Hq, nb_max), dtype=torch.uint8, device=q.device) if with_mask else None
    if workspace is None:
        n = ffd_decode_multi_workspace_bytes(B, Q, Hq, d, max_seq_len, block_size, split_blocks)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    ffd_decode_multi(q, k, v, kq, kscale, seq_lens, max_seq_len=max_seq_len, block_size=block_size, delta=delta,
                     sink=sink, local=local, split_blocks=split_blocks, sm_scale=sm_scale, out=out, lse=lse,
                     kept_mask=mask, workspace=workspace, pseudo_max=pseudo_max, stream=stream)
    return out, lse, mask
