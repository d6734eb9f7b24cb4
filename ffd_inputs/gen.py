"""Seeded synthetic decode-attention inputs.

Recipe (every workload):

* ``numpy.random.SeedSequence(seed)`` is split into ``1 + B*Hkv`` children.
  Child 0 draws the sequence lengths (mixed-length workloads only) and then
  the query ``q ~ N(0,1)`` of shape ``[B, Hq, d]``. Child ``1 + b*Hkv + j``
  draws, for sequence ``b`` and kv head ``j``: ``K ~ N(0,1)`` then
  ``V ~ N(0,1)``, both ``[L_b, d]``, then the key bias of the blocks.
* The key bias pushes whole blocks toward the query direction of the GQA
  group: ``u = unit(mean of the group's bf16 query rows)``; every token of a
  biased block gets ``+amp * u`` added in fp32 before rounding to bf16.
  ``bias="hot"`` picks ``n_hot`` distinct blocks (fixed count, or
  ``max(1, round(hot_frac * NB_b))``) with ``amp ~ U[alpha]``;
  ``bias="lognormal"`` biases every block with ``amp = 0.5 * lognormal(0, 1)``.
* ``qk_sigma`` scales the draws of q and K (q, K ~ N(0, qk_sigma^2); V stays
  N(0, 1)); ``k_outlier = (c, a)`` adds ``a * qk_sigma`` to key channel ``c``
  of every token (one outlier channel). Both are applied to the fp32 draws
  before the block bias.
* Values are fp32 draws rounded to bf16 (round half to even).
* The cache has ``cap = max_b L_b`` rounded up to the block size; rows past
  ``L_b`` are zero, or quiet-NaN when ``poison_tail`` is set (tests use that
  to prove the tail is never read into a result).

These inputs stand in for the long-context workloads the pages evaluate on;
no item of any benchmark suite is reproduced.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Tuple

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round half to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def f32_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload and the selection settings it is run with."""

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    lens: Optional[Tuple[int, ...]] = None          # fixed lengths, one per sequence
    len_range: Optional[Tuple[int, int]] = None     # inclusive range for drawn lengths
    block_size: int = 64
    bias: str = "hot"                               # "hot" | "lognormal" | "none"
    n_hot: Optional[int] = None                     # fixed number of hot blocks
    hot_frac: float = 0.0                           # else fraction of blocks
    alpha: Tuple[float, float] = (2.0, 4.0)         # hot amplitude range (lo == hi: fixed)
    deltas: Tuple[float, ...] = (6.0,)
    sink: int = 1
    local: int = 4
    split_blocks: int = 32
    cap: Optional[int] = None                       # cache capacity; default max len rounded up
    qk_sigma: float = 1.0                           # standard deviation of q and K
    k_outlier: Optional[Tuple[int, float]] = None   # (channel, amplitude in units of qk_sigma)
    diagnostic: str = ""                            # non-empty: not a headline workload; says what it is for

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny_d64_2k": Workload(
        name="tiny_d64_2k", seed=1, B=1, Hq=4, Hkv=1, d=64, lens=(2048,), n_hot=4,
        alpha=(3.0, 3.0), deltas=(8.0, math.inf), sink=1, local=2),
    "llama3_8b_32k": Workload(
        name="llama3_8b_32k", seed=2, B=1, Hq=32, Hkv=8, d=128, lens=(32768,),
        hot_frac=0.02, deltas=(4.0, 8.0), sink=1, local=4),
    "llama3_8b_128k_b4": Workload(
        name="llama3_8b_128k_b4", seed=3, B=4, Hq=32, Hkv=8, d=128, lens=(131072,) * 4,
        hot_frac=0.01, deltas=(6.0,), sink=1, local=4),
    "llama3_8b_256k": Workload(
        name="llama3_8b_256k", seed=4, B=1, Hq=32, Hkv=8, d=128, lens=(262144,),
        hot_frac=0.005, deltas=(2.0, 4.0, 8.0, math.inf), sink=1, local=4),
    "mixed_16x8k_128k": Workload(
        name="mixed_16x8k_128k", seed=5, B=16, Hq=32, Hkv=8, d=128, len_range=(8192, 131072),
        bias="lognormal", deltas=(6.0,), sink=1, local=4),
    # Diagnostic: the 256K head shape with peaked attention (2% of blocks
    # pushed hard toward the group's query), so that Top-δ drops a large,
    # uneven share of the blocks (per split from 1 to all 32 kept); it shows
    # whether time follows the bytes actually read.
    "diag_256k_peaked": Workload(
        name="diag_256k_peaked", seed=6, B=1, Hq=32, Hkv=8, d=128, lens=(262144,),
        hot_frac=0.02, alpha=(6.0, 10.0), deltas=(2.0, 1.0, 4.0, math.inf), sink=1, local=4,
        diagnostic="peaked attention for the skip path (uneven kept counts per split); not a headline workload"),
}


def _unit_group_query(q_bits: np.ndarray, b: int, j: int, G: int) -> np.ndarray:
    qf = f32_from_bf16_bits(q_bits[b, j * G:(j + 1) * G]).astype(np.float64)
    m = qf.mean(axis=0)
    n = np.linalg.norm(m)
    return (m / n if n > 0 else m).astype(np.float32)


def make_inputs(w: Workload, poison_tail: bool = False, threads: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with ``q`` (uint16 bf16 bits ``[B,Hq,d]``), ``k`` and ``v``
    (uint16 ``[B,Hkv,cap,d]``), ``seq_lens`` (int32 ``[B]``), ``cap`` and
    ``biased_blocks`` (per ``(b, j)``: block indices and amplitudes).
    """
    if w.Hq % w.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    root = np.random.SeedSequence(w.seed)
    children = root.spawn(1 + w.B * w.Hkv)
    g0 = np.random.Generator(np.random.PCG64(children[0]))
    if w.lens is not None:
        lens = np.asarray(w.lens, dtype=np.int64)
        if lens.shape != (w.B,):
            raise ValueError("lens must have one entry per sequence")
    elif w.len_range is not None:
        lens = g0.integers(w.len_range[0], w.len_range[1] + 1, size=w.B, dtype=np.int64)
    else:
        raise ValueError("workload needs lens or len_range")
    q32 = g0.standard_normal((w.B, w.Hq, w.d), dtype=np.float32)
    if w.qk_sigma != 1.0:
        q32 = q32 * np.float32(w.qk_sigma)
    q = bf16_bits_from_f32(q32)

    bs = w.block_size
    maxlen = int(lens.max()) if w.B else 0
    cap = w.cap if w.cap is not None else max(bs, -(-maxlen // bs) * bs)
    if cap < maxlen:
        raise ValueError("cap smaller than the longest sequence")
    fill = BF16_QNAN if poison_tail else np.uint16(0)
    k = np.empty((w.B, w.Hkv, cap, w.d), dtype=np.uint16)
    v = np.empty((w.B, w.Hkv, cap, w.d), dtype=np.uint16)
    biased = {}

    def one(bj: int) -> None:
        b, j = divmod(bj, w.Hkv)
        L = int(lens[b])
        g = np.random.Generator(np.random.PCG64(children[1 + bj]))
        K = g.standard_normal((L, w.d), dtype=np.float32)
        V = g.standard_normal((L, w.d), dtype=np.float32)
        if w.qk_sigma != 1.0:
            K *= np.float32(w.qk_sigma)
        if w.k_outlier is not None:
            K[:, w.k_outlier[0]] += np.float32(w.k_outlier[1] * w.qk_sigma)
        nb = -(-L // bs)
        if w.bias == "hot" and nb > 0:
            n_hot = w.n_hot if w.n_hot is not None else max(1, int(round(w.hot_frac * nb)))
            n_hot = min(n_hot, nb)
            picks = np.sort(g.choice(nb, size=n_hot, replace=False))
            lo, hi = w.alpha
            amps = np.full(n_hot, lo, dtype=np.float64) if lo == hi else g.uniform(lo, hi, n_hot)
        elif w.bias == "lognormal" and nb > 0:
            picks = np.arange(nb)
            amps = 0.5 * g.lognormal(0.0, 1.0, nb)
        else:
            picks = np.zeros(0, dtype=np.int64)
            amps = np.zeros(0)
        if len(picks):
            u = _unit_group_query(q, b, j, w.G)
            for p, a in zip(picks, amps):
                K[p * bs:min((p + 1) * bs, L)] += np.float32(a) * u
        k[b, j, :L] = bf16_bits_from_f32(K)
        v[b, j, :L] = bf16_bits_from_f32(V)
        k[b, j, L:] = fill
        v[b, j, L:] = fill
        biased[(b, j)] = (picks, amps)

    n = w.B * w.Hkv
    nthreads = threads or min(16, os.cpu_count() or 1, max(1, n))
    if nthreads > 1 and n > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(n)))
    else:
        for bj in range(n):
            one(bj)
    return {
        "q": q,
        "k": k,
        "v": v,
        "seq_lens": lens.astype(np.int32),
        "cap": cap,
        "biased_blocks": biased,
    }


def make_random_inputs(B: int, Hq: int, Hkv: int, d: int, lens, seed: int, block_size: int = 64,
                       hot_frac: float = 0.05, alpha=(2.0, 4.0), poison_tail: bool = True,
                       cap: Optional[int] = None, qk_sigma: float = 1.0,
                       k_outlier: Optional[Tuple[int, float]] = None) -> dict:
    """Small seeded inputs with arbitrary shapes (test helper)."""
    w = Workload(name="random", seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d,
                 lens=tuple(int(x) for x in lens), block_size=block_size,
                 bias="hot" if hot_frac > 0 else "none", hot_frac=hot_frac, alpha=tuple(alpha),
                 cap=cap, qk_sigma=qk_sigma, k_outlier=k_outlier)
    return make_inputs(w, poison_tail=poison_tail)


def multi_query(inp: dict, Q: int, seed: int, rho: float = 0.8) -> np.ndarray:
    """Q query tokens per sequence for a multi-query step over ``inp``'s cache.

    Token Q-1 (the newest) is ``inp["q"]`` itself, so the workload's hot
    blocks stay aligned with it; the earlier tokens are correlated with it like
    consecutive decode positions: ``rho * q + sqrt(1 - rho^2) * z`` with
    ``z ~ N(0, 1)`` from ``SeedSequence(seed)``, rounded to bf16. Returns bf16
    bits ``[B, Q, Hq, d]``."""
    q = f32_from_bf16_bits(inp["q"])
    B, Hq, d = q.shape
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    out = np.empty((B, Q, Hq, d), dtype=np.uint16)
    for i in range(Q):
        if i == Q - 1:
            out[:, i] = inp["q"]
        else:
            z = rng.standard_normal((B, Hq, d), dtype=np.float32)
            out[:, i] = bf16_bits_from_f32((np.float32(rho) * q + np.float32(math.sqrt(1 - rho * rho)) * z)
                                           .astype(np.float32))
    return out
