"""Run the oracle over whole (sequence, kv head) groups in a thread pool and
merge the rows: the same function on the same inputs, so the result is the
oracle's own, only computed faster (NumPy releases the GIL in its array
loops). Test infrastructure."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import ffd_oracle as O


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def decode(q, k, v, seq_lens, **kw):
    """``O.decode`` on every row, one task per (sequence, kv head) group."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = Hq // Hkv

    def one(bj):
        b, j = bj
        hs = [(b, h) for h in range(j * G, (j + 1) * G)]
        return bj, O.decode(q, k, v, seq_lens, heads=hs, **kw)

    groups = [(b, j) for b in range(B) for j in range(Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(one, groups))
    out = lse = mask = None
    for (b, j), (o, l_, m) in parts:
        if out is None:
            out, lse, mask = np.full_like(o, np.nan), np.full_like(l_, np.nan), np.zeros_like(m)
        sl = slice(j * G, (j + 1) * G)
        out[b, sl], lse[b, sl], mask[b, sl] = o[b, sl], l_[b, sl], m[b, sl]
    return out, lse, mask


def decode_multi(q, k, v, seq_lens, **kw):
    """``O.decode_multi`` on every row, one task per (sequence, kv head) group."""
    B, Q, Hq = q.shape[:3]
    Hkv = k.shape[1]
    G = Hq // Hkv

    def one(bj):
        b, j = bj
        rows = [(b, i, h) for i in range(Q) for h in range(j * G, (j + 1) * G)]
        return bj, O.decode_multi(q, k, v, seq_lens, heads=rows, **kw)

    groups = [(b, j) for b in range(B) for j in range(Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(one, groups))
    out = lse = mask = None
    for (b, j), (o, l_, m) in parts:
        if out is None:
            out, lse, mask = np.full_like(o, np.nan), np.full_like(l_, np.nan), np.zeros_like(m)
        sl = slice(j * G, (j + 1) * G)
        out[b, :, sl], lse[b, :, sl], mask[b, :, sl] = o[b, :, sl], l_[b, :, sl], m[b, :, sl]
    return out, lse, mask
