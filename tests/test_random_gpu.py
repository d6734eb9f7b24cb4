"""Seeded random sweep over the configuration space, every case against the
oracle (mask bit-exact, out/LSE within the bar): entry point (int4 sketch,
thumbnail storage, paged cache, several query tokens, both of the last two), group size, head dim,
split size up to its maximum of 64 blocks, sink/local counts up to the
sink/local mode's limit, δ from 0 to +inf, the three pseudo-max modes, bf16 and
fp32 output, lengths that are empty, a single token, on block boundaries or
ragged, and cache capacities that are not a whole number of blocks."""

import math

import numpy as np
import pytest
from tests.gpu_util import run_case as _run_case

pytestmark = pytest.mark.gpu

N_CASES = 1024


def _case(i):
    rng = np.random.default_rng(20_000 + i)
    kind = ["int4", "thumb", "paged", "multi"][i % 4]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    Q = 1
    if kind == "multi":
        Q = int(rng.integers(2, 16 // G + 1)) if G < 8 else 2
    B = int(rng.integers(1, 4))
    lens = []
    for _ in range(B):
        r = rng.random()
        if r < 0.1:
            lens.append(0)
        elif r < 0.2:
            lens.append(1)
        elif r < 0.35:
            lens.append(64 * int(rng.integers(1, 40)))
        else:
            lens.append(int(rng.integers(2, 4000)))
    S = int(rng.choice([1, 2, 3, 7, 16, 64]))
    delta = float(rng.choice([0.0, 0.5, 1.0, 2.0, 4.0, math.inf]))
    pm = "sink_local" if (rng.random() < 0.35 and not math.isinf(delta)) else "split"
    sink, local = int(rng.integers(0, 3)), int(rng.integers(0, 5))
    if rng.random() < 0.1:
        sink, local = 30, 33   # the sink/local mode's largest total (64 with the query range)
    if pm == "sink_local" and sink + local == 0:
        local = 1
    out_bf16 = bool(rng.random() < 0.25)
    # (drawn last, so the draws above are those of the earlier sweep)
    odd_cap = bool(rng.random() < 0.3) and kind != "paged"
    cap_extra = int(rng.integers(0, 6))
    if pm == "sink_local" and rng.random() < 0.4:
        pm = "max"   # the larger of the split max and the sink/local estimate
    if kind == "paged" and rng.random() < 0.5:
        Q = int(rng.integers(2, 16 // G + 1)) if G < 8 else 2   # several query tokens over the pages
    return dict(kind=kind, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, Q=Q, lens=tuple(lens), S=S, delta=delta, pm=pm,
                sink=sink, local=local, out_bf16=out_bf16, odd_cap=odd_cap, cap_extra=cap_extra, seed=30_000 + i)


def _case_four_waves(i):
    """A case on a grid of more than 1024 (sequence, query head, split) units,
    where the kernel runs 4-wave workgroups (smaller grids run 8-wave ones):
    three ragged sequences, 16 or 32 query heads, one-block splits."""
    rng = np.random.default_rng(40_000 + i)
    kind = ["int4", "thumb", "paged", "multi"][i % 4]
    G = int(rng.choice([2, 4, 8]))
    Hkv = 8 if G == 2 else 4
    d = int(rng.choice([64, 128]))
    Q = (int(rng.integers(2, 16 // G + 1)) if G < 8 else 2) if kind == "multi" else 1
    lens = tuple(int(x) for x in rng.integers(1500, 4000, size=3))
    delta = float(rng.choice([0.0, 1.0, 2.0, 4.0, math.inf]))
    pm = str(rng.choice(["split", "sink_local", "max"])) if not math.isinf(delta) else "split"
    sink, local = int(rng.integers(0, 3)), int(rng.integers(1, 5))
    c = dict(kind=kind, B=3, Hq=G * Hkv, Hkv=Hkv, d=d, Q=Q, lens=lens, S=1, delta=delta, pm=pm, sink=sink,
             local=local, out_bf16=bool(rng.random() < 0.25), odd_cap=False, cap_extra=0, seed=45_000 + i)
    ns = -(-max(lens) // 64)
    assert c["B"] * c["Hq"] * ns > 1024
    return c


@pytest.mark.parametrize("i", range(64))
def test_random_case_four_waves(i):
    _run_case(_case_four_waves(i), f"4-wave {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _run_case(_case(i), str(i))
