"""Cases with large logits, shared by the CPU check that they reach the
regime where the scan's estimate overshoots the exact logits by more than
fp32's exponent range (tests/test_seed_gap.py) and the GPU parity test over
every decode entry point (tests/test_large_logits_gpu.py).

q and K are drawn N(0, sigma^2) (V stays N(0, 1)); with ``outlier`` one key
channel is offset by 30 sigma, which makes the low-bit codes of the other
channels coarse. Plain Python: no torch here."""

import math

SIGMAS = (4.0, 8.0, 16.0, 32.0, 64.0)
OUTLIERS = (None, (5, 30.0))
# entry point, group size, query tokens
KINDS = (("int4", 4, 1), ("thumb", 4, 1), ("paged", 4, 1), ("multi", 4, 2), ("paged", 2, 4))


def case(kind: str, G: int, Q: int, sigma: float, outlier, pm: str, delta: float = 6.0, seed: int = 0) -> dict:
    """A run_case dict: two ragged sequences of several 16-block splits, two kv heads."""
    return dict(kind=kind, B=2, Hq=2 * G, Hkv=2, d=128, Q=Q, lens=(2900, 4100), S=16, delta=delta, pm=pm,
                sink=1, local=2, out_bf16=False, odd_cap=False, cap_extra=0,
                seed=70_000 + seed, sigma=sigma, outlier=outlier)


def all_cases():
    """(test id, case) for every combination; dense (delta = inf) only on the int4 path."""
    out = []
    n = 0
    for kind, G, Q in KINDS:
        for sigma in SIGMAS:
            for outlier in OUTLIERS:
                for pm in ("split", "sink_local"):
                    name = f"{kind}-G{G}-Q{Q}-s{sigma:g}-{'outlier' if outlier else 'plain'}-{pm}"
                    out.append((name, case(kind, G, Q, sigma, outlier, pm, seed=n)))
                    n += 1
    for sigma in SIGMAS:
        for outlier in OUTLIERS:
            name = f"dense-s{sigma:g}-{'outlier' if outlier else 'plain'}"
            out.append((name, case("int4", 4, 1, sigma, outlier, "split", delta=math.inf, seed=n)))
            n += 1
    return out
