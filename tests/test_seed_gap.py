"""The large-logit GPU cases reach the regime they are there for: on their
inputs, the oracle's own scan puts a split's maximum score (the value that
seeds the softmax's running max) above every exact logit of that split's
kept tokens by more than fp32's exponent range (about 87 nats down to the
smallest normal weight, 103 to the smallest denormal), so a running max that
kept the seed would flush every weight of the split to zero."""

import math

import numpy as np
import pytest

from ffd_inputs import make_random_inputs
from oracle import ffd_oracle as O
from tests.large_logit_cases import all_cases


def _largest_gap(c):
    """Largest (seed - max exact kept logit) over the heads and splits of query token 0."""
    inp = make_random_inputs(c["B"], c["Hq"], c["Hkv"], c["d"], c["lens"], seed=c["seed"], block_size=64,
                             hot_frac=0.08, qk_sigma=c["sigma"], k_outlier=c["outlier"])
    G = c["Hq"] // c["Hkv"]
    sm = np.float32(1.0 / math.sqrt(c["d"]))
    storage = "thumb" if c["kind"] == "thumb" else "int4"
    _, _, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=64,
                          delta=c["delta"], sink=c["sink"], local=c["local"], split_blocks=c["S"], sm_scale=sm,
                          pseudo_max=c["pm"], storage=storage, mask_only=True)
    worst = -math.inf
    for b in range(c["B"]):
        L = int(inp["seq_lens"][b])
        for h in range(c["Hq"]):
            j = h // G
            q32 = O.bf16_bits_to_f32(inp["q"][b, h])
            k32 = O.bf16_bits_to_f32(inp["k"][b, j, :L])
            qc, cq = O.quantize_query(q32, sm)
            if storage == "thumb":
                u, t, r8, s8 = O.quantize_keys_thumb(k32)
                tok = O.thumb_token_scores(qc, cq, u, t)
                kx = O.reconstruct_thumb(u, t, r8, s8)
            else:
                codes, scale = O.quantize_keys(k32)
                tok = O.token_scores(qc, cq, codes, scale)
                kx = k32.astype(np.float64)
            z = float(sm) * (kx @ q32.astype(np.float64))
            nb = -(-L // 64)
            keep_tok = np.repeat(mask[b, h, :nb].astype(bool), 64)[:L]
            for s0 in range(0, L, 64 * c["S"]):
                sl = slice(s0, min(L, s0 + 64 * c["S"]))
                if keep_tok[sl].any():
                    worst = max(worst, float(tok[sl].max()) - float(z[sl][keep_tok[sl]].max()))
    return worst


@pytest.mark.parametrize("kind", ["int4", "thumb"])
def test_cases_overshoot_past_fp32_range(kind):
    cases = [c for _, c in all_cases() if c["kind"] == kind and c["pm"] == "split"]
    gaps = [_largest_gap(c) for c in cases]
    # the hardest cases overshoot by far more than exp can span in fp32
    assert max(gaps) > 200.0, gaps
    assert sum(g > 104.0 for g in gaps) >= 3, gaps
