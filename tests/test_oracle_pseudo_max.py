"""The sink/local pseudo-max modes of the oracle: a hand-worked 3-block
example, independence from the split size, monotonicity in δ, the
brute-force token rule with m~ taken over the sink and local tokens, and the
"max" mode (the larger of the split max and the sink/local estimate) keeping
exactly the blocks both other modes keep."""

import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from ffd_inputs import bf16_bits_from_f32, f32_from_bf16_bits, make_random_inputs
from oracle import ffd_oracle as O

SET = settings(max_examples=25, deadline=None)


@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_3block_sink_local.json")) as f:
        return json.load(f)


def test_block_scores(hand):
    k = np.array(hand["inputs"]["k"], np.float32)[0, 0]
    codes, scale = O.quantize_keys(k)
    qc, cq = O.quantize_query(np.array([1.0, 0.0], np.float32), np.float32(1))
    tok = O.token_scores(qc, cq, codes, scale)
    assert O.block_scores(tok, 6, 2).tolist() == hand["block_scores"]


@pytest.mark.parametrize("idx", range(10))
def test_cases(hand, idx):
    c = hand["cases"][idx]
    inp = hand["inputs"]
    f = lambda a: bf16_bits_from_f32(np.array(a, np.float32))
    out, lse, mask = O.decode(f(inp["q"]), f(inp["k"]), f(inp["v"]), np.array(inp["seq_lens"]), max_seq_len=6,
                              block_size=2, delta=c["delta"], sink=c["sink"], local=c["local"],
                              split_blocks=c["split_blocks"], sm_scale=np.float32(1), pseudo_max=c["pseudo_max"])
    assert mask[0, 0].tolist() == c["mask"]
    env = {"e2": math.exp(2.0), "e1": math.e, "ln": math.log}
    cf = hand["closed_forms"][c["out"]]
    np.testing.assert_allclose(out[0, 0], [eval(x, {}, env) for x in cf["out"]], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - eval(cf["lse"], {}, env)) < 1e-14


def test_needs_a_sink_or_local_block():
    with pytest.raises(ValueError):
        O.select_blocks(np.zeros(4, np.float32), 2, 1.0, 0, 0, "sink_local")


def _case(seed, L=None):
    rng = np.random.default_rng(seed)
    L = L or int(rng.integers(1, 240))
    return make_random_inputs(1, 2, 1, 32, (L,), seed=seed, block_size=8, hot_frac=0.15), L


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0, 4), sink=st.integers(0, 2), local=st.integers(0, 3))
def test_independent_of_split_size(seed, delta, sink, local):
    if sink + local == 0:
        local = 1
    inp, L = _case(seed)
    masks = [O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=8,
                      delta=delta, sink=sink, local=local, split_blocks=S, pseudo_max="sink_local",
                      mask_only=True)[2] for S in (1, 3, 64)]
    np.testing.assert_array_equal(masks[0], masks[1])
    np.testing.assert_array_equal(masks[0], masks[2])


@SET
@given(seed=st.integers(0, 10_000), d1=st.floats(0, 5), d2=st.floats(0, 5))
def test_monotone_in_delta(seed, d1, d2):
    lo, hi = sorted((d1, d2))
    inp, L = _case(seed)
    kw = dict(max_seq_len=inp["cap"], block_size=8, sink=1, local=2, split_blocks=4, pseudo_max="sink_local",
              mask_only=True)
    m_lo = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=lo, **kw)[2]
    m_hi = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=hi, **kw)[2]
    assert (m_lo <= m_hi).all()


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0, 4), sink=st.integers(0, 2), local=st.integers(1, 3))
def test_token_rule_with_sink_local_peak(seed, delta, sink, local):
    """Brute force over tokens: m~ = best token score among the sink and local
    blocks; a block is kept iff one of its tokens reaches m~ - δ or it is forced."""
    bs = 8
    inp, L = _case(seed)
    sm = np.float32(1 / math.sqrt(32))
    mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=bs,
                    delta=delta, sink=sink, local=local, split_blocks=2, sm_scale=sm, pseudo_max="sink_local",
                    mask_only=True)[2]
    codes, scale = O.quantize_keys(f32_from_bf16_bits(inp["k"][0, 0, :L]))
    nb = -(-L // bs)
    forced = [j < sink or j >= nb - local for j in range(nb)]
    for h in range(2):
        qc, cq = O.quantize_query(f32_from_bf16_bits(inp["q"][0, h]), sm)
        tok = O.token_scores(qc, cq, codes, scale)
        peak = max(tok[t] for t in range(L) if forced[t // bs])
        thr = np.float32(np.float32(peak) - np.float32(delta))
        for j in range(nb):
            want = forced[j] or any(tok[t] >= thr for t in range(j * bs, min(j * bs + bs, L)))
            assert bool(mask[0, h, j]) == want


def test_splits_may_keep_nothing_and_attention_stays_exact():
    """With the sink/local peak a whole split can be dropped; the output is
    still exact softmax attention over the kept tokens (checked against a
    direct fp64 computation over the kept rows)."""
    inp, L = _case(7, L=8 * 40)
    # make the sink block dominant so that middle splits fall below m~ - δ
    k = f32_from_bf16_bits(inp["k"]).copy()
    qv = f32_from_bf16_bits(inp["q"][0]).mean(0)
    k[0, 0, :8] += 6.0 * qv / np.linalg.norm(qv)
    kb = bf16_bits_from_f32(k)
    sm = np.float32(1 / math.sqrt(32))
    out, lse, mask = O.decode(inp["q"], kb, inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=8,
                              delta=1.0, sink=1, local=1, split_blocks=4, sm_scale=sm, pseudo_max="sink_local")
    empty_splits = [(h, s) for h in range(2) for s in range(10) if not mask[0, h, 4 * s:4 * s + 4].any()]
    assert empty_splits, "the construction should drop at least one whole split"
    for h in range(2):
        keep = np.repeat(mask[0, h].astype(bool), 8)[:L]
        kk = f32_from_bf16_bits(kb[0, 0, :L]).astype(np.float64)[keep]
        vv = f32_from_bf16_bits(inp["v"][0, 0, :L]).astype(np.float64)[keep]
        z = float(sm) * kk @ f32_from_bf16_bits(inp["q"][0, h]).astype(np.float64)
        p = np.exp(z - z.max())
        np.testing.assert_allclose(out[0, h], p @ vv / p.sum(), atol=1e-12)
        assert abs(lse[0, h] - (z.max() + math.log(p.sum()))) < 1e-12


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0, 4), sink=st.integers(0, 2), local=st.integers(0, 3),
       S=st.integers(1, 6))
def test_max_mode_keeps_what_both_modes_keep(seed, delta, sink, local, S):
    """fl32(m - δ) is monotone in m, so the threshold of max(m_split, m_sl) is
    the larger of the two thresholds and a block passes it iff it passes both:
    the kept set of "max" is the intersection of the other two (forced blocks
    in all three)."""
    if sink + local == 0:
        local = 1
    inp, L = _case(seed)
    kw = dict(max_seq_len=L, block_size=8, delta=np.float32(delta), sink=sink, local=local, split_blocks=S,
              sm_scale=np.float32(0.25), mask_only=True)
    masks = {pm: O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], pseudo_max=pm, **kw)[2]
             for pm in ("split", "sink_local", "max")}
    np.testing.assert_array_equal(masks["max"], masks["split"] & masks["sink_local"])


def test_max_mode_multi_query():
    """The same identity per query token with several tokens per sequence."""
    inp, L = _case(77, L=300)
    from ffd_inputs import multi_query
    qm = multi_query(inp, 3, seed=78)
    kw = dict(max_seq_len=L, block_size=8, delta=0.7, sink=1, local=2, split_blocks=4, sm_scale=np.float32(0.25),
              mask_only=True)
    masks = {pm: O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], pseudo_max=pm, **kw)[2]
             for pm in ("split", "sink_local", "max")}
    np.testing.assert_array_equal(masks["max"], masks["split"] & masks["sink_local"])
    assert (masks["max"] != masks["split"]).any() or (masks["max"] != masks["sink_local"]).any()
