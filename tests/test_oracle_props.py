"""Invariants that pin the oracle's quantiser, scan and Top-δ selection.

Each test states a fact that follows from the method's definition, not from
the oracle's code: the kept set grows with δ, every split keeps its argmax
block, the block rule equals the token rule, the quantisers meet their error
bounds, dropped tokens sit below the threshold, and splits do not interact.
"""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from ffd_inputs import f32_from_bf16_bits, make_random_inputs
from oracle import ffd_oracle as O

SET = settings(max_examples=25, deadline=None)


def _rand_case(seed, d=32, bs=8, L=None, G=2):
    rng = np.random.default_rng(seed)
    L = L or int(rng.integers(1, 200))
    inp = make_random_inputs(1, G, 1, d, (L,), seed=seed, block_size=bs, hot_frac=0.1)
    return inp, L


# ---------------------------------------------------------------- selection

@SET
@given(seed=st.integers(0, 10_000), d1=st.floats(0, 6), d2=st.floats(0, 6),
       S=st.integers(1, 9), sink=st.integers(0, 2), local=st.integers(0, 2))
def test_kept_set_monotone_in_delta(seed, d1, d2, S, sink, local):
    lo, hi = sorted((d1, d2))
    inp, L = _rand_case(seed)
    args = dict(max_seq_len=inp["cap"], block_size=8, sink=sink, local=local, split_blocks=S)
    _, _, m_lo = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=lo, **args)
    _, _, m_hi = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=hi, **args)
    assert (m_lo <= m_hi).all()


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0, 4), S=st.integers(1, 9))
def test_every_split_keeps_its_best_block(seed, delta, S):
    inp, L = _rand_case(seed)
    _, _, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                          block_size=8, delta=delta, sink=0, local=0, split_blocks=S)
    nb = -(-L // 8)
    for h in range(mask.shape[1]):
        for s0 in range(0, nb, S):
            assert mask[0, h, s0:min(s0 + S, nb)].any()


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0, 5), S=st.integers(1, 6),
       sink=st.integers(0, 3), local=st.integers(0, 3))
def test_block_rule_equals_token_rule(seed, delta, S, sink, local):
    """Brute force over tokens: a block is kept iff one of its tokens reaches the
    split's best token score minus δ, or it is a sink/local block."""
    bs = 8
    inp, L = _rand_case(seed, bs=bs)
    sm = np.float32(1 / math.sqrt(32))
    _, _, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                          block_size=bs, delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=sm)
    k32 = f32_from_bf16_bits(inp["k"][0, 0, :L])
    codes, scale = O.quantize_keys(k32)
    nb = -(-L // bs)
    for h in range(2):
        qc, cq = O.quantize_query(f32_from_bf16_bits(inp["q"][0, h]), sm)
        tok = O.token_scores(qc, cq, codes, scale)
        for j in range(nb):
            s0 = (j // S) * S * bs
            s1 = min(s0 + S * bs, L)
            thr = np.float32(np.max(tok[s0:s1]) - np.float32(delta))
            want = any(tok[t] >= thr for t in range(j * bs, min(j * bs + bs, L)))
            want = want or j < sink or j >= nb - local
            assert bool(mask[0, h, j]) == want


def test_splits_do_not_interact():
    """Changing every key of one split leaves the other splits' masks alone."""
    inp, L = _rand_case(3, L=8 * 12)
    args = dict(max_seq_len=inp["cap"], block_size=8, delta=1.0, sink=0, local=0, split_blocks=4)
    _, _, m0 = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **args)
    k2 = inp["k"].copy()
    k2[0, 0, 32:64] = inp["k"][0, 0, 64:96][::-1]
    _, _, m1 = O.decode(inp["q"], k2, inp["v"], inp["seq_lens"], **args)
    np.testing.assert_array_equal(m0[..., :4], m1[..., :4])
    np.testing.assert_array_equal(m0[..., 8:], m1[..., 8:])


def test_sink_and_local_forced():
    inp, L = _rand_case(4, L=8 * 20)
    _, _, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                          block_size=8, delta=0.0, sink=2, local=3, split_blocks=5)
    assert mask[0, :, :2].all() and mask[0, :, 17:20].all()


@SET
@given(seed=st.integers(0, 10_000), delta=st.floats(0.5, 6), S=st.integers(1, 9))
def test_dropped_tokens_are_below_peak_by_delta(seed, delta, S):
    """δ semantics: every token of a dropped block scores below m~ - δ, and its
    exact logit is within the scan's error bound of that score, so its exact
    weight relative to the split's best token is below exp(-δ + 2·eps)."""
    bs = 8
    d = 32
    inp, L = _rand_case(seed, bs=bs)
    sm = np.float32(1 / math.sqrt(d))
    _, _, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                          block_size=bs, delta=delta, sink=0, local=0, split_blocks=S, sm_scale=sm)
    k32 = f32_from_bf16_bits(inp["k"][0, 0, :L])
    codes, scale = O.quantize_keys(k32)
    for h in range(2):
        q32 = f32_from_bf16_bits(inp["q"][0, h])
        qc, cq = O.quantize_query(q32, sm)
        tok = O.token_scores(qc, cq, codes, scale)
        z = float(sm) * (k32.astype(np.float64) @ q32.astype(np.float64))
        sq = float(np.max(np.abs(q32))) / 127
        eps = float(sm) * sq * scale.astype(np.float64) * (
            0.5 * np.abs(qc).sum() + 0.5 * np.abs(codes).sum(1) + d / 4) * (1 + 1e-5) + np.abs(tok) * 1e-6
        assert (np.abs(z - tok) <= eps + 1e-12).all()
        nb = -(-L // bs)
        for s0 in range(0, nb, S):
            t0, t1 = s0 * bs, min((s0 + S) * bs, L)
            peak = np.max(tok[t0:t1])
            zmax = np.max(z[t0:t1])
            e = np.max(eps[t0:t1])
            for j in range(s0, min(s0 + S, nb)):
                if mask[0, h, j]:
                    continue
                tt = slice(j * bs, min(j * bs + bs, L))
                assert (tok[tt] < np.float32(peak - np.float32(delta))).all()
                assert (z[tt] - zmax < -delta + 2 * e + 1e-9).all()


# ---------------------------------------------------------------- quantisers

@SET
@given(seed=st.integers(0, 10_000), scale_exp=st.integers(-20, 20))
def test_key_quantiser_error_bound(seed, scale_exp):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((16, 64)) * 2.0 ** scale_exp).astype(np.float32)
    k[0] = 0
    codes, scale = O.quantize_keys(k)
    assert codes.dtype == np.int8 and (np.abs(codes) <= 7).all()
    assert scale[0] == 0 and (codes[0] == 0).all()
    amax = np.abs(k).max(1)
    rec = scale[:, None].astype(np.float64) * codes
    assert (np.abs(k - rec) <= scale[:, None] * 0.5 * (1 + 1e-6) + 1e-45).all()
    for r in range(1, 16):
        i = int(np.argmax(np.abs(k[r])))
        assert codes[r, i] == 7 * np.sign(k[r, i])
        assert abs(float(scale[r]) - float(amax[r]) / 7) <= float(amax[r]) / 7 * 2 ** -23


@SET
@given(seed=st.integers(0, 10_000))
def test_query_quantiser_error_bound(seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(128).astype(np.float32)
    sm = np.float32(0.0883883476)
    qc, cq = O.quantize_query(q, sm)
    sq = float(np.abs(q).max()) / 127
    assert qc.dtype == np.int8 and (np.abs(qc) <= 127).all()
    assert abs(int(qc[np.argmax(np.abs(q))])) == 127
    assert (np.abs(q - sq * qc.astype(np.float64)) <= sq * 0.5 * (1 + 1e-6)).all()
    assert abs(float(cq) - sq * float(sm)) <= sq * float(sm) * 2 ** -22
    zc, zcq = O.quantize_query(np.zeros(8, np.float32), sm)
    assert (zc == 0).all() and zcq == 0


def test_rounding_is_half_to_even():
    # amax 7 -> inv = 1, so codes are rne(k): 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2
    k = np.array([[0.5, 1.5, 2.5, -2.5, 7.0, -3.5]], np.float32)
    codes, scale = O.quantize_keys(k)
    assert codes[0].tolist() == [0, 2, 2, -2, 7, -4]
    assert scale[0] == np.float32(1.0)


def test_pack_unpack_roundtrip_all_pairs():
    vals = np.arange(-8, 8, dtype=np.int8)
    a, b = np.meshgrid(vals, vals, indexing="ij")
    codes = np.stack([a.ravel(), b.ravel()], 1)
    packed = O.pack_int4(codes)
    assert packed.shape == (256, 1)
    assert sorted(packed.ravel().tolist()) == list(range(256))
    np.testing.assert_array_equal(O.unpack_int4(packed), codes)
    # element 0 in the low nibble, element 1 in the high nibble, two's complement
    assert O.pack_int4(np.array([1, -1], np.int8)).tolist() == [0xF1]
    assert O.pack_int4(np.array([-8, 3], np.int8)).tolist() == [0x38]


def test_scan_dot_is_exact_integer():
    rng = np.random.default_rng(0)
    codes = rng.integers(-7, 8, size=(50, 128)).astype(np.int8)
    qc = rng.integers(-127, 128, size=128).astype(np.int8)
    scale = np.ones(50, np.float32)
    tok = O.token_scores(qc, np.float32(1), codes, scale)
    brute = [sum(int(a) * int(b) for a, b in zip(row, qc)) for row in codes]
    assert tok.tolist() == [float(x) for x in brute]
    extreme = np.full((1, 128), 7, np.int8)
    assert O.token_scores(np.full(128, -127, np.int8), np.float32(1), extreme, np.ones(1, np.float32))[0] \
        == -127 * 7 * 128


# ---------------------------------------------------------------- attention

@SET
@given(seed=st.integers(0, 10_000), cut=st.integers(1, 49))
def test_lse_merge_of_a_partition_equals_single_pass(seed, cut):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(16)
    k = rng.standard_normal((50, 16)) * 2
    v = rng.standard_normal((50, 16))
    o, s = O.attend(q, k, v, 0.7)
    o1, s1 = O.attend(q, k[:cut], v[:cut], 0.7)
    o2, s2 = O.attend(q, k[cut:], v[cut:], 0.7)
    m = max(s1, s2)
    lse = m + math.log(math.exp(s1 - m) + math.exp(s2 - m))
    out = math.exp(s1 - lse) * o1 + math.exp(s2 - lse) * o2
    assert abs(lse - s) < 1e-12
    np.testing.assert_allclose(out, o, atol=1e-12)
    # one key: weight 1, out = that value, lse = its logit
    o1k, s1k = O.attend(q, k[:1], v[:1], 0.7)
    np.testing.assert_allclose(o1k, v[0], atol=1e-15)
    assert abs(s1k - 0.7 * float(k[0] @ q)) < 1e-12


def test_tiny_rows_are_zero_rows():
    """Rows whose amax is too small for fl32(QMAX/amax) to stay finite are zero rows."""
    tiny = np.float32(2.0 ** -126)
    ok = np.float32(2.0 ** -125)
    k = np.array([[tiny, -tiny / 2, 0, 0], [ok, -ok, 0, ok / 2]], np.float32)
    codes, scale = O.quantize_keys(k)
    assert (codes[0] == 0).all() and scale[0] == 0
    assert codes[1].tolist() == [7, -7, 0, 4] and np.isfinite(np.float32(7) / ok)
    assert scale[1] == np.float32(ok / np.float32(7))
    qc, cq = O.quantize_query(np.array([2.0 ** -121, 0], np.float32), np.float32(1))
    assert (qc == 0).all() and cq == 0
    qc, cq = O.quantize_query(np.array([2.0 ** -120, 0], np.float32), np.float32(1))
    assert qc.tolist() == [127, 0] and cq > 0
