"""Pins of the oracle's thumbnail + residual key storage: a hand-worked
example, nearest-level and error-bound properties against brute force,
packing, the scan dot, and attention over the reconstructed keys."""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from ffd_inputs import f32_from_bf16_bits, make_random_inputs
from oracle import ffd_oracle as O

SET = settings(max_examples=25, deadline=None)


def test_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "hand_thumb.json")) as f:
        g = json.load(f)
    k = np.array(g["keys"], np.float32)
    u, t, r8, s8 = O.quantize_keys_thumb(k)
    assert u.tolist() == g["u"]
    assert t.tolist() == g["t"]
    assert r8.tolist() == g["r8"]
    for i, flag in enumerate(g["s8_is_2_over_127"]):
        assert (s8[i] == np.float32(np.float32(2) / np.float32(127))) == flag
        if not flag:
            assert s8[i] == 0
    khat = O.reconstruct_thumb(u, t, r8, s8)
    np.testing.assert_array_equal(khat[0], k[0])
    np.testing.assert_array_equal(khat[2], k[2])
    assert khat[1, 3] == 2 - 127 * float(np.float32(np.float32(2) / np.float32(127)))
    qc, cq = O.quantize_query(np.array([1, 0, 0, 0], np.float32), np.float32(1))
    assert O.thumb_token_scores(qc, cq, u, t).tolist() == g["scores"]
    assert O.pack_2bit(u).ravel().tolist() == g["packed"]


@SET
@given(seed=st.integers(0, 10_000), e=st.integers(-30, 30))
def test_levels_residual_and_reconstruction_bounds(seed, e):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((12, 64)) * 2.0 ** e).astype(np.float32)
    k[0] = 0
    u, t, r8, s8 = O.quantize_keys_thumb(k)
    assert (u <= 3).all() and (np.abs(r8.astype(int)) <= 127).all()
    assert t[0] == 0 and s8[0] == 0 and (r8[0] == 0).all()
    amax = np.abs(k).max(1)
    lev = (2 * u.astype(np.float64) - 3) * t[:, None]
    # nearest level, by brute force over the four candidates (ties excepted)
    for r in range(1, 12):
        cand = np.array([-3, -1, 1, 3], np.float64) * float(t[r])
        dist = np.abs(k[r].astype(np.float64)[:, None] - cand[None, :])
        best = dist.min(1)
        assert (np.abs(k[r] - lev[r]) <= best + float(t[r]) * 1e-6).all()
        assert abs(float(t[r]) - float(amax[r]) / 3) <= float(amax[r]) / 3 * 2 ** -23
        # residual: |r - s8 r8| <= s8/2, its amax maps to +-127
        res = k[r].astype(np.float64) - np.float32(lev[r]).astype(np.float64)
        if s8[r] > 0:
            assert (np.abs(res - float(s8[r]) * r8[r]) <= float(s8[r]) * 0.5 * (1 + 1e-6) + 1e-30).all()
            assert np.abs(r8[r]).max() == 127
    khat = O.reconstruct_thumb(u, t, r8, s8)
    bound = s8.astype(np.float64)[:, None] * 0.5 * (1 + 1e-5) + np.abs(k) * 2.0 ** -22 + 1e-300
    assert (np.abs(khat - k) <= bound).all()
    # the residual is small next to the key: at most a level step (2t)
    assert (s8 * 127 <= t * 2 * (1 + 1e-6) + 1e-38).all()


def test_pack_2bit_roundtrip():
    vals = np.array(np.meshgrid(*[np.arange(4)] * 4, indexing="ij")).reshape(4, -1).T.astype(np.uint8)
    packed = O.pack_2bit(vals)
    assert sorted(packed.ravel().tolist()) == list(range(256))
    np.testing.assert_array_equal(O.unpack_2bit(packed), vals)


def test_thumb_dot_is_exact_integer():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 4, size=(40, 128)).astype(np.uint8)
    qc = rng.integers(-127, 128, size=128).astype(np.int8)
    tok = O.thumb_token_scores(qc, np.float32(1), u, np.ones(40, np.float32))
    brute = [sum(int(a) * (2 * int(c) - 3) for a, c in zip(qc, row)) for row in u]
    assert tok.tolist() == [float(x) for x in brute]


def test_dense_limit_over_reconstructed_keys():
    """δ = inf keeps every block; the thumb decode then equals torch's
    attention over K^ (built from the stored codes, residuals and scales)."""
    inp = make_random_inputs(2, 8, 2, 64, (300, 77), seed=3, block_size=16)
    sm = np.float32(0.125)
    out, lse, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=16,
                              delta=math.inf, sink=0, local=0, split_blocks=4, sm_scale=sm, storage="thumb")
    k2, t, kr, s8 = O.quantize_cache_thumb(inp["k"], inp["seq_lens"])
    for b, L in enumerate(inp["seq_lens"]):
        u = O.unpack_2bit(k2[b, :, :L])
        khat = (2.0 * u - 3.0) * t[b, :, :L, None].astype(np.float64) + s8[b, :, :L, None].astype(np.float64) * kr[b, :, :L]
        kt = torch.from_numpy(khat).repeat_interleave(4, 0)
        vt = torch.from_numpy(f32_from_bf16_bits(inp["v"][b, :, :L]).astype(np.float64)).repeat_interleave(4, 0)
        qt = torch.from_numpy(f32_from_bf16_bits(inp["q"][b]).astype(np.float64))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(sm))[:, 0].numpy()
        np.testing.assert_allclose(out[b], ref, atol=1e-12)
        assert mask[b, :, :-(-int(L) // 16)].all()


def test_thumb_attention_close_to_exact_keys():
    """K^ is within half a residual step of K, so attention over K^ stays close
    to attention over the exact keys (loose, scale-aware bound)."""
    inp = make_random_inputs(1, 4, 1, 128, (2048,), seed=4, block_size=64)
    kw = dict(max_seq_len=2048, block_size=64, delta=math.inf, sink=0, local=0, split_blocks=32)
    a = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], storage="thumb", **kw)
    b = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], quantize=False, **kw)
    assert np.abs(a[0] - b[0]).max() < 5e-3
    assert np.abs(a[1] - b[1]).max() < 5e-3


@SET
@given(seed=st.integers(0, 10_000), d1=st.floats(0, 5), d2=st.floats(0, 5))
def test_thumb_selection_monotone(seed, d1, d2):
    lo, hi = sorted((d1, d2))
    inp = make_random_inputs(1, 2, 1, 32, (int(np.random.default_rng(seed).integers(1, 200)),), seed=seed,
                             block_size=8, hot_frac=0.1)
    kw = dict(max_seq_len=inp["cap"], block_size=8, sink=1, local=1, split_blocks=3, storage="thumb",
              mask_only=True)
    m1 = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=lo, **kw)[2]
    m2 = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], delta=hi, **kw)[2]
    assert (m1 <= m2).all()
