"""Dense limits of the oracle against a library attention routine.

With δ = +inf and no quantisation, FFD keeps every block, so the oracle must
equal plain softmax attention; torch's scaled_dot_product_attention (fp64, CPU)
is the independent routine it is compared with.
"""

import math

import numpy as np
import pytest
import torch

from ffd_inputs import f32_from_bf16_bits, make_random_inputs
from oracle import ffd_oracle as O


def _dense_ref(inp, max_seq_len, sm_scale):
    q, k, v, lens = inp["q"], inp["k"], inp["v"], inp["seq_lens"]
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        L = min(int(lens[b]), max_seq_len)
        if L <= 0:
            continue
        qt = torch.from_numpy(f32_from_bf16_bits(q[b]).astype(np.float64))[:, None, :]   # [Hq,1,d]
        kt = torch.from_numpy(f32_from_bf16_bits(k[b, :, :L]).astype(np.float64)).repeat_interleave(G, 0)
        vt = torch.from_numpy(f32_from_bf16_bits(v[b, :, :L]).astype(np.float64)).repeat_interleave(G, 0)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(sm_scale))
        out[b] = o[:, 0].numpy()
        lse[b] = torch.logsumexp(float(sm_scale) * (qt @ kt.transpose(1, 2))[:, 0], dim=-1).numpy()
    return out, lse


SHAPES = [
    (1, 4, 1, 64, (2048,), 64),
    (2, 8, 2, 32, (100, 37), 16),
    (3, 6, 3, 16, (1, 64, 130), 32),
    (2, 2, 2, 8, (5, 0), 4),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,lens,bs", SHAPES)
def test_unquantised_infinite_delta_is_dense(B, Hq, Hkv, d, lens, bs):
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=11, block_size=bs)
    msl = inp["cap"]
    sm = np.float32(1.0 / math.sqrt(d))
    out, lse, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=msl,
                              block_size=bs, delta=math.inf, sink=0, local=0, split_blocks=3,
                              sm_scale=sm, quantize=False)
    ref_out, ref_lse = _dense_ref(inp, msl, sm)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-12)
    for b in range(B):
        nb = -(-min(int(inp["seq_lens"][b]), msl) // bs)
        assert mask[b, :, :nb].all() and not mask[b, :, nb:].any()


@pytest.mark.parametrize("B,Hq,Hkv,d,lens,bs", SHAPES)
def test_quantised_infinite_delta_is_dense(B, Hq, Hkv, d, lens, bs):
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=12, block_size=bs)
    msl = inp["cap"]
    sm = np.float32(1.0 / math.sqrt(d))
    out, lse, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=msl,
                              block_size=bs, delta=math.inf, sink=0, local=0, split_blocks=2, sm_scale=sm)
    ref_out, ref_lse = _dense_ref(inp, msl, sm)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-12)


def test_sink_plus_local_covering_everything_is_dense():
    inp = make_random_inputs(2, 8, 2, 64, (300, 257), seed=13, block_size=64)
    sm = np.float32(0.125)
    out, lse, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                              block_size=64, delta=0.0, sink=2, local=3, split_blocks=1, sm_scale=sm)
    ref_out, ref_lse = _dense_ref(inp, inp["cap"], sm)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    assert mask[0, :, :5].all() and mask[1, :, :5].all()


def test_max_seq_len_truncates():
    inp = make_random_inputs(1, 2, 1, 16, (200,), seed=14, block_size=16)
    sm = np.float32(0.25)
    out, lse, _ = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=70, block_size=16,
                           delta=math.inf, sink=0, local=0, split_blocks=4, sm_scale=sm, quantize=False)
    ref_out, ref_lse = _dense_ref(inp, 70, sm)
    np.testing.assert_allclose(out, ref_out, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_empty_sequence():
    inp = make_random_inputs(2, 4, 2, 16, (0, 10), seed=15, block_size=16)
    out, lse, mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=16, block_size=16,
                              delta=3.0, sink=1, local=1, split_blocks=4)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all() and not mask[0].any()
    assert np.isfinite(lse[1]).all() and mask[1, :, 0].all()
