"""Pins of the oracle's multi-query decode (several query tokens per sequence,
each seeing the cache up to its own position): a hand-worked 2-query example,
the dense limit against a library attention routine with a bottom-right
causal mask, and properties of the definition."""

import json
import math
import os

import numpy as np
import pytest
import torch

from ffd_inputs import bf16_bits_from_f32, f32_from_bf16_bits, make_random_inputs, multi_query
from oracle import ffd_oracle as O


@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_multi.json")) as f:
        return json.load(f)


def _closed(hand, key):
    env = {"e2": math.exp(2.0), "em2": math.exp(-2.0), "ln": math.log}
    cf = hand["closed_forms"][key]
    return np.array([eval(s, {}, env) for s in cf["out"]]), eval(cf["lse"], {}, env)


def _hand_inputs(hand):
    inp = hand["inputs"]
    return (bf16_bits_from_f32(np.array(inp["q"], np.float32)),
            bf16_bits_from_f32(np.array(inp["k"], np.float32)),
            bf16_bits_from_f32(np.array(inp["v"], np.float32)))


def test_hand_block_scores(hand):
    q, k, _ = _hand_inputs(hand)
    k32 = f32_from_bf16_bits(k[0, 0])
    codes, scale = O.quantize_keys(k32)
    for i, L in enumerate((3, 4)):
        qc, cq = O.quantize_query(f32_from_bf16_bits(q[0, i, 0]), np.float32(1.0))
        tok = O.token_scores(qc, cq, codes[:L], scale[:L])
        assert O.block_scores(tok, L, 2).tolist() == hand["block_scores"][i]


@pytest.mark.parametrize("idx", range(8))
def test_hand_cases(hand, idx):
    case = hand["cases"][idx]
    q, k, v = _hand_inputs(hand)
    inp = hand["inputs"]
    delta = math.inf if case["delta"] == "inf" else case["delta"]
    out, lse, mask = O.decode_multi(q, k, v, np.array(inp["seq_lens"]), max_seq_len=4,
                                    block_size=inp["block_size"], delta=delta, sink=case["sink"],
                                    local=case["local"], split_blocks=inp["split_blocks"],
                                    sm_scale=np.float32(inp["sm_scale"]))
    assert mask[0, :, 0].tolist() == case["masks"]
    for i, key in enumerate(case["closed"]):
        o, s = _closed(hand, key)
        np.testing.assert_allclose(out[0, i, 0], o, rtol=0, atol=1e-12)
        assert abs(lse[0, i, 0] - s) <= 1e-12


def test_hand_first_query_sees_nothing(hand):
    q, k, v = _hand_inputs(hand)
    out, lse, mask = O.decode_multi(q, k, v, np.array([1]), max_seq_len=4, block_size=2, delta=1.0, sink=0,
                                    local=0, split_blocks=2, sm_scale=np.float32(1.0))
    assert (out[0, 0, 0] == 0).all() and np.isneginf(lse[0, 0, 0]) and not mask[0, 0].any()
    np.testing.assert_allclose(out[0, 1, 0], [1.0, 0.0], atol=1e-12)
    assert abs(lse[0, 1, 0]) <= 1e-12
    assert mask[0, 1, 0].tolist() == [1, 0]


def _causal_ref(q, k, v, lens, sm):
    """torch SDPA in fp64 with a bottom-right-aligned causal mask: query i of a
    sequence of length L may attend token t iff t <= L - Q + i."""
    B, Q, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Q, Hq, d))
    lse = np.full((B, Q, Hq), -math.inf)
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        qt = torch.from_numpy(f32_from_bf16_bits(q[b]).astype(np.float64)).permute(1, 0, 2)  # [Hq,Q,d]
        kt = torch.from_numpy(f32_from_bf16_bits(k[b, :, :L]).astype(np.float64)).repeat_interleave(G, 0)
        vt = torch.from_numpy(f32_from_bf16_bits(v[b, :, :L]).astype(np.float64)).repeat_interleave(G, 0)
        allowed = torch.arange(L)[None, :] <= (L - Q + torch.arange(Q))[:, None]   # [Q, L]
        rows = allowed.any(dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(qt[:, rows], kt, vt, attn_mask=allowed[rows],
                                                             scale=float(sm))
        z = float(sm) * (qt[:, rows] @ kt.transpose(1, 2))
        z = z.masked_fill(~allowed[rows], -math.inf)
        idx = torch.nonzero(rows)[:, 0].numpy()
        out[b, idx] = o.permute(1, 0, 2).numpy()
        lse[b, idx] = torch.logsumexp(z, dim=-1).permute(1, 0).numpy()
    return out, lse


SHAPES = [
    (1, 4, 1, 64, (130,), 64, 4),
    (2, 8, 2, 32, (100, 37), 16, 3),
    (3, 6, 3, 16, (1, 64, 130), 32, 2),
    (2, 4, 2, 8, (3, 0), 4, 5),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,lens,bs,Q", SHAPES)
@pytest.mark.parametrize("quantize", [False, True])
def test_infinite_delta_is_causal_attention(B, Hq, Hkv, d, lens, bs, Q, quantize):
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=41, block_size=bs)
    q = multi_query(inp, Q, seed=42)
    sm = np.float32(1.0 / math.sqrt(d))
    out, lse, mask = O.decode_multi(q, inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                                    block_size=bs, delta=math.inf, sink=0, local=0, split_blocks=2,
                                    sm_scale=sm, quantize=quantize)
    ref_out, ref_lse = _causal_ref(q, inp["k"], inp["v"], inp["seq_lens"], sm)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-12)
    for b in range(B):
        for i in range(Q):
            nb = -(-max(0, int(inp["seq_lens"][b]) - Q + 1 + i) // bs)
            assert mask[b, i, :, :nb].all() and not mask[b, i, :, nb:].any()


def test_one_query_is_decode():
    inp = make_random_inputs(2, 8, 2, 32, (300, 129), seed=43, block_size=32)
    kw = dict(max_seq_len=inp["cap"], block_size=32, delta=2.0, sink=1, local=2, split_blocks=3,
              sm_scale=np.float32(0.2))
    out, lse, mask = O.decode_multi(inp["q"][:, None], inp["k"], inp["v"], inp["seq_lens"], **kw)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **kw)
    np.testing.assert_array_equal(out[:, 0], r_out)
    np.testing.assert_array_equal(lse[:, 0], r_lse)
    np.testing.assert_array_equal(mask[:, 0], r_mask)


def test_queries_do_not_interact():
    inp = make_random_inputs(1, 4, 1, 32, (500,), seed=44, block_size=32)
    q = multi_query(inp, 4, seed=45)
    kw = dict(max_seq_len=inp["cap"], block_size=32, delta=1.5, sink=1, local=1, split_blocks=4,
              sm_scale=np.float32(0.25))
    out, lse, mask = O.decode_multi(q, inp["k"], inp["v"], inp["seq_lens"], **kw)
    q2 = q.copy()
    q2[:, 1] = multi_query(inp, 4, seed=46)[:, 0]
    out2, lse2, mask2 = O.decode_multi(q2, inp["k"], inp["v"], inp["seq_lens"], **kw)
    for i in (0, 2, 3):
        np.testing.assert_array_equal(out[:, i], out2[:, i])
        np.testing.assert_array_equal(mask[:, i], mask2[:, i])
    assert not np.array_equal(out[:, 1], out2[:, 1])


@pytest.mark.parametrize("d1,d2", [(0.5, 1.0), (1.0, 3.0), (0.0, 8.0)])
def test_monotone_in_delta(d1, d2):
    inp = make_random_inputs(2, 4, 2, 32, (700, 333), seed=47, block_size=32)
    q = multi_query(inp, 3, seed=48)
    kw = dict(max_seq_len=inp["cap"], block_size=32, sink=1, local=1, split_blocks=4, sm_scale=np.float32(0.3),
              mask_only=True)
    _, _, m1 = O.decode_multi(q, inp["k"], inp["v"], inp["seq_lens"], delta=d1, **kw)
    _, _, m2 = O.decode_multi(q, inp["k"], inp["v"], inp["seq_lens"], delta=d2, **kw)
    assert (m1 <= m2).all()


def test_earlier_queries_never_keep_unseen_blocks():
    inp = make_random_inputs(1, 2, 1, 16, (97,), seed=49, block_size=16)
    q = multi_query(inp, 40, seed=50)
    _, _, mask = O.decode_multi(q, inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=16,
                                delta=math.inf, sink=2, local=2, split_blocks=2, mask_only=True)
    for i in range(40):
        nb = -(-(97 - 40 + 1 + i) // 16)
        assert mask[0, i, :, :nb].all() and not mask[0, i, :, nb:].any()
