"""Scale layouts the scan must read correctly: each lane loads one per-token
key scale of a block (tokens past the sequence are not read) and the others
come by lane broadcasts. A cache capacity that is not a multiple of 4 (the last
block runs past the rows), a scale array 4 bytes off a 16-byte boundary, and
blocks past the capacity must keep exactly the oracle's blocks, and aligned
and misaligned copies of one cache must agree bit for bit."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import make_random_inputs, multi_query
from oracle import ffd_oracle as O
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, say, sm_scale_for

pytestmark = pytest.mark.gpu


def _recap(a: np.ndarray, cap: int) -> np.ndarray:
    """The cache rows [B, Hkv, cap0, d] cut or zero-padded to cap rows."""
    if cap <= a.shape[2]:
        return np.ascontiguousarray(a[:, :, :cap])
    pad = np.zeros(a.shape[:2] + (cap - a.shape[2],) + a.shape[3:], dtype=a.dtype)
    return np.concatenate([a, pad], axis=2)


def _device(inp: dict, cap: int, misalign: bool):
    k = dev_bf16(_recap(inp["k"], cap))
    v = dev_bf16(_recap(inp["v"], cap))
    seq = torch.from_numpy(np.ascontiguousarray(inp["seq_lens"], dtype=np.int32)).to("cuda")
    B, Hkv, _, d = k.shape
    if misalign:
        # one float in: the scale array starts 4 bytes past a 16-byte boundary
        flat = torch.zeros(B * Hkv * cap + 1, dtype=torch.float32, device="cuda")
        ks = flat[1:].view(B, Hkv, cap)
        assert ks.data_ptr() % 16 != 0
    else:
        ks = torch.zeros((B, Hkv, cap), dtype=torch.float32, device="cuda")
    kq, ks = ffd.quantize_kv(k, seq, kscale=ks)
    return k, v, seq, kq, ks


def _decode(q, k, v, kq, ks, seq, msl, kw, multi=False):
    fn = ffd.decode_multi if multi else ffd.decode
    out, lse, mask = fn(q, k, v, kq, ks, seq, max_seq_len=msl, block_size=64, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), mask.cpu().numpy()


# (B, Hq, Hkv, d, lens, cap, split, delta, sink, local, pseudo_max, misalign)
CASES = [
    (2, 8, 2, 128, (2045, 1001), 2046, 8, 2.0, 1, 2, "split", False),   # cap = 2 mod 4
    (1, 4, 1, 64, (777,), 779, 4, 1.0, 1, 1, "sink_local", False),      # odd cap, tail past it
    (2, 8, 2, 128, (3000, 1280), 3072, 16, 2.0, 1, 4, "split", True),   # misaligned scales
    (1, 16, 4, 128, (2500,), 2560, 8, 0.5, 2, 2, "sink_local", True),
    (3, 4, 4, 64, (1, 63, 130), 131, 1, 0.0, 0, 1, "split", False),     # blocks past the cap
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_scale_layouts_match_oracle(case):
    B, Hq, Hkv, d, lens, cap, S, delta, sink, local, pm, mis = CASES[case]
    say(f"scale layout case {case}: B={B} Hq={Hq} Hkv={Hkv} d={d} lens={lens} cap={cap} S={S} {pm} misalign={mis}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=700 + case, block_size=64, hot_frac=0.05)
    k, v, seq, kq, ks = _device(inp, cap, mis)
    sm = sm_scale_for(d)
    kw = dict(delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=sm, pseudo_max=pm)
    out, lse, mask = _decode(dev_bf16(inp["q"]), k, v, kq, ks, seq, cap, kw)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=cap, block_size=64,
                                    delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=np.float32(sm),
                                    pseudo_max=pm)
    assert_mask_equal(mask, r_mask, "mask")
    assert_close(out, r_out, "out")
    assert_close(lse, r_lse, "lse")


def test_scale_loads_agree_bit_for_bit():
    """The same cache with aligned scales and with the scales one float off a
    16-byte boundary: identical results."""
    B, Hq, Hkv, d, lens, cap = 2, 16, 4, 128, (4096, 2500), 4096
    say("scale loads: aligned vs misaligned, bit for bit")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=777, block_size=64, hot_frac=0.05)
    kw = dict(delta=1.5, sink=1, local=2, split_blocks=16, sm_scale=sm_scale_for(d))
    res = []
    for mis in (False, True):
        k, v, seq, kq, ks = _device(inp, cap, mis)
        res.append(_decode(dev_bf16(inp["q"]), k, v, kq, ks, seq, cap, kw))
    for a, b, what in zip(res[0], res[1], ("out", "lse", "mask")):
        np.testing.assert_array_equal(a, b, err_msg=what)


def test_multi_query_odd_cap():
    """Several query tokens (rows of different lengths) over a cache whose
    capacity is not a multiple of 4."""
    B, Q, Hq, Hkv, d, lens, cap = 2, 3, 8, 2, 128, (1500, 643), 1501
    say(f"scale layout multi-query: B={B} Q={Q} lens={lens} cap={cap}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=790, block_size=64, hot_frac=0.1)
    qm = multi_query(inp, Q, seed=791)
    k, v, seq, kq, ks = _device(inp, cap, False)
    sm = sm_scale_for(d)
    kw = dict(delta=1.0, sink=1, local=2, split_blocks=4, sm_scale=sm)
    out, lse, mask = _decode(dev_bf16(qm), k, v, kq, ks, seq, cap, kw, multi=True)
    r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], max_seq_len=cap, block_size=64,
                                          delta=1.0, sink=1, local=2, split_blocks=4, sm_scale=np.float32(sm))
    assert_mask_equal(mask, r_mask, "mask")
    assert_close(out, r_out, "out")
    assert_close(lse, r_lse, "lse")
    assert math.isfinite(float(np.nanmax(np.abs(out))))
