"""GPU parity for multi-query decode (ffd_decode_multi): Q query tokens per
sequence, token i seeing the cache up to position L - Q + i. The kept-block
mask must match the oracle bit for bit and out/LSE must be within the bar, on
small ragged cases (padding rows, tokens that see nothing, both pseudo-max
modes, the dense path, bf16 output) and on the 32K and 128K x4 workloads with
four query tokens."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import WORKLOADS, make_inputs, make_random_inputs, multi_query
from oracle import ffd_oracle as O
from tests import oracle_par as P
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu


def _run(dv, qm, *, max_seq_len, delta, sink, local, split_blocks, sm_scale, pseudo_max="split",
         out_dtype=torch.float32, kq=None, ks=None):
    if kq is None and not math.isinf(delta):
        kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    out, lse, mask = ffd.decode_multi(qm, dv["k"], dv["v"], kq, ks, dv["seq_lens"], max_seq_len=max_seq_len,
                                      block_size=64, delta=delta, sink=sink, local=local,
                                      split_blocks=split_blocks, sm_scale=sm_scale, out_dtype=out_dtype,
                                      pseudo_max=pseudo_max)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), mask.cpu().numpy()


# (B, Q, Hq, Hkv, d, lens, split, delta, sink, local, pseudo_max)
CASES = [
    (1, 2, 4, 1, 128, (300,), 2, 1.0, 1, 1, "split"),
    (2, 4, 8, 2, 128, (1000, 70), 3, 0.5, 1, 2, "split"),
    (2, 3, 4, 2, 64, (129, 2), 4, 2.0, 0, 1, "split"),
    (1, 16, 1, 1, 64, (500,), 5, 1.0, 1, 1, "split"),
    (1, 2, 16, 2, 128, (777,), 7, 1.5, 2, 2, "split"),
    (1, 8, 2, 1, 64, (65,), 1, 0.0, 0, 1, "split"),
    (2, 4, 4, 1, 128, (400, 260), 2, 1.0, 1, 2, "sink_local"),
    (1, 16, 1, 1, 128, (200,), 2, 0.5, 1, 1, "sink_local"),
    (2, 4, 8, 2, 128, (300, 5), 3, math.inf, 0, 0, "split"),
    (3, 5, 2, 1, 64, (64, 0, 191), 2, 1.0, 1, 1, "split"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_small(case):
    B, Q, Hq, Hkv, d, lens, S, delta, sink, local, pm = CASES[case]
    say(f"multi small case {case}: B={B} Q={Q} Hq={Hq} Hkv={Hkv} d={d} lens={lens} S={S} delta={delta} {pm}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=300 + case, block_size=64, hot_frac=0.1)
    qm = multi_query(inp, Q, seed=400 + case)
    dv = to_device(inp)
    sm = sm_scale_for(d)
    msl = inp["cap"]
    out, lse, mask = _run(dv, dev_bf16(qm), max_seq_len=msl, delta=delta, sink=sink, local=local, split_blocks=S,
                          sm_scale=sm, pseudo_max=pm)
    r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], max_seq_len=msl, block_size=64,
                                          delta=delta, sink=sink, local=local, split_blocks=S,
                                          sm_scale=np.float32(sm), pseudo_max=pm)
    assert_mask_equal(mask, r_mask, f"case {case} mask")
    assert_close(out, r_out, f"case {case} out")
    assert_close(lse, r_lse, f"case {case} lse")


def test_bf16_output_and_truncation():
    inp = make_random_inputs(2, 8, 2, 64, (300, 150), seed=310, block_size=64, cap=320)
    qm = multi_query(inp, 4, seed=410)
    dv = to_device(inp)
    sm = sm_scale_for(64)
    out, lse, mask = _run(dv, dev_bf16(qm), max_seq_len=256, delta=1.0, sink=1, local=1, split_blocks=2,
                          sm_scale=sm, out_dtype=torch.bfloat16)
    r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], max_seq_len=256, block_size=64,
                                          delta=1.0, sink=1, local=1, split_blocks=2, sm_scale=np.float32(sm))
    assert_mask_equal(mask, r_mask, "bf16/truncation mask")
    assert_close(out, r_out, "bf16/truncation out", bf16_out=True)
    assert_close(lse, r_lse, "bf16/truncation lse")


def test_one_query_equals_decode():
    inp = make_random_inputs(2, 8, 2, 128, (700, 333), seed=311, block_size=64)
    dv = to_device(inp)
    sm = sm_scale_for(128)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    kw = dict(max_seq_len=inp["cap"], block_size=64, delta=1.0, sink=1, local=2, split_blocks=3, sm_scale=sm,
              out_dtype=torch.float32)
    o1, l1, m1 = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], **kw)
    o2, l2, m2 = ffd.decode_multi(dv["q"][:, None].contiguous(), dv["k"], dv["v"], kq, ks, dv["seq_lens"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2[:, 0]) and torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


def test_deterministic():
    inp = make_random_inputs(1, 4, 1, 128, (2000,), seed=312, block_size=64)
    qm = dev_bf16(multi_query(inp, 4, seed=412))
    dv = to_device(inp)
    kw = dict(max_seq_len=inp["cap"], delta=0.5, sink=1, local=1, split_blocks=4, sm_scale=sm_scale_for(128))
    a = _run(dv, qm, **kw)
    b = _run(dv, qm, **kw)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("name,Q", [("llama3_8b_32k", 4), ("llama3_8b_128k_b4", 4)])
def test_workload(name, Q):
    w = WORKLOADS[name]
    say(f"multi-query workload {name} Q={Q}: generating")
    inp = make_inputs(w)
    qm = multi_query(inp, Q, seed=w.seed + 1000)
    dv = to_device(inp)
    sm = sm_scale_for(w.d)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    delta = w.deltas[0]
    say(f"  {name} delta={delta}: GPU")
    out, lse, mask = _run(dv, dev_bf16(qm), max_seq_len=inp["cap"], delta=delta, sink=w.sink, local=w.local,
                          split_blocks=w.split_blocks, sm_scale=sm, kq=kq, ks=ks)
    args = dict(max_seq_len=inp["cap"], block_size=64, delta=delta, sink=w.sink, local=w.local,
                split_blocks=w.split_blocks, sm_scale=np.float32(sm))
    say("  oracle (every row)")
    r_out, r_lse, r_mask = P.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], **args)
    assert_mask_equal(mask, r_mask, f"{name} mask")
    assert_close(out, r_out, f"{name} out")
    assert_close(lse, r_lse, f"{name} lse")


def test_negative_lengths_are_empty():
    """seq_lens are device values and are not validated: any negative length,
    INT_MIN included, is an empty sequence for every query token (out 0, LSE
    -inf, zero mask), in both the several-token and the single-token call;
    the other sequences of the batch are unaffected."""
    B, Q, Hq, Hkv, d = 3, 3, 8, 2, 128
    say("multi: negative lengths")
    inp = make_random_inputs(B, Hq, Hkv, d, (700, 700, 700), seed=61, block_size=64, hot_frac=0.1)
    qm = multi_query(inp, Q, seed=62)
    dv = to_device(inp)
    seq = torch.tensor([-2 ** 31, -5, 700], dtype=torch.int32, device="cuda")
    kq, ks = ffd.quantize_kv(dv["k"], torch.tensor([700, 700, 700], dtype=torch.int32, device="cuda"))
    kw = dict(max_seq_len=inp["cap"], delta=1.0, sink=1, local=2, split_blocks=4, sm_scale=sm_scale_for(d))
    out, lse, mask = ffd.decode_multi(dev_bf16(qm), dv["k"], dv["v"], kq, ks, seq, out_dtype=torch.float32, **kw)
    out1, lse1, mask1 = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, seq, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    for o, l, m in ((out[:2], lse[:2], mask[:2]), (out1[:2], lse1[:2], mask1[:2])):
        assert (o == 0).all() and torch.isneginf(l).all() and (m == 0).all()
    r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], np.array([0, 0, 700]), block_size=64,
                                          max_seq_len=inp["cap"], delta=1.0, sink=1, local=2, split_blocks=4,
                                          sm_scale=np.float32(sm_scale_for(d)))
    assert_mask_equal(mask.cpu().numpy(), r_mask, "mask")
    assert_close(out.cpu().numpy().astype(np.float64), r_out, "out")
    assert_close(lse.cpu().numpy().astype(np.float64), r_lse, "lse")
