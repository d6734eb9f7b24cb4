"""Thumbnail + residual key storage on the GPU: ffd_quantize_kv_thumb is
bit-identical to the oracle's quantiser; ffd_decode_thumb matches the oracle
(mask bit-exact, out/LSE within the bar) on ragged shapes and at full size."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import WORKLOADS, bf16_bits_from_f32, make_inputs, make_random_inputs
from oracle import ffd_oracle as O
from tests import oracle_par as P
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu


def _check_quant(inp):
    dv = to_device(inp)
    k2, k2s, kr, krs = ffd.quantize_kv_thumb(dv["k"], dv["seq_lens"])
    torch.cuda.synchronize()
    r2, r2s, rr, rrs = O.quantize_cache_thumb(inp["k"], inp["seq_lens"])
    np.testing.assert_array_equal(k2.cpu().numpy(), r2)
    np.testing.assert_array_equal(k2s.cpu().numpy().view(np.uint32), r2s.view(np.uint32))
    np.testing.assert_array_equal(kr.cpu().numpy(), rr)
    np.testing.assert_array_equal(krs.cpu().numpy().view(np.uint32), rrs.view(np.uint32))
    return dv, (k2, k2s, kr, krs)


@pytest.mark.parametrize("B,Hkv,d,lens", [(2, 3, 128, (1000, 77)), (3, 2, 64, (1, 0, 130))])
def test_quantize_bit_exact(B, Hkv, d, lens):
    say(f"thumb quantize B={B} Hkv={Hkv} d={d} lens={lens}")
    _check_quant(make_random_inputs(B, Hkv, Hkv, d, lens, seed=71, block_size=64))


def test_quantize_special_rows():
    say("thumb quantize special rows")
    d = 128
    rng = np.random.default_rng(8)
    rows = [np.zeros(d), np.full(d, 2.0 ** -126), np.full(d, 2.0 ** -125), rng.standard_normal(d) * 1e30,
            np.tile([3.0, 1.0, -1.0, -3.0], d // 4), np.tile([6.0, -2.0, 2.0, 0.0], d // 4),
            np.where(np.arange(d) % 3 == 0, 1.5, -0.5), rng.standard_normal(d)]
    rows += [rng.standard_normal(d) * 10.0 ** rng.integers(-20, 20) for _ in range(56)]
    kb = bf16_bits_from_f32(np.stack(rows).astype(np.float32))[None, None]
    inp = {"k": kb, "seq_lens": np.array([kb.shape[2]], np.int32), "q": np.zeros((1, 1, d), np.uint16),
           "v": kb.copy()}
    _check_quant(inp)


CASES = [
    (1, 4, 1, 64, (2048,), 2.0, 1, 2, 32, "split"),
    (3, 8, 8, 128, (1, 63, 65), 1.0, 1, 1, 1, "split"),
    (2, 16, 2, 128, (4000, 1000), 0.5, 2, 3, 3, "split"),
    (4, 32, 8, 128, (0, 5000, 6400, 77), 6.0, 1, 4, 32, "split"),
    (2, 8, 2, 64, (3000, 2999), math.inf, 1, 4, 32, "split"),
    (2, 8, 4, 128, (3000, 1500), 1.5, 1, 2, 8, "sink_local"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_small(case):
    B, Hq, Hkv, d, lens, delta, sink, local, S, pm = CASES[case]
    say(f"thumb decode case {case}: B={B} Hq={Hq} Hkv={Hkv} d={d} lens={lens} delta={delta} S={S} {pm}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=600 + case, block_size=64, hot_frac=0.1)
    dv, (k2, k2s, kr, krs) = _check_quant(inp)
    cap = inp["cap"]
    sm = sm_scale_for(d)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, cap // 64), dtype=torch.uint8, device="cuda")
    ws = ffd.alloc_workspace(B, Hq, d, cap, 64, S)
    ffd.ffd_decode_thumb(dv["q"], k2, k2s, kr, krs, dv["v"], dv["seq_lens"], max_seq_len=cap, block_size=64,
                         delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=sm, out=out, lse=lse,
                         kept_mask=mask, workspace=ws, pseudo_max=pm)
    torch.cuda.synchronize()
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=cap, block_size=64,
                                    delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=np.float32(sm),
                                    pseudo_max=pm, storage="thumb")
    assert_mask_equal(mask.cpu().numpy(), r_mask, "thumb mask")
    assert_close(out.cpu().numpy(), r_out, "thumb out")
    assert_close(lse.cpu().numpy(), r_lse, "thumb lse")


def test_decode_128k_full_size():
    w = WORKLOADS["llama3_8b_128k_b4"]
    say("thumb decode 128K x4 full size")
    inp = make_inputs(w)
    dv = to_device(inp)
    k2, k2s, kr, krs = ffd.quantize_kv_thumb(dv["k"], dv["seq_lens"])
    cap = inp["cap"]
    sm = sm_scale_for(w.d)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((w.B, w.Hq, cap // 64), dtype=torch.uint8, device="cuda")
    ws = ffd.alloc_workspace(w.B, w.Hq, w.d, cap, 64, w.split_blocks)
    ffd.ffd_decode_thumb(dv["q"], k2, k2s, kr, krs, dv["v"], dv["seq_lens"], max_seq_len=cap, block_size=64,
                         delta=6.0, sink=w.sink, local=w.local, split_blocks=w.split_blocks, sm_scale=sm, out=out,
                         lse=lse, kept_mask=mask, workspace=ws)
    torch.cuda.synchronize()
    args = dict(max_seq_len=cap, block_size=64, delta=6.0, sink=w.sink, local=w.local, split_blocks=w.split_blocks,
                sm_scale=np.float32(sm), storage="thumb")
    say("  oracle (every head)")
    r_out, r_lse, r_mask = P.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **args)
    assert_mask_equal(mask.cpu().numpy(), r_mask, "thumb mask 128k")
    assert_close(out.cpu().numpy(), r_out, "thumb out 128k")
    assert_close(lse.cpu().numpy(), r_lse, "thumb lse 128k")
