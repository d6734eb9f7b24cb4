"""ffd_decode_noalloc (partials in the library's static scratch array, no
workspace, no allocation) against ffd_decode with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller input (the array then
still holds the first call's partials), each bit-identical to ffd_decode and
within the bar against the oracle; device memory stays unchanged."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import make_random_inputs
from oracle import ffd_oracle as O
from tests.gpu_util import assert_close, assert_mask_equal, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu


def _setup(B, Hq, Hkv, d, lens, seed, S, delta, pm):
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=seed, block_size=64, hot_frac=0.08)
    dv = to_device(inp)
    cap = inp["cap"]
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    kw = dict(max_seq_len=cap, block_size=64, delta=delta, sink=1, local=2, split_blocks=S,
              sm_scale=sm_scale_for(d), pseudo_max=pm)
    nbm = -(-cap // 64)
    bufs = [dict(out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda"),
                 lse=torch.empty((B, Hq), dtype=torch.float32, device="cuda"),
                 kept_mask=torch.empty((B, Hq, nbm), dtype=torch.uint8, device="cuda")) for _ in range(2)]
    ws = ffd.alloc_workspace(B, Hq, d, cap, 64, S)
    return inp, dv, kq, ks, kw, bufs, ws


def _ref(inp, dv, kq, ks, kw, bufs, ws):
    """ffd_decode (caller workspace) into the first output set."""
    dense = math.isinf(kw["delta"])
    ffd.ffd_decode(dv["q"], dv["k"], dv["v"], None if dense else kq, None if dense else ks, dv["seq_lens"],
                   workspace=ws, **kw, **bufs[0])


def _noalloc(inp, dv, kq, ks, kw, bufs, ws):
    """ffd_decode_noalloc into the second output set."""
    dense = math.isinf(kw["delta"])
    ffd.ffd_decode_noalloc(dv["q"], dv["k"], dv["v"], None if dense else kq, None if dense else ks,
                           dv["seq_lens"], **kw, **bufs[1])


def _compare(name, inp, dv, kq, ks, kw, bufs, ws):
    torch.cuda.synchronize()
    a, b = bufs
    for key in ("out", "lse", "kept_mask"):
        assert torch.equal(a[key], b[key]), f"{name}: {key} differs from ffd_decode"
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                    **{**kw, "sm_scale": np.float32(kw["sm_scale"])})
    assert_mask_equal(b["kept_mask"].cpu().numpy(), r_mask, f"{name} mask")
    assert_close(b["out"].cpu().numpy(), r_out, f"{name} out")
    assert_close(b["lse"].cpu().numpy(), r_lse, f"{name} lse")


def _check(name, *case):
    _ref(*case)
    _noalloc(*case)
    _compare(name, *case)


def test_two_calls_second_smaller():
    say("no-alloc: setting up a large and a small case")
    big = _setup(4, 32, 8, 128, (20000, 13000, 20000, 7), seed=901, S=16, delta=2.0, pm="split")
    small = _setup(1, 8, 2, 64, (3000,), seed=902, S=8, delta=1.0, pm="sink_local")
    need_big = ffd.ffd_decode_workspace_bytes(4, 32, 128, big[0]["cap"], 64, 16)
    need_small = ffd.ffd_decode_workspace_bytes(1, 8, 64, small[0]["cap"], 64, 8)
    assert need_small < need_big <= ffd.NOALLOC_SCRATCH_BYTES
    # the first call on the device looks up the array's address
    say("no-alloc: first call")
    _check("first call", *big)
    _ref(*big)
    _ref(*small)
    torch.cuda.synchronize()
    say("no-alloc: two calls in a row, the second smaller")
    free0 = torch.cuda.mem_get_info()[0]
    _noalloc(*big)
    _noalloc(*small)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, f"device memory changed across the no-alloc calls ({free0} -> {free1})"
    _compare("big", *big)
    _compare("small (after big)", *small)


def test_dense_and_small_grid():
    """The dense path, and a grid small enough for several workgroups per split
    (more partials per head), each after a larger call."""
    say("no-alloc: dense then small grid")
    _check("dense", *_setup(2, 16, 4, 128, (9000, 4100), seed=903, S=32, delta=math.inf, pm="split"))
    _check("small grid", *_setup(1, 4, 1, 128, (2500,), seed=904, S=4, delta=0.5, pm="max"))


def test_over_limit_is_refused():
    B, Hq, d, L = 8, 64, 128, 1 << 20
    assert ffd.ffd_decode_workspace_bytes(B, Hq, d, L, 64, 16) > ffd.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 8, 64, d), dtype=torch.bfloat16, device="cuda")
    seq = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    with pytest.raises(ffd.FFDError) as e:
        ffd.ffd_decode_noalloc(q, k, k, None, None, seq, max_seq_len=L, block_size=64, delta=math.inf, sink=1,
                               local=1, split_blocks=16, sm_scale=0.08, out=out, lse=lse, kept_mask=None)
    assert e.value.status == ffd.FFD_ERR_WORKSPACE and "static scratch" in e.value.message
