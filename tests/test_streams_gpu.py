"""Decode calls on different streams, each with its own workspace and
outputs, may run at the same time: the library allocates nothing and keeps no
state between calls but the thread's error string. Three different problems
(a 4-wave int4 grid, an 8-wave int4 grid with several workgroups per split,
the thumbnail storage) are issued on three streams at once, five times over,
and every result must equal, bit for bit, the same call made alone on the
default stream; the lone calls' masks match the oracle."""

import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import make_random_inputs
from oracle import ffd_oracle as O
from tests.gpu_util import assert_mask_equal, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu

ROUNDS = 5


def _problems():
    # (name, B, Hq, Hkv, d, lens, delta, S, storage)
    return [
        ("int4, 4-wave grid", 2, 32, 8, 128, (20000, 9000), 2.0, 16, "int4"),
        ("int4, 8-wave grid, P > 1", 1, 8, 2, 64, (3000,), 1.0, 8, "int4"),
        ("thumbnail", 2, 16, 4, 128, (7000, 12000), 4.0, 32, "thumb"),
    ]


def _setup(i, prob):
    name, B, Hq, Hkv, d, lens, delta, S, storage = prob
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=600 + i, block_size=64)
    dv = to_device(inp)
    if storage == "thumb":
        dv["store"] = ffd.quantize_kv_thumb(dv["k"], dv["seq_lens"])
    else:
        dv["store"] = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    return inp, dv


def _call(prob, inp, dv, stream):
    name, B, Hq, Hkv, d, lens, delta, S, storage = prob
    cap = inp["cap"]
    kw = dict(max_seq_len=cap, block_size=64, delta=delta, sink=1, local=2, split_blocks=S, sm_scale=sm_scale_for(d))
    ws = ffd.alloc_workspace(B, Hq, d, cap, 64, S)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, -(-cap // 64)), dtype=torch.uint8, device="cuda")
    if storage == "thumb":
        k2, k2s, kr, krs = dv["store"]
        ffd.ffd_decode_thumb(dv["q"], k2, k2s, kr, krs, dv["v"], dv["seq_lens"], out=out, lse=lse, kept_mask=mask,
                             workspace=ws, stream=stream, **kw)
    else:
        kq, ks = dv["store"]
        ffd.ffd_decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], out=out, lse=lse, kept_mask=mask,
                       workspace=ws, stream=stream, **kw)
    return out, lse, mask, ws   # the workspace is returned so that it outlives the call's kernels


def test_concurrent_streams_match_lone_calls():
    probs = _problems()
    data = [_setup(i, p) for i, p in enumerate(probs)]
    torch.cuda.synchronize()
    say("streams: lone calls on the default stream")
    lone = []
    for p, (inp, dv) in zip(probs, data):
        out, lse, mask, _ = _call(p, inp, dv, None)
        torch.cuda.synchronize()
        lone.append((out.clone(), lse.clone(), mask.clone()))
        name, B, Hq, Hkv, d, lens, delta, S, storage = p
        _, _, m_ref = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"], block_size=64,
                               delta=delta, sink=1, local=2, split_blocks=S, sm_scale=sm_scale_for(d),
                               mask_only=True, storage=storage)
        assert_mask_equal(mask.cpu().numpy(), m_ref, f"streams: {name} mask")

    say(f"streams: {len(probs)} problems on {len(probs)} streams, {ROUNDS} rounds")
    streams = [torch.cuda.Stream() for _ in probs]   # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = []
    for r in range(ROUNDS):
        for p, (inp, dv), s in zip(probs, data, streams):
            with torch.cuda.stream(s):
                results.append((p, r, _call(p, inp, dv, s)))
    torch.cuda.synchronize()
    for p, r, (out, lse, mask, _) in results:
        k = probs.index(p)
        lo, ll, lm = lone[k]
        assert torch.equal(mask, lm), f"streams: {p[0]} round {r}: mask differs from the lone call"
        assert torch.equal(out, lo) and torch.equal(lse, ll), f"streams: {p[0]} round {r}: output differs"
