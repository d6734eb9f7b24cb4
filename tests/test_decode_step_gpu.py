"""Decode-step integration: a serving-style loop in which each step -- append
the new token's int4 sketch, advance the lengths on the device, decode -- is
one captured HIP graph, replayed step after step with new queries. A paged
(shuffled block table) cache for single-token decode, and a contiguous cache
for a speculative verify step of Q tokens (ffd_decode_multi). Every replay is
checked against the oracle at that step's lengths."""

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import bf16_bits_from_f32, make_random_inputs
from oracle import ffd_oracle as O
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu

STEPS = 4


def _pages(x, nbs, table_np, num_pages):
    B, Hkv = x.shape[:2]
    pool = torch.full((num_pages, Hkv, 64) + tuple(x.shape[3:]), float("nan"), dtype=x.dtype, device=x.device)
    for b in range(B):
        for jb in range(nbs[b]):
            pool[int(table_np[b, jb])] = x[b, :, 64 * jb:64 * jb + 64]
    return pool


def _random_q(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))


def test_paged_decode_steps_in_a_graph():
    B, Hq, Hkv, d = 2, 16, 4, 128
    final = (2000 + STEPS, 1500 + STEPS)
    say(f"decode steps (paged, graph): lens {final} minus {STEPS}")
    inp = make_random_inputs(B, Hq, Hkv, d, final, seed=71, block_size=64, hot_frac=0.1)
    dv = to_device(inp)
    cap = inp["cap"]
    nbs = [-(-L // 64) for L in final]
    num_pages = sum(nbs) + 3
    perm = np.random.default_rng(5).permutation(num_pages)
    stride = cap // 64
    table_np = np.zeros((B, stride), dtype=np.int32)
    used = 0
    for b in range(B):
        table_np[b, :nbs[b]] = perm[used:used + nbs[b]]
        used += nbs[b]
    table = torch.from_numpy(table_np).cuda()
    kp, vp = _pages(dv["k"], nbs, table_np, num_pages), _pages(dv["v"], nbs, table_np, num_pages)
    kqp = torch.zeros((num_pages, Hkv, 64, d // 2), dtype=torch.uint8, device="cuda")
    ksp = torch.zeros((num_pages, Hkv, 64), dtype=torch.float32, device="cuda")
    L0 = np.array(final, dtype=np.int32) - STEPS
    seq = torch.from_numpy(L0.copy()).cuda()
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    ffd.ffd_quantize_kv_paged(kp, kqp, ksp, table, zeros, seq, int(L0.max()))   # prefill's sketch
    pos_end = torch.empty_like(seq)
    q_static = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, cap // 64), dtype=torch.uint8, device="cuda")
    ws = ffd.alloc_workspace(B, Hq, d, cap, 64, 8)
    kw = dict(max_seq_len=cap, block_size=64, delta=1.5, sink=1, local=2, split_blocks=8, sm_scale=sm_scale_for(d))

    def step():
        torch.add(seq, 1, out=pos_end)
        ffd.ffd_quantize_kv_paged(kp, kqp, ksp, table, seq, pos_end, 1)   # append the new token
        seq.copy_(pos_end)
        ffd.ffd_decode_paged(q_static, kp, vp, kqp, ksp, table, seq, out=out, lse=lse, kept_mask=mask,
                             workspace=ws, **kw)

    # warm every entry point eagerly without changing state (empty append span)
    q_static.zero_()
    ffd.ffd_quantize_kv_paged(kp, kqp, ksp, table, seq, seq, 1)
    ffd.ffd_decode_paged(q_static, kp, vp, kqp, ksp, table, seq, out=out, lse=lse, kept_mask=mask, workspace=ws,
                         **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(seq.cpu(), torch.from_numpy(L0)), "capture must not execute the step"
    rng = np.random.default_rng(8)
    for rep in range(STEPS):
        q_bits = _random_q(rng, (B, Hq, d))
        q_static.copy_(dev_bf16(q_bits))
        g.replay()
        torch.cuda.synchronize()
        lens = L0 + rep + 1
        assert np.array_equal(seq.cpu().numpy(), lens)
        r_out, r_lse, r_mask = O.decode(q_bits, inp["k"], inp["v"], lens, max_seq_len=cap, block_size=64,
                                        delta=kw["delta"], sink=kw["sink"], local=kw["local"],
                                        split_blocks=kw["split_blocks"], sm_scale=np.float32(kw["sm_scale"]))
        assert_mask_equal(mask.cpu().numpy(), r_mask, f"step {rep} mask")
        assert_close(out.cpu().numpy(), r_out, f"step {rep} out")
        assert_close(lse.cpu().numpy(), r_lse, f"step {rep} lse")


def test_speculative_verify_steps_in_a_graph():
    B, Hq, Hkv, d, Q = 2, 8, 2, 128, 4
    final = (1500 + Q * STEPS, 900 + Q * STEPS)
    say(f"verify steps (Q={Q}, graph): lens {final}")
    inp = make_random_inputs(B, Hq, Hkv, d, final, seed=72, block_size=64, hot_frac=0.1)
    dv = to_device(inp)
    cap = inp["cap"]
    kq = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Hkv, cap), dtype=torch.float32, device="cuda")
    L0 = np.array(final, dtype=np.int32) - Q * STEPS
    seq = torch.from_numpy(L0.copy()).cuda()
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    ffd.ffd_quantize_kv(dv["k"], kq, ks, zeros, seq, int(L0.max()))
    pos_end = torch.empty_like(seq)
    q_static = torch.empty((B, Q, Hq, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Q, Hq, cap // 64), dtype=torch.uint8, device="cuda")
    ws = torch.empty(ffd.ffd_decode_multi_workspace_bytes(B, Q, Hq, d, cap, 64, 4), dtype=torch.uint8,
                     device="cuda")
    kw = dict(max_seq_len=cap, block_size=64, delta=1.0, sink=1, local=1, split_blocks=4, sm_scale=sm_scale_for(d))

    def step():
        torch.add(seq, Q, out=pos_end)
        ffd.ffd_quantize_kv(dv["k"], kq, ks, seq, pos_end, Q)   # append the Q draft tokens
        seq.copy_(pos_end)
        ffd.ffd_decode_multi(q_static, dv["k"], dv["v"], kq, ks, seq, out=out, lse=lse, kept_mask=mask,
                             workspace=ws, **kw)

    q_static.zero_()
    ffd.ffd_quantize_kv(dv["k"], kq, ks, seq, seq, Q)
    ffd.ffd_decode_multi(q_static, dv["k"], dv["v"], kq, ks, seq, out=out, lse=lse, kept_mask=mask, workspace=ws,
                         **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(seq.cpu(), torch.from_numpy(L0)), "capture must not execute the step"
    rng = np.random.default_rng(9)
    for rep in range(STEPS):
        q_bits = _random_q(rng, (B, Q, Hq, d))
        q_static.copy_(dev_bf16(q_bits))
        g.replay()
        torch.cuda.synchronize()
        lens = L0 + Q * (rep + 1)
        assert np.array_equal(seq.cpu().numpy(), lens)
        r_out, r_lse, r_mask = O.decode_multi(q_bits, inp["k"], inp["v"], lens, max_seq_len=cap, block_size=64,
                                              delta=kw["delta"], sink=kw["sink"], local=kw["local"],
                                              split_blocks=kw["split_blocks"], sm_scale=np.float32(kw["sm_scale"]))
        assert_mask_equal(mask.cpu().numpy(), r_mask, f"verify step {rep} mask")
        assert_close(out.cpu().numpy(), r_out, f"verify step {rep} out")
        assert_close(lse.cpu().numpy(), r_lse, f"verify step {rep} lse")
