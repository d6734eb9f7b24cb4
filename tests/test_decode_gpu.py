"""ffd_decode on the GPU against the oracle: the kept-block mask bit-exact,
output and LSE within 1e-3 + 2e-3*|ref|, on small ragged shapes that span
several splits, and on the tiny and 32K workloads in full."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import WORKLOADS, make_inputs, make_random_inputs, multi_query
from oracle import ffd_oracle as O
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, run_gpu, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu

INF = math.inf

# (B, Hq, Hkv, d, lens, delta, sink, local, S, extra)
CASES = [
    (1, 4, 1, 64, (2048,), 8.0, 1, 2, 32, {}),
    (3, 8, 8, 128, (1, 63, 65), 2.0, 1, 1, 1, {}),
    (2, 8, 4, 64, (64, 129), 0.0, 0, 0, 2, {}),
    (2, 16, 2, 128, (4000, 1000), 1.0, 2, 3, 3, {}),
    (4, 32, 8, 128, (0, 5000, 6400, 77), 6.0, 1, 4, 32, {}),
    (1, 4, 1, 128, (8192,), 0.5, 0, 0, 64, {}),
    (2, 16, 2, 64, (3000, 2999), INF, 1, 4, 32, {}),
    (1, 8, 2, 128, (300,), 0.0, 3, 3, 2, {}),
    (1, 4, 2, 128, (5000,), 3.0, 1, 2, 5, {"max_seq_len": 3000}),
    (2, 8, 2, 128, (700, 1500), 1.5, 1, 1, 7, {"out_dtype": torch.bfloat16}),
    (1, 2, 1, 64, (4097,), 0.25, 0, 1, 64, {}),
    (1, 4, 4, 128, (64 * 64 + 1,), 4.0, 1, 1, 64, {}),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_small_cases(case):
    B, Hq, Hkv, d, lens, delta, sink, local, S, extra = CASES[case]
    say(f"decode case {case}: B={B} Hq={Hq} Hkv={Hkv} d={d} lens={lens} delta={delta} S={S} {extra}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=100 + case, block_size=64, hot_frac=0.05)
    msl = extra.get("max_seq_len", inp["cap"])
    sm = sm_scale_for(d)
    dv = to_device(inp)
    out_dtype = extra.get("out_dtype", torch.float32)
    out, lse, mask = run_gpu(dv, max_seq_len=msl, delta=delta, sink=sink, local=local, split_blocks=S,
                             sm_scale=sm, out_dtype=out_dtype)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=msl,
                                    block_size=64, delta=delta, sink=sink, local=local, split_blocks=S,
                                    sm_scale=np.float32(sm))
    assert_mask_equal(mask, r_mask, "mask")
    assert_close(out, r_out, "out", bf16_out=out_dtype == torch.bfloat16)
    assert_close(lse, r_lse, "lse")


@pytest.mark.parametrize("case", [0, 3, 4, 6])
def test_bf16_output(case):
    """bf16 output = the fp32 result rounded half to even: within the bar plus
    half a bf16 ulp of the reference, and equal to rounding the fp32 output."""
    B, Hq, Hkv, d, lens, delta, sink, local, S, extra = CASES[case]
    say(f"decode bf16 output case {case}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=100 + case, block_size=64, hot_frac=0.05)
    msl = extra.get("max_seq_len", inp["cap"])
    dv = to_device(inp)
    kw = dict(max_seq_len=msl, delta=delta, sink=sink, local=local, split_blocks=S, sm_scale=sm_scale_for(d))
    out16, lse16, mask16 = run_gpu(dv, out_dtype=torch.bfloat16, **kw)
    out32, lse32, mask32 = run_gpu(dv, out_dtype=torch.float32, **kw)
    np.testing.assert_array_equal(mask16, mask32)
    np.testing.assert_array_equal(lse16, lse32)
    rounded = torch.from_numpy(out32.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(out16, rounded)
    r_out, _, _ = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], block_size=64,
                           sm_scale=np.float32(kw.pop("sm_scale")), **kw)
    assert_close(out16, r_out, "bf16 out", bf16_out=True)


def test_tiny_workload_and_dense_limit():
    w = WORKLOADS["tiny_d64_2k"]
    say(f"decode workload {w.name}")
    inp = make_inputs(w, poison_tail=True)
    dv = to_device(inp)
    sm = sm_scale_for(w.d)
    for delta in w.deltas:
        out, lse, mask = run_gpu(dv, max_seq_len=inp["cap"], delta=delta, sink=w.sink, local=w.local,
                                 split_blocks=w.split_blocks, sm_scale=sm)
        r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                                        block_size=64, delta=delta, sink=w.sink, local=w.local,
                                        split_blocks=w.split_blocks, sm_scale=np.float32(sm))
        assert_mask_equal(mask, r_mask, f"mask delta={delta}")
        assert_close(out, r_out, f"out delta={delta}")
        assert_close(lse, r_lse, f"lse delta={delta}")
        if math.isinf(delta):
            d_out, d_lse, _ = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                                       block_size=64, delta=INF, sink=0, local=0, split_blocks=32,
                                       sm_scale=np.float32(sm), quantize=False)
            assert mask.all()
            assert_close(out, d_out, "dense out")
            assert_close(lse, d_lse, "dense lse")


def test_32k_workload():
    w = WORKLOADS["llama3_8b_32k"]
    say(f"decode workload {w.name}")
    inp = make_inputs(w, poison_tail=True)
    dv = to_device(inp)
    sm = sm_scale_for(w.d)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    for delta in w.deltas:
        out, lse, mask = run_gpu(dv, max_seq_len=inp["cap"], delta=delta, sink=w.sink, local=w.local,
                                 split_blocks=w.split_blocks, sm_scale=sm, kq=kq, kscale=ks)
        r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                                        block_size=64, delta=delta, sink=w.sink, local=w.local,
                                        split_blocks=w.split_blocks, sm_scale=np.float32(sm))
        say(f"  delta={delta}: kept fraction {mask.mean():.4f}")
        assert_mask_equal(mask, r_mask, f"mask delta={delta}")
        assert_close(out, r_out, f"out delta={delta}")
        assert_close(lse, r_lse, f"lse delta={delta}")


def test_deterministic():
    say("decode determinism")
    inp = make_random_inputs(2, 32, 8, 128, (9000, 4000), seed=77, block_size=64)
    dv = to_device(inp)
    res = [run_gpu(dv, max_seq_len=inp["cap"], delta=2.0, sink=1, local=4, split_blocks=32,
                   sm_scale=sm_scale_for(128)) for _ in range(2)]
    for a, b in zip(res[0], res[1]):
        np.testing.assert_array_equal(a, b)


def test_no_mask_pointer_and_reused_workspace():
    say("decode without mask, shared workspace")
    inp = make_random_inputs(1, 8, 2, 128, (3000,), seed=5, block_size=64)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    ws = ffd.alloc_workspace(1, 8, 128, inp["cap"], 64, 16)
    a = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], delta=1.0, split_blocks=16, workspace=ws)
    b = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], delta=1.0, split_blocks=16, workspace=ws,
                   with_mask=False)
    torch.cuda.synchronize()
    assert b[2] is None
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(ffd.FFDError) as ei:
        ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], delta=1.0, split_blocks=16,
                   workspace=ws[:100])
    assert ei.value.status == ffd.FFD_ERR_WORKSPACE


def test_partials_then_combine_equals_decode():
    say("decode = partials + combine")
    inp = make_random_inputs(3, 16, 4, 128, (5000, 0, 2300), seed=21, block_size=64)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    kw = dict(max_seq_len=inp["cap"], block_size=64, delta=2.5, sink=1, local=2, split_blocks=8,
              sm_scale=sm_scale_for(128))
    out_a, lse_a, mask_a = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], out_dtype=torch.float32,
                                      **{k_: v_ for k_, v_ in kw.items() if k_ != "block_size"})
    ws = ffd.alloc_workspace(3, 16, 128, inp["cap"], 64, 8)
    mask_b = torch.empty_like(mask_a)
    out_b = torch.empty_like(out_a)
    lse_b = torch.empty_like(lse_a)
    ffd.ffd_decode_partials(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], kept_mask=mask_b, workspace=ws, **kw)
    ffd.ffd_combine(dv["seq_lens"], max_seq_len=inp["cap"], block_size=64, split_blocks=8, workspace=ws, out=out_b,
                    lse=lse_b)
    torch.cuda.synchronize()
    assert torch.equal(mask_a, mask_b)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    assert torch.isneginf(lse_b[1]).all() and (out_b[1] == 0).all()


def test_workspace_reused_across_calls_with_different_lengths():
    """One workspace serves calls with different lengths (stale partials of an
    earlier, longer call are never read)."""
    say("decode: one workspace, several calls")
    inp = make_random_inputs(3, 8, 2, 128, (7000, 300, 4100), seed=31, block_size=64)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    ws = ffd.alloc_workspace(3, 8, 128, inp["cap"], 64, 4)
    sm = sm_scale_for(128)
    for lens in [(7000, 300, 4100), (64, 0, 4100), (6999, 300, 1), (7000, 300, 4100)]:
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        a = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, seq, delta=1.0, split_blocks=4, workspace=ws,
                       out_dtype=torch.float32)
        b = ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, seq, delta=1.0, split_blocks=4, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), lens
        r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], np.array(lens), max_seq_len=inp["cap"],
                                        block_size=64, delta=1.0, sink=1, local=4, split_blocks=4,
                                        sm_scale=np.float32(sm))
        assert_mask_equal(a[2].cpu().numpy(), r_mask, f"mask {lens}")
        assert_close(a[0].cpu().numpy(), r_out, f"out {lens}")
        assert_close(a[1].cpu().numpy(), r_lse, f"lse {lens}")


def test_workspace_garbage_is_never_used():
    """The combine reads each row's partial slots past the sequence's own
    (they lie inside the row's workspace) and drops them: a workspace full of
    NaN bytes gives bit-identical results to a zeroed one, for rows with no
    tokens, short rows and long rows (several query tokens too)."""
    say("decode: NaN-filled workspace")
    lens = (6000, 0, 130, 64 * 32 * 3)
    inp = make_random_inputs(4, 16, 4, 128, lens, seed=51, block_size=64)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    res = []
    for fill in (0x00, 0xFF):
        ws = ffd.alloc_workspace(4, 16, 128, inp["cap"], 64, 8)
        ws.fill_(fill)
        res.append(ffd.decode(dv["q"], dv["k"], dv["v"], kq, ks, dv["seq_lens"], delta=1.5, split_blocks=8,
                              workspace=ws, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for a, b, what in zip(res[0], res[1], ("out", "lse", "mask")):
        assert torch.equal(a, b), what
    assert not torch.isnan(res[1][0]).any() and not torch.isnan(res[1][1]).any()
    assert torch.isneginf(res[1][1][1]).all() and (res[1][0][1] == 0).all()
    Q = 3
    qm = dev_bf16(multi_query(inp, Q, seed=52))
    res = []
    for fill in (0x00, 0xFF):
        ws = torch.full((ffd.ffd_decode_multi_workspace_bytes(4, Q, 16, 128, inp["cap"], 64, 8),), fill,
                        dtype=torch.uint8, device="cuda")
        res.append(ffd.decode_multi(qm, dv["k"], dv["v"], kq, ks, dv["seq_lens"], delta=1.5, split_blocks=8,
                                    workspace=ws, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for a, b, what in zip(res[0], res[1], ("out", "lse", "mask")):
        assert torch.equal(a, b), "multi " + what


def test_graph_capture_and_replay():
    """ffd_decode allocates nothing and never synchronises, so it can be
    captured in a HIP graph; every replay (with new query data copied in
    between, eager work and syncs interleaved) matches an eager call."""
    say("decode: HIP graph capture and replay")
    inp = make_random_inputs(2, 16, 4, 128, (5000, 3000), seed=41, block_size=64)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    torch.cuda.synchronize()
    B, Hq, d = dv["q"].shape
    msl = inp["cap"]
    ws = ffd.alloc_workspace(B, Hq, d, msl, 64, 16)
    q_static = dv["q"].clone()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, -(-msl // 64)), dtype=torch.uint8, device="cuda")
    kw = dict(max_seq_len=msl, block_size=64, delta=2.0, sink=1, local=2, split_blocks=16,
              sm_scale=sm_scale_for(d))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the stream before capture
        ffd.ffd_decode(q_static, dv["k"], dv["v"], kq, ks, dv["seq_lens"], out=out, lse=lse, kept_mask=mask,
                       workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffd.ffd_decode(q_static, dv["k"], dv["v"], kq, ks, dv["seq_lens"], out=out, lse=lse, kept_mask=mask,
                       workspace=ws, **kw)
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        q_new = torch.randn(dv["q"].shape, device="cuda", generator=gen).to(torch.bfloat16)
        q_static.copy_(q_new)
        g.replay()
        torch.cuda.synchronize()
        ref = ffd.decode(q_new, dv["k"], dv["v"], kq, ks, dv["seq_lens"], out_dtype=torch.float32,
                         **{k_: v_ for k_, v_ in kw.items() if k_ != "block_size"})
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), rep
        assert torch.equal(lse, ref[1]), rep
        assert torch.equal(mask, ref[2]), rep
