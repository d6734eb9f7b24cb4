"""Seeded random sweep over the configuration space, every case against the
oracle (mask bit-exact, out/LSE within the bar): entry point (int4 sketch,
thumbnail storage, paged cache, several query tokens, both of the last two), group size, head dim,
split size up to its maximum of 64 blocks, sink/local counts up to the
sink/local mode's limit, δ from 0 to +inf, the three pseudo-max modes, bf16 and
fp32 output, lengths that are empty, a single token, on block boundaries or
ragged, and cache capacities that are not a whole number of blocks."""

import math

import numpy as np
import pytest
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import make_random_inputs, multi_query
from oracle import ffd_oracle as O
from tests.gpu_util import assert_close, assert_mask_equal, dev_bf16, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu

N_CASES = 1024


def _case(i):
    rng = np.random.default_rng(20_000 + i)
    kind = ["int4", "thumb", "paged", "multi"][i % 4]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    Q = 1
    if kind == "multi":
        Q = int(rng.integers(2, 16 // G + 1)) if G < 8 else 2
    B = int(rng.integers(1, 4))
    lens = []
    for _ in range(B):
        r = rng.random()
        if r < 0.1:
            lens.append(0)
        elif r < 0.2:
            lens.append(1)
        elif r < 0.35:
            lens.append(64 * int(rng.integers(1, 40)))
        else:
            lens.append(int(rng.integers(2, 4000)))
    S = int(rng.choice([1, 2, 3, 7, 16, 64]))
    delta = float(rng.choice([0.0, 0.5, 1.0, 2.0, 4.0, math.inf]))
    pm = "sink_local" if (rng.random() < 0.35 and not math.isinf(delta)) else "split"
    sink, local = int(rng.integers(0, 3)), int(rng.integers(0, 5))
    if rng.random() < 0.1:
        sink, local = 30, 33   # the sink/local mode's largest total (64 with the query range)
    if pm == "sink_local" and sink + local == 0:
        local = 1
    out_bf16 = bool(rng.random() < 0.25)
    # (drawn last, so the draws above are those of the earlier sweep)
    odd_cap = bool(rng.random() < 0.3) and kind != "paged"
    cap_extra = int(rng.integers(0, 6))
    if pm == "sink_local" and rng.random() < 0.4:
        pm = "max"   # the larger of the split max and the sink/local estimate
    if kind == "paged" and rng.random() < 0.5:
        Q = int(rng.integers(2, 16 // G + 1)) if G < 8 else 2   # several query tokens over the pages
    return dict(kind=kind, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, Q=Q, lens=tuple(lens), S=S, delta=delta, pm=pm,
                sink=sink, local=local, out_bf16=out_bf16, odd_cap=odd_cap, cap_extra=cap_extra, seed=30_000 + i)


def _recap(x: torch.Tensor, cap: int) -> torch.Tensor:
    """Cache rows [B, Hkv, cap0, d] cut, or padded with NaN, to cap rows."""
    if cap <= x.shape[2]:
        return x[:, :, :cap].contiguous()
    pad = torch.full(x.shape[:2] + (cap - x.shape[2],) + x.shape[3:], float("nan"), dtype=x.dtype, device=x.device)
    return torch.cat([x, pad], dim=2)


def _pages(x, nbs, table_np, num_pages):
    B, Hkv = x.shape[:2]
    pool = torch.full((num_pages, Hkv, 64) + tuple(x.shape[3:]), 0, dtype=x.dtype, device=x.device)
    if x.dtype == torch.bfloat16:
        pool.fill_(float("nan"))
    for b in range(B):
        for jb in range(nbs[b]):
            pool[int(table_np[b, jb])] = x[b, :, 64 * jb:64 * jb + 64]
    return pool


def _paged_pools(c, dv, kq, ks, nbm):
    """The cache rows on shuffled 64-token pages (unused page slots NaN) and the block table."""
    B = c["B"]
    nbs = [-(-L // 64) for L in c["lens"]]
    num_pages = max(1, sum(nbs))
    perm = np.random.default_rng(c["seed"]).permutation(num_pages)
    table_np = np.zeros((B, nbm), dtype=np.int32)
    used = 0
    for b in range(B):
        table_np[b, :nbs[b]] = perm[used:used + nbs[b]]
        used += nbs[b]
    pools = [_pages(x, nbs, table_np, num_pages) for x in (dv["k"], dv["v"], kq, ks)]
    return pools, torch.from_numpy(table_np).cuda()


def _case_four_waves(i):
    """A case on a grid of more than 1024 (sequence, query head, split) units,
    where the kernel runs 4-wave workgroups (smaller grids run 8-wave ones):
    three ragged sequences, 16 or 32 query heads, one-block splits."""
    rng = np.random.default_rng(40_000 + i)
    kind = ["int4", "thumb", "paged", "multi"][i % 4]
    G = int(rng.choice([2, 4, 8]))
    Hkv = 8 if G == 2 else 4
    d = int(rng.choice([64, 128]))
    Q = (int(rng.integers(2, 16 // G + 1)) if G < 8 else 2) if kind == "multi" else 1
    lens = tuple(int(x) for x in rng.integers(1500, 4000, size=3))
    delta = float(rng.choice([0.0, 1.0, 2.0, 4.0, math.inf]))
    pm = str(rng.choice(["split", "sink_local", "max"])) if not math.isinf(delta) else "split"
    sink, local = int(rng.integers(0, 3)), int(rng.integers(1, 5))
    c = dict(kind=kind, B=3, Hq=G * Hkv, Hkv=Hkv, d=d, Q=Q, lens=lens, S=1, delta=delta, pm=pm, sink=sink,
             local=local, out_bf16=bool(rng.random() < 0.25), odd_cap=False, cap_extra=0, seed=45_000 + i)
    ns = -(-max(lens) // 64)
    assert c["B"] * c["Hq"] * ns > 1024
    return c


@pytest.mark.parametrize("i", range(64))
def test_random_case_four_waves(i):
    _run_case(_case_four_waves(i), f"4-wave {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _run_case(_case(i), str(i))


def _run_case(c, i):
    if c["pm"] != "split" and c["sink"] + c["local"] + (c["Q"] > 1) > 64:
        c["local"] -= 1
    say(f"random case {i}: {c}")
    inp = make_random_inputs(c["B"], c["Hq"], c["Hkv"], c["d"], c["lens"], seed=c["seed"], block_size=64,
                             hot_frac=0.08)
    dv = to_device(inp)
    cap = inp["cap"]
    if c["odd_cap"]:
        # a capacity that is not a whole number of blocks (or of 4-token groups)
        cap = max(max(c["lens"]), 1) + c["cap_extra"]
        dv["k"], dv["v"] = _recap(dv["k"], cap), _recap(dv["v"], cap)
    sm = sm_scale_for(c["d"])
    odt = torch.bfloat16 if c["out_bf16"] else torch.float32
    kw = dict(max_seq_len=cap, block_size=64, delta=c["delta"], sink=c["sink"], local=c["local"],
              split_blocks=c["S"], sm_scale=sm, pseudo_max=c["pm"])
    rkw = dict(max_seq_len=cap, block_size=64, delta=c["delta"], sink=c["sink"], local=c["local"],
               split_blocks=c["S"], sm_scale=np.float32(sm), pseudo_max=c["pm"])
    dense = math.isinf(c["delta"])
    B, Hq, d = c["B"], c["Hq"], c["d"]
    nbm = -(-cap // 64)
    if c["kind"] == "multi":
        qm = multi_query(inp, c["Q"], seed=c["seed"] + 1)
        kq, ks = (None, None) if dense else ffd.quantize_kv(dv["k"], dv["seq_lens"])
        out, lse, mask = ffd.decode_multi(dev_bf16(qm), dv["k"], dv["v"], kq, ks, dv["seq_lens"], out_dtype=odt,
                                          **kw)
        r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], **rkw)
    else:
        out = torch.empty((B, Hq, d), dtype=odt, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        mask = torch.empty((B, Hq, nbm), dtype=torch.uint8, device="cuda")
        ws = ffd.alloc_workspace(B, Hq, d, cap, 64, c["S"])
        io = dict(out=out, lse=lse, kept_mask=mask, workspace=ws)
        if c["kind"] == "thumb":
            k2, k2s, kr, krs = ffd.quantize_kv_thumb(dv["k"], dv["seq_lens"])
            ffd.ffd_decode_thumb(dv["q"], k2, k2s, kr, krs, dv["v"], dv["seq_lens"], **kw, **io)
            r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], storage="thumb", **rkw)
        else:
            kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
            if c["kind"] == "paged" and c["Q"] > 1:
                pools, table = _paged_pools(c, dv, kq, ks, nbm)
                Q = c["Q"]
                qm = multi_query(inp, Q, seed=c["seed"] + 1)
                out = torch.empty((B, Q, Hq, d), dtype=odt, device="cuda")
                lse = torch.empty((B, Q, Hq), dtype=torch.float32, device="cuda")
                mask = torch.empty((B, Q, Hq, nbm), dtype=torch.uint8, device="cuda")
                ws = torch.empty(ffd.ffd_decode_multi_workspace_bytes(B, Q, Hq, d, cap, 64, c["S"]),
                                 dtype=torch.uint8, device="cuda")
                ffd.ffd_decode_paged_multi(dev_bf16(qm), pools[0], pools[1], None if dense else pools[2],
                                           None if dense else pools[3], table, dv["seq_lens"], out=out, lse=lse,
                                           kept_mask=mask, workspace=ws, **kw)
                r_out, r_lse, r_mask = O.decode_multi(qm, inp["k"], inp["v"], inp["seq_lens"], **rkw)
            elif c["kind"] == "paged":
                pools, table = _paged_pools(c, dv, kq, ks, nbm)
                ffd.ffd_decode_paged(dv["q"], pools[0], pools[1], None if dense else pools[2],
                                     None if dense else pools[3], table, dv["seq_lens"], **kw, **io)
                r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **rkw)
            else:
                ffd.ffd_decode(dv["q"], dv["k"], dv["v"], None if dense else kq, None if dense else ks,
                               dv["seq_lens"], **kw, **io)
                r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **rkw)
    torch.cuda.synchronize()
    assert_mask_equal(mask.cpu().numpy(), r_mask, f"case {i} mask")
    assert_close(out.float().cpu().numpy(), r_out, f"case {i} out", bf16_out=c["out_bf16"])
    assert_close(lse.cpu().numpy(), r_lse, f"case {i} lse")
