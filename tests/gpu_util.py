"""Helpers for the GPU parity tests: move generated inputs to the device, run
the library through its C ABI, and compare against the oracle."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import make_random_inputs, multi_query
from oracle import ffd_oracle as O

RTOL = 2e-3
ATOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def to_device(inp: dict) -> dict:
    return {
        "q": dev_bf16(inp["q"]),
        "k": dev_bf16(inp["k"]),
        "v": dev_bf16(inp["v"]),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(inp["seq_lens"], dtype=np.int32)).to("cuda"),
    }


def sm_scale_for(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def run_gpu(dv: dict, *, max_seq_len: int, delta: float, sink: int, local: int, split_blocks: int,
            sm_scale: float, out_dtype=torch.float32, kq=None, kscale=None, pseudo_max: str = "split"):
    if kq is None and not math.isinf(delta):
        kq, kscale = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    out, lse, mask = ffd.decode(dv["q"], dv["k"], dv["v"], kq, kscale, dv["seq_lens"], max_seq_len=max_seq_len,
                                block_size=64, delta=delta, sink=sink, local=local, split_blocks=split_blocks,
                                sm_scale=sm_scale, out_dtype=out_dtype, pseudo_max=pseudo_max)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), mask.cpu().numpy()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 8).astype(int))


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, rtol: float = RTOL, atol: float = ATOL,
                 bf16_out: bool = False) -> None:
    """|gpu - ref| <= atol + rtol*|ref| elementwise. With ``bf16_out`` the GPU
    value was rounded to bf16 after the computation, so half a bf16 ulp of ref
    is added to the bound (bf16 keeps 8 significant bits: up to 3.9e-3
    relative, more than the 2e-3 relative bar alone allows)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_r = np.isinf(ref)
    assert (np.isinf(gpu) == inf_r).all() and (np.sign(gpu[inf_r]) == np.sign(ref[inf_r])).all(), \
        f"{what}: infinities differ"
    fin = ~inf_r
    err = np.abs(gpu[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    if bf16_out:
        bound = bound + bf16_half_ulp(ref[fin])
    bad = err > bound
    assert not np.isnan(gpu[fin]).any(), f"{what}: NaN in GPU result"
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside {atol}+{rtol}|ref|; "
                           f"worst err {err.max():.3e} (bound there {bound[np.argmax(err - bound)]:.3e})")


def assert_mask_equal(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    if not np.array_equal(gpu, ref):
        diff = np.argwhere(gpu != ref)
        raise AssertionError(f"{what}: mask differs at {len(diff)} entries, first {diff[:5].tolist()}")


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


def run_case(c, i):
    """One seeded case (a dict: entry point ``kind`` in int4 / thumb / paged /
    multi, shapes, selection settings, optional ``sigma`` and ``outlier`` of
    the q/K draws) against the oracle: mask bit-exact, out/LSE within the bar."""
    if c["pm"] != "split" and c["sink"] + c["local"] + (c["Q"] > 1) > 64:
        c["local"] -= 1
    say(f"random case {i}: {c}")
    inp = make_random_inputs(c["B"], c["Hq"], c["Hkv"], c["d"], c["lens"], seed=c["seed"], block_size=64,
                             hot_frac=0.08,
                             qk_sigma=c.get("sigma", 1.0), k_outlier=c.get("outlier"))
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
