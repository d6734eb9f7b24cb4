"""Helpers for the GPU parity tests: move generated inputs to the device, run
the library through its C ABI, and compare against the oracle."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import sparse_long_context_ffd_amd as ffd

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
