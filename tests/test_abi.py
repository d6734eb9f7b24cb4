"""The C-ABI library loads, exports every entry point ``include/ffd.h``
declares, and rejects bad arguments on the host before any GPU work."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import sparse_long_context_ffd_amd as ffd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "ffd.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ffd_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = ffd.lib()
    names = _declared()
    assert set(names) >= {"ffd_quantize_kv", "ffd_decode", "ffd_decode_workspace_bytes", "ffd_decode_partials",
                          "ffd_combine"}
    for n in names:
        assert hasattr(L, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", ffd.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(ffd_[a-z_0-9]+)\b", dyn))
    assert set(names) <= exported
    assert set(ffd.EXPORTED_SYMBOLS) == set(names)
    assert ffd.ffd_abi_version() == 2


def test_workspace_bytes():
    ns = -(-(-(-131072 // 64)) // 32)
    exp = 4 * 32 * ns * 128 * 4 + (-(-4 * 32 * ns * 4 // 256)) * 256   # partials, lse
    assert ffd.ffd_decode_workspace_bytes(4, 32, 128, 131072, 64, 32) == exp
    assert ffd.ffd_decode_workspace_bytes(4, 32, 128, 131072, 32, 32) == 0   # unsupported block size
    assert ffd.ffd_decode_workspace_bytes(0, 32, 128, 131072, 64, 32) == 0


def _decode(**kw):
    args = dict(q=None, k=None, v=None, kq=None, kscale=None, seq_lens=None, max_seq_len=128, B=1, Hq=4, Hkv=1,
                d=128, cap=128, block_size=64, delta=6.0, sink=1, local=4, pm=0, split=32, sm_scale=0.088388,
                out=None, out_dtype=0, lse=None, mask=None, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    L = ffd.lib()
    return L.ffd_decode(args["q"], args["k"], args["v"], args["kq"], args["kscale"], args["seq_lens"],
                        args["max_seq_len"], args["B"], args["Hq"], args["Hkv"], args["d"], args["cap"],
                        args["block_size"], ctypes.c_float(args["delta"]), args["sink"], args["local"], args["pm"],
                        args["split"], ctypes.c_float(args["sm_scale"]), args["out"], args["out_dtype"],
                        args["lse"], args["mask"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Hq=6, Hkv=4), ffd.FFD_ERR_INVALID_ARG, "multiple"),
    (dict(d=65), ffd.FFD_ERR_INVALID_ARG, "even"),
    (dict(cap=64), ffd.FFD_ERR_INVALID_ARG, "cap"),
    (dict(delta=-1.0), ffd.FFD_ERR_INVALID_ARG, "delta"),
    (dict(delta=math.nan), ffd.FFD_ERR_INVALID_ARG, "delta"),
    (dict(sink=-1), ffd.FFD_ERR_INVALID_ARG, "sink"),
    (dict(split=0), ffd.FFD_ERR_INVALID_ARG, "split_blocks"),
    (dict(sm_scale=0.0), ffd.FFD_ERR_INVALID_ARG, "sm_scale"),
    (dict(sm_scale=math.inf), ffd.FFD_ERR_INVALID_ARG, "sm_scale"),
    (dict(out_dtype=7), ffd.FFD_ERR_INVALID_ARG, "out_dtype"),
    (dict(d=96), ffd.FFD_ERR_UNSUPPORTED, "d=96"),
    (dict(block_size=32), ffd.FFD_ERR_UNSUPPORTED, "block_size"),
    (dict(Hq=12, Hkv=4), ffd.FFD_ERR_UNSUPPORTED, "group size"),
    (dict(split=65), ffd.FFD_ERR_UNSUPPORTED, "split_blocks"),
    (dict(pm=3), ffd.FFD_ERR_INVALID_ARG, "pseudo_max"),
    (dict(pm=1, sink=0, local=0), ffd.FFD_ERR_INVALID_ARG, "sink/local"),
    (dict(pm=2, sink=0, local=0), ffd.FFD_ERR_INVALID_ARG, "sink/local"),
    (dict(pm=2, sink=40, local=30), ffd.FFD_ERR_UNSUPPORTED, "exceeds"),
    (dict(pm=1, sink=40, local=30), ffd.FFD_ERR_UNSUPPORTED, "exceeds"),
    (dict(), ffd.FFD_ERR_INVALID_ARG, "null"),
])
def test_host_validation(kw, status, needle):
    assert _decode(**kw) == status
    assert needle in ffd.ffd_last_error()


def test_workspace_too_small_and_misaligned():
    fake = 1 << 20  # never dereferenced: validation fails before any launch
    common = dict(q=fake, k=fake, v=fake, kq=fake, kscale=fake, seq_lens=fake, out=fake, lse=fake)
    assert _decode(**common, ws=fake, ws_bytes=16) == ffd.FFD_ERR_WORKSPACE
    assert "workspace" in ffd.ffd_last_error()
    assert _decode(**common, ws=fake + 16, ws_bytes=1 << 30) == ffd.FFD_ERR_INVALID_ARG
    assert "aligned" in ffd.ffd_last_error()
    assert _decode(**{**common, "kq": None}, ws=fake, ws_bytes=1 << 30) == ffd.FFD_ERR_INVALID_ARG
    assert "kq" in ffd.ffd_last_error()


def test_empty_batch_is_a_no_op():
    assert _decode(B=0) == ffd.FFD_OK
    assert ffd.ffd_last_error() == ""
    L = ffd.lib()
    assert L.ffd_quantize_kv(None, None, None, None, None, 0, 8, 128, 128, 10, None) == ffd.FFD_OK
    assert L.ffd_quantize_kv(None, None, None, None, None, 1, 8, 128, 96, 10, None) == ffd.FFD_ERR_UNSUPPORTED
    assert L.ffd_quantize_kv(None, None, None, None, None, 1, 8, 128, 128, 10, None) == ffd.FFD_ERR_INVALID_ARG


def test_paged_validation():
    L = ffd.lib()
    f = ctypes.c_float
    fake = 1 << 20
    # null block table
    st = L.ffd_decode_paged(fake, fake, fake, fake, fake, None, 4, 10, fake, 256, 1, 4, 1, 128, 64, f(2.0), 1, 1, 0,
                            32, f(0.1), fake, 0, fake, None, fake, 1 << 30, None)
    assert st == ffd.FFD_ERR_INVALID_ARG and "block_table" in ffd.ffd_last_error()
    # table too narrow for max_seq_len
    st = L.ffd_decode_paged(fake, fake, fake, fake, fake, fake, 3, 10, fake, 256, 1, 4, 1, 128, 64, f(2.0), 1, 1, 0,
                            32, f(0.1), fake, 0, fake, None, fake, 1 << 30, None)
    assert st == ffd.FFD_ERR_INVALID_ARG and "table_stride" in ffd.ffd_last_error()
    st = L.ffd_decode_paged(fake, fake, fake, fake, fake, fake, 4, 0, fake, 256, 1, 4, 1, 128, 64, f(2.0), 1, 1, 0,
                            32, f(0.1), fake, 0, fake, None, fake, 1 << 30, None)
    assert st == ffd.FFD_ERR_INVALID_ARG and "num_pages" in ffd.ffd_last_error()
    st = L.ffd_quantize_kv_paged(fake, fake, fake, None, 4, 10, fake, fake, 1, 8, 128, 64, None)
    assert st == ffd.FFD_ERR_INVALID_ARG and "block_table" in ffd.ffd_last_error()


def test_paged_multi_validation():
    """The multi-query block-table call checks its table and its query count
    like the single-token one, before any launch."""
    L = ffd.lib()
    f = ctypes.c_float
    fake = 1 << 20

    def call(table, stride, num_pages, Q, Hq=8, Hkv=2, ws_bytes=1 << 30):
        return L.ffd_decode_paged_multi(fake, fake, fake, fake, fake, table, stride, num_pages, fake, 256, 1, Q, Hq,
                                        Hkv, 128, 64, f(2.0), 1, 1, 0, 32, f(0.1), fake, 0, fake, fake, fake,
                                        ws_bytes, None)

    assert call(None, 4, 10, 2) == ffd.FFD_ERR_INVALID_ARG and "block_table" in ffd.ffd_last_error()
    assert call(fake, 3, 10, 2) == ffd.FFD_ERR_INVALID_ARG and "table_stride" in ffd.ffd_last_error()
    assert call(fake, 4, 0, 2) == ffd.FFD_ERR_INVALID_ARG and "num_pages" in ffd.ffd_last_error()
    assert call(fake, 4, 2 ** 30, 2, Hq=8, Hkv=2) == ffd.FFD_ERR_UNSUPPORTED and "num_pages" in ffd.ffd_last_error()
    assert call(fake, 4, 10, 0) == ffd.FFD_ERR_INVALID_ARG and "Q=0" in ffd.ffd_last_error()
    assert call(fake, 4, 10, 5, Hq=4, Hkv=1) == ffd.FFD_ERR_UNSUPPORTED
    assert "ffd_decode_paged_multi" in ffd.ffd_last_error()
    one = ffd.ffd_decode_workspace_bytes(1, 8, 128, 256, 64, 32)
    assert call(fake, 4, 10, 2, ws_bytes=one) == ffd.FFD_ERR_WORKSPACE


def test_package_reexports_every_entry_point():
    """Each C entry point has a wrapper of the same name at package level."""
    for n in ffd.EXPORTED_SYMBOLS:
        assert callable(getattr(ffd, n, None)), n


def _decode_multi(**kw):
    args = dict(q=None, k=None, v=None, kq=None, kscale=None, seq_lens=None, max_seq_len=128, B=1, Q=2, Hq=4, Hkv=1,
                d=128, cap=128, block_size=64, delta=6.0, sink=1, local=4, pm=0, split=32, sm_scale=0.088388,
                out=None, out_dtype=0, lse=None, mask=None, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    L = ffd.lib()
    return L.ffd_decode_multi(args["q"], args["k"], args["v"], args["kq"], args["kscale"], args["seq_lens"],
                              args["max_seq_len"], args["B"], args["Q"], args["Hq"], args["Hkv"], args["d"],
                              args["cap"], args["block_size"], ctypes.c_float(args["delta"]), args["sink"],
                              args["local"], args["pm"], args["split"], ctypes.c_float(args["sm_scale"]), args["out"],
                              args["out_dtype"], args["lse"], args["mask"], args["ws"], args["ws_bytes"],
                              args["stream"])


def _ws_expected(B, rows, Hq, L, S, d):
    ns = -(-(-(-L // 64)) // S)
    units = B * Hq * ns
    # workgroups per split: one, or on grids of at most 1024 units (8-wave
    # workgroups) up to four, about one round of them
    parts = min(4, max(1, 1024 // units)) if units <= 1024 else 1
    n = B * rows * ns * parts
    return -(-n * d * 4 // 256) * 256 + -(-n * 4 // 256) * 256


def test_multi_workspace_bytes():
    for B, Q, Hq, L in ((4, 4, 32, 131072), (1, 16, 8, 131072), (2, 1, 32, 131072), (1, 4, 32, 32768)):
        assert ffd.ffd_decode_multi_workspace_bytes(B, Q, Hq, 128, L, 64, 32) == _ws_expected(B, Q * Hq, Hq, L, 32, 128)
    assert ffd.ffd_decode_multi_workspace_bytes(1, 1, 32, 128, 32768, 64, 32) == \
        ffd.ffd_decode_workspace_bytes(1, 32, 128, 32768, 64, 32)
    assert ffd.ffd_decode_multi_workspace_bytes(4, 0, 32, 128, 131072, 64, 32) == 0


def test_small_grids_get_more_partials():
    # 32K tokens, one sequence: 16 splits x 32 heads = 512 units -> 2 workgroups per split
    assert ffd.ffd_decode_workspace_bytes(1, 32, 128, 32768, 64, 32) == _ws_expected(1, 32, 32, 32768, 32, 128)
    assert _ws_expected(1, 32, 32, 32768, 32, 128) >= 2 * 32 * 16 * 128 * 4
    # 128K x4: 8192 units -> one workgroup per split
    assert ffd.ffd_decode_workspace_bytes(4, 32, 128, 131072, 64, 32) == _ws_expected(4, 32, 32, 131072, 32, 128)
    assert _ws_expected(4, 32, 32, 131072, 32, 128) < 2 * 4 * 32 * 64 * 128 * 4


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Q=0), ffd.FFD_ERR_INVALID_ARG, "Q=0"),
    (dict(Q=5, Hq=4, Hkv=1), ffd.FFD_ERR_UNSUPPORTED, "rows per workgroup"),
    (dict(Q=3, Hq=8, Hkv=1), ffd.FFD_ERR_UNSUPPORTED, "rows per workgroup"),
    (dict(Q=16, Hq=2, Hkv=2, pm=1, sink=32, local=32), ffd.FFD_ERR_UNSUPPORTED, "exceeds"),
    (dict(Q=2), ffd.FFD_ERR_INVALID_ARG, "null"),
])
def test_multi_host_validation(kw, status, needle):
    assert _decode_multi(**kw) == status
    assert needle in ffd.ffd_last_error()


def test_multi_workspace_covers_every_query_row():
    fake = 1 << 20  # never dereferenced: validation fails before any launch
    common = dict(q=fake, k=fake, v=fake, kq=fake, kscale=fake, seq_lens=fake, out=fake, lse=fake, ws=fake)
    one = ffd.ffd_decode_workspace_bytes(1, 4, 128, 128, 64, 32)
    assert _decode_multi(**common, ws_bytes=one, Q=2) == ffd.FFD_ERR_WORKSPACE
    assert _decode_multi(**common, ws_bytes=one, Q=4, pm=1, sink=0, local=0) == ffd.FFD_ERR_INVALID_ARG
    assert _decode_multi(B=0, Q=4) == ffd.FFD_OK


def test_token_counts_above_2_30_are_rejected_not_overflowed():
    """Block counts and grid sizes are computed without int overflow; lengths
    past 2^30 tokens are refused before anything is launched."""
    big = 2 ** 31 - 1
    fake = 1 << 20
    common = dict(q=fake, k=fake, v=fake, kq=fake, kscale=fake, seq_lens=fake, out=fake, lse=fake, ws=fake,
                  ws_bytes=1 << 40)
    assert _decode(**common, max_seq_len=big, cap=big) == ffd.FFD_ERR_UNSUPPORTED
    assert "2^30" in ffd.ffd_last_error()
    assert ffd.ffd_decode_workspace_bytes(1, 32, 128, big, 64, 1) == 0
    assert ffd.ffd_decode_multi_workspace_bytes(1, 2, 32, 128, big, 64, 1) == 0
    assert ffd.ffd_decode_workspace_bytes(1, 32, 128, 2 ** 30, 64, 1) > 0
    L = ffd.lib()
    assert L.ffd_quantize_kv(fake, fake, fake, fake, fake, 1, 8, 128, 128, big, None) == ffd.FFD_ERR_UNSUPPORTED
    assert L.ffd_quantize_kv(fake, fake, fake, fake, fake, 1, 8, big, 128, 16, None) == ffd.FFD_ERR_UNSUPPORTED
    assert L.ffd_quantize_kv_paged(fake, fake, fake, fake, 2 ** 25, 4, fake, fake, 1, 8, 128, 16,
                                   None) == ffd.FFD_ERR_UNSUPPORTED
    assert L.ffd_combine(fake, big, 1, 32, 128, 64, 32, fake, 1 << 40, fake, 0, fake, None) == ffd.FFD_ERR_UNSUPPORTED


def _noalloc(**kw):
    """ffd_decode_noalloc with stand-in (never dereferenced) device pointers."""
    fake = ctypes.c_void_p(1 << 20)
    args = dict(max_seq_len=128, B=1, Hq=4, Hkv=1, d=128, cap=128, block_size=64, delta=6.0, pm=0, split=32)
    args.update(kw)
    return ffd.lib().ffd_decode_noalloc(fake, fake, fake, fake, fake, fake, args["max_seq_len"], args["B"],
                                        args["Hq"], args["Hkv"], args["d"], args["cap"], args["block_size"],
                                        ctypes.c_float(args["delta"]), 1, 4, args["pm"], args["split"],
                                        ctypes.c_float(0.088388), fake, 0, fake, None, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=8, Hq=64, max_seq_len=1 << 20, cap=1 << 20, split=16), ffd.FFD_ERR_WORKSPACE, "static scratch"),
    (dict(Hq=6, Hkv=4), ffd.FFD_ERR_INVALID_ARG, "multiple"),
    (dict(split=0), ffd.FFD_ERR_INVALID_ARG, "split_blocks"),
    (dict(d=96), ffd.FFD_ERR_UNSUPPORTED, "d=96"),
    (dict(cap=64), ffd.FFD_ERR_INVALID_ARG, "cap"),
])
def test_noalloc_rejects_on_host(kw, status, needle):
    """Sizes beyond the static array and bad arguments are refused before any
    device call (these run without a GPU)."""
    assert _noalloc(**kw) == status
    assert needle in ffd.ffd_last_error()


def test_noalloc_scratch_size_matches_header():
    with open(os.path.join(ROOT, "include", "ffd.h")) as f:
        src = f.read()
    m = re.search(r"#define FFD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ffd.NOALLOC_SCRATCH_BYTES
