"""The Python binding refuses tensors whose shapes do not match the call
before anything reaches the library: a pool or vector too small would
otherwise be read past its end on the GPU."""

import pytest
import torch

import sparse_long_context_ffd_amd as ffd

pytestmark = pytest.mark.gpu


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_paged_shapes_are_checked():
    B, Hq, Hkv, d, P = 2, 8, 2, 128, 6
    q = _t((B, Hq, d), torch.bfloat16)
    kp, vp = _t((P, Hkv, 64, d), torch.bfloat16), _t((P, Hkv, 64, d), torch.bfloat16)
    kqp, ksp = _t((P, Hkv, 64, d // 2), torch.uint8), _t((P, Hkv, 64), torch.float32)
    table, seq = _t((B, 3), torch.int32), _t((B,), torch.int32)
    out, lse = _t((B, Hq, d), torch.float32), _t((B, Hq), torch.float32)
    ws = _t(ffd.ffd_decode_workspace_bytes(B, Hq, d, 192, 64, 2), torch.uint8)
    kw = dict(max_seq_len=192, block_size=64, delta=1.0, sink=1, local=1, split_blocks=2, sm_scale=0.1, out=out,
              lse=lse, kept_mask=None, workspace=ws)
    ffd.ffd_decode_paged(q, kp, vp, kqp, ksp, table, seq, **kw)   # well-formed: runs (all lengths 0)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="kq/kscale pages"):
        ffd.ffd_decode_paged(q, kp, vp, kqp[:P - 1], ksp, table, seq, **kw)
    with pytest.raises(ValueError, match="kq/kscale pages"):
        ffd.ffd_decode_paged(q, kp, vp, kqp, ksp[:, :1].contiguous(), table, seq, **kw)
    with pytest.raises(ValueError, match="seq_lens"):
        ffd.ffd_decode_paged(q, kp, vp, kqp, ksp, table, seq[:1], **kw)
    q4 = _t((B, 2, Hq, d), torch.bfloat16)
    out4, lse4 = _t((B, 2, Hq, d), torch.float32), _t((B, 2, Hq), torch.float32)
    kw4 = dict(kw, out=out4, lse=lse4)
    with pytest.raises(ValueError, match="kq/kscale pages"):
        ffd.ffd_decode_paged_multi(q4, kp, vp, kqp[:, :1].contiguous(), ksp, table, seq, **kw4)
    with pytest.raises(ValueError, match="pos_end"):
        ffd.ffd_quantize_kv_paged(kp, kqp, ksp, table, _t((B,), torch.int32), _t((B - 1,), torch.int32), 64)


def test_thumb_and_combine_shapes_are_checked():
    B, Hq, Hkv, cap, d = 2, 4, 1, 128, 64
    k = _t((B, Hkv, cap, d), torch.bfloat16)
    k2, k2s = _t((B, Hkv, cap, d // 4), torch.uint8), _t((B, Hkv, cap), torch.float32)
    kr, krs = _t((B, Hkv, cap, d), torch.int8), _t((B, Hkv, cap), torch.float32)
    seq = _t((B,), torch.int32)
    with pytest.raises(ValueError, match="pos_begin"):
        ffd.ffd_quantize_kv_thumb(k, k2, k2s, kr, krs, _t((1,), torch.int32), seq, 64)
    q = _t((B, Hq, d), torch.bfloat16)
    out, lse = _t((B, Hq, d), torch.float32), _t((B, Hq), torch.float32)
    ws = _t(ffd.ffd_decode_workspace_bytes(B, Hq, d, cap, 64, 1), torch.uint8)
    kw = dict(max_seq_len=cap, block_size=64, delta=1.0, sink=1, local=1, split_blocks=1, sm_scale=0.1, out=out,
              lse=lse, kept_mask=None, workspace=ws)
    with pytest.raises(ValueError, match="shapes"):
        ffd.ffd_decode_thumb(q, k2, k2s[:, :, :cap - 1].contiguous(), kr, krs, k, seq, **kw)
    with pytest.raises(ValueError, match="seq_lens"):
        ffd.ffd_decode_thumb(q, k2, k2s, kr, krs, k, seq[:1], **kw)
    with pytest.raises(ValueError, match="seq_lens"):
        ffd.ffd_combine(seq[:1], max_seq_len=cap, block_size=64, split_blocks=1, workspace=ws, out=out, lse=lse)
