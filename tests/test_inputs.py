"""The seeded input generator: reproducible, bf16 rounding as torch does it,
tails poisoned on request, and hot blocks biased toward the group query."""

import numpy as np
import torch

from ffd_inputs import WORKLOADS, Workload, bf16_bits_from_f32, f32_from_bf16_bits, make_inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38, 1e-40], np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(f32_from_bf16_bits(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_poisoned():
    w = Workload(name="t", seed=7, B=2, Hq=4, Hkv=2, d=16, lens=(40, 17), block_size=8, hot_frac=0.3)
    a = make_inputs(w, poison_tail=True)
    b = make_inputs(w, poison_tail=True, threads=1)
    for key in ("q", "k", "v", "seq_lens"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["cap"] == 40
    assert np.isnan(f32_from_bf16_bits(a["k"][1, :, 17:])).all()
    assert not np.isnan(f32_from_bf16_bits(a["k"][1, :, :17])).any()
    c = make_inputs(w, poison_tail=False)
    assert (c["k"][1, :, 17:] == 0).all()


def test_hot_blocks_lean_toward_the_query():
    w = Workload(name="t", seed=3, B=1, Hq=4, Hkv=1, d=64, lens=(2048,), n_hot=4, alpha=(3.0, 3.0))
    inp = make_inputs(w)
    picks, amps = inp["biased_blocks"][(0, 0)]
    assert len(picks) == 4 and (amps == 3.0).all()
    qm = f32_from_bf16_bits(inp["q"][0]).mean(0)
    u = qm / np.linalg.norm(qm)
    proj = f32_from_bf16_bits(inp["k"][0, 0]) @ u
    blk = proj.reshape(32, 64).mean(1)
    assert set(np.argsort(blk)[-4:].tolist()) == set(picks.tolist())
    assert abs(blk[picks].mean() - 3.0) < 0.5


def test_workload_table():
    assert WORKLOADS["llama3_8b_128k_b4"].B == 4 and WORKLOADS["llama3_8b_128k_b4"].lens == (131072,) * 4
    w5 = WORKLOADS["mixed_16x8k_128k"]
    small = Workload(**{**w5.__dict__, "len_range": (64, 512), "name": "small5"})
    inp = make_inputs(small)
    assert inp["seq_lens"].shape == (16,)
    assert ((inp["seq_lens"] >= 64) & (inp["seq_lens"] <= 512)).all()
