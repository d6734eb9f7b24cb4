"""GPU parity for the sink/local pseudo-max modes ("sink_local", and "max":
the larger of the split max and the sink/local estimate): mask bit-exact and
out/LSE within the bar against the oracle, including splits that keep no
block at all, and the 128K x4 workload at full size."""

import math

import numpy as np
import pytest

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import WORKLOADS, bf16_bits_from_f32, f32_from_bf16_bits, make_inputs, make_random_inputs
from oracle import ffd_oracle as O
from tests import oracle_par as P
from tests.gpu_util import assert_close, assert_mask_equal, run_gpu, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu

CASES = [
    (1, 4, 1, 64, (2048,), 2.0, 1, 2, 32),
    (3, 8, 8, 128, (1, 63, 700), 1.0, 1, 1, 1),
    (2, 16, 2, 128, (4000, 1000), 0.5, 2, 3, 3),
    (2, 8, 2, 64, (3000, 2999), 3.0, 0, 4, 7),
    (1, 8, 4, 128, (9000,), 1.5, 4, 0, 16),
    (4, 32, 8, 128, (0, 5000, 6400, 77), 6.0, 1, 4, 32),
]


@pytest.mark.parametrize("pm", ["sink_local", "max"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_small_cases(case, pm):
    B, Hq, Hkv, d, lens, delta, sink, local, S = CASES[case]
    say(f"{pm} case {case}: B={B} Hq={Hq} Hkv={Hkv} d={d} lens={lens} delta={delta} S={S}")
    inp = make_random_inputs(B, Hq, Hkv, d, lens, seed=500 + case, block_size=64, hot_frac=0.1)
    sm = sm_scale_for(d)
    out, lse, mask = run_gpu(to_device(inp), max_seq_len=inp["cap"], delta=delta, sink=sink, local=local,
                             split_blocks=S, sm_scale=sm, pseudo_max=pm)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], max_seq_len=inp["cap"],
                                    block_size=64, delta=delta, sink=sink, local=local, split_blocks=S,
                                    sm_scale=np.float32(sm), pseudo_max=pm)
    assert_mask_equal(mask, r_mask, "mask")
    assert_close(out, r_out, "out")
    assert_close(lse, r_lse, "lse")


def test_max_mode_is_the_intersection_on_the_gpu():
    """On the GPU too, the "max" mode keeps exactly the blocks both the split
    and the sink/local modes keep (same cache, same query)."""
    say("max mode = split AND sink_local (GPU)")
    inp = make_random_inputs(2, 16, 4, 128, (6000, 2500), seed=520, block_size=64, hot_frac=0.1)
    dv = to_device(inp)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    kw = dict(max_seq_len=inp["cap"], delta=0.75, sink=1, local=3, split_blocks=8, sm_scale=sm_scale_for(128),
              kq=kq, kscale=ks)
    m = {pm: run_gpu(dv, pseudo_max=pm, **kw)[2] for pm in ("split", "sink_local", "max")}
    np.testing.assert_array_equal(m["max"], m["split"] & m["sink_local"])
    assert (m["max"] != m["split"]).any() and (m["max"] != m["sink_local"]).any()


def test_whole_splits_dropped():
    """A dominant sink block pushes m~ up so that whole splits keep nothing;
    their partials must carry zero weight."""
    say("sink_local: whole splits dropped")
    inp = make_random_inputs(2, 8, 2, 128, (64 * 48, 64 * 20 + 5), seed=77, block_size=64, hot_frac=0.05)
    k = f32_from_bf16_bits(inp["k"]).copy()
    for b in range(2):
        for j in range(2):
            qv = f32_from_bf16_bits(inp["q"][b, 4 * j:4 * j + 4]).mean(0)
            k[b, j, :64] += 5.0 * qv / np.linalg.norm(qv)
    inp["k"] = bf16_bits_from_f32(k)
    sm = sm_scale_for(128)
    kw = dict(max_seq_len=inp["cap"], delta=1.0, sink=1, local=1, split_blocks=4, sm_scale=sm)
    out, lse, mask = run_gpu(to_device(inp), pseudo_max="sink_local", **kw)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], block_size=64,
                                    pseudo_max="sink_local", **{**kw, "sm_scale": np.float32(sm)})
    nb = 48
    empty = [(h, s) for h in range(8) for s in range(nb // 4) if not r_mask[0, h, 4 * s:4 * s + 4].any()]
    assert empty, "construction should drop at least one whole split"
    assert_mask_equal(mask, r_mask, "mask")
    assert_close(out, r_out, "out")
    assert_close(lse, r_lse, "lse")


def test_128k_workload_full_size():
    w = WORKLOADS["llama3_8b_128k_b4"]
    say("sink_local: 128K x4 full size")
    inp = make_inputs(w)
    dv = to_device(inp)
    sm = sm_scale_for(w.d)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    for delta in (2.0, 6.0):
        out, lse, mask = run_gpu(dv, max_seq_len=inp["cap"], delta=delta, sink=w.sink, local=w.local,
                                 split_blocks=w.split_blocks, sm_scale=sm, kq=kq, kscale=ks, pseudo_max="sink_local")
        args = dict(max_seq_len=inp["cap"], block_size=64, delta=delta, sink=w.sink, local=w.local,
                    split_blocks=w.split_blocks, sm_scale=np.float32(sm), pseudo_max="sink_local")
        say(f"  delta={delta}: kept fraction {mask.mean():.4f}; oracle (every head)")
        r_out, r_lse, r_mask = P.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **args)
        assert_mask_equal(mask, r_mask, f"mask delta={delta}")
        assert_close(out, r_out, f"out delta={delta}")
        assert_close(lse, r_lse, f"lse delta={delta}")
