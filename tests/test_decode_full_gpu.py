"""Full-size workloads (128K x4, 256K, mixed 8K-128K x16, and the peaked
256K diagnostic) in the launch configuration the benchmark times: the whole
kept-block mask bit-exact against the oracle, output and LSE within the bar
on every head. Also the skip path's benchmark lines (256K at low delta),
where most blocks are dropped and the kept counts differ from split to
split."""

import numpy as np
import pytest

import sparse_long_context_ffd_amd as ffd
from ffd_inputs import WORKLOADS, make_inputs
from oracle import ffd_oracle as O
from tests import oracle_par as P
from tests.gpu_util import assert_close, assert_mask_equal, run_gpu, say, sm_scale_for, to_device

pytestmark = pytest.mark.gpu


def _check_workload(name, deltas):
    w = WORKLOADS[name]
    say(f"full-size workload {name}: generating")
    inp = make_inputs(w)
    dv = to_device(inp)
    sm = sm_scale_for(w.d)
    kq, ks = ffd.quantize_kv(dv["k"], dv["seq_lens"])
    keeps = []
    for delta in deltas:
        say(f"  {name} delta={delta}: GPU")
        out, lse, mask = run_gpu(dv, max_seq_len=inp["cap"], delta=delta, sink=w.sink, local=w.local,
                                 split_blocks=w.split_blocks, sm_scale=sm, kq=kq, kscale=ks)
        say(f"  kept fraction {mask[mask.sum(-1) > 0].mean() if mask.any() else 0:.4f}; oracle (every head)")
        args = dict(max_seq_len=inp["cap"], block_size=64, delta=delta, sink=w.sink, local=w.local,
                    split_blocks=w.split_blocks, sm_scale=np.float32(sm))
        r_out, r_lse, r_mask = P.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], **args)
        assert_mask_equal(mask, r_mask, f"{name} mask delta={delta}")
        assert_close(out, r_out, f"{name} out delta={delta}")
        assert_close(lse, r_lse, f"{name} lse delta={delta}")
        keeps.append(float(mask.mean()))
    return keeps


@pytest.mark.parametrize("name", ["llama3_8b_128k_b4", "llama3_8b_256k", "mixed_16x8k_128k", "diag_256k_peaked"])
def test_full_size(name):
    _check_workload(name, WORKLOADS[name].deltas)


def test_skip_path_low_delta():
    """256K at the deltas of the skip-path measurements: per-head keeps of
    about 0.03 to 0.4 (at delta 0 each head keeps its best block per split
    and the sink/local blocks), kept counts from 1 to 17 blocks per split."""
    keeps = _check_workload("llama3_8b_256k", (0.0, 0.25, 0.5, 1.0))
    assert keeps[0] < 0.05 and keeps[0] < keeps[1] < keeps[2] < keeps[3] < 0.5, keeps


@pytest.fixture(scope="module")
def longest_inputs():
    from ffd_inputs import make_random_inputs

    L = (1 << 20) + 37
    say(f"longest sequence L={L}: generating")
    inp = make_random_inputs(1, 8, 1, 128, (L,), seed=4242, block_size=64, hot_frac=0.01)
    return inp, to_device(inp)


@pytest.mark.parametrize("pm", ["split", "max"])
def test_longest_sequence_widest_split(pm, longest_inputs):
    """Sizes at the top of what one call handles in one piece: a single
    sequence of 2^20 + 37 tokens (16385 blocks, a ragged last block), the
    widest split (64 blocks), eight query heads on one kv head, and many sink
    and local blocks; mask bit-exact on every head, output and LSE on all."""
    inp, dv = longest_inputs
    say(f"longest sequence, S=64, {pm}: GPU")
    sm = sm_scale_for(128)
    kw = dict(max_seq_len=inp["cap"], delta=2.0, sink=4, local=12, split_blocks=64, pseudo_max=pm)
    out, lse, mask = run_gpu(dv, sm_scale=sm, **kw)
    say(f"  kept fraction {mask.mean():.4f}; oracle")
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], block_size=64,
                                    sm_scale=np.float32(sm), **kw)
    assert 0.0 < mask.mean() < 1.0
    assert_mask_equal(mask, r_mask, f"longest sequence mask ({pm})")
    assert_close(out, r_out, f"longest sequence out ({pm})")
    assert_close(lse, r_lse, f"longest sequence lse ({pm})")


def test_many_short_sequences():
    """A wide batch: 300 sequences of 0 to 3000 tokens (empty ones included)
    in one call, against the oracle on every row."""
    from ffd_inputs import make_random_inputs

    rng = np.random.default_rng(77)
    lens = rng.integers(0, 3001, size=300)
    lens[::37] = 0
    say(f"many short sequences: B={len(lens)}, {int(lens.sum())} tokens")
    inp = make_random_inputs(len(lens), 8, 2, 64, tuple(int(x) for x in lens), seed=78, block_size=64,
                             hot_frac=0.05)
    dv = to_device(inp)
    sm = sm_scale_for(64)
    kw = dict(max_seq_len=inp["cap"], delta=1.0, sink=1, local=2, split_blocks=8)
    out, lse, mask = run_gpu(dv, sm_scale=sm, **kw)
    r_out, r_lse, r_mask = O.decode(inp["q"], inp["k"], inp["v"], inp["seq_lens"], block_size=64,
                                    sm_scale=np.float32(sm), **kw)
    assert_mask_equal(mask, r_mask, "many sequences mask")
    assert_close(out, r_out, "many sequences out")
    assert_close(lse, r_lse, "many sequences lse")
