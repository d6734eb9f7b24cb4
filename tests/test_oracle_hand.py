"""The hand-worked 2-block example pins the oracle's quantiser, scan, Top-δ
rule (including the tie at the threshold) and exact attention."""

import json
import math
import os

import numpy as np
import pytest

from ffd_inputs import bf16_bits_from_f32
from oracle import ffd_oracle as O


@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_2block.json")) as f:
        return json.load(f)


def _closed(hand, key):
    e2, em2 = math.exp(2.0), math.exp(-2.0)
    env = {"e2": e2, "em2": em2, "ln": math.log}
    cf = hand["closed_forms"][key]
    return np.array([eval(s, {}, env) for s in cf["out"]]), eval(cf["lse"], {}, env)


def _inputs(hand):
    inp = hand["inputs"]
    return (bf16_bits_from_f32(np.array(inp["q"], np.float32)),
            bf16_bits_from_f32(np.array(inp["k"], np.float32)),
            bf16_bits_from_f32(np.array(inp["v"], np.float32)),
            np.array(inp["seq_lens"]))


def test_intermediates(hand):
    it = hand["intermediates"]
    qc, cq = O.quantize_query(np.array([1.0, 0.0], np.float32), np.float32(1.0))
    assert qc.tolist() == it["qc"]
    assert float(cq) == float.fromhex(it["cq_hex"])
    k = np.array(hand["inputs"]["k"], np.float32)[0, 0]
    codes, scale = O.quantize_keys(k)
    assert codes.tolist() == it["codes"]
    assert all(float(s) == float.fromhex(it["scale_hex"]) for s in scale)
    assert O.pack_int4(codes.reshape(-1)).tolist() == it["packed"]
    tok = O.token_scores(qc, cq, codes, scale)
    assert tok.dtype == np.float32
    assert tok.tolist() == it["token_scores"]
    assert O.block_scores(tok, 4, 2).tolist() == it["block_scores"]


@pytest.mark.parametrize("case_idx", range(7))
def test_cases(hand, case_idx):
    case = hand["cases"][case_idx]
    q, k, v, lens = _inputs(hand)
    inp = hand["inputs"]
    delta = math.inf if case["delta"] == "inf" else case["delta"]
    out, lse, mask = O.decode(q, k, v, lens, max_seq_len=4, block_size=inp["block_size"], delta=delta,
                              sink=case["sink"], local=case["local"], split_blocks=inp["split_blocks"],
                              sm_scale=np.float32(inp["sm_scale"]))
    assert mask[0, 0].tolist() == case["mask"]
    ref_out, ref_lse = _closed(hand, case["out"])
    np.testing.assert_allclose(out[0, 0], ref_out, rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - ref_lse) < 1e-14
