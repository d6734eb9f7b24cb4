"""The rocprofv3 summaries in profiles/ and the code that derives HBM bytes
from their counters (CPU only): request counts weighted by request size give
back the bytes of the copy of known size, per-dispatch means are taken per
kernel, every committed summary is consistent with its own counters and was
taken on the current kernel source (so the benchmark reports its traffic)."""

import glob
import json
import os

import pytest

import bench
import bench_profiles as BP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PMC = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.json")))


def test_summaries_exist():
    assert len(PMC) >= 5
    for p in PMC:
        assert os.path.exists(p.replace("_pmc.json", "_pmc.md"))
        assert os.path.exists(p.replace("_pmc.json", "_kernel_stats.md"))


def test_copy_probe_counters_give_its_bytes():
    """1 GiB read + 1 GiB written by a plain elementwise kernel: the
    size-weighted request counts recorded with each summary return both."""
    for p in PMC:
        rec = json.load(open(p))
        d = BP.derived_bytes(rec["copy_probe"]["counters_per_dispatch"])
        assert abs(d["read_bytes"] / (1 << 30) - 1) < 1e-4, p
        assert abs(d["dram_read_bytes"] / (1 << 30) - 1) < 1e-4, p
        assert d["write_bytes"] == 1 << 30 and d["dram_write_bytes"] == 1 << 30, p


def test_derived_bytes_weights():
    c = {"TCC_EA0_RDREQ_32B_sum": 1, "TCC_EA0_RDREQ_64B_sum": 2, "TCC_EA0_RDREQ_128B_sum": 3,
         "TCC_EA0_RDREQ_DRAM_32B_sum": 5, "TCC_EA0_WRREQ_sum": 7, "TCC_EA0_WRREQ_64B_sum": 4,
         "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": 11}
    d = BP.derived_bytes(c)
    assert d["read_bytes"] == 32 + 128 + 384
    assert d["dram_read_bytes"] == 160
    assert d["write_bytes"] == 32 * 3 + 64 * 4
    assert d["dram_write_bytes"] == 352


def test_counters_per_dispatch(tmp_path):
    rows = [("1", "fused_decode_kernel<128>", "A", "10"), ("1", "fused_decode_kernel<128>", "A", "2"),
            ("2", "fused_decode_kernel<128>", "A", "20"), ("3", "combine_kernel<128>", "A", "99"),
            ("3", "fused_decode_kernel<128>", "B", "1")]
    with open(tmp_path / "x_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            f.write(",".join(r) + "\n")
    k = BP.counters_per_dispatch([str(tmp_path)], "fused_decode_kernel")
    assert k["counters"]["A"] == (12 + 20) / 2   # values of one dispatch add up (one per XCD or SE)
    assert k["counters"]["B"] == 1
    last = BP.counters_per_dispatch([str(tmp_path)], "fused_decode_kernel", last=1)
    assert last["counters"]["A"] == 20


@pytest.mark.parametrize("path", PMC, ids=[os.path.basename(p) for p in PMC])
def test_summary_is_consistent_and_current(path):
    rec = json.load(open(path))
    d = rec["derived_bytes_per_dispatch"]
    assert rec["traffic_bytes_per_launch"] == int(round(d["dram_read_bytes"] + d["dram_write_bytes"]))
    assert rec["traffic_over_algorithmic"] == round(rec["traffic_bytes_per_launch"]
                                                    / rec["algorithmic_bytes_per_launch"], 4)
    # reads at least the algorithmic bytes, and no more than a few percent beyond
    assert 1.0 <= rec["traffic_over_algorithmic"] < 1.07
    assert rec["kernel_source_hash"] == bench.kernel_source_hash(), \
        "profile taken on another kernel source: re-run the rocprofv3 passes"


def _traffic(stem):
    return json.load(open(os.path.join(ROOT, "profiles", stem + "_pmc.json")))["traffic_bytes_per_launch"]


def test_bench_finds_the_summary_of_its_mode():
    """Each bench line takes the summary of its own workload, δ, storage, KV
    layout, pseudo-max and query-token count, and none when there is none."""
    mode = {"storage": "int4", "pseudo_max": "split", "paged": False}
    c3 = "llama3_8b_128k_b4"
    assert bench.load_traffic(c3, 6.0, mode) == _traffic("fused_decode_llama3_8b_128k_b4")
    assert bench.load_traffic(c3, 6.0, {**mode, "paged": True}) == _traffic("fused_decode_llama3_8b_128k_b4_paged")
    assert bench.load_traffic(c3, 6.0, mode, 4) == _traffic("fused_decode_llama3_8b_128k_b4_q4")
    assert bench.load_traffic(c3, 6.0, {**mode, "pseudo_max": "sink_local"}) == \
        _traffic("fused_decode_llama3_8b_128k_b4_sink_local")
    assert bench.load_traffic("llama3_8b_256k", 0.25, mode) == _traffic("fused_decode_llama3_8b_256k_delta0.25")
    assert bench.load_traffic(c3, 5.0, mode) is None
    assert bench.load_traffic(c3, 6.0, mode, 2) is None
    assert bench.load_traffic(c3, 6.0, {**mode, "paged": True, "pseudo_max": "sink_local"}) is None
