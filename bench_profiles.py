"""Summaries of rocprofv3 runs of ``bench.py`` for ``profiles/``.

``python bench.py --profile-summary STEM --trace-dir D --pmc-dirs D1,D2
--copy-pmc-dirs C1,C2 --bench-json F --commands F`` reads the CSV files that
rocprofv3 wrote (``--kernel-trace --stats``: ``*kernel_stats.csv``;
``--pmc``: ``*counter_collection.csv``) and the JSON line of the profiled
bench run, and writes ``profiles/STEM_kernel_stats.md`` and
``profiles/STEM_pmc.{json,md}``. No GPU work.

Bytes are derived from request counts at the L2's memory interface (the
TCC/EA counters), each request weighted by its size:

* reads:  32*RDREQ_32B + 64*RDREQ_64B + 128*RDREQ_128B  (all L2 misses);
  32*RDREQ_DRAM_32B  (those bound for DRAM, the counter's unit is 32 B);
* writes: 32*(WRREQ - WRREQ_64B) + 64*WRREQ_64B;  32*WRREQ_WRITE_DRAM_32B.

The DRAM-bound reads and writes are the traffic figure. A plain elementwise
copy of known size (``bench.py --copy-probe``) is read with the same counters
as a check of the derivation, not as a scale factor. FETCH_SIZE and
WRITE_SIZE (rocprofv3's derived KiB) are kept beside them for comparison:
on gfx950 FETCH_SIZE weighs a 128-byte request as 64 bytes.
"""

from __future__ import annotations

import csv
import glob
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_DIR = os.path.join(ROOT, "profiles")
FUSED = "fused_decode_kernel"
COPY = "neg"


def _rows(pattern_dir: str, suffix: str):
    files = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {pattern_dir}")
    out = []
    for fn in files:
        with open(fn, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def counters_per_dispatch(dirs, match: str, last: int = 0) -> dict:
    """Mean per dispatch of every counter collected in ``dirs`` for the
    kernels whose name contains ``match`` (only the last ``last`` dispatches
    if given), and the dispatch count."""
    per = {}
    for d in dirs:
        for r in _rows(d, "counter_collection.csv"):
            if match not in r["Kernel_Name"]:
                continue
            key = (d, int(r["Dispatch_Id"]))
            per.setdefault(r["Counter_Name"], {})
            per[r["Counter_Name"]][key] = per[r["Counter_Name"]].get(key, 0.0) + float(r["Counter_Value"])
    res = {}
    n = None
    for name, vals in per.items():
        keys = sorted(vals)
        if last:
            keys = keys[-last:]
        res[name] = sum(vals[k] for k in keys) / len(keys)
        n = len(keys)
    return {"counters": res, "dispatches": n}


def derived_bytes(c: dict) -> dict:
    g = lambda k: c.get(k)  # noqa: E731
    out = {}
    if all(g(k) is not None for k in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")):
        out["read_bytes"] = (32 * g("TCC_EA0_RDREQ_32B_sum") + 64 * g("TCC_EA0_RDREQ_64B_sum")
                             + 128 * g("TCC_EA0_RDREQ_128B_sum"))
    if g("TCC_EA0_RDREQ_DRAM_32B_sum") is not None:
        out["dram_read_bytes"] = 32 * g("TCC_EA0_RDREQ_DRAM_32B_sum")
    if g("TCC_EA0_WRREQ_sum") is not None and g("TCC_EA0_WRREQ_64B_sum") is not None:
        out["write_bytes"] = 32 * (g("TCC_EA0_WRREQ_sum") - g("TCC_EA0_WRREQ_64B_sum")) + 64 * g("TCC_EA0_WRREQ_64B_sum")
    if g("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum") is not None:
        out["dram_write_bytes"] = 32 * g("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    if g("FETCH_SIZE") is not None:
        out["fetch_size_kib"] = g("FETCH_SIZE")
    if g("WRITE_SIZE") is not None:
        out["write_size_kib"] = g("WRITE_SIZE")
    return out


def _bench_record(path: str) -> dict:
    with open(path) as f:
        lines = [ln for ln in f if ln.lstrip().startswith("{")]
    return json.loads(lines[-1])


def kernel_stats_md(trace_dir: str, rec: dict, commands: str) -> str:
    rows = _rows(trace_dir, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    cfg = rec["config"]
    lines = [f"# rocprofv3 kernel trace: FFD decode ({cfg['key_storage']}), workload {cfg['workload']} "
             f"(delta={cfg['delta']}, pseudo-max {cfg['pseudo_max']}, {cfg['kv_layout']}, "
             f"{cfg['query_tokens']} query token(s))", "",
             "Command (from the repository root on the GPU host, `$REPO` = repository path):", "", "```",
             commands.strip(), "```", "",
             "| Kernel | Calls | Avg (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    fused_avg = None
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        short = name.replace("void ", "").replace("(anonymous namespace)::", "")
        short = short.split("(")[0][:90]
        avg = float(r["AverageNs"]) / 1e3
        if FUSED in name and fused_avg is None:
            fused_avg = avg
        lines.append(f"| `{short}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    rl, t = rec["roofline"], rec["timing_us"]
    lines += ["", f"Same run, HIP events inside bench.py around each fused-kernel launch (flushed steps): "
                  f"mean {t['fused_mean']} us, median {t['fused_median']} us; rocprofv3 average "
                  f"{fused_avg:.1f} us.",
              f"Algorithmic bytes per launch {rl['algorithmic_bytes_per_launch']} ({rec['bytes']['scan']} scan + "
              f"{rec['bytes']['kv']} refinement); kept fraction per head {rec['kept_fraction']['per_head']}, "
              f"GQA union {rec['kept_fraction']['gqa_union']}.",
              f"Kernel source hash {rec['kernel_source_hash']}.", ""]
    return "\n".join(lines), fused_avg


def write_summaries(args) -> int:
    rec = _bench_record(args.bench_json)
    commands = open(args.commands).read() if args.commands else ""
    stem = args.profile_summary
    os.makedirs(PROFILE_DIR, exist_ok=True)
    trace_cmds = "\n".join(c for c in commands.splitlines() if "--kernel-trace" in c)
    pmc_cmds = "\n".join(c for c in commands.splitlines() if "--pmc" in c)
    if args.trace_dir:
        md, fused_avg = kernel_stats_md(args.trace_dir, rec, trace_cmds)
        with open(os.path.join(PROFILE_DIR, stem + "_kernel_stats.md"), "w") as f:
            f.write(md)
        print(f"wrote {stem}_kernel_stats.md (rocprof fused avg {fused_avg:.1f} us)")
    pmc = [d for d in args.pmc_dirs.split(",") if d]
    if not pmc:
        return 0
    k = counters_per_dispatch(pmc, FUSED)
    kb = derived_bytes(k["counters"])
    cp = [d for d in args.copy_pmc_dirs.split(",") if d]
    copy = None
    if cp:
        c = counters_per_dispatch(cp, COPY, last=5)
        cb = derived_bytes(c["counters"])
        known = 1 << 30
        copy = {"bytes_read": known, "bytes_written": known, "counters_per_dispatch": c["counters"],
                "derived": cb,
                "derived_over_known": {key: round(v / known, 5) for key, v in cb.items() if key.endswith("bytes")}}
        if "fetch_size_kib" in cb:
            copy["fetch_size_over_known"] = round(cb["fetch_size_kib"] * 1024 / known, 5)
        if "write_size_kib" in cb:
            copy["write_size_over_known"] = round(cb["write_size_kib"] * 1024 / known, 5)
    alg = rec["roofline"]["algorithmic_bytes_per_launch"]
    traffic = None
    if "dram_read_bytes" in kb and "dram_write_bytes" in kb:
        traffic = int(round(kb["dram_read_bytes"] + kb["dram_write_bytes"]))
    # cross-check: FETCH_SIZE and WRITE_SIZE scaled by what they read on the
    # copy of known size
    fw = None
    if copy and "fetch_size_kib" in kb and "write_size_kib" in kb and "fetch_size_over_known" in copy:
        fw = int(round(kb["fetch_size_kib"] * 1024 / copy["fetch_size_over_known"]
                       + kb["write_size_kib"] * 1024 / copy["write_size_over_known"]))
    cfg = rec["config"]
    out = {
        "kernel": FUSED,
        "mode": {"storage": "thumb" if "thumbnail" in cfg["key_storage"] else "int4",
                 "pseudo_max": cfg["pseudo_max"], "paged": cfg["kv_layout"] != "contiguous"},
        "workload": cfg["workload"],
        "delta": cfg["delta"],
        "query_tokens": cfg["query_tokens"],
        "kernel_source_hash": rec["kernel_source_hash"],
        "dispatches": k["dispatches"],
        "counters_per_dispatch": k["counters"],
        "derived_bytes_per_dispatch": kb,
        "copy_probe": copy,
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": None if traffic is None else round(traffic / alg, 4),
        "traffic_fetch_write_size_scaled": fw,
        "flush": rec["timing_us"]["flush"],
        "commands": [c for c in pmc_cmds.splitlines() if c.strip()],
    }
    with open(os.path.join(PROFILE_DIR, stem + "_pmc.json"), "w") as f:
        json.dump(out, f, indent=1)
    md = [f"# rocprofv3 memory counters: fused decode kernel ({cfg['key_storage']}), workload {cfg['workload']} "
          f"(delta={cfg['delta']}, pseudo-max {cfg['pseudo_max']}, {cfg['kv_layout']})", "",
          "Commands (`$REPO` = repository path on the GPU host):", "", "```", pmc_cmds.strip(), "```", "",
          "Bytes per fused-kernel dispatch, from request counts at the L2's memory interface weighted by request "
          "size (the DRAM-bound counters count 32-byte units).", "",
          "| Quantity | Fused kernel | Copy probe (1 GiB read + 1 GiB written) |", "|---|---|---|"]

    def fmt(x):
        return "—" if x is None else f"{x / 1e9:.4f} GB"

    cbd = copy["derived"] if copy else {}
    for key, label in (("read_bytes", "all reads (32/64/128-byte requests)"),
                       ("dram_read_bytes", "reads bound for DRAM"),
                       ("write_bytes", "all writes (32/64-byte requests)"),
                       ("dram_write_bytes", "writes bound for DRAM")):
        md.append(f"| {label} | {fmt(kb.get(key))} | {fmt(cbd.get(key))} |")
    if "fetch_size_kib" in kb:
        md.append(f"| FETCH_SIZE (rocprofv3 derived) | {kb['fetch_size_kib'] * 1024 / 1e9:.4f} GB | "
                  f"{fmt(cbd['fetch_size_kib'] * 1024) if 'fetch_size_kib' in cbd else '—'} |")
    md += ["", f"Traffic (DRAM reads + writes) per launch: {fmt(traffic)}; algorithmic bytes {alg / 1e9:.4f} GB; "
               f"traffic / algorithmic = {out['traffic_over_algorithmic']}.",
           f"Cross-check: FETCH_SIZE and WRITE_SIZE, each scaled by what it reads on the copy of known size "
           f"(x{1 / copy['fetch_size_over_known']:.4f} and x{1 / copy['write_size_over_known']:.4f}): "
           f"{fmt(fw)}." if fw is not None else "",
           f"Timed steps in bench.py: {out['flush']}.",
           f"Kernel source hash {rec['kernel_source_hash']}; {k['dispatches']} dispatches averaged.", ""]
    with open(os.path.join(PROFILE_DIR, stem + "_pmc.md"), "w") as f:
        f.write("\n".join(md))
    print(f"wrote {stem}_pmc.json/.md: traffic {traffic} B, alg {alg} B")
    return 0
