"""Summarises rocprofv3 output of a bench.py run into a short text profile and a traffic table.

Inputs (directories written by rocprofv3 --output-format csv -o run):
  --kt     kernel trace + stats run        (run_kernel_stats.csv, run_kernel_trace.csv)
  --fetch  optional --pmc FETCH_SIZE run   (run_counter_collection.csv)
  --write  optional --pmc WRITE_SIZE run   (run_counter_collection.csv)
  --sq     optional --pmc SQ_* run         (run_counter_collection.csv)
  --bench  optional bench.py JSON line of the same workload (algorithmic bytes per kernel)

HBM traffic per dispatch = counter KiB x 1024 x calibration, where the calibration of each
counter is taken from the library's streaming copy kernel in the same run, whose true traffic
is known (bytes read = bytes written = its size): calibration = true bytes / counted bytes.

Outputs: a markdown summary (--out) and, with --traffic, a JSON table {kernel: {HBM bytes per
launch, hash of the kernel's defining source and the internal header}}, which bench.py reports
as `traffic` only while that kernel's source is unchanged.

Usage: python -m rank_kv_cache_layer_amd.profsum --kt D --fetch D --write D [--sq D]
           [--bench F] --copy-bytes N --cmd "..." --out profiles/X.md
           [--traffic profiles/traffic.json [--merge]]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
HOT = ("split_score", "split_score_sliced", "split_apply", "score_cos_mfma", "score_cos_gemm", "fused_hop")
N_SE, N_SIMD = 32, 1024   # MI355X: 8 XCDs x 4 shader engines; 256 CUs x 4 SIMDs


def short_name(k: str) -> str:
    """'void kvc::(anonymous namespace)::split_score<128, 2>(kvc::SplitArgs)' -> 'split_score'."""
    k = k.replace("(anonymous namespace)::", "").replace("void ", "")
    k = re.sub(r"[(<].*$", "", k)
    return k.split("::")[-1].strip()


_KERNEL_DEF = re.compile(r"__global__\s+void\s+__launch_bounds__\([^)]*\)\s+(\w+)\s*\(")


def kernel_source_hash(name: str) -> str:
    """Hash of the shared internal header and of the source file(s) that define kernel `name`
    (none for runtime or torch kernels), so a counter figure goes stale only when that
    kernel's own source changes."""
    csrc = os.path.join(PKG, "csrc")
    h = hashlib.sha256(open(os.path.join(csrc, "kvc_internal.h"), "rb").read())
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".hip"):
            text = open(os.path.join(csrc, f), "rb").read()
            if name in _KERNEL_DEF.findall(text.decode()):
                h.update(f.encode() + text)
    return h.hexdigest()[:16]


def counters(d: str):
    """{short kernel name: {counter: [per-dispatch values]}} from a --pmc run."""
    out = defaultdict(lambda: defaultdict(list))
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            out[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def kernel_stats(d: str):
    rows = {}
    with open(os.path.join(d, "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows[short_name(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]), float(r["Percentage"]))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kt", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--sq")
    ap.add_argument("--bench")
    ap.add_argument("--copy-bytes", type=int, default=0, help="size of one peak_copy dispatch")
    ap.add_argument("--cmd", required=True, help="the profiled command, for the record")
    ap.add_argument("--title", default="per-hop correction, 32768-token Llama-3.1-8B-shaped hop")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic")
    ap.add_argument("--merge", action="store_true",
                    help="keep the traffic table's entries for kernels this run did not launch")
    a = ap.parse_args()

    ks = kernel_stats(a.kt)
    counted = bool(a.fetch and a.write)
    fe, wr = (counters(a.fetch), counters(a.write)) if counted else ({}, {})
    sq = counters(a.sq) if a.sq else {}
    bench = json.loads(open(a.bench).read().strip().splitlines()[-1]) if a.bench else None

    cal_f = cal_w = None
    if counted:
        copy_f = statistics.median(fe["peak_copy"]["FETCH_SIZE"]) * 1024
        copy_w = statistics.median(wr["peak_copy"]["WRITE_SIZE"]) * 1024
        cal_f, cal_w = a.copy_bytes / copy_f, a.copy_bytes / copy_w

    lines = [f"# rocprofv3 profile: {a.title}", "",
             "Commands (run from the repository root on one MI355X, `export TMPDIR=/tmp`):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv -d <kt> -o run -- {a.cmd}"]
    if counted:
        lines += [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- {a.cmd}",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- {a.cmd}"]
    if a.sq:
        names = sorted({c for k in sq.values() for c in k})
        lines.append(f"rocprofv3 --pmc {' '.join(names)} --output-format csv -d <sq> -o run -- {a.cmd}")
    if counted:
        lines += ["python -m rank_kv_cache_layer_amd.profsum --kt <kt> --fetch <fetch> --write <write> "
                  f"{'--sq <sq> ' if a.sq else ''}--copy-bytes {a.copy_bytes} ...", "```", "",
                  f"Counter calibration from the streaming copy kernel ({a.copy_bytes} bytes read and written per "
                  f"dispatch): FETCH_SIZE x {cal_f:.3f}, WRITE_SIZE x {cal_w:.3f}.", "",
                  "| kernel | calls | avg ms | % time | HBM read GB/launch | HBM write GB/launch | algorithmic GB/launch |",
                  "|---|---|---|---|---|---|---|"]
    else:
        lines += [f"python -m rank_kv_cache_layer_amd.profsum --kt <kt> {'--sq <sq> ' if a.sq else ''}...", "```", "",
                  "| kernel | calls | avg ms | % time |", "|---|---|---|---|"]
    traffic = {}
    algo = (bench or {}).get("kernels", {})
    for name, (calls, avg_ns, pct) in sorted(ks.items(), key=lambda x: -x[1][2]):
        f = statistics.median(fe[name]["FETCH_SIZE"]) * 1024 * cal_f if name in fe else None
        w = statistics.median(wr[name]["WRITE_SIZE"]) * 1024 * cal_w if name in wr else None
        if f is not None and w is not None:
            traffic[name] = {"bytes": int(f + w), "source_hash": kernel_source_hash(name)}
        alg = algo.get(name, {}).get("algorithmic_bytes")
        fmt = lambda x: "" if x is None else f"{x / 1e9:.3f}"
        if counted:
            lines.append(f"| {name} | {calls} | {avg_ns / 1e6:.4f} | {pct:.1f} | {fmt(f)} | {fmt(w)} | {fmt(alg)} |")
        else:
            lines.append(f"| {name} | {calls} | {avg_ns / 1e6:.4f} | {pct:.1f} |")
    if sq:
        lines += ["", "SQ counters (per dispatch, median):", "", "| kernel | counter | value |", "|---|---|---|"]
        for name in HOT:
            for c, v in sorted(sq.get(name, {}).items()):
                lines.append(f"| {name} | {c} | {statistics.median(v):.0f} |")
        derived = []
        for name in HOT:
            c = sq.get(name, {})
            if name in ks and "SQ_BUSY_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                dur = ks[name][1] / 1e9
                clk = statistics.median(c["SQ_BUSY_CYCLES"]) / N_SE / dur
                busy = statistics.median(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / (N_SIMD * clk * dur)
                derived.append(f"| {name} | {clk / 1e9:.2f} | {busy:.3f} |")
        if derived:
            lines += ["", f"Derived: shader clock = SQ_BUSY_CYCLES / {N_SE} shader engines / average duration; "
                          f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (matrix-core cycles summed over SIMDs) / "
                          f"({N_SIMD} SIMDs x clock x duration).", "",
                      "| kernel | clock GHz | MFMA busy |", "|---|---|---|", *derived]
    if bench and bench.get("roofline"):
        lines += ["", f"bench.py line of the same workload: {bench['ms_per_step']} ms/hop, {bench['value']} tokens/s; "
                      f"dominant kernel {bench['roofline']['kernel']}: {bench['roofline']['achieved']} "
                      f"{bench['roofline']['unit']} of {bench['roofline']['peak']} "
                      f"({bench['roofline']['bound']} bound, frac {bench['roofline']['frac']})."]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    open(a.out, "w").write("\n".join(lines) + "\n")
    if a.traffic and counted:
        if a.merge and os.path.exists(a.traffic):
            old = json.load(open(a.traffic)).get("kernels", {})
            traffic = {**{k: v for k, v in old.items() if isinstance(v, dict)}, **traffic}
        json.dump({"calibration": {"fetch": cal_f, "write": cal_w}, "kernels": traffic}, open(a.traffic, "w"),
                  indent=1)
        open(a.traffic, "a").write("\n")


if __name__ == "__main__":
    main()
