"""Turn rocprofv3 CSV output into the short text summaries kept with the sources.

    python3 -m dropless_grouped_gemm_amd.profsum kernels  DIR --command CMD [--bench LOG] --out F
    python3 -m dropless_grouped_gemm_amd.profsum traffic  FETCH_DIR WRITE_DIR --kernel K
            --label L --workload W --command CMD --out F

`kernels` reads DIR/run_kernel_stats.csv (and run_kernel_trace.csv for medians) of a
`rocprofv3 --kernel-trace --stats` run; with --bench, the JSON line the benchmark
printed under the profiler is appended, so its event-timed stage durations sit next
to the trace's.

`traffic` reads the run_counter_collection.csv of two `rocprofv3 --pmc` runs, one
with FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch).  Each counter is scaled
by the ratio of known to counted bytes of a plain elementwise kernel that reads and
writes 1 GiB (torch.neg over 2^28 fp32 values, launched by the benchmark's
--copy-probe), giving HBM bytes per launch of kernel K.  The summary ends with a
JSON block that the benchmark reads; it carries the SHA-256 of the grouped-GEMM
sources so that a figure taken before the kernels changed is not reported.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
from collections import defaultdict

PROBE_KERNEL = "neg_kernel"
PROBE_BYTES = 1 << 30           # read, and written, by the probe kernel
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# every source the grouped-GEMM kernels are built from
GEMM_SOURCE = [os.path.join("dropless_grouped_gemm_amd", "csrc", f)
               for f in ("moe_gemm.hip", "moe_gemm_wide.hip", "moe_gemm_common.h")]


def source_digest(rel_paths) -> str:
    """SHA-256 over the concatenated bytes of one source file or a list of them."""
    if isinstance(rel_paths, str):
        rel_paths = [rel_paths]
    h = hashlib.sha256()
    for rel in rel_paths:
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return ""
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without its parameter list (templates kept)."""
    name = name.replace("(anonymous namespace)", "{anon}")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    name = name[5:] if name.startswith("void ") else name
    return name if len(name) <= 96 else name[:93] + "..."


def kernels_summary(d: str, command: str, bench_log: str | None) -> str:
    stats = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    med = {}
    trace = os.path.join(d, "run_kernel_trace.csv")
    if os.path.exists(trace):
        per = defaultdict(list)
        for r in csv.DictReader(open(trace)):
            per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        med = {k: statistics.median(v) for k, v in per.items()}
    lines = ["| kernel | calls | avg us | median us | min us | max us | share % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in stats:
        n = r["Name"]
        lines.append(f"| `{short_name(n)}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{med.get(n, float('nan')):.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    out = ["Command (from the repository root):", "",
           "```", command, "```", ""] + lines
    if bench_log and os.path.exists(bench_log):
        js = [l for l in open(bench_log).read().splitlines() if l.startswith("{")]
        if js:
            b = json.loads(js[-1])
            out += ["", "Event-timed stage averages printed by the benchmark in the same run (us):",
                    "", "```", json.dumps(b.get("stages_us")), "```",
                    f"roofline: {json.dumps(b.get('roofline'))}"]
            for name, w in (b.get("workloads") or {}).items():
                out += [f"{name}: stages (us) {json.dumps(w.get('stages_us'))}"]
            bw = b.get("backward")
            if bw:
                out += ["", "Backward stages in the same run (us), and each backward GEMM launch's "
                        "TFLOP/s:", "", "```", json.dumps(bw.get("stages_us")),
                        json.dumps({k: round(v["tflops"], 1) for k, v in bw.get("gemm", {}).items()}),
                        "```"]
    return "\n".join(out) + "\n"


def _per_kernel(csv_path: str, counter: str):
    vals = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _pick(vals, needle):
    hits = [k for k in vals if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel '{needle}': {len(hits)} matches in the counter file")
    v = vals[hits[0]]
    return hits[0], sum(v) / len(v), len(v)


def traffic_summary(fetch_dir, write_dir, kernel, label, workload, command, algo_bytes=None,
                    source=None):
    source = source or GEMM_SOURCE
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _per_kernel(os.path.join(d, "run_counter_collection.csv"), counter)
        # the probe is the largest elementwise negation (a workload's input generator may
        # negate small tensors of its own)
        probe_kib = max(max(v) for k, v in vals.items() if PROBE_KERNEL in k)
        name, kib, n = _pick(vals, kernel)
        factor = PROBE_BYTES / (probe_kib * 1024.0)
        res[counter] = dict(kib=kib, dispatches=n, probe_kib=probe_kib, factor=factor,
                            bytes=kib * 1024.0 * factor, name=name)
    total = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    out = ["Command (from the repository root):", "",
           "```", command, "```", "",
           f"Kernel `{short_name(res['FETCH_SIZE']['name'])}` ({label}), workload {workload}.", "",
           "| counter | KiB / dispatch | dispatches | probe KiB | scale | bytes / launch |",
           "|---|---:|---:|---:|---:|---:|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        out.append(f"| {c} | {r['kib']:.0f} | {r['dispatches']} | {r['probe_kib']:.0f} | "
                   f"{r['factor']:.3f} | {r['bytes']:.4e} |")
    out += ["", f"Probe: torch.neg over 2^28 fp32 values, {PROBE_BYTES} bytes read and "
                f"{PROBE_BYTES} bytes written; scale = known bytes / counted bytes.",
            f"HBM traffic per launch: {total:.4e} bytes"]
    if algo_bytes:
        out.append(f"Algorithmic bytes per launch: {algo_bytes:.4e} (traffic / algorithmic = "
                   f"{total / algo_bytes:.2f})")
    blob = {"kernel": label, "config": workload, "source": source,
            "source_sha256": source_digest(source), "bytes_per_launch": total,
            "fetch_bytes": res["FETCH_SIZE"]["bytes"], "write_bytes": res["WRITE_SIZE"]["bytes"]}
    out += ["", "```json", json.dumps(blob), "```"]
    return "\n".join(out) + "\n"


def read_traffic(path: str, kernel: str, workload: str):
    """bytes_per_launch from a traffic summary, or None when it is missing, covers
    another kernel or workload, or was taken from a different kernel source."""
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    if "```json" not in text:
        return None
    blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if blob.get("kernel") != kernel or blob.get("config") != workload:
        return None
    if blob.get("source_sha256") != source_digest(blob.get("source", GEMM_SOURCE)):
        return None
    return blob.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--command", required=True)
    k.add_argument("--bench", default=None)
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True, help="substring of the kernel name")
    t.add_argument("--label", required=True, help="stage name the benchmark uses")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--algo-bytes", type=float, default=None)
    t.add_argument("--source", action="append", default=None,
                   help="source file (from the repository root) the kernel is built from, "
                        "repeatable; default: the grouped-GEMM sources")
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "kernels":
        text = kernels_summary(a.dir, a.command, a.bench)
    else:
        text = traffic_summary(a.fetch_dir, a.write_dir, a.kernel, a.label, a.workload, a.command,
                               a.algo_bytes, a.source)
    with open(a.out, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
