"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m mxfp4_weight_streaming_amd.profiling stats  <kernel_stats.csv> <out.txt> "<command>" [note ...]
    python -m mxfp4_weight_streaming_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <copy_mib> <out.txt> "<fetch command>" "<write command>"

`stats` keeps the per-kernel rows of a `--kernel-trace --stats` run.
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a command
that first copies <copy_mib> MiB device-to-device (bench.py --copy-mb) and
scales each counter so that the copy reads and writes exactly its size; it
reports HBM bytes per dispatch of the gate/up kernel, tagged with the hash of
the kernel source it was measured on.
"""
from __future__ import annotations

import csv
import json
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the gate/up kernel's code and its launch geometry
KERNEL_SOURCES = ["mxfp4_weight_streaming_amd/csrc/gemv_kernels.hpp",
                  "mxfp4_weight_streaming_amd/csrc/moe_kernels.hip",
                  "mxfp4_weight_streaming_amd/csrc/moe_types.hpp",
                  "mxfp4_weight_streaming_amd/csrc/device_common.hpp",
                  "mxfp4_weight_streaming_amd/csrc/topk_wave.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0][:80]


def stats(csv_path: str, out_path: str, command: str, notes=()) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"command: {command}"] + [f"note: {n}" for n in notes] + ["",
             f"{'kernel':80s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        name = _short(r.get("Name") or r.get("KERNEL_NAME") or "")
        calls = int(float(r.get("Calls", 0)))
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        lines.append(f"{name:80s} {calls:7d} {avg:9.3f} {mn:9.3f} {mx:9.3f} {pct:6.2f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path: str):
    out = {}
    for r in csv.DictReader(open(csv_path)):
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, out_path: str, fetch_cmd: str, write_cmd: str,
            kernel_prefix: str = "void moe::gate_up_kernel<2560, 768, 1>") -> None:
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy_kib = copy_mib * 1024.0
    # the reference copies are the largest copy dispatches
    f_copy = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    w_copy = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    lines = ["# HBM traffic from rocprofv3 counters (KiB per dispatch), scaled by a plain copy of known size",
             f"fetch command: {fetch_cmd}", f"write command: {write_cmd}",
             f"reference copy: {copy_mib} MiB; FETCH_SIZE read {f_copy:.1f} KiB (scale {f_scale:.4f}); "
             f"WRITE_SIZE read {w_copy:.1f} KiB (scale {w_scale:.4f})", ""]
    lines.append(f"{'kernel':60s} {'n':>6s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'fetch_MB':>9s} {'write_MB':>9s}")
    target = None
    for k in sorted(fetch):
        if "moe::" not in k:
            continue
        fv, wv = fetch[k], write.get(k, [0.0])
        fm, wm = statistics.mean(fv), statistics.mean(wv)
        fb, wb = fm * 1024 * f_scale, wm * 1024 * w_scale
        lines.append(f"{_short(k):60s} {len(fv):6d} {fm:11.1f} {wm:11.1f} {fb / 1e6:9.3f} {wb / 1e6:9.3f}")
        if k.startswith(kernel_prefix):
            target = (fb, wb)
    lines.append("")
    lines.append(f"kernel_source_sha256: {kernel_source_hash()}")
    if target is not None:
        lines.append(f"gate_up_fetch_bytes_per_launch: {target[0]:.0f}")
        lines.append(f"gate_up_write_bytes_per_launch: {target[1]:.0f}")
        lines.append(f"traffic_bytes_per_launch: {target[0] + target[1]:.0f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def phases(trace_csv: str, out_path: str, kernel_prefix: str, sizes, names) -> None:
    """Appends to out_path the mean and median duration of one kernel's
    dispatches in each phase of the bench run, in dispatch order (phase i
    holds the next sizes[i] dispatches)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if r["Kernel_Name"].startswith(kernel_prefix)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    lines = ["", f"per-phase durations of {_short(kernel_prefix)} (us), in dispatch order:"]
    at = 0
    for n, name in zip(sizes, names):
        seg = d[at:at + n]
        at += n
        if seg:
            lines.append(f"  {name:32s} n={len(seg):5d} mean={statistics.mean(seg):8.3f} median={statistics.median(seg):8.3f}")
    open(out_path, "a").write("\n".join(lines) + "\n")


def sweep(out_path: str, runs) -> None:
    """Writes a token-sweep table from bench.py JSON lines: runs is a list of
    (command, json_path) pairs."""
    lines = ["# Decode token sweep (bench.py, one MI355X, cold walk over independent layers, HIP graph replay)"]
    lines += [f"command: {cmd}" for cmd, _ in runs]
    lines += ["table: python3 -m mxfp4_weight_streaming_amd.profiling sweep <this file> <command> <its JSON line> ..."]
    lines += ["timing: HIP events around the graph replays; GB/s = algorithmic bytes (selected experts' MXFP4 codes "
              "+ scales, bf16 router, x, out) / time; kernel columns: start/stop events stamped by each launch", "",
              f"{'experts':>7s} {'tokens':>6s} {'distinct':>8s} {'us/layer':>9s} {'GB/s':>7s} {'%8TB/s':>7s} "
              f"{'router':>7s} {'gate_up':>8s} {'down':>7s}"]
    chunks = []
    for _, path in runs:
        d = json.loads(open(path).read().strip().splitlines()[-1])
        E = d["config"]["experts"]
        for M, r in sorted(d["by_tokens"].items(), key=lambda kv: int(kv[0])):
            k = r["kernel_us"]
            lines.append(f"{E:7d} {int(M):6d} {r['mean_distinct_experts']:8.2f} {r['us_per_layer']:9.2f} {r['gbs']:7.0f} "
                         f"{r['pct_of_hbm_peak']:7.2f} {k['router']:7.2f} {k['gate_up']:8.2f} {k['down']:7.2f}")
        if d.get("chunk"):
            c = d["chunk"]
            chunks.append(f"{c['tokens']}-token chunk, {E} experts: {c['us_per_layer']:.2f} us/layer, {c['gbs']:.1f} GB/s, "
                          f"{c['mean_experts_touched']:.1f} experts touched, kernels (us) {c['kernel_us']}, matrix cores "
                          f"{c['mfma']['tflops_layer']:.1f} TFLOP/s")
    lines += [""] + chunks
    open(out_path, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    elif sys.argv[1] == "phases":
        # phases TRACE OUT KERNEL_PREFIX name=count name=count ...
        pairs = [a.split("=") for a in sys.argv[5:]]
        phases(sys.argv[2], sys.argv[3], sys.argv[4], [int(c) for _, c in pairs], [n for n, _ in pairs])
    elif sys.argv[1] == "sweep":
        # sweep OUT CMD1 JSON1 [CMD2 JSON2 ...]
        rest = sys.argv[3:]
        sweep(sys.argv[2], list(zip(rest[0::2], rest[1::2])))
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7])
    else:
        raise SystemExit(__doc__)
