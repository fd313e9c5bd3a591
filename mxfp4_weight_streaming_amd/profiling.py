"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m mxfp4_weight_streaming_amd.profiling stats  <kernel_stats.csv> <out.txt> "<command>" [note ...]
    python -m mxfp4_weight_streaming_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <copy_mib> <out.txt> "<fetch command>" "<write command>" \
        ["label|kernel prefix|dispatches|algorithmic bytes" ...]

`stats` keeps the per-kernel rows of a `--kernel-trace --stats` run.
`reqsize` sums the L2 read requests by size (32/64/128 bytes) per dispatch.
`mfma` summarises the matrix-core counters of the chunk kernels.
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


def _code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed:
    what the compiler sees, so that a comment edit keeps a kernel's counters
    valid while any change to its code invalidates them.  (The kernel sources
    hold no string or character literals containing comment markers.)"""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def _sources_hash(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def kernel_source_hash() -> str:
    return _sources_hash(KERNEL_SOURCES)


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
    """Counter values per kernel name, in dispatch order."""
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"]))
    out = {}
    for r in rows:
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, out_path: str, fetch_cmd: str, write_cmd: str,
            groups=(), kernel_prefix: str = "void moe::gate_up_kernel<2560, 768, 1>") -> None:
    """groups: (label, kernel prefix, dispatches, algorithmic fetch bytes) in
    dispatch order per kernel: a kernel's dispatches are cut into consecutive
    groups of that many (one group per workload of the run)."""
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
    if groups:
        lines += ["", "per workload (consecutive dispatches of one kernel; algorithmic = the weight bytes the "
                  "dispatch must read, n_act experts x per-expert bytes, plus its small inputs):",
                  f"{'workload':10s} {'kernel':44s} {'n':>5s} {'fetch_MB':>9s} {'algorithmic_MB':>14s} "
                  f"{'fetch/alg':>9s} {'write_MB':>9s}"]
        at = {}
        for label, prefix, n, alg in groups:
            name = next(k for k in fetch if k.startswith(prefix))
            i = at.get(name, 0)
            fv, wv = fetch[name][i:i + n], write.get(name, [0.0] * (i + n))[i:i + n]
            at[name] = i + n
            fb = statistics.mean(fv) * 1024 * f_scale
            wb = statistics.mean(wv) * 1024 * w_scale
            lines.append(f"{label:10s} {_short(name)[:44]:44s} {len(fv):5d} {fb / 1e6:9.3f} {alg / 1e6:14.3f} "
                         f"{fb / alg:9.3f} {wb / 1e6:9.3f}")
    lines.append("")
    lines.append(f"kernel_source_sha256: {kernel_source_hash()}")
    if target is not None:
        lines.append(f"gate_up_fetch_bytes_per_launch: {target[0]:.0f}")
        lines.append(f"gate_up_write_bytes_per_launch: {target[1]:.0f}")
        lines.append(f"traffic_bytes_per_launch: {target[0] + target[1]:.0f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def _per_kernel_counters(csv_path: str):
    """{kernel: {counter: [values in dispatch order]}}."""
    out = {}
    for r in sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"])):
        out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def reqsize(sizes_csv: str, bubble_csv: str, copy_mib: int, out_path: str, sizes_cmd: str, bubble_cmd: str) -> None:
    """Read bytes per dispatch from the L2's read-request counters by size
    (TCC_EA0_RDREQ_32B/_64B/_128B), next to TCC_BUBBLE, which FETCH_SIZE's
    expression takes as the count of 128-byte requests."""
    sz, bub = _per_kernel_counters(sizes_csv), _per_kernel_counters(bubble_csv)
    lines = ["# L2 read requests by size (rocprofv3 --pmc), per dispatch",
             f"sizes command: {sizes_cmd}", f"bubble command: {bubble_cmd}",
             "FETCH_SIZE = (TCC_BUBBLE*128 + (TCC_EA0_RDREQ - TCC_BUBBLE - TCC_EA0_RDREQ_32B)*64 "
             "+ TCC_EA0_RDREQ_32B*32) / 1024 KiB (rocprofv3 --list-avail on this box)",
             "bytes = 32 * RDREQ_32B + 64 * RDREQ_64B + 128 * RDREQ_128B", ""]
    cp = next(k for k in sz if "copyBuffer" in k)
    i = max(range(len(sz[cp]["TCC_EA0_RDREQ_sum"])), key=lambda j: sz[cp]["TCC_EA0_RDREQ_sum"][j])
    c = {n: v[i] for n, v in sz[cp].items()}
    b = {n: v[i] for n, v in bub.get(cp, {}).items()}
    cb = 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]
    lines.append(f"reference copy of {copy_mib} MiB (its largest dispatch): RDREQ {c['TCC_EA0_RDREQ_sum']:.0f}, "
                 f"32B {c['TCC_EA0_RDREQ_32B_sum']:.0f}, 64B {c['TCC_EA0_RDREQ_64B_sum']:.0f}, "
                 f"128B {c['TCC_EA0_RDREQ_128B_sum']:.0f}, BUBBLE {b.get('TCC_BUBBLE_sum', float('nan')):.0f}; "
                 f"bytes by size {cb:.0f} = {cb / (copy_mib << 20):.5f} x the copy")
    lines += ["", f"{'kernel':60s} {'n':>5s} {'RDREQ':>9s} {'32B':>7s} {'64B':>7s} {'128B':>9s} {'BUBBLE':>7s} "
              f"{'read_MB':>9s}"]
    for k in sorted(sz):
        if "moe::" not in k:
            continue
        m = {n: statistics.mean(v) for n, v in sz[k].items()}
        bb = statistics.mean(bub.get(k, {}).get("TCC_BUBBLE_sum", [float("nan")]))
        rb = 32 * m["TCC_EA0_RDREQ_32B_sum"] + 64 * m["TCC_EA0_RDREQ_64B_sum"] + 128 * m["TCC_EA0_RDREQ_128B_sum"]
        lines.append(f"{_short(k):60s} {len(sz[k]['TCC_EA0_RDREQ_sum']):5d} {m['TCC_EA0_RDREQ_sum']:9.0f} "
                     f"{m['TCC_EA0_RDREQ_32B_sum']:7.0f} {m['TCC_EA0_RDREQ_64B_sum']:7.0f} "
                     f"{m['TCC_EA0_RDREQ_128B_sum']:9.0f} {bb:7.0f} {rb / 1e6:9.3f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


# the chunk path's matrix-core kernels, for the MFMA counter summary
CHUNK_SOURCES = ["mxfp4_weight_streaming_amd/csrc/chunk_kernels.hpp",
                 "mxfp4_weight_streaming_amd/csrc/moe_chunk.hip",
                 "mxfp4_weight_streaming_amd/csrc/moe_types.hpp",
                 "mxfp4_weight_streaming_amd/csrc/device_common.hpp"]


def chunk_source_hash() -> str:
    return _sources_hash(CHUNK_SOURCES)


def mfma(counters_csv: str, out_path: str, command: str, xcds: int, simds: int, alg_flops) -> None:
    """Matrix-core counters per dispatch of the chunk kernels: instructions
    and operations (MOPS x 512) by type, busy cycles of the matrix cores
    (summed over SIMDs), and GRBM_GUI_ACTIVE (summed over the XCDs, so one
    XCD's active cycles are that / xcds).  utilisation = busy / (active per
    XCD x SIMDs).  alg_flops: {kernel prefix: algorithmic flops per dispatch}."""
    d = _per_kernel_counters(counters_csv)
    lines = ["# matrix-core counters of the chunk kernels (rocprofv3 --pmc), means per dispatch",
             f"command: {command}",
             f"utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} XCDs x {simds} SIMDs); "
             "ops = MOPS x 512; cycles per instruction = busy / instructions (per SIMD)", "",
             f"{'kernel':44s} {'n':>4s} {'insts_F8':>10s} {'ops_F8_G':>9s} {'ops_F6F4_G':>10s} {'ops_BF16_G':>10s} "
             f"{'alg_G':>7s} {'ops/alg':>7s} {'cyc/inst':>8s} {'util':>7s}"]
    keys = []
    for k in sorted(d):
        c = d[k]
        if "moe::" not in k or statistics.mean(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0])) == 0:
            continue
        m = {n: statistics.mean(v) for n, v in c.items()}
        ins = m.get("SQ_INSTS_VALU_MFMA_F8", 0.0) + m.get("SQ_INSTS_VALU_MFMA_F6F4", 0.0)
        o8 = m.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512
        o4 = m.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) * 512
        ob = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        alg = next((v for p, v in alg_flops.items() if k.startswith(p)), float("nan"))
        util = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / xcds * simds)
        cpi = m["SQ_VALU_MFMA_BUSY_CYCLES"] / ins if ins else float("nan")
        lines.append(f"{_short(k)[:44]:44s} {len(c['GRBM_GUI_ACTIVE']):4d} {ins:10.0f} {o8 / 1e9:9.3f} "
                     f"{o4 / 1e9:10.3f} {ob / 1e9:10.3f} {alg / 1e9:7.3f} {(o8 + o4 + ob) / alg:7.3f} {cpi:8.1f} "
                     f"{util:7.4f}")
        keys.append((_short(k), util, (o8 + o4 + ob) / alg))
    lines.append("")
    lines.append(f"chunk_source_sha256: {chunk_source_hash()}")
    for name, util, ratio in keys:
        tag = "gate_up" if "gate_up" in name else ("down" if "down" in name else "router")
        lines.append(f"{tag}_mfma_busy_util: {util:.4f}")
        lines.append(f"{tag}_executed_over_algorithmic_ops: {ratio:.4f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def phases(trace_csv: str, out_path: str, kernel_prefix: str, sizes, names) -> None:
    """Appends to out_path the mean and median duration of one kernel's
    dispatches in each phase of the bench run, in dispatch order (phase i
    holds the next sizes[i] dispatches).

    Two durations per dispatch: the trace's own (end - start), and the
    exclusive one, end - max(start, end of every earlier dispatch).  When
    dispatches are queued back to back (graph replay, plain launches), a
    dispatch's start stamp can precede the end of the one before it, which
    the kernel still has to wait for; the exclusive duration leaves that wait
    out.  `overlapped` counts the dispatches whose start stamp came first."""
    every = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    raw, excl, early = [], [], []
    last_end = 0
    for r in every:
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if _short(r["Kernel_Name"]).startswith(_short(kernel_prefix)):   # with or without "void "
            raw.append((e - s) / 1e3)
            excl.append((e - max(s, last_end)) / 1e3)
            early.append(s < last_end)
        last_end = max(last_end, e)
    lines = ["", f"per-phase durations of {_short(kernel_prefix)} (us), in dispatch order "
                 "(trace: end - start; exclusive: end - max(start, previous dispatch's end)):"]
    at = 0
    for n, name in zip(sizes, names):
        seg, sx, se = raw[at:at + n], excl[at:at + n], early[at:at + n]
        at += n
        if seg:
            lines.append(f"  {name:32s} n={len(seg):5d} trace mean={statistics.mean(seg):8.3f} "
                         f"median={statistics.median(seg):8.3f}  exclusive mean={statistics.mean(sx):8.3f} "
                         f"median={statistics.median(sx):8.3f}  overlapped={sum(se):5d}")
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
              f"{'router':>7s} {'gate_up':>8s} {'down':>7s}",
              "(tokens 4x32 / 4x20: the 4-token verify routers with 32 / 20 distinct experts)"]
    chunks = []
    for _, path in runs:
        d = json.loads(open(path).read().strip().splitlines()[-1])
        E = d["config"]["experts"]
        for M, r in sorted(d["by_tokens"].items(), key=lambda kv: (int(kv[0].split("x")[0]), kv[0])):
            k = r["kernel_us"]
            lines.append(f"{E:7d} {M:>6s} {r['distinct_experts']:8.2f} {r['us_per_layer']:9.2f} {r['gbs']:7.0f} "
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
        # traffic FETCH WRITE COPY_MIB OUT FETCH_CMD WRITE_CMD [label|kernel prefix|dispatches|algorithmic bytes ...]
        grp = [g.split("|") for g in sys.argv[8:]]
        traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7],
                [(a, b, int(c), float(d)) for a, b, c, d in grp])
    elif sys.argv[1] == "reqsize":
        # reqsize SIZES_CSV BUBBLE_CSV COPY_MIB OUT SIZES_CMD BUBBLE_CMD
        reqsize(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7])
    elif sys.argv[1] == "mfma":
        # mfma CSV OUT CMD XCDS SIMDS "kernel prefix|algorithmic flops" ...
        grp = [g.split("|") for g in sys.argv[7:]]
        mfma(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), int(sys.argv[6]), {a: float(b) for a, b in grp})
    else:
        raise SystemExit(__doc__)
