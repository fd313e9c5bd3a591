#!/usr/bin/env python3
"""Benchmark of the MI355X MoE decode layer (W4A8: MXFP4 experts, FP8 activations).

Workload: the Ling-shaped decode layer (hidden 2560, expert intermediate 768,
256 experts, top-8) streamed cold: 40 independent layers (about 30 GiB of MXFP4
weights, far above the 256 MB Infinity Cache) are walked in turn, every layer
with its own freshly drawn hidden state, so no layer's weights are cache-warm
when it runs.  One step = one layer forward (router, top-K, compaction, FP8
quantisation, gate/up + SiLU + requantisation, down + combine) through the C
ABI.  The walk of 40 layers is captured once per hidden set in a HIP graph and
replayed; plain launches are timed too.

Reported (one JSON line on stdout):
  value        algorithmic HBM GB/s at 1 token (bytes the layer must read or
               write: the 8 selected experts' MXFP4 codes and scales, the bf16
               router, x and out) / wall time
  us_per_layer wall time per layer
  steps        exactly --steps layer forwards are timed (whole-walk graph
               replays, then a graph of the remaining layers); every hidden
               set is also walked once in a timed region of its own
               (per_set_walk_us_per_layer)
  m4           the same at 4 tokens (the speculative-decoding verify window)
               with natural routing; m4_32 and m4_20 with the verify-window
               router construction (32 distinct experts, or 4 shared + 4 own
               per token: 20)
  roofline     the dominant kernel against 8 TB/s: its algorithmic bytes over
               its execution time, from start/stop HIP events its launch
               stamps on the bench stream
  by_tokens    the same per workload
  shared_expert  the walk again with the model's shared expert in every layer
  chunk        the 512-token chunk layer (grouped scaled FP4xFP8 MFMA) and its
               matrix-core rate against the FP4 and FP8 dense peaks
  lm_head      the FP8 LM-head GEMV (vocabulary 157,184) per token count
  cpu_baseline the CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

H, I, E, K = 2560, 768, 256, 8
HBM_PEAK_GBS = 8000.0
W13_BYTES = 2 * I * H // 2 + 2 * I * H // 32          # codes + E8M0 scales of one expert's gate/up
W2_BYTES = H * I // 2 + H * I // 32
EXPERT_BYTES = W13_BYTES + W2_BYTES                     # 3,133,440
ROUTER_BYTES = E * H * 2


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def layer_bytes(n_act: int, M: int) -> int:
    return n_act * EXPERT_BYTES + ROUTER_BYTES + M * H * 2 + M * H * 4


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20000, help="timed layer forwards (exactly this many)")
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--layers", type=int, default=40)
    p.add_argument("--reps", type=int, default=8, help="independent hidden sets (one graph each)")
    p.add_argument("--plain-steps", type=int, default=2000, help="layer forwards timed with plain launches")
    p.add_argument("--cpu-runs", type=int, default=3,
                   help="oracle runs per token count in the CPU baseline, median reported (0: skip)")
    p.add_argument("--no-verify", dest="verify", action="store_false",
                   help="skip the 4-token verify-window router constructions (32 and 20 distinct experts)")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="first run a plain device copy of this many MiB (a known-size reference for HBM counters)")
    p.add_argument("--tokens", type=str, default="1,4",
                   help="token counts to time (the first is the reported value); 4 also times 4x32 and 4x20 "
                        "(the verify-window routers) unless --no-verify; 4x32 or 4x20 alone time just that one")
    p.add_argument("--experts", type=int, default=256, help="routed experts per layer (512 is Ling-3.0-flash's own)")
    p.add_argument("--chunk-tokens", type=int, default=512, help="tokens of the chunk measurement (0: skip)")
    p.add_argument("--chunk-steps", type=int, default=400, help="timed chunk layer forwards")
    p.add_argument("--lm-head-vocab", type=int, default=157184, help="vocabulary of the FP8 LM-head GEMV (0: skip)")
    p.add_argument("--lm-head-steps", type=int, default=400, help="timed LM-head GEMV calls per token count")
    p.add_argument("--shared-steps", type=int, default=4000,
                   help="layer forwards timed again with a shared expert per layer (0: skip)")
    p.add_argument("--one-kernel", action="store_true",
                   help="time the one-kernel M <= 8 layer (layer_kernel) instead of the default three kernels")
    return p.parse_args()


def main() -> int:
    args = parse()
    global E, ROUTER_BYTES
    E = args.experts
    ROUTER_BYTES = E * H * 2
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer is not sharded "
              "across GPUs in this library)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mxfp4_weight_streaming_amd import binding as moe
    from mxfp4_weight_streaming_amd import synth

    torch.cuda.set_device(0)
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"reference copy: {args.copy_mb} MiB x 3")
        del src, dst
    if args.one_kernel:
        moe.moe_set_decode_path(moe.PATH_ONE_KERNEL)
    shp = moe.shape(H, I, E, K)
    L, reps = args.layers, args.reps
    st, path = moe.moe_path_info(shp, 1)
    assert st == 0, path
    log(f"path: {path}")
    log(f"drawing {L} layers of weights on the GPU ({L * (EXPERT_BYTES * E + ROUTER_BYTES) / 2**30:.1f} GiB)")
    stack = synth.device_stack(L, H, I, E, seed=1234)
    shared_layers = synth.device_shared(L, H, I, seed=4321) if args.shared_steps > 0 else None
    stream = torch.cuda.Stream()
    ws = moe.workspace(shp, 8)
    out = torch.empty((8, H), dtype=torch.float32, device="cuda")

    workloads = []
    for tok in args.tokens.split(","):
        if "x" in tok:                      # "4x32": 4 tokens, verify router with 32 distinct experts
            m, d = (int(v) for v in tok.split("x"))
            if m != 4 or d not in (20, 32):
                raise SystemExit(f"--tokens {tok}: the verify construction is 4x32 or 4x20")
            workloads.append((tok, m, d))
            continue
        M = int(tok)
        workloads.append((str(M), M, None))
        if M == 4 and args.verify:
            # the verify window as configured: biased routers giving 32
            # distinct experts, or 4 shared + 4 own per token (20 distinct)
            workloads += [("4x32", 4, 32), ("4x20", 4, 20)]
    results = {}
    for name, M, distinct in workloads:
        results[name] = time_walks(args, moe, synth, stack, shared_layers, shp, stream, ws, out, name, M, distinct)

    lm_head = None
    if args.lm_head_vocab > 0:
        lm_head = lm_head_bench(args, moe, stream)

    chunk = None
    if args.chunk_tokens > 0:
        chunk = chunk_bench(args, moe, synth, stack, shp, stream)

    cpu = None
    if args.cpu_runs > 0:
        cpu = cpu_baseline(args.cpu_runs)

    head = results[workloads[0][0]]

    def summary(r):
        return {"us_per_layer": round(r["us_per_layer"], 3), "gbs": round(r["gbs"], 1),
                "pct_of_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
                "distinct_experts": round(r["mean_distinct_experts"], 2),
                "per_set_walk_us_per_layer": r["per_set"],
                "plain_us_per_layer": round(r["plain_us_per_layer"], 3),
                "kernel_us": {k: round(v, 3) for k, v in r["kernel_us"].items()}}

    traffic = measured_traffic()
    rl = head["roofline"]
    line = {
        "metric": "MoE-layer decode us + weight-stream HBM GB/s (% of peak), M=1 and M=4",
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms"] / head["steps"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 x e4m3 -> f32",
        "data": "synthetic",
        "config": {"workload": f"ling-shaped MoE decode layer, {workloads[0][1]} token(s), cold walk over {L} layers",
                   "hidden": H, "expert_inter": I, "experts": E, "topk": K, "tokens": workloads[0][1], "layers": L,
                   "launch": f"hip graphs of the {L}-layer walk; the timed region is exactly --steps layers"},
        "us_per_layer": round(head["us_per_layer"], 3),
        "pct_of_hbm_peak": round(100 * head["gbs"] / HBM_PEAK_GBS, 2),
        "per_set_walk_us_per_layer": head["per_set"],
        "plain_launch": {"us_per_layer": round(head["plain_us_per_layer"], 3), "gbs": round(head["plain_gbs"], 1)},
        "m4": summary(results["4"]) if "4" in results else None,
        "m4_32": summary(results["4x32"]) if "4x32" in results else None,
        "m4_20": summary(results["4x20"]) if "4x20" in results else None,
        "by_tokens": {n: summary(r) for n, r in results.items()},
        "kernel_us": {k: round(v, 3) for k, v in head["kernel_us"].items()},
        "roofline": {"kernel": rl["kernel"], "bound": "hbm", "achieved": round(rl["gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(rl["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": rl["bytes"], "us_per_launch": round(rl["us"], 3),
                     "timing": rl["timing"],
                     # the headline's own launch mode (graph replay) leaves gate/up the layer's time
                     # less the other two kernels' launch-stamped times: the same within a few %
                     "graph_layer_less_router_and_down_us": (
                         round(head["us_per_layer"] - head["kernel_us"]["router"] - head["kernel_us"]["down"], 3)
                         if "router" in head["kernel_us"] else None)},
        "shared_expert": {"by_tokens": {n: r["shared"] for n, r in results.items() if r.get("shared")}} or None,
        "chunk": chunk,
        "lm_head": lm_head,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def time_walks(args, moe, synth, stack, shared_layers, shp, stream, ws, out, name, M, distinct) -> dict:
    """One decode workload (M tokens; natural routing, or the verify-window
    router construction with `distinct` experts) over the cold walk: a HIP
    graph per hidden set of the whole walk; exactly args.steps layers timed
    (whole walks, then a prefix graph for the rest); every hidden set timed as
    one walk of its own; plain launches; per-kernel launch-stamped events."""
    import numpy as np
    import torch
    L, reps = len(stack), args.reps
    xs = synth.device_hidden(L * reps, M, H, seed=10_000 + M + (0 if distinct is None else 1000 * distinct))
    if distinct is None:
        routers = [[stack[l]["wr"] for l in range(L)] for _ in range(reps)]
    else:
        g = torch.Generator(device="cuda")
        g.manual_seed(20_000 + distinct)
        routers = [[synth.device_verify_router(stack[l]["wr"], xs[r * L + l], distinct, g, K=K) for l in range(L)]
                   for r in range(reps)]
    torch.cuda.synchronize()

    def fwd(r, l, events=None, shared=False):
        Ly, x, wr = stack[l], xs[r * L + l], routers[r][l]
        if shared:
            moe.moe_decode_forward_shared(shp, M, x, wr, Ly["w13"], Ly["s13"], Ly["w2"], Ly["s2"],
                                          shared_layers[l], out, ws)
        elif events is None:
            moe.moe_decode_forward(shp, M, x, wr, Ly["w13"], Ly["s13"], Ly["w2"], Ly["s2"], out, ws)
        else:
            moe.moe_decode_forward_events(shp, M, x, wr, Ly["w13"], Ly["s13"], Ly["w2"], Ly["s2"], out, ws, events)

    # routing pre-pass: distinct experts of every (hidden set, layer)
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, K), dtype=torch.float32, device="cuda")
    n_active = torch.zeros((reps, L), dtype=torch.int32, device="cuda")
    stream.wait_stream(torch.cuda.current_stream())      # inputs were made on the default stream
    with torch.cuda.stream(stream):
        for r in range(reps):
            for l in range(L):
                moe.moe_route(shp, M, xs[r * L + l], routers[r][l], ids, wts, ws,
                              taps={"n_active": n_active[r, l:l + 1]})
    torch.cuda.synchronize()
    n_act = n_active.cpu().numpy().astype(np.int64)
    lo, hi = (K, min(E, M * K)) if distinct is None else (distinct, distinct)
    if n_act.min() < lo or n_act.max() > hi:
        raise RuntimeError(f"{name}: routing pre-pass read back distinct-expert counts outside [{lo}, {hi}]: "
                           f"min {n_act.min()}, max {n_act.max()}")
    lb = [[layer_bytes(int(n_act[r, l]), M) for l in range(L)] for r in range(reps)]

    with torch.cuda.stream(stream):
        for r in range(reps):                               # eager warm-up walk of every set
            for l in range(L):
                fwd(r, l)
        torch.cuda.synchronize()
        graphs = []
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for l in range(L):
                    fwd(r, l)
            graphs.append(g)
        n_full, rest = divmod(args.steps, L)
        prefix = None
        if rest:
            prefix = torch.cuda.CUDAGraph()
            with torch.cuda.graph(prefix, stream=stream):
                for l in range(rest):
                    fwd(n_full % reps, l)
        # untimed warm-up: --warmup layers, as whole walks
        for i in range(max(1, math.ceil(args.warmup / L))):
            graphs[i % reps].replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(n_full):
            graphs[i % reps].replay()
        if prefix is not None:
            prefix.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        steps = n_full * L + rest
        total = sum(sum(lb[i % reps]) for i in range(n_full)) + sum(lb[n_full % reps][:rest])
        # every hidden set walked once, each in a timed region of its own
        per_set = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs[r].replay()
            b.record(stream)
            torch.cuda.synchronize()
            per_set.append(a.elapsed_time(b) * 1e3 / L)
    gbs = total / (ms * 1e-3) / 1e9
    log(f"{name}: graph replay of exactly {steps} layers in {ms:.3f} ms ({ms * 1e3 / steps:.2f} us/layer, "
        f"{gbs:.0f} GB/s); every set walked once: median {np.median(per_set):.2f} us/layer "
        f"(min {min(per_set):.2f}, max {max(per_set):.2f}); mean distinct experts {n_act.mean():.2f}")

    # plain launches (no graph)
    n_plain = max(L, args.plain_steps)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        pbytes = 0
        for i in range(n_plain):
            r, l = (i // L) % reps, i % L
            fwd(r, l)
            pbytes += lb[r][l]
        p1.record(stream)
        torch.cuda.synchronize()
    pms = p0.elapsed_time(p1)

    # per-kernel durations from start/stop HIP events stamped by each kernel's
    # own launch (plain launches on the bench stream; a spin kernel at the
    # head of the stream lets the host queue the whole walk first, so the
    # kernels run back to back as in the timed walk)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)]
    one_kernel = "one-kernel" in moe.moe_path_info(shp, M)[1]
    names = ("layer",) if one_kernel else ("router", "gate_up", "down")
    dur = {k: [] for k in names}
    gu_launch_bytes, layer_launch_bytes = [], []
    with torch.cuda.stream(stream):
        for row in evs:
            for e in row:
                e.record(stream)          # torch creates the HIP event on first record
        for ps in range(max(2, 400 // L)):
            r = ps % reps
            torch.cuda._sleep(50_000_000)
            for l in range(L):
                fwd(r, l, events=evs[l])
            torch.cuda.synchronize()
            for l in range(L):
                for k, kn in enumerate(names):
                    dur[kn].append(evs[l][2 * k].elapsed_time(evs[l][2 * k + 1]))
                gu_launch_bytes.append(int(n_act[r, l]) * W13_BYTES)
                layer_launch_bytes.append(lb[r][l])
    kus = {k: float(np.mean(v)) * 1e3 for k, v in dur.items()}
    gu_bytes = float(np.mean(gu_launch_bytes))
    log(f"{name}: kernel means (us) {kus}")

    shared = None
    if shared_layers is not None and distinct is None:
        # the same walk with the model's shared expert in every layer
        with torch.cuda.stream(stream):
            for r in range(reps):
                for l in range(L):
                    fwd(r, l, shared=True)
            torch.cuda.synchronize()
            gsh = []
            for r in range(reps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for l in range(L):
                        fwd(r, l, shared=True)
                gsh.append(g)
            for i in range(reps):
                gsh[i].replay()
            torch.cuda.synchronize()
            n_sh = max(reps, math.ceil(args.shared_steps / L))
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for i in range(n_sh):
                gsh[i % reps].replay()
            s1.record(stream)
            torch.cuda.synchronize()
        sms = s0.elapsed_time(s1)
        sbytes = sum(sum(lb[i % reps]) + L * EXPERT_BYTES for i in range(n_sh))
        shared = {"us_per_layer": round(sms * 1e3 / (n_sh * L), 3), "gbs": round(sbytes / (sms * 1e-3) / 1e9, 1),
                  "pct_of_hbm_peak": round(100 * sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2), "layers": n_sh * L}
        log(f"{name} with a shared expert: {shared['us_per_layer']:.2f} us/layer, {shared['gbs']:.0f} GB/s")
        del gsh
    del graphs, prefix
    errs = moe.sync_errors(ws)
    if errs:
        raise RuntimeError(f"{name}: the layer kernel's waits ran out (sync error bits {errs:#x}); results invalid")
    return {"us_per_layer": ms * 1e3 / steps, "gbs": gbs, "steps": steps, "ms": ms,
            "per_set": {"median": round(float(np.median(per_set)), 3), "min": round(min(per_set), 3),
                        "max": round(max(per_set), 3), "sets": reps},
            "mean_distinct_experts": float(n_act.mean()),
            "plain_us_per_layer": pms * 1e3 / n_plain, "plain_gbs": pbytes / (pms * 1e-3) / 1e9,
            "kernel_us": kus, "shared": shared,
            "roofline": ({"kernel": f"layer_kernel<H=2560,I=768> ({M} token(s), the whole layer)",
                          "bytes": float(np.mean(layer_launch_bytes)), "us": kus["layer"],
                          "gbs": float(np.mean(layer_launch_bytes)) / (kus["layer"] * 1e-6) / 1e9,
                          "timing": "launch-stamped HIP events, plain launches queued behind a spin kernel"}
                         if one_kernel else
                         {"kernel": f"gate_up_kernel<H=2560,I=768> ({M} token(s))", "bytes": gu_bytes,
                          "us": kus["gate_up"], "gbs": gu_bytes / (kus["gate_up"] * 1e-6) / 1e9,
                          "timing": "launch-stamped HIP events, plain launches queued behind a spin kernel"})}


def lm_head_bench(args, moe, stream) -> dict:
    """The FP8 LM head (vocabulary x 2560, quantised once from bf16): GEMV
    time per call at 1 and 4 tokens, alternating between two quantised copies
    (together above the memory-side cache) so every call streams cold rows."""
    import torch
    V = args.lm_head_vocab
    g = torch.Generator(device="cuda")
    g.manual_seed(777)
    copies = []
    for _ in range(2):
        w = (torch.randn((V, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
        q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
        sc = torch.empty(V, dtype=torch.float32, device="cuda")
        moe.moe_lm_head_quantize(w, q, sc)
        torch.cuda.synchronize()
        del w
        copies.append((q, sc))
    res = {}
    for M in (1, 4):
        x = (torch.randn((M, H), generator=g, device="cuda")).to(torch.bfloat16).view(torch.int16)
        logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
        stream.wait_stream(torch.cuda.current_stream())   # x was made on the default stream
        with torch.cuda.stream(stream):
            for i in range(20):
                q, sc = copies[i % 2]
                moe.moe_lm_head_forward(x, q, sc, logits)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(2):
                    q, sc = copies[i]
                    moe.moe_lm_head_forward(x, q, sc, logits)
            graph.replay()
            torch.cuda.synchronize()
            n = max(1, args.lm_head_steps // 2)
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(n):
                graph.replay()
            t1.record(stream)
            torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / (2 * n)
        nbytes = V * H + V * 4 + M * H * 2 + M * V * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        res[str(M)] = {"us_per_call": round(us, 2), "gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        log(f"lm head V={V} M={M}: {us:.1f} us per call, {gbs:.0f} GB/s")
    bf16_bytes = V * H * 2
    return {"vocab": V, "hidden": H, "by_tokens": res,
            "weight_bytes_fp8": V * H, "weight_bytes_bf16": bf16_bytes,
            "workload": "FP8 LM-head GEMV (per-row fp32 scales, bf16 activations), two quantised copies alternated"}


FP4_PEAK_TFLOPS = 10100.0     # dense FP4 matrix peak of the chip
FP8_PEAK_TFLOPS = 5000.0      # dense FP8 matrix peak (the mixed FP8 x FP4 form is not faster than this)


def chunk_bench(args, moe, synth, stack, shp, stream) -> dict:
    """A chunk of M tokens per layer (Zipf-skewed routing) through the chunk
    path, over the same cold 40-layer walk."""
    import numpy as np
    import torch
    M, L = args.chunk_tokens, len(stack)
    # per-layer routers with a popularity bias channel: token channel 0 is 1.0
    # and expert e's channel-0 weight is tau * (-1.1 * ln rank_e)
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    routers, xs = [], []
    for l in range(L):
        wr = stack[l]["wr"].view(torch.bfloat16).float()
        ranks = torch.randperm(E, generator=g, device="cuda").float() + 1.0
        wr[:, 0] = 0.5 * (-1.1 * torch.log(ranks))
        routers.append(wr.to(torch.bfloat16).view(torch.uint16).contiguous())
        x = torch.randn((M, H), generator=g, device="cuda")
        x[:, 0] = 1.0
        xs.append(x.to(torch.bfloat16).view(torch.uint16).contiguous())
    ws = moe.workspace(shp, M)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((M, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, K), dtype=torch.float32, device="cuda")
    n_active = torch.zeros(L, dtype=torch.int32, device="cuda")
    stream.wait_stream(torch.cuda.current_stream())       # inputs were made on the default stream
    with torch.cuda.stream(stream):
        for l in range(L):
            moe.moe_route(shp, M, xs[l], routers[l], ids, wts, ws, taps={"n_active": n_active[l:l + 1]})
    torch.cuda.synchronize()
    n_act = n_active.cpu().numpy().astype(np.int64)
    if n_act.min() < K or n_act.max() > E:
        raise RuntimeError(f"chunk routing pre-pass read back distinct-expert counts outside [{K}, {E}]")
    layer_b = [int(n) * EXPERT_BYTES + ROUTER_BYTES + M * H * 2 + M * H * 4 for n in n_act]
    P = M * K
    flops_gu = 2.0 * P * (2 * I) * H
    flops_down = 2.0 * P * H * I

    def fwd(l, events=None):
        Ly = stack[l]
        if events is None:
            moe.moe_decode_forward(shp, M, xs[l], routers[l], Ly["w13"], Ly["s13"], Ly["w2"], Ly["s2"], out, ws)
        else:
            moe.moe_decode_forward_events(shp, M, xs[l], routers[l], Ly["w13"], Ly["s13"], Ly["w2"], Ly["s2"],
                                          out, ws, events)

    with torch.cuda.stream(stream):
        for l in range(L):
            fwd(l)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for l in range(L):
                fwd(l)
        graph.replay()
        torch.cuda.synchronize()
        n_rep = max(1, math.ceil(args.chunk_steps / L))
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(n_rep):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    us_layer = ms * 1e3 / (n_rep * L)
    gbs = n_rep * sum(layer_b) / (ms * 1e-3) / 1e9
    # per-kernel execution times from launch-stamped events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)]
    dur = {"router": [], "gate_up": [], "down": []}
    with torch.cuda.stream(stream):
        for row in evs:
            for e in row:
                e.record(stream)
        torch.cuda._sleep(50_000_000)
        for l in range(L):
            fwd(l, events=evs[l])
        torch.cuda.synchronize()
    for l in range(L):
        for k, name in enumerate(("router", "gate_up", "down")):
            dur[name].append(evs[l][2 * k].elapsed_time(evs[l][2 * k + 1]))
    kus = {k: float(np.mean(v)) * 1e3 for k, v in dur.items()}
    gu_bytes = float(np.mean(n_act)) * W13_BYTES
    dn_bytes = float(np.mean(n_act)) * W2_BYTES
    mfma_layer = (flops_gu + flops_down) / (us_layer * 1e-6) / 1e12
    log(f"chunk M={M}: {us_layer:.1f} us/layer, {gbs:.0f} GB/s, experts touched {n_act.mean():.1f}, "
        f"kernels (us) {kus}, matrix-core {mfma_layer:.1f} TFLOP/s over the layer")
    return {"tokens": M, "us_per_layer": round(us_layer, 2), "gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "mean_experts_touched": round(float(n_act.mean()), 1),
            "kernel_us": {k: round(v, 2) for k, v in kus.items()},
            "gate_up_gbs": round(gu_bytes / (kus["gate_up"] * 1e-6) / 1e9, 1),
            "down_gbs": round(dn_bytes / (kus["down"] * 1e-6) / 1e9, 1),
            "mfma": {"flops_per_layer": flops_gu + flops_down,
                     "tflops_layer": round(mfma_layer, 1),
                     "tflops_gate_up_kernel": round(flops_gu / (kus["gate_up"] * 1e-6) / 1e12, 1),
                     "tflops_down_kernel": round(flops_down / (kus["down"] * 1e-6) / 1e12, 1),
                     "util_vs_fp4_peak": round(mfma_layer / FP4_PEAK_TFLOPS, 4),
                     "util_vs_fp8_peak": round(mfma_layer / FP8_PEAK_TFLOPS, 4)},
            "mfma_counters": measured_chunk_mfma(),
            "workload": f"{M}-token chunk per layer, Zipf-1.1 routing through a bias channel, cold 40-layer walk, "
                        "hip graph"}


# HBM traffic of the gate/up kernel comes from hardware counters taken with
# rocprofv3 (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size)
# and is only reported while the kernel source is the one it was taken on.
TRAFFIC_FILE = "profiles/gate_up_hbm_traffic.txt"


def kernel_source_hash() -> str:
    from mxfp4_weight_streaming_amd.profiling import kernel_source_hash as h
    return h()


def measured_traffic():
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Matrix-core counters of the chunk kernels (rocprofv3 --pmc), reported only
# while the chunk kernels' sources are the ones they were taken on.
CHUNK_MFMA_FILE = "profiles/chunk_mfma_counters_ling_zipf512.txt"


def measured_chunk_mfma():
    from mxfp4_weight_streaming_amd.profiling import chunk_source_hash
    path = os.path.join(ROOT, CHUNK_MFMA_FILE)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "command")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("chunk_source_sha256") != chunk_source_hash():
        return None
    try:
        return {"gate_up_busy_util": float(fields["gate_up_mfma_busy_util"]),
                "down_busy_util": float(fields["down_mfma_busy_util"]),
                "executed_over_algorithmic_ops": float(fields["gate_up_executed_over_algorithmic_ops"]),
                "basis": "SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' active cycles; the FP8 x FP4 scaled MFMA issues "
                         "at 32 cycles per 16x16x128 (the dense FP8 rate), and the 16-row tiles are padded"}
    except (KeyError, ValueError):
        return None


def cpu_baseline(runs: int) -> dict:
    """The oracle on the bench's own workload: one Ling-shaped layer at 1 token
    (natural routing) and at 4 tokens (the verify construction with 32 distinct
    experts), each timed `runs` times inside the oracle library around the
    layer call only, with the process pinned to one host core; the median is
    reported.  The oracle is single-threaded."""
    import platform

    import numpy as np

    import oracle
    from mxfp4_weight_streaming_amd import synth
    log("cpu baseline: drawing the oracle's inputs")
    w = synth.expert_weights(77, H, I, E)
    x1 = synth.decode_tokens(500, w, 1, K).x
    v4 = synth.verify_router(501, w, 32, M=4, K=K)
    oracle.lib()
    model = platform.processor() or "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        s1 = oracle.time_layer(x1, w.wr, w.w13, w.s13, w.w2, w.s2, K, runs=runs)
        s4 = oracle.time_layer(v4.x, v4.wts.wr, w.w13, w.s13, w.w2, w.s2, K, runs=runs)
    finally:
        os.sched_setaffinity(0, allowed)
    m1, m4 = float(np.median(s1)), float(np.median(s4))
    log(f"cpu baseline: 1 token {m1:.3f} s, 4 tokens {m4:.3f} s per layer on core {core} ({model})")
    b1, b4 = layer_bytes(K, 1), layer_bytes(32, 4)
    return {"value": round(b1 / m1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one Ling-shaped layer (H=2560, I=768, E=256, K=8) at 1 token: median of {runs} runs "
                      f"{m1 * 1e3:.0f} ms ({[round(v * 1e3) for v in s1]} ms); at 4 tokens with 32 distinct "
                      f"experts: {m4 * 1e3:.0f} ms ({b4 / m4 / 1e9:.4f} GB/s); timed inside the oracle library "
                      f"(CLOCK_MONOTONIC around the layer call), process pinned to core {core}",
            "us_per_layer": {"1": round(m1 * 1e6, 1), "4x32": round(m4 * 1e6, 1)},
            "host": {"cpu_model": model, "nproc": os.cpu_count(), "cores_allowed": len(allowed),
                     "pinned_core": core}}


if __name__ == "__main__":
    sys.exit(main())
