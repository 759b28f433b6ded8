#!/usr/bin/env python3
"""Throughput of the deflated-ASP NVFP4 W4A4 linear on one MI355X.

Default workload: the 600-layer two-expert set (30 blocks x 10 linears per
expert; video d 3072 / ffn 14336 at M = 4096 tokens, rank 0; action d 1024 /
ffn 4096 at M = 256 tokens, rank 32).  One step = one denoising step: the
whole per-call path (activation prep, then the 4-bit GEMM with its
low-rank/bias epilogue) for all 600 linears as one stream, every weight and
input resident in HBM (each layer its own, about 24 GB in all, so every read
comes from HBM).  W eager warm-up steps, then exactly K steps captured in one
HIP graph and replayed once between synchronize() and HIP events on the
launch stream.  The same K steps then run once more, eagerly, with HIP
events around every launch of the dominant kernel (the video expert's 4-bit
GEMM): its per-launch durations in the step's own sequence give the roofline
figure.

--workload 0..3 times one of the smaller workloads instead (layers that read
one input run as one group; steps rotate through replicas of every buffer,
>= 1 GiB, so reads come from HBM rather than the 256 MB Infinity Cache; each
kernel is then also timed alone for its roofline figure).  --eigen, --svdq
and --search time the adjacent parts.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "deflated-ASP NVFP4 linear effective TFLOP/s + % of roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA
RIDGE = F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
CSRC = os.path.join(ROOT, "wam_asp_w4a4_amd", "csrc")
# the sources each kernel is built from: a traffic figure measured with
# hardware counters stays valid only while these files are unchanged
KERNEL_SOURCES = {
    "k_prep_u": ["asp_prep.hip", "asp_device.h", "nvfp4_codec.h", "asp_internal.h"],
    "k_prep_q": ["asp_prep.hip", "asp_device.h", "nvfp4_codec.h", "asp_internal.h"],
    "k_gemm": ["asp_gemm.hip", "asp_device.h", "nvfp4_codec.h", "asp_internal.h"],
    "k_eig_gv": ["asp_eig.hip", "asp_device.h", "nvfp4_codec.h", "asp_internal.h"],
    "k_svdq_gemm": ["asp_svdq.hip", "asp_device.h", "nvfp4_codec.h", "asp_internal.h"],
}
WORKLOAD_SLUGS = {0: "single_M64_K512_N512", 1: "action_attn_M256_K1024_N1024",
                  2: "action_ffn_M256", 3: "video_attn_M4096_K3072_N3072"}
COPY_CALIBRATION_BYTES = 256 << 20
F64_PEAK_TFLOPS = 78.6      # MI355X dense fp64 MFMA
I8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA
# the basis solve: the action expert's widest layer input (ffn.2, K = 4096),
# rank 32 with a block of 64, 8 products with the metric
EIG_K, EIG_P, EIG_R, EIG_ITERS = 4096, 64, 32, 8
EIG_SLUG = "metric_K4096_p64"


def layer_flops(M, N, K, r):
    """Algorithmic FLOPs of one layer call: 2MNK + 2MKr (u) + 2MKr (deflation) + 2MNr (low rank)."""
    return 2 * M * N * K + 4 * M * K * r + 2 * M * N * r


def layer_bytes(M, N, K, r, xb, yb):
    """Minimum HBM bytes of one layer call: x, y, codes, scales, W~V, V, s, b (no FP4 activation)."""
    return M * K * xb + M * N * yb + N * K // 2 + N * K // 16 + 2 * N * r + 4 * K * r + 4 * K + 4 * N


def prep_u_bytes(M, K, r, xb):
    """Algorithmic bytes of the u stage: x and diag(1/s) H V (three bf16 terms) in, u out."""
    return M * K * xb + 6 * K * r + 4 * M * r


def prep_q_bytes(M, K, r, xb):
    """Algorithmic bytes of the quantise stage: x, 1/(s sqrt 128) (float64), V (three bf16
    terms) and u in; codes, scales and u out."""
    return M * K * xb + 8 * K + 6 * K * r + 4 * M * r + M * K // 2 + M * K // 16 + 4 * M * r


def gemm_bytes(M, N, K, r, yb):
    """Algorithmic bytes of one GEMM launch: both operands' codes and scales, u, W~V, bias, y."""
    return (M * K // 2 + M * K // 16 + 4 * M * r + N * K // 2 + N * K // 16 + 2 * N * r + 4 * N
            + M * N * yb)


def gemm_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * N * r


def prep_u_flops(M, K, r):
    return 2 * M * K * r


def prep_q_flops(M, K, r):
    return 2 * M * K * r


def roofline_of(nbytes, nflops, ms):
    """The bound a kernel's arithmetic intensity puts it under, and its fraction of that peak."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = nflops / (ms * 1e-3) / 1e12
    if nflops / nbytes >= RIDGE:
        return {"bound": "mfma", "achieved": round(tfs, 2), "peak": F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tfs / F16_PEAK_TFLOPS, 4)}, gbs, tfs
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}, gbs, tfs


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 10 denoising steps of the 600-layer set, or "
                         "400 steps of a --workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=None, choices=[0, 1, 2, 3],
                    help="time one of the smaller workloads instead of the 600-layer set")
    ap.add_argument("--min-replica-gib", type=float, default=1.0)
    ap.add_argument("--kernel-timing-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--search", action="store_true",
                    help="time the per-layer smoothing search (the 39-candidate grid) on the "
                         "workload's first layer instead of the forward step")
    ap.add_argument("--eigen", action="store_true",
                    help="time the basis solve instead: the top-32 eigenspace of a synthetic "
                         "4096 x 4096 action metric (block 64, 8 iterations)")
    ap.add_argument("--svdq", action="store_true",
                    help="time the SVDQuant-style INT4 (group 64) W4A4 arm on the workload's "
                         "layer shapes instead of the deflated-ASP NVFP4 path")
    ap.add_argument("--mot", action="store_true",
                    help="the 600-layer two-expert set (the default workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy three times (the reference "
                         "kernel that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    small = args.workload is not None or args.search or args.svdq
    if args.workload is None:
        args.workload = 1
    if args.steps is None:
        args.steps = 400 if small else 10
    if args.warmup is None:
        args.warmup = 40 if small else 2
    args.mot = not small and not args.eigen
    return args


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    slug = workload if isinstance(workload, str) else WORKLOAD_SLUGS[workload]
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{slug}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_digest(kernel):
        return None
    return int(val.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by token rows with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from wam_asp_w4a4_amd import binding as B
    from wam_asp_w4a4_amd import synth
    from wam_asp_w4a4_amd.layer import PackedLayer

    if not os.path.exists(B.LIB_PATH):
        from wam_asp_w4a4_amd import build as _build
        _build.build()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.eigen:
        eigen_bench(args, dev)
        return
    if args.svdq:
        svdq_bench(args, dev)
        return
    if args.mot:
        mot_bench(args, dev)
        return
    layers = synth.workload(args.workload)
    if args.search:
        search_bench(args, layers[0], dev)
        return
    y_dtype = "bf16"
    yb = 2

    # ---- pack once per layer on the host, upload R replicas of every buffer
    host = []
    for lay in layers:
        pk = PackedLayer.pack_host(lay.w, lay.s, lay.v)
        xh = synth.bf16_bits(lay.x) if lay.x_dtype == "bf16" else lay.x
        host.append((lay, pk, xh))

    def replica_bytes():
        tot = 0
        for lay, pk, xh in host:
            tot += xh.nbytes + pk["w_codes"].nbytes + pk["w_scales"].nbytes
            tot += 0 if pk["wv"] is None else pk["wv"].nbytes
            tot += pk["prep"].nbytes
            tot += lay.M * lay.N * yb + B.asp_workspace_bytes(lay.M, lay.N, lay.K, lay.r)
        return tot

    per = replica_bytes()
    R = int(min(512, max(2, np.ceil(args.min_replica_gib * 2 ** 30 / per))))

    def t(a, dtype=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        return (x.view(dtype) if dtype is not None else x).to(dev)

    # layers that read one x (and share K and rank) run as one group: one
    # launch per kernel for the whole group
    group_keys = []
    for lay, _, _ in host:
        key = (id(lay.x), lay.K, lay.r, lay.x_dtype)
        if key not in group_keys:
            group_keys.append(key)
    group_of = [group_keys.index((id(l.x), l.K, l.r, l.x_dtype)) for l, _, _ in host]

    replicas = []
    for _ in range(R):
        groups = [{"layers": [], "packed": [], "ys": [], "wss": [], "x": None}
                  for _ in group_keys]
        for (lay, pk, xh), gi in zip(host, group_of):
            g = groups[gi]
            if g["x"] is None:
                g["x"] = t(xh, torch.bfloat16 if lay.x_dtype == "bf16" else None)
            p = PackedLayer(lay.N, lay.K, lay.r, t(pk["w_codes"]), t(pk["w_scales"]),
                            None if pk["wv"] is None else t(pk["wv"], torch.int16),
                            t(pk["prep"]), t(lay.b))
            g["layers"].append(lay)
            g["packed"].append(p)
            g["ys"].append(torch.empty((lay.M, lay.N), dtype=torch.bfloat16, device=dev))
            g["wss"].append(p.workspace(lay.M))
        replicas.append(groups)

    def run_group(g, stages):
        lay0, ps = g["layers"][0], g["packed"]
        B.asp_forward_group_stages(
            stages, [g["x"]] * len(ps), B.DTYPES[lay0.x_dtype], lay0.M, lay0.K, lay0.r,
            [p.prep for p in ps], [p.w_codes for p in ps], [p.w_scales for p in ps],
            [p.wv for p in ps] if lay0.r else None, [p.bias for p in ps], [p.N for p in ps],
            g["ys"], B.DTYPES[y_dtype], g["wss"], [w.numel() for w in g["wss"]])

    def step(i):
        for g in replicas[i % R]:
            run_group(g, 7)

    # ---- warm-up, then K steps from one graph
    for i in range(args.warmup):
        step(i)
    if args.calibrate_copy:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    # spread: the same graph replayed a few more times (value keeps the first)
    replays = [ms_per_step]
    for _ in range(4):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        replays.append(e0.elapsed_time(e1) / args.steps)
    replays.sort()

    # secondary bandwidth denominator: a plain 256 MiB device-to-device copy
    csrc = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(3):
        cdst.copy_(csrc)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * 3 * COPY_CALIBRATION_BYTES / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del csrc, cdst

    flops_step = sum(layer_flops(l.M, l.N, l.K, l.r) for l, _, _ in host)
    bytes_step = sum(layer_bytes(l.M, l.N, l.K, l.r, 2 if l.x_dtype == "bf16" else 4, yb)
                     for l, _, _ in host)
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12

    # ---- per-kernel durations: each kernel alone (asp_forward_group_stages),
    # nk steps' worth of its launches cycling through the replicas, replayed
    # from a graph of its own between two events on the launch stream (graph
    # replay keeps host launch cost out of the figure).  The u stage goes
    # first, so the quantise stage and then the GEMM read valid partial sums
    # and codes.
    nk = max(1, min(args.kernel_timing_steps, args.steps))

    def graph_ms(stages, sel):
        todo = [g for i in range(nk) for g in replicas[i % R] if sel(g)]
        for g in todo[: len(group_keys)]:  # warm the code path outside the capture
            run_group(g, stages)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for g in todo:
                run_group(g, stages)
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        gr.replay()
        eb.record(stream)
        torch.cuda.synchronize()
        return ea.elapsed_time(eb), todo

    xbytes = lambda l: 2 if l.x_dtype == "bf16" else 4
    gemm_names = sorted({B.asp_gemm_kernel_name(g["layers"][0].M, sum(l.N for l in g["layers"]),
                                                g["layers"][0].K) for g in replicas[0]})
    kernels = [
        ("k_prep_u", "k_prep_u", 1, lambda g: g["layers"][0].r > 0,
         lambda l: prep_u_bytes(l.M, l.K, l.r, xbytes(l)), lambda l: prep_u_flops(l.M, l.K, l.r)),
        ("k_prep_q", "k_prep_q", 2, lambda g: True,
         lambda l: prep_q_bytes(l.M, l.K, l.r, xbytes(l)), lambda l: prep_q_flops(l.M, l.K, l.r)),
        (" + ".join(gemm_names), "k_gemm", 4, lambda g: True,
         lambda l: gemm_bytes(l.M, l.N, l.K, l.r, yb), lambda l: gemm_flops(l.M, l.N, l.K, l.r)),
    ]
    timed = []
    for name, family, stages, sel, fb, ff in kernels:
        if not any(sel(g) for g in replicas[0]):
            continue
        ms, todo = graph_ms(stages, sel)
        nbytes = sum(fb(l) for g in todo for l in g["layers"])
        nflops = sum(ff(l) for g in todo for l in g["layers"])
        timed.append((name, family, ms, len(todo), nbytes, nflops))
    name, family, ms, n_launch, nbytes, nflops = max(timed, key=lambda k: k[2])
    roof, gbs, tfs = roofline_of(nbytes, nflops, ms)
    roof.update({
        "traffic": measured_traffic(family, args.workload),
        "kernel": name,
        "source_digest": kernel_source_digest(family),
        "avg_launch_us": round(ms / n_launch * 1e3, 3),
        "launches": n_launch,
        "algorithmic_bytes_per_launch": nbytes // n_launch,
        "algorithmic_flops_per_launch": nflops // n_launch,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_f16_frac": round(tfs / F16_PEAK_TFLOPS, 4),
        # the roofline the kernel's arithmetic intensity allows, min(P, AI * BW)
        "attainable": round(min(F16_PEAK_TFLOPS, nflops / nbytes * HBM_PEAK_GBS / 1e3), 2)
        if roof["bound"] == "mfma" else HBM_PEAK_GBS,
        "frac_of_attainable": round((tfs if roof["bound"] == "mfma" else gbs)
                                    / (min(F16_PEAK_TFLOPS, nflops / nbytes * HBM_PEAK_GBS / 1e3)
                                       if roof["bound"] == "mfma" else HBM_PEAK_GBS), 4),
        "copy_GBps": round(copy_gbs, 1),
        "hbm_frac_of_copy": round(gbs / copy_gbs, 4),
        "kernels": {k[0]: {"avg_launch_us": round(k[2] / k[3] * 1e3, 3),
                           "frac": roofline_of(k[4], k[5], k[2])[0]["frac"],
                           "bound": roofline_of(k[4], k[5], k[2])[0]["bound"]} for k in timed},
    })

    # ---- CPU baseline: the oracle, on the host cores, on a bounded sample
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(layers, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": synth.WORKLOADS[args.workload],
            "layers": [{"name": l.name, "M": l.M, "K": l.K, "N": l.N, "r": l.r,
                        "x": l.x_dtype, "y": y_dtype} for l, _, _ in host],
            "operands": "NVFP4 (E2M1, block 16, E4M3 scales) decoded to exact fp16 for MFMA, fp32 accumulate",
            "flops_per_step": flops_step,
            "algorithmic_bytes_per_step": bytes_step,
            "effective_GBps": round(bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
            "groups": [[l.name for l in g["layers"]] for g in replicas[0]],
            "replicas": R,
            "replica_bytes": per,
            "timing": "one HIP graph of K steps, events on the capture stream",
            "ms_per_step_replays": {"min": round(replays[0], 6), "median": round(replays[2], 6),
                                    "max": round(replays[-1], 6), "replays": len(replays)},
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def search_bench(args, lay, dev):
    """Wall time of the per-layer smoothing search (host packing of every candidate
    plus the device forward and error per candidate), and the oracle's search on a
    bounded subset of the same grid."""
    import torch
    from wam_asp_w4a4_amd import synth
    from wam_asp_w4a4_amd.layer import smoothing_grid, smoothing_search
    xh = synth.bf16_bits(lay.x) if lay.x_dtype == "bf16" else lay.x
    x = torch.from_numpy(np.ascontiguousarray(xh))
    x = (x.view(torch.bfloat16) if lay.x_dtype == "bf16" else x).to(dev)
    grid = smoothing_grid()
    smoothing_search(x, lay.w, lay.b, lay.v, grid[:2])  # warm-up (code objects, pools)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a, b, mse, best = smoothing_search(x, lay.w, lay.b, lay.v, grid)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    cpu = None
    if args.cpu_seconds > 0:
        from oracle import smoothing as oracle_smoothing
        n = 0
        t1 = time.perf_counter()
        while n < len(grid) and time.perf_counter() - t1 < args.cpu_seconds:
            oracle_smoothing.search(lay.x, lay.w, lay.b, lay.v, [grid[n]])
            n += 1
        cel = time.perf_counter() - t1
        cpu = {"value": round(n / cel, 4), "unit": "candidates/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{n} of the {len(grid)} candidates, {cel:.1f} s"}
    out = {
        "metric": "per-layer smoothing search, candidates per second",
        "value": round(len(grid) / el, 3), "unit": "candidates/s", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": synth.WORKLOADS[args.workload], "layer": lay.name, "M": lay.M,
                   "K": lay.K, "N": lay.N, "r": lay.r, "candidates": len(grid),
                   "seconds": round(el, 4), "best": [a, b],
                   "note": "each candidate: host float64 packing of the weight, upload, "
                           "device forward and squared-error reduction"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def eigen_bench(args, dev):
    """Solves per second of the top-r eigenspace (subspace iteration, Rayleigh-Ritz)
    of a synthetic action metric resident in HBM, the metric-product kernel timed
    alone for the roofline, and the oracle's solve (float64 eigh) on the host."""
    import torch
    from wam_asp_w4a4_amd import binding as B
    from wam_asp_w4a4_amd import synth
    K, p, r, iters = EIG_K, EIG_P, EIG_R, EIG_ITERS
    steps = max(1, min(args.steps, 200))
    warm = max(1, min(args.warmup, 20))
    rng = np.random.default_rng(synth.DEFAULT_SEED)
    g, lam, _ = synth.draw_metric(rng, K)
    v0 = synth.draw_start(rng, K, p)
    gd = torch.from_numpy(g).to(dev)
    vd = torch.from_numpy(v0).to(dev)
    nbytes = B.asp_top_eigenspace_workspace_bytes(K, p, r)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    v = torch.empty((K, r), dtype=torch.float32, device=dev)
    ev = torch.empty(r, dtype=torch.float32, device=dev)
    res = torch.empty(r, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def solve():
        B.asp_top_eigenspace(gd, K, vd, p, r, iters, v, ev, res, ws, nbytes, sp)

    if args.calibrate_copy:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(warm):
        solve()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        solve()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev_h = ev.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(ev_h - lam[:r])) / lam[0])

    # the metric product alone (the kernel the solve spends most of its time in)
    S = B.asp_top_eigenspace_slices(K, p)
    v64 = torch.from_numpy(np.linalg.qr(v0.astype(np.float64))[0]).to(dev)
    yp = torch.empty((S, K, p), dtype=torch.float64, device=dev)
    n_launch = max(10, min(args.kernel_timing_steps, 400))
    for _ in range(3):
        B.asp_metric_product_partials(gd, K, v64, p, yp, sp)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_launch):
        B.asp_metric_product_partials(gd, K, v64, p, yp, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    kms = e0.elapsed_time(e1) / n_launch
    kflops = 2 * K * K * p
    kbytes = 4 * K * K + 8 * K * p + 8 * S * K * p
    tfs = kflops / (kms * 1e-3) / 1e12
    gbs = kbytes / (kms * 1e-3) / 1e9
    ridge = F64_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if kflops / kbytes >= ridge:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": F64_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tfs / F64_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof.update({
        "traffic": measured_traffic("k_eig_gv", EIG_SLUG),
        "kernel": f"k_eig_gv<{p}>",
        "source_digest": kernel_source_digest("k_eig_gv"),
        "avg_launch_us": round(kms * 1e3, 3),
        "launches": n_launch,
        "algorithmic_bytes_per_launch": kbytes,
        "algorithmic_flops_per_launch": kflops,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "dtype": "f64 MFMA (float32 metric widened in registers)",
        "slices": S,
        "timing": "HIP events on the launch stream around back-to-back launches; the "
                  "67 MB metric stays in the 256 MB Infinity Cache between launches, as it "
                  "does between the iterations of a solve",
    })
    cpu = None
    if args.cpu_seconds > 0:
        from oracle import eigen as oracle_eigen
        try:
            from threadpoolctl import threadpool_info
            threads = max([q.get("num_threads", 1) for q in threadpool_info()] or [1])
        except Exception:
            threads = 1
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle_eigen.top_eigenspace(g, r)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n >= 100:
                break
        cpu = {"value": round(n / el, 4), "unit": "solves/s", "cores": int(threads),
               "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{n} full solves of the same metric (float64 NumPy eigh), "
                         f"{el:.1f} s; cores = BLAS threads"}
    out = {
        "metric": f"top-{r} eigenspace of a {K}x{K} action metric, solves per second",
        "value": round(1e3 / ms, 3), "unit": "solves/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"basis solve: K={K}, block p={p}, r={r}, {iters} products with "
                               f"G, spectrum exp(-i/8) + 1e-6 (synthetic metric)",
                   "K": K, "p": p, "r": r, "iters": iters,
                   "max_eigenvalue_error_rel_lam1": err,
                   "max_residual": float(res.max().item()),
                   "timing": "HIP events on the launch stream around back-to-back solves"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def svdq_bench(args, dev):
    """The SVDQuant-style INT4 W4A4 arm on the workload's layer shapes: one step =
    u (k_prep_u), the group quantiser and the INT8 GEMM for every layer, on
    replicas of every buffer resident in HBM; then each kernel timed alone."""
    import torch
    from wam_asp_w4a4_amd import binding as B
    from wam_asp_w4a4_amd import synth
    from wam_asp_w4a4_amd.layer import SvdqLayer
    base = synth.workload(args.workload)
    layers = [synth.make_svdq_layer(l.name, l.M, l.K, l.N, l.r or 32, seed=synth.DEFAULT_SEED + i)
              for i, l in enumerate(base)]
    packed = []
    for lay in layers:
        v = SvdqLayer.right_basis(lay.w, lay.s, lay.r)
        packed.append(SvdqLayer.pack_host(lay.w, lay.s, lay.r, v, lay.b))
    flops = sum(2 * l.M * l.N * l.K + 2 * l.M * l.K * l.r + 2 * l.M * l.N * l.r for l in layers)

    def per_replica(l, h):
        return (h.codes.nbytes + h.scales.nbytes + h.l1.nbytes + h.prep.nbytes + l.M * l.K * 2
                + l.M * l.N * 2 + B.asp_svdq_workspace_bytes(l.M, l.N, l.K, l.r))
    per = sum(per_replica(l, h) for l, h in zip(layers, packed))
    R = max(2, int(np.ceil(args.min_replica_gib * 2 ** 30 / per)))
    reps = []
    for _ in range(R):
        rep = []
        for l, h in zip(layers, packed):
            d = h.to(dev)
            x = torch.from_numpy(synth.bf16_bits(l.x)).view(torch.bfloat16).to(dev)
            nb = B.asp_svdq_workspace_bytes(l.M, l.N, l.K, l.r)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            y = torch.empty((l.M, l.N), dtype=torch.bfloat16, device=dev)
            rep.append((l, d, x, ws, nb, y))
        reps.append(rep)
    # launches go to torch's current stream (the capture stream inside a graph)
    sp = None

    def step(i):
        for l, d, x, ws, nb, y in reps[i % R]:
            B.asp_svdq_forward(x, B.ASP_BF16, l.M, l.K, l.r, d.prep, d.codes, d.scales, d.l1, d.bias,
                               l.N, y, B.ASP_BF16, ws, nb, sp)

    for i in range(args.warmup):
        step(i)
    if args.calibrate_copy:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # each kernel alone: graphs of its launches over the replicas
    nk = max(R, min(args.kernel_timing_steps, 4 * R))
    ubufs = [[torch.zeros((l.M, (l.r + 31) // 32 * 32), dtype=torch.float32, device=dev)
              for l in layers] for _ in range(R)]

    def timed(fn):
        fn(0)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(nk):
                fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nk

    def k_u(i):
        for l, d, x, ws, nb, y in reps[i % R]:
            B.asp_act_prep_u(x, B.ASP_BF16, l.M, l.K, l.r, d.prep, ws, nb, sp)

    def k_q(i):
        for l, d, x, ws, nb, y in reps[i % R]:
            B.asp_svdq_act_quant(x, B.ASP_BF16, l.M, l.K, d.prep, ws, ws[l.M * l.K // 2:], sp)

    def k_g(i):
        for (l, d, x, ws, nb, y), u in zip(reps[i % R], ubufs[i % R]):
            xs_off = (l.M * l.K // 2 + 255) // 256 * 256
            B.asp_svdq_gemm(ws, ws[xs_off:], u, l.M, l.N, l.K, l.r, d.codes, d.scales, d.l1,
                            d.bias, y, B.ASP_BF16, sp)

    t_u, t_q, t_g = timed(k_u), timed(k_q), timed(k_g)
    gflops = sum(2 * l.M * l.N * l.K + 2 * l.M * l.N * l.r for l in layers)
    gbytes = sum(l.M * l.K // 2 + l.M * l.K // 32 + l.N * l.K // 2 + l.N * l.K // 32
                 + l.M * l.r * 4 + l.N * ((l.r + 31) // 32 * 32) * 2 + l.M * l.N * 2 + l.N * 4
                 for l in layers)
    tops = gflops / (t_g * 1e-3) / 1e12
    gbs = gbytes / (t_g * 1e-3) / 1e9
    ridge = I8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gflops / gbytes >= ridge:
        roof = {"bound": "mfma", "achieved": round(tops, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(tops / I8_PEAK_TOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    names = sorted({f"k_svdq_gemm<2, {(l.r + 31) // 32}>" for l in layers})
    roof.update({
        "traffic": measured_traffic("k_svdq_gemm", f"svdq_{WORKLOAD_SLUGS[args.workload]}"),
        "kernel": " + ".join(names),
        "source_digest": kernel_source_digest("k_svdq_gemm"),
        "avg_launch_us": round(t_g * 1e3 / len(layers), 3),
        "launches": nk * len(layers),
        "algorithmic_bytes_per_launch": gbytes // len(layers),
        "algorithmic_flops_per_launch": gflops // len(layers),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "dtype": "int8 MFMA on INT4 codes (exact), float32 group scaling, bf16 low-rank branch",
        "kernels": {"k_prep_u": {"avg_launch_us": round(t_u * 1e3 / len(layers), 3)},
                    "k_svdq_quant": {"avg_launch_us": round(t_q * 1e3 / len(layers), 3)},
                    "k_svdq_gemm": {"avg_launch_us": round(t_g * 1e3 / len(layers), 3)}},
    })
    cpu = None
    if args.cpu_seconds > 0:
        from oracle import svdquant as oracle_sq
        try:
            from threadpoolctl import threadpool_info
            threads = max([q.get("num_threads", 1) for q in threadpool_info()] or [1])
        except Exception:
            threads = 1
        opk = [oracle_sq.pack_weight(l.w, l.s, l.r) for l in layers]
        # the oracle's exact integer group products are slow: large-M layers
        # run on their first 64 rows (rows are independent), FLOPs counted to match
        rows = [l.M if l.M <= 256 else 64 for l in layers]
        sflops = sum(2 * m * l.N * l.K + 2 * m * l.K * l.r + 2 * m * l.N * l.r
                     for m, l in zip(rows, layers))
        n = 0
        t0 = time.perf_counter()
        while True:
            for l, pk, m in zip(layers, opk, rows):
                oracle_sq.forward(l.x[:m], l.w, l.b, l.s, l.r, packed=pk)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n >= 1000:
                break
        cpu = {"value": round(sflops * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
               "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{n} passes over {rows} rows of the layers (float64 NumPy oracle with "
                         f"exact integer group products, weights pre-packed), {el:.1f} s; "
                         "cores = BLAS threads"}
    out = {
        "metric": "SVDQuant-style INT4 W4A4 linear effective TFLOP/s + % of roofline, 1 MI355X",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": synth.WORKLOADS[args.workload] + " (SVDQuant-style INT4 arm)",
                   "layers": [{"name": l.name, "M": l.M, "K": l.K, "N": l.N, "r": l.r} for l in layers],
                   "flops_per_step": flops, "replicas": R,
                   "timing": "one HIP graph of K steps, events on the capture stream"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# Calls per block of one expert in the 600-layer set, in the order a block's
# data dependencies allow.  The first call holds every projection whose input
# is ready when the block starts: self-attention q, k and v read the block's
# input, and cross-attention k and v read the conditioning context, which no
# projection of the block produces.  Each later projection reads the output of
# the attention or residual step before it, so it is a call of its own.
MOT_GROUPS = [("self_attn.q", "self_attn.k", "self_attn.v", "cross_attn.k", "cross_attn.v"),
              ("self_attn.o",), ("cross_attn.q",), ("cross_attn.o",), ("ffn.0",), ("ffn.2",)]
MOT_SLUG = "mot_600_layers"
MOT_WORKLOAD = ("600-layer two-expert MoT set: 30 blocks x {self_attn q/k/v/o, cross_attn "
                "q/k/v/o, ffn.0, ffn.2} per expert, run as one stream of quantised linears; "
                "video d 3072, ffn 14336, M 4096, r 0 (smoothed + Hadamard NVFP4); action "
                "d 1024, ffn 4096, M 256, r 32 (deflated ASP); one step = one denoising step "
                "of all 600 linears; bf16 in and out")


def mot_bench(args, dev):
    """The 600-layer two-expert set (video: d 3072, ffn 14336, M 4096, r 0;
    action: d 1024, ffn 4096, M 256, r 32) as one stream of quantised linears
    per denoising step, every weight and input resident in HBM.  Every layer
    has its own packed weight, prep pack, input and output; the inputs are
    random device tensors drawn like the workloads' (N(0, 1), a fraction of
    channels scaled as outliers) and the packed weights random codes and
    scales (the kernels' timing does not depend on the values; parity on
    sampled layers of this set is in the GPU tests).

    Timing: W eager warm-up steps, then K steps captured in one HIP graph and
    replayed once between synchronisations and events (value).  The same K
    steps then run once more eagerly with HIP events around every launch of
    the video expert's 4-bit GEMM (the dominant kernel): the per-kernel
    figures (roofline).  The experts' split comes from a graph of each expert's half alone.  The
    rocprofv3 kernel trace of the same command gives the kernel's average
    over the graph's and the eager pass's launches alike."""
    import torch
    from wam_asp_w4a4_amd import binding as B
    from wam_asp_w4a4_amd import synth

    gen = torch.Generator(device=dev).manual_seed(synth.DEFAULT_SEED)
    prep_host = {}

    def prep_pack(K, r):
        if (K, r) not in prep_host:
            rng = np.random.default_rng(K + r)
            s_ = (1.0 + rng.random(K)).astype(np.float32)
            v = np.linalg.qr(rng.standard_normal((K, r)))[0].astype(np.float32) if r else None
            pack = np.empty(B.asp_prep_pack_bytes(K, r), np.uint8)
            B.asp_pack_prep(K, r, s_, v, pack)
            prep_host[(K, r)] = torch.from_numpy(pack)
        return prep_host[(K, r)].to(dev)

    layers = {}
    for (name, M, K, N, r, frac, gain, gelu) in synth.mot_shapes():
        x = torch.randn(M, K, generator=gen, device=dev)
        if gelu:
            x = torch.nn.functional.gelu(x)
        n_out = int(round(frac * K))
        if n_out:
            x[:, torch.randperm(K, generator=gen, device=dev)[:n_out]] *= gain
        wv = None
        if r:
            wv = (torch.randn(N, r, generator=gen, device=dev) * 0.05).to(torch.bfloat16)
            wv = wv.view(torch.int16).contiguous()
        layers[name] = {
            "M": M, "K": K, "N": N, "r": r, "x": x.to(torch.bfloat16), "wv": wv,
            "codes": torch.randint(0, 256, (N, K // 2), generator=gen, device=dev,
                                   dtype=torch.uint8),
            "scales": torch.randint(0x30, 0x40, (N, K // 16), generator=gen, device=dev,
                                    dtype=torch.uint8),
            "bias": torch.randn(N, generator=gen, device=dev) * 0.1,
            "prep": prep_pack(K, r),
            "y": torch.empty(M, N, dtype=torch.bfloat16, device=dev)}
        del x
    # workspaces (no dependence on N), one set per (M, K, r), reused by every
    # call in stream order
    wspool = {}

    def workspaces(M, K, r, n):
        key = (M, K, r)
        if key not in wspool:
            nb = B.asp_workspace_bytes(M, 1, K, r)
            wspool[key] = [torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
                           for _ in range(max(len(g) for g in MOT_GROUPS))]
        return wspool[key][:n]

    calls = {"video": [], "action": []}
    for expert in calls:
        for blk in range(synth.MOT_BLOCKS):
            for grp in MOT_GROUPS:
                calls[expert].append([layers[f"{expert}.{blk}.{p}"] for p in grp])
    flops = {e: sum(layer_flops(L["M"], L["N"], L["K"], L["r"]) for c in cs for L in c)
             for e, cs in calls.items()}
    hbm_bytes = {e: sum(layer_bytes(L["M"], L["N"], L["K"], L["r"], 2, 2) for c in cs for L in c)
                 for e, cs in calls.items()}
    gemm_kernel = {B.asp_gemm_kernel_name(c[0]["M"], sum(L["N"] for L in c), c[0]["K"])
                   for c in calls["video"]}
    assert len(gemm_kernel) == 1, gemm_kernel
    gemm_kernel = gemm_kernel.pop()

    def run(c, stages):
        L0 = c[0]
        ws = workspaces(L0["M"], L0["K"], L0["r"], len(c))
        B.asp_forward_group_stages(
            stages, [L["x"] for L in c], B.DTYPES["bf16"], L0["M"], L0["K"], L0["r"],
            [L["prep"] for L in c], [L["codes"] for L in c], [L["scales"] for L in c],
            [L["wv"] for L in c] if L0["r"] else None, [L["bias"] for L in c],
            [L["N"] for L in c], [L["y"] for L in c], B.DTYPES["bf16"], ws,
            [w.numel() for w in ws])

    def step(ev=None):
        """One denoising step.  ev: one (a, b) pair of HIP events per video call,
        recorded around its GEMM launch."""
        for i, c in enumerate(calls["video"]):
            if ev:
                run(c, 3)               # the activation prep
                ev[i][0].record()
                run(c, 4)               # the 4-bit GEMM with its epilogue
                ev[i][1].record()
            else:
                run(c, 7)
        for c in calls["action"]:
            run(c, 7)

    def new_events():
        mk = lambda: torch.cuda.Event(enable_timing=True)
        return [(mk(), mk()) for _ in calls["video"]]

    K_steps, W_steps = args.steps, args.warmup
    for _ in range(max(1, W_steps)):
        step()
    if args.calibrate_copy:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timing = "one HIP graph of K denoising steps, replayed once; events on the capture stream"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(K_steps):
            step()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    # Per-launch durations: the same K steps once more, launched eagerly on the
    # same stream with HIP events around every launch of the video GEMM and
    # around each expert's half (torch declines external events on ROCm, and
    # the runtime rejects event-record nodes in an instantiated graph, so the
    # graph itself carries none).
    evs = [new_events() for _ in range(K_steps)]
    for i in range(K_steps):
        step(evs[i])
    torch.cuda.synchronize()
    per_gemm = [a.elapsed_time(b) for ev in evs for a, b in ev]
    kernel_timing = ("HIP events on the launch stream around every launch of the video GEMM in an "
                     "eager pass of the same K steps right after the timed graph")
    # each expert's half of a step alone, as a graph of its own (3 replays)
    half_ms = {}
    for expert in ("video", "action"):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls[expert]:
                run(c, 7)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        half_ms[expert] = e0.elapsed_time(e1) / 3
        del g
    ms = ms_total / K_steps
    ms_video, ms_action = half_ms["video"], half_ms["action"]
    total = flops["video"] + flops["action"]

    # ---- the dominant kernel: the video expert's 4-bit GEMM, per launch
    gflops = [sum(gemm_flops(L["M"], L["N"], L["K"], L["r"]) for L in c) for c in calls["video"]]
    gbytes = [sum(gemm_bytes(L["M"], L["N"], L["K"], L["r"], 2) for L in c) for c in calls["video"]]
    n_launch = len(per_gemm)
    fl_all = sum(gflops) * K_steps
    by_all = sum(gbytes) * K_steps
    dur_ms = float(np.sum(per_gemm))
    tfs = fl_all / (dur_ms * 1e-3) / 1e12
    shapes = {}
    for i, c in enumerate(calls["video"]):
        key = f"{len(c)} x {c[0]['M']}x{c[0]['K']}->{c[0]['N']}"
        d = shapes.setdefault(key, {"launches": 0, "ms": 0.0, "flops": 0})
        for s_ in range(K_steps):
            d["launches"] += 1
            d["ms"] += per_gemm[s_ * len(calls["video"]) + i]
            d["flops"] += gflops[i]
    per_shape = {k: {"launches": v["launches"],
                     "avg_launch_us": round(v["ms"] / v["launches"] * 1e3, 2),
                     "TFLOPs": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 1),
                     "frac": round(v["flops"] / (v["ms"] * 1e-3) / 1e12 / F16_PEAK_TFLOPS, 4)}
                 for k, v in shapes.items()}
    roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": F16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tfs / F16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("k_gemm", MOT_SLUG),
            "kernel": gemm_kernel,
            "source_digest": kernel_source_digest("k_gemm"),
            "avg_launch_us": round(dur_ms / n_launch * 1e3, 3),
            "launches": n_launch,
            "algorithmic_flops_per_launch": fl_all // n_launch,
            "algorithmic_bytes_per_launch": by_all // n_launch,
            "share_of_step": round(dur_ms / ms_total, 4),
            "per_shape": per_shape,
            "timing": kernel_timing,
            "counters": measured_counters("k_gemm", MOT_SLUG),
            "action_expert": {
                "ms_per_step": round(ms_action, 4),
                "algorithmic_bytes_per_step": hbm_bytes["action"],
                "GBps": round(hbm_bytes["action"] / (ms_action * 1e-3) / 1e9, 1),
                "hbm_frac": round(hbm_bytes["action"] / (ms_action * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "TFLOPs": round(flops["action"] / (ms_action * 1e-3) / 1e12, 2),
                "note": "the 300 rank-32 layers at M = 256 (the small-M target is "
                        "60% of HBM bandwidth); bytes are the layers' algorithmic minimum"}}
    cpu = None
    if args.cpu_seconds > 0:
        cpu = mot_cpu_baseline(args.cpu_seconds, total)
    out = {
        "metric": METRIC,
        "value": round(total / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K_steps, "warmup": W_steps, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic: random device-resident bf16 inputs (outlier channels as in the "
                "workloads) and random packed NVFP4 weights",
        "config": {
            "workload": MOT_WORKLOAD,
            "layers": 600, "calls_per_step": sum(len(v) for v in calls.values()),
            "flops_per_step": total,
            "algorithmic_bytes_per_step": hbm_bytes["video"] + hbm_bytes["action"],
            "video_ms": round(ms_video, 4), "action_ms": round(ms_action, 4),
            "video_TFLOPs": round(flops["video"] / (ms_video * 1e-3) / 1e12, 1),
            "action_TFLOPs": round(flops["action"] / (ms_action * 1e-3) / 1e12, 2),
            # the model card's inference schedule: the video expert once, the action
            # expert for each of the 10 denoising steps (3 300 GEMM calls)
            "schedule_video1_action10_ms": round(ms_video + 10 * ms_action, 3),
            "operands": "NVFP4 (E2M1, block 16, E4M3 scales) decoded to exact fp16 for MFMA, "
                        "fp32 accumulate",
            "timing": timing,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def measured_counters(kernel, slug):
    """MFMA-utilisation figures from the committed counter summary, or None when
    there is none or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{slug}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    if not sha or sha.group(1) != kernel_source_digest(kernel):
        return None
    out = {}
    for key in ("mfma_busy_frac", "mfma_f16_mops_frac", "lds_bank_conflict_per_launch"):
        m = re.search(rf"^{key}:\s*(\S+)", text, re.M)
        if m:
            out[key] = float(m.group(1))
    return out or None


def mot_cpu_baseline(budget_s, step_flops):
    """The oracle on sampled layers of the 600-layer set, its FLOP rate taken
    as the rate of the whole set (extrapolated by FLOPs, stated so), plus the
    single-thread figure for workloads 0-2 and the weight-packing time of the
    oracle against the C++ packer."""
    from oracle import asp as oracle_asp
    from wam_asp_w4a4_amd import synth
    from wam_asp_w4a4_amd.layer import PackedLayer
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits, threads = None, 1
    # one attention projection and both FFN layers of each expert at block 0,
    # each on 256 rows (all of an action layer's; 256 of a video layer's 4096 --
    # rows are independent, but the oracle decodes the whole weight once per
    # call, which 256 rows amortise less than 4096)
    pick = {"video.0.self_attn.q", "video.0.ffn.0", "video.0.ffn.2",
            "action.0.self_attn.q", "action.0.ffn.0", "action.0.ffn.2"}
    sample = []
    for i, (name, M, K, N, r, frac, gain, gelu) in enumerate(synth.mot_shapes()):
        if name in pick:
            rows = 256
            sample.append(synth.make_layer(name, rows, K, N, r, seed=synth.DEFAULT_SEED + i,
                                           outlier_frac=frac, outlier_gain=gain, gelu=gelu))
    # weight packing, timed once per sampled layer of each expert: oracle vs C++
    pack = {}
    for lay in (sample[1], sample[4]):   # video ffn.0 (14336 x 3072), action ffn.0
        t0 = time.perf_counter()
        oracle_asp.pack_weight(lay.w, lay.s, lay.v)
        t1 = time.perf_counter()
        PackedLayer.pack_host(lay.w, lay.s, lay.v)
        t2 = time.perf_counter()
        pack[lay.name] = {"N": lay.N, "K": lay.K, "r": lay.r, "oracle_s": round(t1 - t0, 3),
                          "cpp_packer_s": round(t2 - t1, 3)}
    packed = [oracle_asp.pack_weight(l.w, l.s, l.v) for l in sample]
    flops = sum(layer_flops(l.M, l.N, l.K, l.r) for l in sample)
    n = 0
    t0 = time.perf_counter()
    while True:
        for lay, pk in zip(sample, packed):
            oracle_asp.forward(lay.x, lay.w, lay.b, lay.s, lay.v, packed=pk)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    rate = flops * n / el
    # single-thread oracle on workloads 0-2 (one pass each)
    single = {}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            for w in (0, 1, 2):
                lays = synth.workload(w)
                pks = [oracle_asp.pack_weight(l.w, l.s, l.v) for l in lays]
                t0 = time.perf_counter()
                for l, pk in zip(lays, pks):
                    oracle_asp.forward(l.x, l.w, l.b, l.s, l.v, packed=pk)
                dt = time.perf_counter() - t0
                fl = sum(layer_flops(l.M, l.N, l.K, l.r) for l in lays)
                single[f"workload_{w}"] = {"seconds": round(dt, 4),
                                           "GFLOPs": round(fl / dt / 1e9, 3)}
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": (f"{n} passes over 6 sampled layers of the set (the self-attention q "
                       "projection, ffn.0 and ffn.2 of block 0 of each expert; the video "
                       f"layers on 256 of their 4096 rows), {el:.1f} s on {threads} BLAS "
                       "threads, weights pre-packed; extrapolated by FLOPs to the whole "
                       f"set: {step_flops / rate:.0f} s per denoising step"),
            "single_thread": single,
            "weight_pack_seconds": pack}


def cpu_baseline(layers, budget_s):
    """Time the oracle's per-call path (activation side + NVFP4 contraction) on the host."""
    from oracle import asp as oracle_asp
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    packed = [oracle_asp.pack_weight(l.w, l.s, l.v) for l in layers]
    flops = sum(layer_flops(l.M, l.N, l.K, l.r) for l in layers)
    n = 0
    t0 = time.perf_counter()
    while True:
        for lay, pk in zip(layers, packed):
            oracle_asp.forward(lay.x, lay.w, lay.b, lay.s, lay.v, packed=pk)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    return {"value": round(flops * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{n} full steps of the same workload (float64 NumPy oracle, weights "
                      f"pre-packed), {el:.1f} s; cores = BLAS threads"}


if __name__ == "__main__":
    main()
