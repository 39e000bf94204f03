"""Throughput of the fused Single-Pass mHC step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
pack the next sublayer's projection (mhc_pack_wmix) and run mhc_fused_step on
all tokens (hc_post, hc_mixes with its 4x4 Sinkhorn, hc_pre and RMSNorm, in
one pass over the streams). Inputs are drawn by the seeded generators of
``stream_hyper_connections_amd.workloads`` and are resident in HBM before the
timed region starts; the prior coefficients come from the library's own
mhc_mixes on the same streams.

Prints one JSON line. ``value`` is tokens/s; ``roofline`` reports the fused
kernel's achieved HBM bandwidth (algorithmic bytes per launch / average
launch duration, from HIP events on the launch stream) against 8 TB/s;
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_step_large_prefill_traffic.txt")
BACKWARD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "backward_large_prefill_traffic.txt")
KERNEL_DIR = os.path.join(ROOT, "stream_hyper_connections_amd", "csrc")


def measured_traffic(workload: str, path=None, sources=None):
    """HBM bytes per launch of the fused kernel (or, with the backward's record
    and sources, per backward call) from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by the same counters on a plain copy of known size;
    None unless they were taken on the current kernel source and this
    workload."""
    import json as _json
    try:
        rec = _json.load(open(path or TRAFFIC_FILE))
        src = kernel_source_hash(sources or FUSED_SOURCES)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != src or rec.get("workload") != workload:
        return None
    return int(rec["traffic_bytes"])


# the sources the measured fused-step kernels are built from (the feature-split
# kernel, its clear and tail kernels, the packing kernel and their launch code);
# the general-n, backward and three-kernel sources do not enter them
FUSED_SOURCES = ("mhc.hip", "split_kernel.h")
# the backward's kernels and their launch code
BACKWARD_SOURCES = ("mhc.hip", "backward.h")


def kernel_source_hash(sources=FUSED_SOURCES) -> str:
    """sha256 over kernel sources (names and contents), by default those of the
    fused step."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        h.update(name.encode())
        h.update(open(os.path.join(KERNEL_DIR, name), "rb").read())
    return h.hexdigest()


def algorithmic_bytes_three_kernel(tokens: int, d: int, elem: int) -> int:
    """Bytes the separate kernels must move: hc_post reads x, f and writes x'
    (9d), hc_mixes reads x' (4d), hc_pre reads x' and writes h (5d), RMSNorm
    reads h and writes y (2d): (4n+4)*d elements per token, plus the same 192 B
    of coefficients and the per-call parameters."""
    per_token = (4 * N + 4) * d * elem + 2 * 24 * 4
    per_call = (24 * N * d + 24 + 3 + d) * 4
    return tokens * per_token + per_call


def algorithmic_bytes(tokens: int, d: int, elem: int) -> int:
    """Bytes one fused-step launch must move: read x [T,4,d] and f [T,d], write
    x_out and y ((2n+2)*d elements per token), read the 24 prior coefficients
    and write the 24 new ones (float32), plus the float32 parameters once
    (W [24,4d], base [24], scale [3], gamma [d])."""
    per_token = (2 * N + 2) * d * elem + 2 * 24 * 4
    per_call = (24 * N * d + 24 + 3 + d) * 4
    return tokens * per_token + per_call


def algorithmic_bytes_n(tokens: int, d: int, elem: int, n: int) -> int:
    """Bytes one call of the general-n step must move: the streams ((2n+2)*d
    elements per token), the prior coefficients read and the new ones written
    ((2n + n^2) floats each way), the mixes written ((2+n)n floats, an output
    of that entry point), plus the float32 parameters once."""
    nm = (2 + n) * n
    per_token = (2 * n + 2) * d * elem + (2 * (2 * n + n * n) + nm) * 4
    per_call = (nm * n * d + nm + 3 + d) * 4
    return tokens * per_token + per_call


N_SWEEP = (2, 4, 8)


def general_n_bench(w0, steps, warmup):
    """mhc_fused_step_n at the workload's shape for n = 2, 4, 8: one JSON line
    per n and kernel (HIP events around the call): the token-block kernel
    ("block") for every n, and the feature-split kernel ("split") and the
    chunked block kernel ("chunk", up to 8192 tokens) where they apply, with a
    workspace; each followed by the split/Sinkhorn kernel."""
    import dataclasses
    import torch
    import stream_hyper_connections_amd as mhc
    from stream_hyper_connections_amd import workloads as wl
    dev = torch.device("cuda:0")
    for n in N_SWEEP:
        w = dataclasses.replace(w0, name=f"{w0.name}_n{n}", n=n)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        elem = 2 if w.dtype == "bf16" else 4
        x = upload_tokens(w, wl.X, 0, dev, dt).view(w.tokens, n, w.d)
        f = upload_tokens(w, wl.F, 0, dev, dt)
        prev = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w, prev=True).items()}
        cur = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w).items()}
        prior = mhc.mixes_n(x, mhc.pack_wmix_n(prev["w_mix"], w.dtype), prev["base"],
                            prev["scale"], w.iters, w.norm_eps, w.hc_eps)
        wp = mhc.pack_wmix_n(cur["w_mix"], w.dtype)
        outs = dict(x_out=torch.empty_like(x), y_out=torch.empty_like(f),
                    pre_out=torch.empty_like(prior["pre"]),
                    post_out=torch.empty_like(prior["post"]),
                    comb_out=torch.empty_like(prior["comb"]),
                    mix_out=torch.empty_like(prior["mix"]))

        paths = ["block"]
        for p in ("split", "chunk"):
            try:
                mhc.fused_step_route_n(n, p, w.tokens, w.d, w.dtype)
                paths.append(p)
            except ValueError:
                pass
        kernels = {"block": "gen::block_kernel + gen::sinkhorn_kernel",
                   "split": "fsn::split_kernel + gen::sinkhorn_kernel (feature-split)",
                   "chunk": "gen::block_kernel (chunked) + gen::chunk_finish_kernel + "
                            "gen::sinkhorn_kernel"}
        for path in paths:
            def call():
                mhc.fused_step_n(x, f, prior["pre"], prior["post"], prior["comb"], wp,
                                 cur["base"], cur["scale"], cur["gamma"], w.iters, w.norm_eps,
                                 w.hc_eps, path=path, **outs)

            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            for i in range(steps):
                a[i].record()
                call()
                b[i].record()
            torch.cuda.synchronize()
            ms = np.array([x0.elapsed_time(x1) for x0, x1 in zip(a, b)])
            alg = algorithmic_bytes_n(w.tokens, w.d, elem, n)
            achieved = alg / (ms.mean() / 1e3) / 1e9
            print(json.dumps({
                "metric": f"tokens/s of the general-n fused step, n={n} d={w.d}",
                "value": round(w.tokens / (ms.mean() / 1e3), 1), "unit": "tokens/s",
                "n_streams": n, "path": path, "tokens": w.tokens, "d": w.d, "dtype": w.dtype,
                "call_ms_avg": round(float(ms.mean()), 5),
                "call_ms_p50": round(float(np.percentile(ms, 50)), 5),
                "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                             "algorithmic_bytes_per_launch": alg, "kernel": kernels[path]},
                "config": {"workload": w.name, "sinkhorn_iters": w.iters}}), flush=True)
        del x, f, prior, outs
        torch.cuda.empty_cache()


def algorithmic_bytes_backward(tokens: int, d: int, elem: int, n: int) -> int:
    """Bytes the backward must move at least: read X, F and the upstream dX',
    dy, write dX and dF ((3n+3)*d elements per token; the new streams and h are
    recomputable from X and F), the per-token coefficients (forward's pre, post,
    comb in, mixes out, upstream coefficient gradients, and the coefficient
    gradients written), plus the parameters read and their gradients written."""
    nm = (2 + n) * n
    per_token = (3 * n + 3) * d * elem + (3 * (2 * n + n * n) + nm + (2 * n + n * n)) * 4
    per_call = 2 * (nm * n * d + nm + 3 + d) * 4
    return tokens * per_token + per_call


def backward_bench(w, steps, warmup):
    """mhc_fused_step_backward_n at the workload's shape (its stream count, 4
    unless --n says otherwise): one JSON line, HIP events around the call (all
    backward kernels)."""
    import torch
    import stream_hyper_connections_amd as mhc
    from stream_hyper_connections_amd import workloads as wl
    dev = torch.device("cuda:0")
    n = w.n
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elem = 2 if w.dtype == "bf16" else 4
    x = upload_tokens(w, wl.X, 0, dev, dt).view(w.tokens, n, w.d)
    f = upload_tokens(w, wl.F, 0, dev, dt)
    prev = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w, prev=True).items()}
    cur = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w).items()}
    prior = mhc.mixes_n(x, mhc.pack_wmix_n(prev["w_mix"], w.dtype), prev["base"], prev["scale"],
                        w.iters, w.norm_eps, w.hc_eps)
    fwd = mhc.fused_step_n(x, f, prior["pre"], prior["post"], prior["comb"],
                           mhc.pack_wmix_n(cur["w_mix"], w.dtype), cur["base"], cur["scale"],
                           cur["gamma"], w.iters, w.norm_eps, w.hc_eps)
    # upstream gradients: the forward's own outputs serve as seeded, finite data
    d_x_out, d_y = fwd["x_out"].clone(), fwd["y"].clone()
    d_pre, d_post, d_comb = fwd["pre"].clone(), fwd["post"].clone(), fwd["comb"].clone()
    ws = torch.empty(mhc.fused_step_backward_workspace_bytes_n(n, w.tokens, w.d),
                     dtype=torch.uint8, device=dev)

    def call():
        mhc.fused_step_backward_n(x, f, prior["pre"], prior["post"], prior["comb"], fwd["x_out"],
                                  fwd["mix"], cur["w_mix"], cur["base"], cur["scale"],
                                  cur["gamma"], d_x_out, d_y, d_pre, d_post, d_comb, w.iters,
                                  w.norm_eps, w.hc_eps, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        a[i].record()
        call()
        b[i].record()
    torch.cuda.synchronize()
    ms = np.array([x0.elapsed_time(x1) for x0, x1 in zip(a, b)])
    alg = algorithmic_bytes_backward(w.tokens, w.d, elem, n)
    achieved = alg / (ms.mean() / 1e3) / 1e9
    print(json.dumps({
        "metric": f"tokens/s of the fused-step backward, n={n} d={w.d}",
        "value": round(w.tokens / (ms.mean() / 1e3), 1), "unit": "tokens/s",
        "n_streams": n, "tokens": w.tokens, "d": w.d, "dtype": w.dtype,
        "call_ms_avg": round(float(ms.mean()), 5),
        "call_ms_p50": round(float(np.percentile(ms, 50)), 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic(w.name, BACKWARD_TRAFFIC_FILE, BACKWARD_SOURCES)
                                 if n == 4 else None),
                     "algorithmic_bytes_per_launch": alg,
                     "kernel": "bwd:: split + stats + stream + param + reductions"},
        "config": {"workload": w.name, "sinkhorn_iters": w.iters}}), flush=True)


CONFIG_NAMES = ("tiny", "prefill", "decode", "large_prefill", "chain")


# the kernel that dominates each route of mhc_fused_step
ROUTE_KERNELS = {
    "split": "fsplit::split_kernel (feature-split fused step)",
    "chunk": "pipe::chunk_kernel + pipe::chunk_finish_kernel (chunked fused step)",
    "tile": "pipe::fused_bf16_kernel (tile fused step)",
}


def all_configs_bench(reps_min=50, min_ms=200.0, flush_bytes=512 << 20, path="auto",
                      cooperative=False):
    """mhc_fused_step alone on each workload (the chain: its first step), with
    HIP events around the C-ABI call: warm (10 warm-up calls, then at least
    `reps_min` calls or `min_ms` of calls) and cache-flushed (a write of
    `flush_bytes` between calls, outside the timed events, so that the inputs
    are not served from the 256 MB Infinity Cache). One JSON line per workload
    with p50 / p95 / p99 in microseconds and tokens/s, GB/s and % of peak at
    the p50, and the time per call of 200 calls back to back, eager and as
    replays of the call captured in a graph. cooperative: the feature-split
    kernel launched cooperatively (MHC_PATH_COOPERATIVE) instead of as an
    ordinary kernel."""
    import torch
    import stream_hyper_connections_amd as mhc
    from stream_hyper_connections_amd import workloads as wl
    dev = torch.device("cuda:0")
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    for name in CONFIG_NAMES:
        w = wl.WORKLOADS[name]
        try:
            route = mhc.fused_step_route(path, w.tokens, w.d, w.dtype, cooperative=cooperative)
        except ValueError as e:
            print(f"[bench] {name}: skipped ({e})", file=sys.stderr, flush=True)
            continue
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        elem = 2 if w.dtype == "bf16" else 4
        x = upload_tokens(w, wl.X, 0, dev, dt).view(w.tokens, N, w.d)
        f = upload_tokens(w, wl.F, 0, dev, dt)
        prev = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w, prev=True).items()}
        cur = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w).items()}
        prior = mhc.mixes(x, mhc.pack_wmix(prev["w_mix"], w.dtype), prev["base"], prev["scale"],
                          w.iters, w.norm_eps, w.hc_eps)
        wp = mhc.pack_wmix(cur["w_mix"], w.dtype)
        outs = dict(x_out=torch.empty_like(x), y_out=torch.empty_like(f),
                    pre_out=torch.empty_like(prior["pre"]),
                    post_out=torch.empty_like(prior["post"]),
                    comb_out=torch.empty_like(prior["comb"]))

        need = mhc.fused_step_workspace_bytes(w.tokens, w.d, w.dtype)
        ws = mhc.workspace_for(dev, need) if need > 0 and route != "tile" else None

        def call():
            mhc.fused_step(x, f, prior["pre"], prior["post"], prior["comb"], wp, cur["base"],
                           cur["scale"], cur["gamma"], w.iters, w.norm_eps, w.hc_eps, path=path,
                           workspace=ws, cooperative=cooperative, **outs)

        line = {"metric": "fused mHC step latency per workload, n=4", "workload": name,
                "tokens": w.tokens, "d": w.d, "dtype": w.dtype,
                "route": route}
        if route == "split":
            line["launch"] = "cooperative" if cooperative else "plain"
        alg = algorithmic_bytes(w.tokens, w.d, elem)
        for mode in ("warm", "flushed"):
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            times, total = [], 0.0
            while len(times) < reps_min or total < min_ms:
                if mode == "flushed":
                    scratch.fill_(len(times) & 255)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                b.synchronize()
                ms = a.elapsed_time(b)
                times.append(ms)
                total += ms
            us = np.array(times) * 1e3
            p50 = float(np.percentile(us, 50))
            line[mode] = {"reps": len(times), "p50_us": round(p50, 2),
                          "p95_us": round(float(np.percentile(us, 95)), 2),
                          "p99_us": round(float(np.percentile(us, 99)), 2),
                          "tokens_per_s": round(w.tokens / (p50 / 1e6), 1),
                          "GBps": round(alg / (p50 / 1e6) / 1e9, 1),
                          "frac_of_peak": round(alg / (p50 / 1e6) / 1e9 / HBM_PEAK_GBS, 4)}
        # eager calls back to back (no synchronisation between calls)
        per_call = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(200):
                call()
            b.record()
            b.synchronize()
            per_call.append(a.elapsed_time(b) * 1e3 / 200)
        line["back_to_back_us_per_call"] = round(float(np.median(per_call)), 2)
        # the call captured once into a graph, then replayed back to back
        # (a serving loop's view, no host issue time)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        per_call = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(200):
                graph.replay()
            b.record()
            b.synchronize()
            per_call.append(a.elapsed_time(b) * 1e3 / 200)
        line["graph_replay_us_per_call"] = round(float(np.median(per_call)), 2)
        del graph
        line["algorithmic_bytes"] = alg
        print(json.dumps(line), flush=True)
        del x, f, outs, prior
        torch.cuda.empty_cache()


def crossover_bench(d=5120, sizes=(256, 512, 768, 1024, 1536, 2048, 2560, 3072, 4096), calls=40,
                    runs=5):
    """mhc_fused_step on the chunked and the feature-split route (launched
    as an ordinary kernel: "split", and cooperatively: "split_coop") for a
    range of token counts (seeded random bf16 inputs of width d): per route
    and size, `calls` calls back to back between two events, median over
    `runs` runs. One JSON line per size; the routes' crossing points are where
    path "auto" should switch, with and without MHC_PATH_COOPERATIVE."""
    import torch
    import stream_hyper_connections_amd as mhc
    for t in sizes:
        g = torch.Generator(device="cuda").manual_seed(t)
        x = torch.randn((t, N, d), device="cuda", generator=g).bfloat16()
        f = torch.randn((t, d), device="cuda", generator=g).bfloat16()
        pre = torch.rand((t, N), device="cuda", generator=g)
        post = torch.rand((t, N), device="cuda", generator=g)
        comb = torch.rand((t, N, N), device="cuda", generator=g)
        comb = comb / comb.sum(1, keepdim=True)
        wp = mhc.pack_wmix(0.02 * torch.randn((24, N * d), device="cuda", generator=g), "bf16")
        base = 0.1 * torch.randn(24, device="cuda", generator=g)
        scale, gamma = torch.ones(3, device="cuda"), torch.ones(d, device="cuda")
        ws = torch.zeros(mhc.fused_step_workspace_bytes(t, d, "bf16"), dtype=torch.uint8,
                         device="cuda")
        outs = dict(x_out=torch.empty_like(x), y_out=torch.empty_like(f),
                    pre_out=torch.empty_like(pre), post_out=torch.empty_like(post),
                    comb_out=torch.empty_like(comb))
        line = {"metric": "fused step call time by route, back to back", "tokens": t, "d": d,
                "unit": "us per call", "auto_route": mhc.fused_step_route("auto", t, d, "bf16")}
        for name in ("chunk", "split", "split_coop"):
            def call():
                mhc.fused_step(x, f, pre, post, comb, wp, base, scale, gamma,
                               path=name.split("_")[0], workspace=ws,
                               cooperative=name == "split_coop", **outs)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            per = []
            for _ in range(runs):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(calls):
                    call()
                b.record()
                b.synchronize()
                per.append(a.elapsed_time(b) * 1e3 / calls)
            if mhc.split_status(ws) != 0:   # sticky: covers every call above
                raise RuntimeError("a cross-workgroup wait of the feature-split kernel gave up")
            line[name] = round(float(np.median(per)), 1)
        print(json.dumps(line), flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_prefill")
    ap.add_argument("--path", choices=("auto", "tile", "split", "chunk"), default="auto",
                    help="kernel family of mhc_fused_step (auto: the library's choice by size)")
    ap.add_argument("--cooperative", action="store_true",
                    help="launch the feature-split kernel cooperatively "
                         "(MHC_PATH_COOPERATIVE) instead of as an ordinary kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="minimum oracle time for the cpu_baseline sample")
    ap.add_argument("--form", choices=("fused", "three-kernel"), default="fused",
                    help="fused: the single-pass step (the headline); three-kernel: hc_post, "
                         "hc_mixes, hc_pre and RMSNorm as separate kernels (the comparison)")
    ap.add_argument("--sinkhorn-sweep", action="store_true",
                    help="time the split/Sinkhorn kernel (mhc_sinkhorn4) on the workload's mixes "
                         "for a range of iteration counts and report row-sum convergence; one "
                         "JSON line per count")
    ap.add_argument("--n-sweep", action="store_true",
                    help="time the general stream-count step (mhc_fused_step_n) at the "
                         "workload's shape for n = 2, 4, 8; one JSON line per n")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the step (mhc_fused_step_backward_n) at the "
                         "workload's shape; one JSON line")
    ap.add_argument("--n", type=int, choices=(2, 4), default=None,
                    help="stream count of --backward (default: the workload's, 4)")
    ap.add_argument("--all-configs", action="store_true",
                    help="latency of the fused step alone on every workload, warm and "
                         "cache-flushed (p50/p95/p99); one JSON line per workload")
    ap.add_argument("--crossover", action="store_true",
                    help="call time of the chunked and feature-split routes from 512 to 4,096 "
                         "tokens, back to back; one JSON line per size")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of 2 GiB instead (the reference "
                         "kernel for scaling the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(steps):
    """A plain copy of known size: 2 GiB read + 2 GiB written per launch."""
    import torch
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}), flush=True)


def sinkhorn_sweep(w, mix, base, scale, steps, warmup):
    """mhc_sinkhorn4 on the mixes [T, 24] for every count in SWEEP_ITERS: time
    (HIP events over `steps` calls) and row-sum deviation of the output comb."""
    import torch
    import stream_hyper_connections_amd as mhc
    t = mix.shape[0]
    for iters in SWEEP_ITERS:
        for _ in range(warmup):
            out = mhc.sinkhorn4(mix, base, scale, iters, w.hc_eps)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            out = mhc.sinkhorn4(mix, base, scale, iters, w.hc_eps)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        rdev = (out["comb"].double().sum(dim=2) - 1).abs().amax(dim=1)
        cdev = (out["comb"].double().sum(dim=1) - 1).abs().amax()
        print(json.dumps({
            "metric": "split + Sinkhorn kernel time and comb row-sum deviation vs iterations",
            "sinkhorn_iters": iters, "tokens": t, "ms": round(ms, 5),
            "tokens_per_s": round(t / ms * 1e3, 1),
            "row_dev_median": float(rdev.median()), "row_dev_p99": float(rdev.quantile(0.99)),
            "row_dev_max": float(rdev.max()), "col_dev_max": float(cdev),
            "config": {"workload": w.name, "hc_eps": w.hc_eps}}), flush=True)


def upload_tokens(w, tensor, step, dev, dtype_t):
    """Draw a token-indexed tensor chunk by chunk straight into device memory."""
    import torch
    from stream_hyper_connections_amd import workloads as wl
    width = w.n * w.d if tensor == wl.X else w.d
    out = torch.empty((w.tokens, width), dtype=dtype_t, device=dev)
    for t0, blk in wl.token_tensor_chunks(w, tensor, step):
        out[t0:t0 + len(blk)].copy_(wl.to_dtype(blk, w.dtype))
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, min_seconds):
    """The float64 oracle on consecutive 1,024-token chunks of the same
    workload until at least ``min_seconds`` of oracle time has accumulated.
    Per chunk the inputs and the prior coefficients are prepared outside the
    timed region; only ``oracle.fused_step`` is timed."""
    import oracle
    from threadpoolctl import threadpool_info
    from stream_hyper_connections_amd import workloads as wl

    prev, cur = wl.params(w, prev=True), wl.params(w)
    chunk, done, secs = wl.CHUNK, 0, 0.0
    while secs < min_seconds and done < w.tokens:
        idx = np.arange(done, min(done + chunk, w.tokens))
        x = wl.streams(w, 0, idx).double().numpy()
        f = wl.sublayer_out(w, 0, idx).double().numpy()
        _, pre, post, comb = oracle.mixes(x, prev["w_mix"], prev["base"], prev["scale"], w.iters,
                                          w.norm_eps, w.hc_eps)
        pre, post, comb = (a.astype(np.float32) for a in (pre, post, comb))
        t0 = time.perf_counter()
        oracle.fused_step(x, f, pre, post, comb, cur["w_mix"], cur["base"], cur["scale"],
                          cur["gamma"], w.iters, w.norm_eps, w.hc_eps, w.dtype)
        secs += time.perf_counter() - t0
        done += len(idx)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    # one core, on one chunk, for context
    from threadpoolctl import threadpool_limits
    idx = np.arange(0, min(chunk, w.tokens))
    x = wl.streams(w, 0, idx).double().numpy()
    f = wl.sublayer_out(w, 0, idx).double().numpy()
    _, pre, post, comb = oracle.mixes(x, prev["w_mix"], prev["base"], prev["scale"], w.iters,
                                      w.norm_eps, w.hc_eps)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.fused_step(x, f, pre.astype(np.float32), post.astype(np.float32),
                          comb.astype(np.float32), cur["w_mix"], cur["base"], cur["scale"],
                          cur["gamma"], w.iters, w.norm_eps, w.hc_eps, w.dtype)
        one = len(idx) / (time.perf_counter() - t0)
    return {"value": done / secs, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle, full step on the first {done} tokens of {w.name} in "
                      f"chunks of {chunk} ({secs:.2f} s of oracle time; inputs and prior prepared "
                      f"outside the timed region), host CPUs {os.cpu_count()}",
            "cpu_model": cpu_model(), "single_core_value": round(one, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the step shards over "
              "tokens with no communication, so a multi-GPU figure would be N independent "
              "copies of the one-GPU run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import stream_hyper_connections_amd as mhc
    from stream_hyper_connections_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    mhc.load()
    w = wl.WORKLOADS[args.workload]
    if args.n_sweep:
        general_n_bench(w, args.steps, args.warmup)
        return
    if args.backward:
        if args.n is not None:
            w = dataclasses.replace(w, n=args.n)
        backward_bench(w, args.steps, args.warmup)
        return
    if args.all_configs:
        all_configs_bench(path=args.path, cooperative=args.cooperative)
        return
    if args.crossover:
        crossover_bench()
        return
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elem = 2 if w.dtype == "bf16" else 4

    t_prep = time.time()
    x = upload_tokens(w, wl.X, 0, dev, dt).view(w.tokens, N, w.d)
    f = upload_tokens(w, wl.F, 0, dev, dt)
    prev = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w, prev=True).items()}
    cur = {k: torch.as_tensor(v).to(dev) for k, v in wl.params(w).items()}
    wp_prev = mhc.pack_wmix(prev["w_mix"], w.dtype)
    prior = mhc.mixes(x, wp_prev, prev["base"], prev["scale"], w.iters, w.norm_eps, w.hc_eps)
    wp = torch.empty(mhc.wmix_packed_bytes(w.d, w.dtype), dtype=torch.uint8, device=dev)
    outs = dict(x_out=torch.empty_like(x), y_out=torch.empty_like(f),
                pre_out=torch.empty_like(prior["pre"]), post_out=torch.empty_like(prior["post"]),
                comb_out=torch.empty_like(prior["comb"]))
    route = mhc.fused_step_route(args.path, w.tokens, w.d, w.dtype, cooperative=args.cooperative)
    kernel_name = ROUTE_KERNELS[route]
    if args.form != "fused":
        kernel_name = "hc_post + hc_mixes + hc_pre + RMSNorm kernels (three-kernel form)"
    if args.sinkhorn_sweep:
        cur_mix = mhc.mixes(x, mhc.pack_wmix(cur["w_mix"], w.dtype), cur["base"], cur["scale"],
                            w.iters, w.norm_eps, w.hc_eps, want_mix=True)["mix"]
        torch.cuda.synchronize()
        sinkhorn_sweep(w, cur_mix, cur["base"], cur["scale"], args.steps, args.warmup)
        return
    torch.cuda.synchronize()
    print(f"[bench] inputs resident after {time.time() - t_prep:.1f}s: {w.name} T={w.tokens} "
          f"d={w.d} {w.dtype}", file=sys.stderr, flush=True)

    h_buf = torch.empty_like(f)

    def step():
        mhc.pack_wmix(cur["w_mix"], w.dtype, out=wp)
        e1.record()
        if args.form == "fused":
            mhc.fused_step(x, f, prior["pre"], prior["post"], prior["comb"], wp, cur["base"],
                           cur["scale"], cur["gamma"], w.iters, w.norm_eps, w.hc_eps,
                           path=args.path, cooperative=args.cooperative, **outs)
        else:
            mhc.three_kernel_step(x, f, prior["pre"], prior["post"], prior["comb"], wp,
                                  cur["base"], cur["scale"], cur["gamma"], w.iters, w.norm_eps,
                                  w.hc_eps, x_out=outs["x_out"], h_out=h_buf, y_out=outs["y_out"])

    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        e1 = mids[i]
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if route != "tile" and args.form == "fused":
        # the status word is sticky (no call clears it), so this one read
        # covers every warm-up and timed call on the workspace
        ws = mhc.workspace_for(dev, mhc.fused_step_workspace_bytes(w.tokens, w.d, w.dtype))
        if mhc.split_status(ws) != 0:
            print("bench.py: a cross-workgroup wait of the feature-split kernel gave up; the "
                  "outputs and the timing are invalid", file=sys.stderr)
            sys.exit(1)

    step_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    kern_ms = np.array([m.elapsed_time(e) for m, e in zip(mids, ends)])
    total_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = total_ms / args.steps
    value = w.tokens / (ms_per_step / 1e3)
    alg = (algorithmic_bytes(w.tokens, w.d, elem) if args.form == "fused"
           else algorithmic_bytes_three_kernel(w.tokens, w.d, elem))
    kern_avg_s = kern_ms.mean() / 1e3
    achieved = alg / kern_avg_s / 1e9

    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak) for fused mHC step, n=4 d=5120",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch,
                   "seq_len": w.tokens // w.batch, "n_streams": N, "d": w.d,
                   "sinkhorn_iters": w.iters, "stream_dtype": w.dtype, "form": args.form,
                   "split_launch": (("cooperative" if args.cooperative else "plain")
                                    if route == "split" else None)},
        "step_ms_p50": round(float(np.percentile(step_ms, 50)), 5),
        "step_ms_p95": round(float(np.percentile(step_ms, 95)), 5),
        "step_ms_p99": round(float(np.percentile(step_ms, 99)), 5),
        "fused_kernel_ms_avg": round(float(kern_ms.mean()), 5),
        "fused_kernel_ms_p50": round(float(np.percentile(kern_ms, 50)), 5),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name) if args.form == "fused" else None,
                     "algorithmic_bytes_per_launch": alg,
                     "kernel": kernel_name},
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
