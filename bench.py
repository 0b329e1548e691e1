#!/usr/bin/env python3
"""Benchmark of the NVFP4 grouped-MoE path on one MI355X.

Headline workload: one rank's share of the 16-token grouped-MoE decode. That is 16 tokens, 512
experts, top-10 uniform routing, hidden K = 2048, expert intermediate I = 512, NVFP4 W13/W2 and
FP16 activations. One step is one MoE layer call: routing plan, grouped W13 + SwiGLU, grouped W2,
and the top-k weighted reduction (4 kernels). Steps are captured in one HIP graph. They cycle
through 48 seeded route patterns and through several distinct weight sets, so the 256 MB
Infinity Cache cannot serve repeated weights (the rotating-weights lesson of the "[Kernel][SM70]
Improve Qwen3.8 no-MTP concurrency" page, "Test Result").

value = weight HBM GB/s: the bytes of the distinct active experts' weights (W13 1,179,648 B plus
W2 589,824 B per expert) summed over the steps of one graph, divided by the median time of 20 (or
--trials) timed replays of that graph (p10 / median / p90 in `trials`). The JSON line also carries:
  - us_per_layer and the M = 1..16 sweep (uniform routing);
  - the routing-stress rows (Zipf, all-singleton, shared ids, repeats + invalid) at M = 1..16;
  - the tiny layer's latency;
  - a measured copy-kernel ceiling (torch's copy of the same byte counts) and each GB/s figure's
    fraction of it beside its fraction of the 8 TB/s peak;
  - the 8192-token prefill in TFLOP/s;
  - the dense 4352x5120 projection, its channel-FP8 form, the dense gated MLP, the router;
  - the roofline of the dominant kernel (grouped W13 + SwiGLU with the plan built in the
    launch), timed with HIP events on its launch stream;
  - the fp64 CPU oracle timed on a bounded sample (cpu_baseline).
--counters decode|prefill runs only a calibration copy and a few eager layer calls, for
rocprofv3 --pmc counter runs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE W13+W2 µs/layer + weight HBM GB/s (M=1..16), TFLOP/s at 8192 tok"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 MFMA
E, TOPK, K, I = 512, 10, 2048, 512
W13_EXPERT_BYTES = 2 * I * K // 2 + 2 * I * K // 16   # 1,179,648
W2_EXPERT_BYTES = K * I // 2 + K * I // 16            # 589,824
EXPERT_BYTES = W13_EXPERT_BYTES + W2_EXPERT_BYTES     # 1,769,472
FLOP_PER_PAIR = 6 * I * K                             # 2*2I*K (W13) + 2*K*I (W2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--weight-sets", type=int, default=12)
    p.add_argument("--patterns", type=int, default=48)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-route", action="store_true")
    p.add_argument("--no-mlp", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--trials", type=int, default=20, help="timed replays of each graph (at least 20 for the headline)")
    p.add_argument("--no-stress", action="store_true")
    p.add_argument("--counters", choices=("decode", "prefill"), default=None,
                   help="counter-collection mode for rocprofv3 --pmc runs: a 256 MiB device copy (the calibration "
                        "kernel), then eager layer calls (decode: 12 calls of the 16-token layer on distinct weight "
                        "sets; prefill: 2 calls of the 8192-token layer); prints only what it ran")
    p.add_argument("--traffic", action="store_true", help="same as --counters decode")
    return p.parse_args()


class Routes:
    """Seeded route patterns for M tokens (device tensors + per-pattern active-expert counts)."""

    def __init__(self, M, n, seed_base, routing="uniform"):
        import torch
        from synth import inputs as S
        self.M, self.x, self.ids, self.tw, self.active, self.valid, self.np_ids = M, [], [], [], [], [], []
        for p in range(n):
            rng = S.rng_for(S.WORKLOAD_IDS["decode"] if M <= 16 else S.WORKLOAD_IDS["prefill"], 0, seed_base + p)
            x = S.activations(rng, M, K)
            ids = S.ROUTINGS[routing](rng, M, TOPK, E)
            tw = S.softmax_weights(rng, M, TOPK)
            self.np_ids.append(ids)
            self.x.append(torch.from_numpy(x).cuda())
            self.ids.append(torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda())
            self.tw.append(torch.from_numpy(tw).cuda())
            self.active.append(S.active_experts(ids, E))
            self.valid.append(int(((ids >= 0) & (ids < E)).sum()))


def time_graph(build_fn, steps, warmup_fn=None, trials=20):
    """Capture build_fn() (which enqueues `steps` steps) in one graph, replay it once untimed, then
    time `trials` replays, each alone: HIP events on the replay stream around the replay, with a
    synchronize before and after. Returns the per-replay milliseconds."""
    import torch
    if warmup_fn is not None:
        warmup_fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        build_fn()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(max(1, trials)):
        torch.cuda.synchronize()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms.append(t0.elapsed_time(t1))
    del g
    return ms


def med(ms):
    return float(np.median(ms))


def spread(ms, steps):
    """p10 / median / p90 of per-replay times, in µs per step."""
    q = np.percentile(np.asarray(ms) * 1e3 / steps, [10, 50, 90])
    return {"n": len(ms), "us_p10": round(float(q[0]), 3), "us_median": round(float(q[1]), 3),
            "us_p90": round(float(q[2]), 3)}


def weight_sets(n, seed0=1000):
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    w13 = [G.NVFP4Tensor(*S.device_nvfp4_weights(seed0 + r, E, 2 * I, K)) for r in range(n)]
    w2 = [G.NVFP4Tensor(*S.device_nvfp4_weights(seed0 + 500 + r, E, K, I)) for r in range(n)]
    return w13, w2


def moe_layer_timing(M, steps, warmup, W13, W2, routes, trials=20):
    """µs per MoE layer and weight GB/s over graphs of `steps` layer calls: the median of `trials`
    timed replays (p10 / p90 beside it)."""
    import gemm_nvfp4_amd as G
    R, P = len(W13), len(routes.x)
    layer = G.MoELayer(M, TOPK, W13[0], W2[0])

    def step(i):
        p = i % P
        layer(routes.x[p], routes.ids[p], routes.tw[p], W13[i % R], W2[i % R])

    def warm():
        for i in range(warmup):
            step(i)

    ms_all = time_graph(lambda: [step(i) for i in range(steps)], steps, warm, trials=trials)
    ms = med(ms_all)
    wbytes = sum(routes.active[i % P] * EXPERT_BYTES for i in range(steps))
    pairs = sum(routes.valid[i % P] for i in range(steps))
    us = ms * 1e3 / steps
    return {"M": M, "us_per_layer": round(us, 3), "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(pairs * FLOP_PER_PAIR / (ms * 1e-3) / 1e12, 2),
            "mean_active_experts": round(float(np.mean(routes.active)), 2), "steps": steps,
            "trials": spread(ms_all, steps)}


def stress_timing(steps, warmup, W13, W2, patterns):
    """The routing-stress workload (512 experts, top-10, K=2048, I=512) at M = 1, 2, 4, 8, 16 for each
    routing: Zipf(1.2), all-singleton, every token on the same 10 experts, repeated ids with -1
    slots. Weight GB/s counts each layer's distinct active experts."""
    res = []
    for r, routing in enumerate(("zipf", "singleton", "shared", "repeat_invalid")):
        for M in (1, 2, 4, 8, 16):
            routes = Routes(M, patterns, 6000 + 100 * r + M, routing=routing)
            t = moe_layer_timing(M, steps, warmup, W13, W2, routes)
            res.append({"routing": routing, "M": M, "us_per_layer": t["us_per_layer"],
                        "weight_GBps": t["weight_GBps"], "hbm_frac": t["hbm_frac"],
                        "mean_active_experts": t["mean_active_experts"], "us_p90": t["trials"]["us_p90"]})
    return res


def tiny_timing(steps, copies=64):
    """The tiny layer (1 token, 8 experts, top-2, K=256, I=128): µs per layer call in a graph that
    rotates `copies` weight sets. Its 442 KB of weights make it a latency figure, not a roofline one."""
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    sh = S.TINY
    w13 = [G.NVFP4Tensor(*S.device_nvfp4_weights(11000 + c, sh.e, 2 * sh.i, sh.k)) for c in range(copies)]
    w2 = [G.NVFP4Tensor(*S.device_nvfp4_weights(11500 + c, sh.e, sh.k, sh.i)) for c in range(copies)]
    import torch
    xs, ids, tws = [], [], []
    for p in range(16):
        rng = S.rng_for(S.WORKLOAD_IDS["tiny"], 0, 500 + p)
        xs.append(torch.from_numpy(S.activations(rng, 1, sh.k)).cuda())
        ids.append(torch.from_numpy(np.ascontiguousarray(S.routing_uniform(rng, 1, sh.topk, sh.e), np.int32)).cuda())
        tws.append(torch.from_numpy(S.softmax_weights(rng, 1, sh.topk)).cuda())
    layer = G.MoELayer(1, sh.topk, w13[0], w2[0])

    def step(i):
        layer(xs[i % 16], ids[i % 16], tws[i % 16], w13[i % copies], w2[i % copies])

    ms = time_graph(lambda: [step(i) for i in range(steps)], steps, lambda: [step(i) for i in range(4)])
    return {"workload": "1 token, 8 experts, top-2, K=256, I=128", "us_per_layer": round(med(ms) * 1e3 / steps, 3),
            "trials": spread(ms, steps)}


def copy_ceiling(nbytes_list=(12533760, 245194752), sets=8, launches=64):
    """A plain device copy (torch's copy kernel) of the same byte counts as the dense projection's
    weights and the 16-token layer's weights, rotating `sets` source/destination pairs. GB/s counts
    the bytes read plus the bytes written, the HBM traffic of the copy."""
    import torch
    res = []
    for nb in nbytes_list:
        src = [torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(sets)]
        dst = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(sets)]
        n = launches if nb < (64 << 20) else 16
        ms = time_graph(lambda: [dst[i % sets].copy_(src[i % sets]) for i in range(n)], n)
        us = med(ms) * 1e3 / n
        res.append({"bytes": nb, "copy_us": round(us, 3), "copy_GBps": round(2 * nb / (us * 1e-6) / 1e9, 1)})
        del src, dst
        torch.cuda.empty_cache()
    return res


def eager_latency(M, W13, W2, routes, calls=20):
    """Median µs of single eager layer calls (host launch work included), each bracketed by HIP
    events and a synchronize."""
    import torch
    import gemm_nvfp4_amd as G
    layer = G.MoELayer(M, TOPK, W13[0], W2[0])
    P = len(routes.x)
    for i in range(3):
        layer(routes.x[i % P], routes.ids[i % P], routes.tw[i % P], W13[i % len(W13)], W2[i % len(W2)])
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for i in range(calls):
        t0.record()
        layer(routes.x[i % P], routes.ids[i % P], routes.tw[i % P], W13[i % len(W13)], W2[i % len(W2)])
        t1.record()
        torch.cuda.synchronize()
        us.append(t0.elapsed_time(t1) * 1e3)
    return round(float(np.median(us)), 3)


def w13_kernel_timing(M, launches, W13, routes):
    """Average duration of the layer's grouped W13 + SwiGLU launch alone, the one that builds the
    routing plan itself (HIP events around a graph of back-to-back launches on the capture/replay
    stream), and its algorithmic bytes per launch."""
    import torch
    import gemm_nvfp4_amd as G
    R, P = len(W13), len(routes.x)
    plan = torch.empty(max(G.nvfp4_moe_plan_bytes(M, TOPK, E), 4) // 4, dtype=torch.int32, device="cuda")
    h = torch.empty((M * TOPK, I), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()

    def build():
        for i in range(launches):
            p = i % P
            G.nvfp4_moe_plan_w13_swiglu(routes.ids[p], E, routes.x[p], W13[i % R], 0, plan=plan, h=h)

    ms = med(time_graph(build, launches))
    algo = [routes.active[p] * W13_EXPERT_BYTES + M * K * 2 + routes.valid[p] * I * 2 for p in range(P)]
    bytes_per_launch = float(np.mean([algo[i % P] for i in range(launches)]))
    us = ms * 1e3 / launches
    return us, bytes_per_launch


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w13_swiglu_stream_decode16_traffic.txt")
ROOFLINE_KERNEL = "w13_swiglu_stream_kernel<4, 1, false, true, false> (routing plan built in the launch)"
KERNEL_SOURCES = ("gemm_nvfp4_amd/csrc/moe_gemm.hip", "gemm_nvfp4_amd/csrc/nvfp4_device.hpp",
                  "gemm_nvfp4_amd/csrc/internal.hpp", "gemm_nvfp4_amd/csrc/plan_device.hpp",
                  "gemm_nvfp4_amd/csrc/stream_schedule.hpp")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the headline W13 kernel from the committed counter summary, or None
    when the kernel sources changed since the counters were taken."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def counters_mode(kind, W13, W2):
    """Eager launches for rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, SQ_*): a device copy of known
    size first (the calibration kernel), then the layer calls of one workload."""
    import torch
    import gemm_nvfp4_amd as G
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    if kind == "decode":
        M, calls = 16, 12
        routes = Routes(M, calls, 1000)
    else:
        M, calls = 8192, 2
        routes = Routes(M, calls, 5000)
    layer = G.MoELayer(M, TOPK, W13[0], W2[0])
    for i in range(calls):
        layer(routes.x[i], routes.ids[i], routes.tw[i], W13[i % len(W13)], W2[i % len(W2)])
    torch.cuda.synchronize()
    w13 = [routes.active[p] * W13_EXPERT_BYTES + M * K * 2 + routes.valid[p] * I * 2 for p in range(calls)]
    w2 = [routes.active[p] * W2_EXPERT_BYTES + routes.valid[p] * I * 2 + routes.valid[p] * K * 4 for p in range(calls)]
    log(f"counters mode ({kind}): copy 268435456 B x3; {calls} layer calls at M={M}; algorithmic bytes per "
        f"launch: W13 {np.mean(w13):.0f}, W2 (weights + h + FP32 results) {np.mean(w2):.0f}; "
        f"FLOP per layer {np.mean(routes.valid) * FLOP_PER_PAIR:.4g}")


def eager_launch_floor(calls=50):
    """Median µs of one eager launch of a one-element kernel (torch's in-place add) bracketed by HIP
    events and a synchronize, as eager_latency brackets a layer call: the runtime's own latency of
    a single launch, which an eager layer call pays once more than its graph replay."""
    import torch
    t = torch.zeros(1, device="cuda")
    for _ in range(5):
        t.add_(1.0)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for _ in range(calls):
        t0.record()
        t.add_(1.0)
        t1.record()
        torch.cuda.synchronize()
        us.append(t0.elapsed_time(t1) * 1e3)
    return round(float(np.median(us)), 3)


def launch_floor(launches=480):
    import torch
    t = torch.zeros(1, device="cuda")
    ms = med(time_graph(lambda: [t.add_(1.0) for _ in range(launches)], launches))
    return ms * 1e3 / launches


def prefill_timing(W13, W2, steps=4):
    import gemm_nvfp4_amd as G
    M = 8192
    routes = Routes(M, 2, 5000)
    layer = G.MoELayer(M, TOPK, W13[0], W2[0])
    R = len(W13)

    def step(i):
        layer(routes.x[i % 2], routes.ids[i % 2], routes.tw[i % 2], W13[i % R], W2[i % R])

    ms_all = time_graph(lambda: [step(i) for i in range(steps)], steps, lambda: step(0), trials=10)
    ms = med(ms_all)
    pairs = sum(routes.valid[i % 2] for i in range(steps))
    return {"M": M, "ms_per_layer": round(ms / steps, 3),
            "tflops": round(pairs * FLOP_PER_PAIR / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(pairs * FLOP_PER_PAIR / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "gflop_per_layer": round(routes.valid[0] * FLOP_PER_PAIR / 1e9, 2),
            "trials": {k.replace("us_", "ms_"): round(v / 1e3, 4) if k != "n" else v
                       for k, v in spread(ms_all, steps).items()}}


def dense_timing(copies=64, launches=256):
    import torch
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    N, Kd = S.DENSE_N, S.DENSE_K
    ws = [G.NVFP4Tensor(*S.device_nvfp4_weights(7000 + c, 1, N, Kd)) for c in range(copies)]
    wbytes = N * Kd // 2 + N * Kd // 16
    res = []
    for M in S.DENSE_MS:
        x = torch.from_numpy(S.activations(S.rng_for(1, 0, 1000 + M), M, Kd)).cuda()
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ms = med(time_graph(lambda: [G.nvfp4_linear(x, ws[i % copies], y=y) for i in range(launches)], launches))
        us = ms * 1e3 / launches
        # the split-K form (nvfp4_linear_ws: same results, per-chunk partials in a workspace, then
        # their ordered sum; up to 8 rows it runs the one-launch kernel)
        wsb = torch.empty(max(G.nvfp4_linear_ws_bytes(M, N, Kd), 16), dtype=torch.uint8, device="cuda")
        ms_ws = med(time_graph(lambda: [G.nvfp4_linear_ws(x, ws[i % copies], y=y, ws=wsb) for i in range(launches)],
                               launches))
        us_ws = ms_ws * 1e3 / launches
        res.append({"M": M, "us": round(us, 3), "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "split_k_us": round(us_ws, 3),
                    "split_k_hbm_frac": round(wbytes / (us_ws * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    return res


def shared_layer_timing(steps, W13, W2, routes, i_shared=512):
    """The 16-token decode layer with a shared expert (K=2048, 512 intermediate columns) and its gate:
    plan + W13 (one launch), shared expert, W2 with the shared term. Weight sets rotate as in the headline; the
    shared expert rotates over as many copies. Three forms: the shared expert's own launches in the
    same stream (serial), on a second stream (overlapped), and inside the routed launches (fused)."""
    import torch
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    R, P, M = len(W13), len(routes.x), 16
    sw13 = [G.NVFP4Tensor(*S.device_nvfp4_weights(8000 + r, 1, 2 * i_shared, K)) for r in range(R)]
    sw2 = [G.NVFP4Tensor(*S.device_nvfp4_weights(8500 + r, 1, K, i_shared)) for r in range(R)]
    g = torch.from_numpy((np.random.default_rng(3).standard_normal(K) / np.sqrt(K)).astype(np.float16)).cuda()
    layer = G.MoELayer(M, TOPK, W13[0], W2[0])
    hs = torch.empty((M, i_shared), dtype=torch.float16, device="cuda")
    ys = torch.empty((M, K), dtype=torch.float32, device="cuda")
    sg = torch.empty((M,), dtype=torch.float32, device="cuda")

    side = torch.cuda.Stream()  # default priority

    def step_fused(i):  # the shared expert as extra tiles of the routed W13 and W2 launches
        p, r = i % P, i % R
        G.nvfp4_moe_plan_w13_swiglu_with_shared(routes.ids[p], E, routes.x[p], W13[r], sw13[r], g, plan=layer.plan,
                                                h=layer.h, shared_h=hs, shared_sigma=sg)
        G.nvfp4_moe_w2_reduce_with_shared(layer.plan, M, TOPK, E, layer.h, W2[r], routes.tw[p], hs, sw2[r], sg,
                                          shared_y=ys, out=layer.out, ws=layer.ws)

    def step(i, overlap):
        if overlap is None:
            return step_fused(i)
        p, r = i % P, i % R
        cur = torch.cuda.current_stream()
        if overlap:  # the shared expert depends on x only: run it beside plan + W13
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                G.nvfp4_moe_shared_expert(routes.x[p], sw13[r], sw2[r], g, h=hs, shared_y=ys, shared_sigma=sg,
                                          stream=side)
        else:
            G.nvfp4_moe_shared_expert(routes.x[p], sw13[r], sw2[r], g, h=hs, shared_y=ys, shared_sigma=sg)
        G.nvfp4_moe_plan_w13_swiglu(routes.ids[p], E, routes.x[p], W13[r], 0, plan=layer.plan, h=layer.h)
        if overlap:
            cur.wait_stream(side)
        G.nvfp4_moe_w2_reduce_shared(layer.plan, M, TOPK, E, layer.h, W2[r], routes.tw[p], ys, sg, out=layer.out,
                                     ws=layer.ws)

    wbytes = sum(routes.active[i % P] * EXPERT_BYTES + 3 * i_shared * K * 9 // 16 for i in range(steps))
    res = {"M": M, "shared_intermediate": i_shared}
    for name, ov in (("serial", False), ("overlapped", True), ("fused", None)):
        ms = med(time_graph(lambda: [step(i, ov) for i in range(steps)], steps,
                            lambda: [step(i, ov) for i in range(8)]))
        res[f"us_per_layer_{name}"] = round(ms * 1e3 / steps, 3)
        res[f"weight_GBps_{name}"] = round(wbytes / (ms * 1e-3) / 1e9, 1)
    return res


def fp8_timing(copies=40, launches=192):
    """Channel-FP8 dense projection 4352 x 5120 (22.3 MB of E4M3 bytes + scales), µs per call in
    graphs that rotate `copies` weight copies (about 0.9 GB)."""
    import torch
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    N, Kd = S.DENSE_N, S.DENSE_K
    ws = []
    for c in range(copies):
        codes, scale = S.fp8_channel_weights(S.rng_for(S.WORKLOAD_IDS["dense"], 700 + c, 0), N, Kd)
        ws.append(G.FP8ChannelTensor.from_numpy((codes, scale)))
    wbytes = N * Kd + N * 4
    res = []
    for M in (1, 16, 32):
        x = torch.from_numpy(S.activations(S.rng_for(1, 0, 3000 + M), M, Kd)).cuda()
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ms = med(time_graph(lambda: [G.nvfp4_linear_fp8(x, ws[i % copies], y=y) for i in range(launches)],
                            launches))
        us = ms * 1e3 / launches
        res.append({"M": M, "us": round(us, 3), "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    return res


def mlp_timing(copies=48, launches=192):
    """Dense gated MLP shard (hidden 5120, 2176 intermediate columns): the gated gate/up projection
    (4352 x 5120 packed weights) and the down projection (5120 x 2176), µs per call in graphs that
    rotate `copies` weight sets (about 0.9 GB, beyond the 256 MB MALL)."""
    import torch
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    Kd, Id = S.DENSE_K, S.DENSE_N // 2
    w13 = [G.NVFP4Tensor(*S.device_nvfp4_weights(9000 + c, 1, 2 * Id, Kd)) for c in range(copies)]
    w2 = [G.NVFP4Tensor(*S.device_nvfp4_weights(9500 + c, 1, Kd, Id)) for c in range(copies)]
    b13, b2 = 2 * Id * Kd * 9 // 16, Kd * Id * 9 // 16
    res = []
    for M in (1, 16, 32):
        x = torch.from_numpy(S.activations(S.rng_for(1, 0, 2000 + M), M, Kd)).cuda()
        h = torch.empty((M, Id), dtype=torch.float16, device="cuda")
        y = torch.empty((M, Kd), dtype=torch.float16, device="cuda")
        g_ms = med(time_graph(lambda: [G.nvfp4_linear_swiglu(x, w13[i % copies], h=h) for i in range(launches)],
                              launches))
        d_ms = med(time_graph(lambda: [G.nvfp4_linear(h, w2[i % copies], y=y) for i in range(launches)], launches))
        g_us, d_us = g_ms * 1e3 / launches, d_ms * 1e3 / launches
        # the split-K forms of both projections, one workspace sized for the larger
        wsb = torch.empty(max(G.nvfp4_linear_ws_bytes(M, 2 * Id, Kd), G.nvfp4_linear_ws_bytes(M, Kd, Id), 16),
                          dtype=torch.uint8, device="cuda")
        gs_ms = med(time_graph(lambda: [G.nvfp4_linear_swiglu_ws(x, w13[i % copies], h=h, ws=wsb)
                                        for i in range(launches)], launches))
        ds_ms = med(time_graph(lambda: [G.nvfp4_linear_ws(h, w2[i % copies], y=y, ws=wsb) for i in range(launches)],
                               launches))
        gs_us, ds_us = gs_ms * 1e3 / launches, ds_ms * 1e3 / launches
        res.append({"M": M, "gate_up_swiglu_us": round(g_us, 3), "down_us": round(d_us, 3),
                    "weight_GBps": round((b13 + b2) / ((g_us + d_us) * 1e-6) / 1e9, 1),
                    "split_k_gate_up_swiglu_us": round(gs_us, 3), "split_k_down_us": round(ds_us, 3)})
    return res


def route_timing(launches=256, patterns=8):
    """Router fused with the plan (fp32 logits -> ids, weights, plan) against the plan alone from
    ids, µs per call in graphs of `launches` calls, at 1, 16 and 8192 tokens (512 experts, top-10)."""
    import torch
    import gemm_nvfp4_amd as G
    from synth import inputs as S
    res = []
    for M in (1, 16, 8192):
        xs = [torch.from_numpy(S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 20, 100 * M + p), M, E)).cuda()
              for p in range(patterns)]
        ids = torch.empty((M, TOPK), dtype=torch.int32, device="cuda")
        w = torch.empty((M, TOPK), dtype=torch.float32, device="cuda")
        plan = torch.empty(G.nvfp4_moe_plan_bytes(M, TOPK, E) // 4, dtype=torch.int32, device="cuda")
        n = launches if M <= 16 else 16
        route_ms = med(time_graph(lambda: [G.nvfp4_moe_route(xs[i % patterns], TOPK, ids=ids, weights=w, plan=plan)
                                           for i in range(n)], n))
        id_sets = [G.nvfp4_moe_route(x, TOPK)[0] for x in xs]
        plan_ms = med(time_graph(lambda: [G.nvfp4_moe_plan(id_sets[i % patterns], E, plan=plan) for i in range(n)], n))
        res.append({"M": M, "route_plan_us": round(route_ms * 1e3 / n, 3), "plan_us": round(plan_ms * 1e3 / n, 3)})
    return res


def cpu_baseline(W13, W2, seconds):
    """The fp64 oracle (grouped form) on the headline workload's route patterns, on the host's
    cores, for about `seconds` of CPU work; reported in the same unit (weight GB/s)."""
    from oracle import oracle as O
    from synth import inputs as S
    w13 = tuple(t.cpu().numpy() for t in (W13[0].codes, W13[0].scales, W13[0].global_scale))
    w2 = tuple(t.cpu().numpy() for t in (W2[0].codes, W2[0].scales, W2[0].global_scale))
    threads = O._threads(None)
    done, wbytes, t0 = 0, 0, time.perf_counter()
    while True:
        rng = S.rng_for(S.WORKLOAD_IDS["decode"], 0, 1000 + done)
        case = {"shape": S.DECODE, "x": S.activations(rng, 16, K), "ids": S.routing_uniform(rng, 16, TOPK, E),
                "topk_weights": S.softmax_weights(rng, 16, TOPK), "w13": w13, "w2": w2}
        pl = O.plan(case["ids"], E, 16)
        O.moe_grouped(case, pl, nthreads=threads)
        done += 1
        wbytes += pl["n_active"] * EXPERT_BYTES
        el = time.perf_counter() - t0
        if el >= seconds or done >= 200:
            break
    # The same on one thread, for a few layers.
    done1, wbytes1, t1 = 0, 0, time.perf_counter()
    while True:
        rng = S.rng_for(S.WORKLOAD_IDS["decode"], 0, 1000 + done1)
        case = {"shape": S.DECODE, "x": S.activations(rng, 16, K), "ids": S.routing_uniform(rng, 16, TOPK, E),
                "topk_weights": S.softmax_weights(rng, 16, TOPK), "w13": w13, "w2": w2}
        pl = O.plan(case["ids"], E, 16)
        O.moe_grouped(case, pl, nthreads=1)
        done1 += 1
        wbytes1 += pl["n_active"] * EXPERT_BYTES
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 3 or done1 >= 50:
            break
    model = "unknown"
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(wbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} route patterns of the 16-token decode layer (fp64 grouped oracle, "
                      f"{el:.1f} s wall, {el / done * 1e3:.1f} ms per layer)",
            "one_thread_GBps": round(wbytes1 / el1 / 1e9, 4), "nproc": os.cpu_count(), "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; multi-GPU runs are not supported "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_nvfp4_amd as G
    G.lib()  # raises if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    W13, W2 = weight_sets(args.weight_sets)
    torch.cuda.synchronize()
    log(f"weight sets: {args.weight_sets} x {E * EXPERT_BYTES / 2**20:.0f} MiB")
    if args.counters or args.traffic:
        counters_mode(args.counters or "decode", W13, W2)
        return

    routes16 = Routes(16, args.patterns, 1000)
    head = moe_layer_timing(16, args.steps, args.warmup, W13, W2, routes16, trials=max(20, args.trials))
    log(f"headline M=16: {head}")
    eager = {"M1_us": eager_latency(1, W13, W2, Routes(1, 8, 4000)), "M16_us": eager_latency(16, W13, W2, routes16),
             "one_kernel_us": eager_launch_floor()}
    log(f"eager single-call latency: {eager}")
    k_us, k_bytes = w13_kernel_timing(16, args.steps, W13, routes16)
    achieved = k_bytes / (k_us * 1e-6) / 1e9
    log(f"w13 kernel: {k_us:.3f} us/launch, {k_bytes / 1e6:.2f} MB/launch -> {achieved:.1f} GB/s")
    floor = launch_floor()
    log(f"graph launch floor: {floor:.3f} us")
    copies = copy_ceiling()
    log(f"copy ceiling: {copies}")
    copy_dense, copy_layer = copies[0]["copy_GBps"], copies[1]["copy_GBps"]

    shared = shared_layer_timing(args.steps, W13, W2, routes16)
    log(f"layer with shared expert: {shared}")

    sweep = []
    if not args.no_sweep:
        for M in (1, 2, 4, 8, 16):
            r = moe_layer_timing(M, args.steps, args.warmup, W13, W2, Routes(M, args.patterns, 3000 + 97 * M))
            r["copy_frac"] = round(r["weight_GBps"] / copy_layer, 4)
            log(f"sweep: {r}")
            sweep.append(r)
    stress = None
    if not args.no_stress:
        stress = stress_timing(args.steps, args.warmup, W13, W2, args.patterns)
        log(f"stress: {stress}")
    tiny = tiny_timing(args.steps)
    log(f"tiny layer: {tiny}")
    prefill = None
    if not args.no_prefill:
        prefill = prefill_timing(W13, W2)
        log(f"prefill: {prefill}")
    dense = None
    if not args.no_dense:
        dense = dense_timing()
        for r in dense:
            r["copy_frac"] = round(r["weight_GBps"] / copy_dense, 4)
        log(f"dense: {dense}")
    fp8 = None
    if not args.no_dense:
        fp8 = fp8_timing()
        log(f"dense channel-FP8: {fp8}")
    mlp = None
    if not args.no_mlp:
        mlp = mlp_timing()
        log(f"dense gated MLP: {mlp}")
    route = None
    if not args.no_route:
        route = route_timing()
        log(f"route: {route}")
    cpu = None if args.no_cpu else cpu_baseline(W13, W2, args.cpu_seconds)
    if cpu:
        log(f"cpu baseline: {cpu}")

    ms_step = head["us_per_layer"] / 1e3
    line = {
        "metric": METRIC, "value": head["weight_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "grouped NVFP4 MoE decode layer (plan + W13/SwiGLU + W2/reduce): 16 tokens, "
                               "512 experts, top-10 uniform, K=2048, I=512",
                   "tokens": 16, "experts": E, "topk": TOPK, "hidden": K, "intermediate": I,
                   "weight_sets": args.weight_sets, "route_patterns": args.patterns},
        "value_is": "median of the timed replays of one graph of `steps` layer calls",
        "us_per_layer": head["us_per_layer"], "hbm_frac": head["hbm_frac"],
        "copy_frac": round(head["weight_GBps"] / copy_layer, 4), "trials": head["trials"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": ROOFLINE_KERNEL, "us_per_launch": round(k_us, 3),
                     "algorithmic_bytes_per_launch": round(k_bytes),
                     "copy_frac": round(achieved / copy_layer, 4)},
        "copy_ceiling": copies, "launch_floor_us": round(floor, 3), "eager_layer_latency": eager,
        "sweep": sweep, "stress": stress, "tiny": tiny, "prefill": prefill, "dense": dense, "dense_fp8": fp8,
        "mlp": mlp, "with_shared_expert": shared, "route": route, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
