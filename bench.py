"""Benchmark of the routed MoE layer on one MI355X.

One step = one pass of the whole layer (router, top-k, permutation + FP8
activations, grouped gate/up GEMM + SwiGLU + FP8 requantisation, grouped down
GEMM, weighted combine) through moe_forward, on one synthetic batch already
resident in HBM.

Prints ONE JSON line:
  value        tokens/s of the whole layer: T tokens / the median step time, each
               step timed alone with HIP events around moe_forward after a 1 GiB
               read that evicts the L2s and the 256 MB last-level cache (the
               timed loop is exactly `steps` such steps, bracketed by device
               synchronisations); `warm` is the rate of `steps` back-to-back
               steps with no flush
  roofline     the dominant kernel (the gate/up expert GEMM), timed with HIP
               events on the stream it runs on: algorithmic bytes (below the
               625 FLOP/byte ridge point: HBM-bound) or FLOPs (above it:
               MFMA-bound) per launch / mean launch duration, against the
               MI355X peak; traffic = HBM bytes per launch from the counter
               summaries in profiles/ while the GEMM sources are unchanged
  cold_cache_step  the per-step HIP-event times behind `value` (median, p10, p90)
  graph_replay the same step captured once as a HIP graph and replayed
  cpu_baseline the CPU oracle on a bounded sample of the same workload
Workloads: tiny, flash_decode, flash_prefill, pro_decode,
pro_skewed_prefill (default: the largest), their one-GPU tensor-parallel shares (*_tp4), the
speculative-verify blocks flash_verify, pro_verify, and the FP8 block-scaled
expert format (*_fp8: e4m3 weights, float32 128 x 128 block scales) (see
synthetic/__init__.py).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 (the FP8 x FP4 scaled MFMA issues at the FP8 rate)
METRIC = "MoE-layer tokens/s at 1 MI355X; % HBM peak (decode), % MFMA peak (prefill)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="pro_skewed_prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps without the 1 GiB cache flush before each (value = warm rate)")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="how the cache flush touches its 1 GiB: read it (default; leaves no dirty lines whose "
                         "write-back the next step would pay for) or write it")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens for the CPU oracle (0 = auto)")
    ap.add_argument("--canonical-weights", action="store_true",
                    help="run on the canonical (row-major) weight layout instead of the packed one")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch one plain 1 GiB copy kernel (for scaling HBM byte counters)")
    ap.add_argument("--power", action="store_true",
                    help="sample the board power and graphics clock (amd-smi) while the workload's gate/up GEMM, "
                         "down GEMM and whole forward, and the FP4 x FP8 MFMA microbenchmark, each run back to back "
                         "for --power-seconds; print their JSON line")
    ap.add_argument("--power-seconds", type=float, default=5.0)
    ap.add_argument("--micro", action="store_true",
                    help="run the microbenchmarks of the HBM and MFMA ceilings (include/moe_micro.h) instead, "
                         "and print their JSON line")
    return ap.parse_args()


# the sources the gate/up GEMM's HBM traffic depends on: the kernel that runs
# (streaming on decode-sized batches, LDS-tiled on prefill-sized ones), the
# shared headers and, for the tiled kernels, the tile plan
_CSRC = "sparse_moe_expert_route_amd/csrc/"
GEMM_SOURCES = {
    ("mxfp4", "stream"): [_CSRC + "expert_gemm.hip", _CSRC + "moe_internal.h", _CSRC + "moe_launch.h"],
    ("mxfp4", "tiled"): [_CSRC + "expert_gemm_tiled.hip", _CSRC + "moe_internal.h", _CSRC + "moe_launch.h",
                         _CSRC + "permute.hip"],
    ("fp8_block", "stream"): [_CSRC + "expert_gemm_fp8.hip", _CSRC + "moe_internal.h", _CSRC + "moe_launch.h"],
    ("fp8_block", "tiled"): [_CSRC + "expert_gemm_fp8_tiled.hip", _CSRC + "moe_internal.h", _CSRC + "moe_launch.h",
                             _CSRC + "permute.hip"],
}


def measured_traffic(workload, sources):
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3 counter summary
    (profiles/traffic_<workload>.md: FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), or None
    when there is none or the GEMM sources have changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        parts = line.strip().split(": ", 1)
        if len(parts) == 2 and parts[0] in ("gemm1_hbm_bytes_per_launch", "sources_sha256"):
            fields[parts[0]] = parts[1].strip()
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(here, f), "rb").read())
    if fields.get("sources_sha256") != h.hexdigest() or "gemm1_hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["gemm1_hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (one layer's expert set fits one "
              "MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.micro:
        print(json.dumps(micro()), flush=True)
        return
    if args.power:
        print(json.dumps(power(args)), flush=True)
        return
    import numpy as np
    import torch

    import sparse_moe_expert_route_amd as moe
    import synthetic as S

    cfg = S.config(args.config)
    T, H, E, k, inter = cfg["T"], cfg["H"], cfg["E"], cfg["k"], cfg["I"]
    fp8 = cfg["format"] == "fp8_block"
    N = T * k
    log("bench: workload %s T=%d H=%d E=%d k=%d I=%d" % (args.config, T, H, E, k, inter))
    t0 = time.time()
    lay = S.make_layer(args.config, seed=args.seed)
    log("bench: generated inputs in %.1f s" % (time.time() - t0))

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wr = dev(lay["x"]), dev(lay["w_router"])
    bias = None if lay["bias"] is None else dev(lay["bias"])
    W = moe.ExpertWeights(dev(lay["w13"]), dev(lay["w13_s"]), dev(lay["w2"]), dev(lay["w2_s"]))
    p = moe.Problem.make(T, H, inter, E, k, 0, moe.EXPERTS_FP8_BLOCK if fp8 else moe.EXPERTS_MXFP4)
    prepack_ms = None
    if not args.canonical_weights:
        # one-time reordering of the expert code bytes at load time (untimed; reported)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        Wp = moe.prepack_weights(p, W)
        e1.record()
        torch.cuda.synchronize()
        prepack_ms = e0.elapsed_time(e1)
        del W
        W = Wp
        log("bench: prepacked expert weights in %.2f ms" % prepack_ms)
    ws = moe.alloc_workspace(p)
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    if args.calibrate_copy:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # ---- whole layer, warm: warmup, then `steps` back-to-back steps ----
    for _ in range(args.warmup):
        moe.forward(p, x, wr, bias, W, y, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        moe.forward(p, x, wr, bias, W, y, ws)
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - t0
    warm = {"ms_per_step": round(warm_wall / args.steps * 1e3, 4), "value": round(T * args.steps / warm_wall, 1)}
    log("bench: warm %.3f ms/step, %.0f tokens/s" % (warm["ms_per_step"], warm["value"]))

    # ---- the timed loop: exactly `steps` steps with cold caches.  Before each step a
    # 1 GiB read evicts the L2s and the 256 MB last-level cache (a write would leave dirty
    # lines there whose write-back lands in the next step), then HIP events on the
    # launching stream bracket moe_forward alone; value = T / median step time ----
    flushed = None
    scratch = None if args.no_flush else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if scratch is not None:
            if args.flush == "read":
                torch.sum(scratch, dtype=torch.float32)
            else:
                scratch.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        moe.forward(p, x, wr, bias, W, y, ws)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    loop_wall = time.perf_counter() - t0
    del scratch
    q = np.percentile(np.array(times), [10, 50, 90])
    ms_per_step = float(q[1])
    tokens_per_s = T / (ms_per_step * 1e-3)
    flushed = {"ms_p10": round(float(q[0]), 4), "ms_median": round(float(q[1]), 4), "ms_p90": round(float(q[2]), 4),
               "flush": None if args.no_flush else "%s 1 GiB" % args.flush,
               "loop_wall_ms_per_step": round(loop_wall / args.steps * 1e3, 4)}
    log("bench: %s step median %.3f ms (p10 %.3f, p90 %.3f), %.0f tokens/s"
        % ("cold-cache" if not args.no_flush else "event-timed", q[1], q[0], q[2], tokens_per_s))

    # ---- the same step captured once as a HIP graph and replayed (no launch overhead) ----
    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            moe.forward(p, x, wr, bias, W, y, ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            moe.forward(p, x, wr, bias, W, y, ws)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        graph = {"ms_per_step": round(gwall / args.steps * 1e3, 4), "value": round(T * args.steps / gwall, 1)}
        log("bench: graph replay %.3f ms/step" % graph["ms_per_step"])
        del g

    # ---- dominant kernel: gate/up expert GEMM, timed with HIP events on its stream ----
    logits = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(N, dtype=torch.int32, device="cuda")
    ros = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(N, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(N, H // 128, dtype=moe.scale_dtype(p), device="cuda")
    hq = torch.empty(N, inter, dtype=torch.uint8, device="cuda")
    hs = torch.empty(N, inter // 128, dtype=moe.scale_dtype(p), device="cuda")
    moe.route(p, x, wr, bias, logits, ids, w)
    moe.permute(p, ids, x, off, st, ros, xq, xs, ws)
    torch.cuda.synchronize()
    counts = np.diff(off.cpu().numpy())
    touched = int(np.count_nonzero(counts))
    # one event pair around the K back-to-back launches on the kernel's stream:
    # an event pair around every launch adds its own gap (about 10 us on a
    # 0.36 ms decode launch) that the kernel trace does not show
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    gemm1_ms = e0.elapsed_time(e1) / args.steps

    if fp8:
        # e4m3 codes + one float32 per 128 x 128 block; activation and h scales float32
        w13_bytes_per_expert = 2 * inter * H + (2 * inter // 128) * (H // 128) * 4
        gemm1_bytes = touched * w13_bytes_per_expert + N * (H + 4 * H // 128) + N * (inter + 4 * inter // 128)
    else:
        w13_bytes_per_expert = 2 * inter * (H // 2 + H // 32)
        gemm1_bytes = touched * w13_bytes_per_expert + N * (H + H // 128) + N * (inter + inter // 128)
    gemm1_flops = 2.0 * N * 2 * inter * H
    # the kernel's bound: below the ridge point (peak FLOP/s over peak bytes/s, 625 FLOP/byte)
    # the weight and activation bytes take longer than the MFMA work
    ridge = MFMA_FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gemm1_flops / gemm1_bytes < ridge:
        achieved = gemm1_bytes / (gemm1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = gemm1_flops / (gemm1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None}
    tiled = N >= 32 * E and H % 512 == 0 and inter % 512 == 0 and max(H, inter) <= (8192 if fp8 else 6144)
    roof["traffic"] = None if args.canonical_weights else \
        measured_traffic(args.config, GEMM_SOURCES[("fp8_block" if fp8 else "mxfp4", "tiled" if tiled else "stream")])
    roof["kernel"] = "expert_gemm_%s%s_kernel<gate/up + SwiGLU + FP8 requant>" % ("fp8_" if fp8 else "",
                                                                                   "tiled" if tiled else "stream")
    roof["launch_ms"] = round(gemm1_ms, 4)
    roof["algorithmic_bytes"] = int(gemm1_bytes)
    roof["algorithmic_flops"] = gemm1_flops

    # whole-layer work per step (touched experts' weights + router + x + y; FLOPs of both expert GEMMs)
    expert_bytes = 3 * H * inter + 3 * (H // 128) * (inter // 128) * 4 if fp8 else 3 * H * inter * 17 // 32
    layer_bytes = touched * expert_bytes + E * H * 2 + T * H * 2 + T * H * 4
    layer_flops = 2.0 * N * 3 * inter * H
    step_s = ms_per_step * 1e-3
    layer = {"bytes": int(layer_bytes), "flops": layer_flops, "experts_touched": touched,
             "GB/s": round(layer_bytes / step_s / 1e9, 1), "TFLOP/s": round(layer_flops / step_s / 1e12, 1),
             "hbm_frac": round(layer_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac": round(layer_flops / step_s / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4)}

    out = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8e4m3 x fp8e4m3 block-scaled (fp32 acc)" if fp8 else "fp8e4m3 x mxfp4 (fp32 acc)",
           "data": "synthetic (seeded; N(0,1) bf16 activations, 0.02*N(0,1) bf16 router and %s experts)"
                   % ("FP8 block-scaled" if fp8 else "MXFP4"),
           "config": {"workload": args.config, "T": T, "H": H, "E": E, "k": k, "I": inter, "seed": args.seed,
                      "bias": cfg["bias"], "experts": cfg["format"]},
           "roofline": roof, "layer": layer,
           "warm": warm,
           "graph_replay": graph,
           "cold_cache_step": flushed,
           "weight_layout": "canonical" if args.canonical_weights else "packed",
           "prepack_ms": None if prepack_ms is None else round(prepack_ms, 3)}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lay, args, T)
    print(json.dumps(out), flush=True)


def _smi_sample():
    """(socket power W, mean graphics clock MHz over the XCDs) from amd-smi, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=5)
        d = json.loads(r.stdout)["gpu_data"][0]
        clk = [v["clk"]["value"] for k_, v in d["clock"].items() if k_.startswith("gfx")]
        return float(d["power"]["socket_power"]["value"]), float(sum(clk) / len(clk))
    except Exception:
        return None


def power(args):
    """Board power and graphics clock while each of the workload's GEMMs, its whole forward and
    the FP4 x FP8 MFMA microbenchmark (register operands, no memory traffic) run back to back:
    a sampling thread polls amd-smi about every 0.1 s; each phase reports the medians of the
    samples taken inside it (its first 0.5 s left out) and its time per call."""
    import ctypes
    import threading
    import numpy as np
    import torch
    import sparse_moe_expert_route_amd as moe
    from sparse_moe_expert_route_amd import build as B
    import synthetic as S

    if _smi_sample() is None:
        raise RuntimeError("amd-smi is not available")
    cfg = S.config(args.config)
    T, H, E, k, inter = cfg["T"], cfg["H"], cfg["E"], cfg["k"], cfg["I"]
    fp8 = cfg["format"] == "fp8_block"
    N = T * k
    lay = S.make_layer(args.config, seed=args.seed)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wr = dev(lay["x"]), dev(lay["w_router"])
    bias = None if lay["bias"] is None else dev(lay["bias"])
    p = moe.Problem.make(T, H, inter, E, k, 0, moe.EXPERTS_FP8_BLOCK if fp8 else moe.EXPERTS_MXFP4)
    W = moe.prepack_weights(p, moe.ExpertWeights(dev(lay["w13"]), dev(lay["w13_s"]), dev(lay["w2"]), dev(lay["w2_s"])))
    del lay
    ws = moe.alloc_workspace(p)
    sd = moe.scale_dtype(p)
    L = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(N, dtype=torch.int32, device="cuda")
    ros = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(N, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(N, H // 128, dtype=sd, device="cuda")
    hq = torch.empty(N, inter, dtype=torch.uint8, device="cuda")
    hs = torch.empty(N, inter // 128, dtype=sd, device="cuda")
    yp = torch.empty(N, H, device="cuda")
    y = torch.empty(T, H, device="cuda")
    moe.route(p, x, wr, bias, L, ids, w)
    moe.permute(p, ids, x, off, st, ros, xq, xs, ws)
    moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)
    torch.cuda.synchronize()

    micro_lib = ctypes.CDLL(B.MICRO_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    micro_lib.moe_micro_mfma.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fo = torch.empty(cus * 2 * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    sp = vp(torch.cuda.current_stream().cuda_stream)

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            s_ = _smi_sample()
            if s_ is not None:
                samples.append((time.time(),) + s_)
            time.sleep(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(1.0)
    idle = [s_ for s_ in samples]
    phases = [
        ("gemm1_swiglu", lambda: moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)),
        ("gemm2", lambda: moe.grouped_gemm2(p, hq, hs, off, W, yp, ws)),
        ("forward", lambda: moe.forward(p, x, wr, bias, W, y, ws)),
        ("mfma_microbenchmark_32x32x64_fp4xfp8",
         lambda: micro_lib.moe_micro_mfma(4, 0, 32, 4096, cus * 2, vp(fo.data_ptr()), vp(clk.data_ptr()), sp)),
    ]
    out = {"workload": args.config, "idle_W": round(float(np.median([s_[1] for s_ in idle])), 1) if idle else None,
           "phases": {}}
    for name, fn in phases:
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        while time.time() - t0 < args.power_seconds:
            for _ in range(4):
                fn()
                n += 1
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        inside = [s_ for s_ in samples if t0 + 0.5 < s_[0] < t1]
        out["phases"][name] = {
            "ms_per_call": round(e0.elapsed_time(e1) / n, 4),
            "samples": len(inside),
            "power_W_median": round(float(np.median([s_[1] for s_ in inside])), 1) if inside else None,
            "gfx_clock_MHz_median": round(float(np.median([s_[2] for s_ in inside])), 1) if inside else None,
        }
        log("power: %s %s" % (name, out["phases"][name]))
        time.sleep(1.0)
    stop.set()
    th.join(timeout=10)
    return {"power": out}


def micro():
    """The ceilings the layer is measured against, on this GPU: HBM stream bandwidth (16-byte
    reads over 4 GiB, two access patterns, a sweep of grid sizes; 16-byte writes) and the
    block-scaled MFMA issue rate with the shader clock it ran at (libmoe_micro.so)."""
    import ctypes
    import numpy as np
    import torch
    from sparse_moe_expert_route_amd import build as B
    if not os.path.exists(B.MICRO_LIB):
        raise RuntimeError("libmoe_micro.so is not built: run python -m sparse_moe_expert_route_amd.build")
    L = ctypes.CDLL(B.MICRO_LIB)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.moe_micro_hbm_read.argtypes = [vp, sz, vp, i32, i32, vp]
    L.moe_micro_hbm_write.argtypes = [vp, sz, i32, vp]
    L.moe_micro_mfma.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp]
    stream = torch.cuda.current_stream()
    sp = vp(stream.cuda_stream)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    out = {"device": torch.cuda.get_device_name(0), "cus": torch.cuda.get_device_properties(0).multi_processor_count}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(16384 * 256, dtype=torch.int32, device="cuda")
    hbm = {}
    for pattern, name in ((0, "read_grid_stride"), (1, "read_chunk_per_workgroup"),
                          (2, "read_grid_stride_nontemporal"), (3, "read_chunk_per_workgroup_nontemporal")):
        res = {}
        for grid in (1024, 2048, 4096, 8192, 16384):
            def run(g=grid, pt=pattern):
                assert L.moe_micro_hbm_read(vp(buf.data_ptr()), nbytes, vp(sink.data_ptr()), g, pt, sp) == 0
            res[grid] = round(nbytes / timed(run) / 1e9, 1)
        hbm[name] = {"GB/s by grid": res, "best GB/s": max(res.values())}
        log("micro: %s %s" % (name, res))
    # the packed-weight read pattern of the streaming GEMMs: 16 groups of one
    # 16-row weight group each per workgroup (group bytes 16 K/2: 16 KiB for
    # K = 2048, 32 KiB for 4096, 48 KiB for 6144), groups back to back or
    # spaced by one extra KiB, waves walking the stages in step or staggered
    L.moe_micro_hbm_read_groups.argtypes = [vp, sz, sz, sz, i32, vp, i32, vp]
    gb = 2 << 30
    groups = {}
    for gk in (16, 32, 48):
        for pad in (0, 1):
            for skew in (0, 1, 2):
                for nt in (0, 1):
                    def rung(g=gk << 10, st=(gk + pad) << 10, sk=skew, n=nt):
                        assert L.moe_micro_hbm_read_groups(vp(buf.data_ptr()), gb, g, st, sk, vp(sink.data_ptr()),
                                                           n, sp) == 0
                    nreg = gb // (16 * ((gk + pad) << 10))
                    key = "group %d KiB%s, skew %d, %s" % (gk, " +1 KiB" if pad else "", skew,
                                                         "non-temporal" if nt else "cached")
                    groups[key] = round(nreg * 16 * (gk << 10) / timed(rung) / 1e9, 1)
                    log("micro: read_gemm_groups %s: %s GB/s" % (key, groups[key]))
    hbm["read_gemm_groups"] = groups
    res = {}
    for grid in (2048, 8192):
        def runw(g=grid):
            assert L.moe_micro_hbm_write(vp(buf.data_ptr()), nbytes, g, sp) == 0
        res[grid] = round(nbytes / timed(runw) / 1e9, 1)
    hbm["write_grid_stride"] = {"GB/s by grid": res, "best GB/s": max(res.values())}
    log("micro: write %s" % res)
    hbm["bytes"] = nbytes
    out["hbm"] = hbm
    del buf
    cus = out["cus"]
    mf = {}
    fo = torch.empty(cus * 2 * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    for shape, per in ((32, 8 * 2 * 32 * 32 * 64), (16, 16 * 2 * 16 * 16 * 128)):
        for fa, fb, fname in ((4, 0, "fp4 x fp8"), (0, 0, "fp8 x fp8"), (4, 4, "fp4 x fp4")):
            for wg_per_cu in (1, 2):
                grid, iters = cus * wg_per_cu, 4096
                def runm(g=grid, it=iters, a=fa, b=fb, sh=shape):
                    assert L.moe_micro_mfma(a, b, sh, it, g, vp(fo.data_ptr()), vp(clk.data_ptr()), sp) == 0
                t = timed(runm, reps=3)
                c = clk.cpu().tolist()
                ghz = c[0] / (c[1] / 100e6) / 1e9 if c[1] else None
                flops = grid * 4 * iters * per
                key = "%dx%dx%d %s, %d wave%s per SIMD" % (shape, shape, 64 if shape == 32 else 128, fname, wg_per_cu,
                                                          "s" if wg_per_cu > 1 else "")
                mf[key] = {"TFLOP/s": round(flops / t / 1e12, 1), "shader_clock_GHz": round(ghz, 3) if ghz else None}
                log("micro: %s %s" % (key, mf[key]))
    out["mfma"] = mf
    return {"micro": out}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(lay, args, T):
    """The oracle, as it stands, on a bounded sample of tokens of the same workload, with
    BLAS on every core this process may run on."""
    import numpy as np
    from oracle import layer as OL
    cores = len(os.sched_getaffinity(0))
    n = args.cpu_sample_tokens or 8
    n = min(n, T)
    toks = np.arange(n)
    blas = {"vendor": None, "threads": None}
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:   # pragma: no cover
        threadpool_info = threadpool_limits = None
    log("bench: CPU oracle on %d tokens, %d cores" % (n, cores))
    # time split: the oracle's expert-weight decoding, its per-expert work (the
    # decoding, both GEMMs, SwiGLU and the FP8 requantisation of h) and the rest
    # (router logits, top-k, FP8 quantisation of x, combine), by timing wrappers
    # around two of its functions for the length of this call (its arithmetic
    # is untouched)
    spent = {"decode": 0.0, "experts": 0.0}
    orig = {"decode_expert_matrix": OL.decode_expert_matrix, "expert_ffn": OL.expert_ffn}

    def timed(name, key):
        f = orig[name]

        def g(*a, **kw):
            t = time.perf_counter()
            try:
                return f(*a, **kw)
            finally:
                spent[key] += time.perf_counter() - t
        return g

    OL.decode_expert_matrix = timed("decode_expert_matrix", "decode")
    OL.expert_ffn = timed("expert_ffn", "experts")
    try:
        t0 = time.perf_counter()
        if threadpool_limits:
            with threadpool_limits(limits=cores, user_api="blas"):
                info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
                if info:
                    blas = {"vendor": "%s %s" % (info[0].get("internal_api"), info[0].get("version")),
                            "threads": info[0].get("num_threads")}
                OL.forward_tokens(lay, toks)
        else:
            OL.forward_tokens(lay, toks)
        sec = time.perf_counter() - t0
    finally:
        OL.decode_expert_matrix = orig["decode_expert_matrix"]
        OL.expert_ffn = orig["expert_ffn"]
    split = {"expert_decode": round(spent["decode"], 3),
             "expert_gemms_swiglu_requant": round(spent["experts"] - spent["decode"], 3),
             "rest": round(sec - spent["experts"], 3)}
    return {"value": round(n / sec, 4), "unit": "tokens/s", "cores": blas["threads"] or cores, "kind": "oracle",
            "cpu": _cpu_model(), "blas": blas["vendor"], "affinity_cores": cores, "split_s": split,
            "sample": "first %d tokens of the %s workload, whole layer (router, routing, FP8 quantisation, all "
                      "their experts decoded from %s and run in float64 with BLAS on %s threads, combine); %.1f s"
                      % (n, args.config, "FP8 blocks" if lay.get("format") == "fp8_block" else "MXFP4",
                         blas["threads"] or cores, sec)}


if __name__ == "__main__":
    main()
