"""Benchmark of the routed MoE layer on one MI355X.

One step = one pass of the whole layer (router, top-k, permutation + FP8
activations, grouped gate/up GEMM + SwiGLU + FP8 requantisation, grouped down
GEMM, weighted combine) through moe_forward, on one synthetic batch already
resident in HBM.

Prints ONE JSON line:
  value        tokens/s of the whole layer (T tokens per step / wall time per step)
  roofline     the dominant kernel (the gate/up expert GEMM), timed with HIP
               events on the stream it runs on: algorithmic bytes (below the
               625 FLOP/byte ridge point: HBM-bound) or FLOPs (above it:
               MFMA-bound) per launch / mean launch duration, against the
               MI355X peak; traffic = HBM bytes per launch from the counter
               summaries in profiles/ while the GEMM sources are unchanged
  cold_cache_step  per-step HIP-event times of moe_forward with a 1 GiB cache
               flush before each step (median, p10, p90)
  graph_replay the same step captured once as a HIP graph and replayed
  cpu_baseline the CPU oracle on a bounded sample of the same workload
Workloads: tiny, flash_decode (default), flash_prefill, pro_decode,
pro_skewed_prefill, their one-GPU tensor-parallel shares (*_tp4), the
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
    ap.add_argument("--config", default="flash_decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cold-cache per-step timing (1 GiB cache flush before each step)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens for the CPU oracle (0 = auto)")
    ap.add_argument("--canonical-weights", action="store_true",
                    help="run on the canonical (row-major) weight layout instead of the packed one")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch one plain 1 GiB copy kernel (for scaling HBM byte counters)")
    return ap.parse_args()


GEMM_SOURCES = ["sparse_moe_expert_route_amd/csrc/expert_gemm.hip",
                "sparse_moe_expert_route_amd/csrc/expert_gemm_tiled.hip",
                "sparse_moe_expert_route_amd/csrc/moe_internal.h"]
FP8_GEMM_SOURCES = ["sparse_moe_expert_route_amd/csrc/expert_gemm_fp8.hip",
                    "sparse_moe_expert_route_amd/csrc/expert_gemm_fp8_tiled.hip",
                    "sparse_moe_expert_route_amd/csrc/moe_internal.h"]


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

    # ---- whole layer: warmup, then exactly `steps` timed steps ----
    for _ in range(args.warmup):
        moe.forward(p, x, wr, bias, W, y, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        moe.forward(p, x, wr, bias, W, y, ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    tokens_per_s = T * args.steps / wall
    log("bench: %.3f ms/step, %.0f tokens/s" % (ms_per_step, tokens_per_s))

    # ---- per-step times with cold caches: before each step a 1 GiB write evicts the
    # L2s and the 256 MB last-level cache, then HIP events bracket moe_forward alone ----
    flushed = None
    if not args.no_flush:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        times = []
        for _ in range(args.steps):
            scratch.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.forward(p, x, wr, bias, W, y, ws)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        q = np.percentile(np.array(times), [10, 50, 90])
        flushed = {"ms_p10": round(float(q[0]), 4), "ms_median": round(float(q[1]), 4),
                   "ms_p90": round(float(q[2]), 4), "value_median": round(T / (float(q[1]) * 1e-3), 1)}
        log("bench: cold-cache step median %.3f ms (p10 %.3f, p90 %.3f)" % (q[1], q[0], q[2]))

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
    roof["traffic"] = None if args.canonical_weights else \
        measured_traffic(args.config, FP8_GEMM_SOURCES if fp8 else GEMM_SOURCES)
    tiled = N >= 32 * E and H % 512 == 0 and inter % 512 == 0 and max(H, inter) <= (8192 if fp8 else 6144)
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
           "graph_replay": graph,
           "cold_cache_step": flushed,
           "weight_layout": "canonical" if args.canonical_weights else "packed",
           "prepack_ms": None if prepack_ms is None else round(prepack_ms, 3)}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lay, args, T)
    print(json.dumps(out), flush=True)


def cpu_baseline(lay, args, T):
    """The oracle, as it stands, on a bounded sample of tokens of the same workload (single thread)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # pragma: no cover
        threadpool_limits = None
    from oracle import layer as OL
    n = args.cpu_sample_tokens or (32 if T <= 256 else 8)
    n = min(n, T)
    toks = np.arange(n)
    log("bench: CPU oracle on %d tokens" % n)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx:
        with ctx:
            OL.forward_tokens(lay, toks)
    else:
        OL.forward_tokens(lay, toks)
    sec = time.perf_counter() - t0
    return {"value": round(n / sec, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "first %d tokens of the %s workload, whole layer (router, routing, FP8 quantisation, all "
                      "their experts decoded from %s and run in float64, combine); %.1f s"
                      % (n, args.config, "FP8 blocks" if lay.get("format") == "fp8_block" else "MXFP4", sec)}


if __name__ == "__main__":
    main()
