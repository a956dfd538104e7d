#!/usr/bin/env python3
"""Benchmark of the quantized GEMV / GEMM hot path on one MI355X.

Headline workload: the Qwen3-0.6B-shaped Q4 decode projection set (28 layers
x {q, k, v, o, gate, up, down} + the 151936 x 1024 LM head, group 64, M = 1,
597 M weights, 337.8 MB of compressed weights), synthetic seeded inputs
resident in HBM.  One step = every GEMV of the set once, issued as one
batched launch (each GEMV with its own lane layout for its K).  The headline value is the
set's algorithmic bytes (compressed weights + fp16 x + fp32 y) per second.

Also measured (outside the timed region, reported in the same JSON line):
  * the roofline of the dominant kernel (that batched launch, the only
    kernel of a step): its average launch duration is the timed region's
    HIP-event time over K;
  * the same set as 197 separate qmm_gemv launches replayed from a HIP graph;
  * the set in decode dependency order (per layer: q|k|v, o, gate|up, down;
    then the LM head) replayed from a HIP graph: per-token projection time,
    also as a fused decode step (q|k|v stored as one matrix, o and down
    adding the residual, gate/up as one SiLU-gated launch);
  * the LM head alone with four rotating copies (steady state);
  * the single 3072 x 1024 Q4 GEMV;
  * the Llama-3.2-3B-shaped bit-width sweep (Q2/Q3/Q4/Q5/Q6/Q8 and fp16
    weights);
  * Llama-3.2-1B-shaped prefill GEMMs at M = 128 and 512: TFLOP/s, % MFMA,
    with Q4 weights and again with fp16 weights, and at M = 2048 with fp32
    and fp16 output, the dense fp16 library matmul of each shape beside them,
    and the layer with q|k|v and gate|up as grouped GEMMs;
  * the fused gate/up projection (silu(Wg x) * (Wu x), one launch) against
    two GEMV launches, Q4, on Qwen3-0.6B and Llama-3.2-3B shapes;
  * Qwen3-30B-A3B-shaped MoE expert projections at 1 and 16 tokens, also with
    gate and up fused with the SiLU-gated product;
  * the CPU oracle on the host cores over the same projection set;
  * measured ceilings (a plain streaming read and an fp16 MFMA loop built
    here), reported beside the spec peaks as second denominators.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick | --decode-graphs]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense fp16 flop/clk/CU
METRIC = "Q4 dequant-GEMV HBM GB/s (% of peak); prefill qGEMM TFLOP/s (% MFMA)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_batched_q4_qwen3_decode_set.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# The sources the batched GEMV kernel is compiled and launched from (its
# device code, shared device helpers, the launch plumbing and the host plan).
TRAFFIC_SOURCES = ("gemv_bits.hip", "gemv_kernels.h", "qmm_api.hip", "qmm_device.h", "qmm_kernels.h")


def kernel_source_digest() -> str:
    """sha256 over the batched GEMV's sources; ties stored counter readings to
    a build of that kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_qmm_gemv_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when missing or taken on different kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha256") != kernel_source_digest():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Timer:
    """Average milliseconds per call of fn(), measured on the GPU side.

    `reps` calls are captured into one HIP graph (a caller that rotates
    through several input copies bakes that rotation into the graph), the
    graph is replayed `replays` times between two events, and the elapsed
    time is divided by the number of calls.  Replaying a graph keeps the host
    out of the measurement: each call costs its kernels plus the dispatch gap
    between graph nodes, which is what a captured decode or prefill step pays.
    """

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps=20, warmup=3, replays=5, settle_ms=20.0):
        t = self.torch
        for _ in range(warmup):
            fn()
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            for _ in range(reps):
                fn()
        # Untimed replays for at least settle_ms, so that the timed ones run
        # at steady-state clocks (inputs are generated on the host between
        # measurements, and the GPU idles meanwhile).
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        t.cuda.synchronize()
        once = max(a.elapsed_time(b), 1e-3)
        for _ in range(min(200, int(settle_ms / once) + 1)):
            g.replay()
        t.cuda.synchronize()
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / (replays * reps)

    def replay(self, g, replays=20, settle_ms=20.0):
        """Average milliseconds per replay of an already captured graph
        (after untimed replays for at least settle_ms, as in __call__)."""
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        t.cuda.synchronize()
        once = max(a.elapsed_time(b), 1e-3)
        for _ in range(min(200, int(settle_ms / once) + 1)):
            g.replay()
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / replays


# Working sets of at least this many bytes per timing loop keep every HBM
# rate honest: twice the 256 MB last-level cache, so no replay finds its
# weights still cached from the previous one.
CACHE_BUST_BYTES = 540 * 2**20


def copies_for(nbytes: int, cap: int = 4096) -> int:
    """Device copies of an nbytes working set that together exceed CACHE_BUST_BYTES."""
    return max(2, min(cap, -(-CACHE_BUST_BYTES // max(nbytes, 1))))


def device_copies(dq: dict, count: int) -> list:
    """dq plus count - 1 device-side clones of its weight, scale and min tensors."""
    clone = lambda t: None if t is None else t.clone()
    return [dq] + [{**dq, "w": dq["w"].clone(), "scales": clone(dq["scales"]), "mins": clone(dq["mins"])}
                   for _ in range(count - 1)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: about 0.1 s of warm-up launches (identical to the timed ones)
    # so the GPU runs at its steady-state clocks, then 1000 timed launches.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiler runs)")
    ap.add_argument("--decode-graphs", action="store_true",
                    help="headline plus the decode-order graphs only (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter scale reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here "
              "(the projections would shard by output rows, with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import configs, inputs, tensors

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # A plain copy of known size: hardware byte counters read against it
        # give the factor that turns their readings into bytes.
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel(), "launches": 3}))
        return
    qmm.load()
    timer = Timer(torch)
    G = configs.GROUP

    # ---- headline workload: the decode projection set --------------------------
    t0 = time.time()
    mats, xs, ys = [], [], []
    for layer, j, name, n, k in configs.decode_set():
        key = (configs.CFG_DECODE_SET, layer, j, 4)
        q = inputs.quantized_matrix(n, k, 4, G, key=key)
        dq = tensors.upload_matrix(q)
        x = tensors.device_tensor(inputs.activation_rows(1, k, key=key)[0])
        mats.append((layer, name, dq))
        xs.append(x)
        ys.append(torch.empty(n, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    log("decode set generated and uploaded in %.1f s" % (time.time() - t0))
    set_bytes = sum(configs.gemv_bytes(dq["n"], dq["k"], 4) for _, _, dq in mats)
    set_weight_bytes = sum(configs.weight_bytes(dq["n"], dq["k"], 4) for _, _, dq in mats)

    # The whole set is one batched launch: every GEMV gets its own lane layout
    # (by its K) inside the same kernel.
    batch = tensors.GemvBatch(list(zip([d for _, _, d in mats], xs, ys)), 4, G)
    total_rows = sum(d["n"] for _, _, d in mats)
    plan = qmm.qmm_get_plan(3, 1, total_rows, max(d["k"] for _, _, d in mats), 4, G)
    st = torch.cuda.current_stream().cuda_stream

    for _ in range(args.warmup):
        batch(stream=st)
    torch.cuda.synchronize()
    # Timed region: K steps back to back, bracketed by events and syncs.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        batch(stream=st)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps
    value = set_bytes / (ms_per_step * 1e-3) / 1e9
    # The step is one launch of the dominant kernel, so its average launch
    # duration is the timed region's event time over K (it includes the
    # inter-launch gap of about a microsecond, so it slightly understates the
    # kernel's own rate as a profiler's kernel trace reports it).
    dom_ms = ms_per_step
    dom_bytes = set_bytes
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    log("step %.3f us (wall %.3f us), %.1f GB/s; batched launch %.3f us, %.1f GB/s"
        % (ms_per_step * 1e3, wall / args.steps * 1e6, value, dom_ms * 1e3, dom_gbs))

    traffic = stored_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4 weights, fp16 x, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "qwen3_0.6b_q4_decode_projection_set",
            "gemvs": len(mats), "layers": configs.QWEN3_06B_LAYERS, "hidden": 1024,
            "lm_head": "151936x1024", "bits": 4, "group": G, "m": 1,
            "weight_bytes": set_weight_bytes, "algorithmic_bytes_per_step": set_bytes,
            "launches_per_step": 1, "parallelism": "none (1 GPU)",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": "gemv_batched_kernel<4,%d,%d,%d> (one launch, 197 GEMVs)" % (
                plan["unit_codes"], plan["units_per_lane"], plan["rows_per_iter"]),
            "bound": "hbm",
            "achieved": round(dom_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_ms * 1e3, 3),
        },
    }

    if args.decode_graphs:
        result["extras"] = extras(torch, np, qmm, configs, inputs, tensors, timer, mats, xs, ys, set_bytes,
                                  decode_graphs_only=True)
    elif not args.quick:
        ceil = measured_ceilings(torch, set_bytes)
        result["measured_ceilings"] = ceil
        result["roofline"]["measured_peak"] = ceil["hbm_read_GBps"]
        result["roofline"]["frac_of_measured"] = round(dom_gbs / ceil["hbm_read_GBps"], 4)
        result["extras"] = extras(torch, np, qmm, configs, inputs, tensors, timer, mats, xs, ys,
                                  set_bytes)
        for key, per_m in result["extras"].items():
            if key.startswith("prefill_"):
                for row in per_m.values():
                    row["pct_of_measured_mfma"] = round(100 * row["TFLOPs"] / ceil["mfma_f16_TFLOPs"], 2)
                    if "grouped" in row:
                        row["grouped"]["pct_of_measured_mfma"] = round(
                            100 * row["grouped"]["TFLOPs"] / ceil["mfma_f16_TFLOPs"], 2)
    if not args.no_cpu_baseline and not args.quick and not args.decode_graphs:
        result["cpu_baseline"] = cpu_baseline(np, configs, inputs, set_bytes)
    print(json.dumps(result), flush=True)


def measured_ceilings(torch, set_bytes):
    """Second denominators, measured here: a plain streaming read of a buffer
    of the decode set's size (larger than the last-level cache) and of 2 GiB,
    and a loop of independent fp16 32x32x16 MFMAs on every SIMD.  Each is the
    best of a few launch shapes (work-groups per CU), after warm-up."""
    import ctypes
    from gemm_qmm_gemv_amd import build as qbuild
    if not os.path.exists(qbuild.CEILING_LIB):
        raise RuntimeError("%s is missing: run gemm_qmm_gemv_amd.build first" % qbuild.CEILING_LIB)
    lib = ctypes.CDLL(qbuild.CEILING_LIB)
    p, u64, ci = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
    lib.qmm_ceiling_read.argtypes = [p, u64, ci, p, p]
    lib.qmm_ceiling_mfma.argtypes = [ci, ci, p, p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")

    def best_ms(calls, reps):
        best = float("inf")
        for fn in calls:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) / reps)
        return best

    out = {}
    for label, nbytes in (("hbm_read_GBps", set_bytes // 16 * 16), ("hbm_read_2GiB_GBps", 2 << 30)):
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")  # XOR-folds to 0: sink untouched
        calls = [lambda blocks=cus * mult: lib.qmm_ceiling_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), st)
                 for mult in (1, 2, 4, 8, 32)]
        ms = best_ms(calls, 20)
        out[label] = round(nbytes / ms / 1e6, 1)
        del buf, calls
    iters = 4000
    tf = 0.0
    for mult in (2, 8):
        blocks = cus * mult  # four waves each, 4 * iters MFMAs of 32768 flops per wave
        ms = best_ms([lambda: lib.qmm_ceiling_mfma(blocks, iters, sink.data_ptr(), st)], 5)
        tf = max(tf, blocks * 4 * iters * 4 * 32768.0 / ms / 1e9)
    out["mfma_f16_TFLOPs"] = round(tf, 1)
    out["read_buffer_bytes"] = set_bytes // 16 * 16
    log("measured ceilings: read %.0f GB/s (set-sized), %.0f GB/s (2 GiB); fp16 MFMA %.0f TFLOP/s"
        % (out["hbm_read_GBps"], out["hbm_read_2GiB_GBps"], out["mfma_f16_TFLOPs"]))
    return out


def extras(torch, np, qmm, configs, inputs, tensors, timer, mats, xs, ys, set_bytes, decode_graphs_only=False):
    G = configs.GROUP
    out = {}

    # 197 separate launches, replayed from a HIP graph.
    def per_call():
        for (layer, name, dq), x, y in zip(mats, xs, ys):
            tensors.gemv(dq, x, y)
    per_call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        per_call()
    ms = timer.replay(g)
    out["decode_set_per_call_graph"] = {"us": round(ms * 1e3, 2),
                                        "GBps": round(set_bytes / ms / 1e6, 1)}
    log("per-call graph: %.1f us" % (ms * 1e3))

    # Decode dependency order: per layer q|k|v, o, gate|up, down; then LM head.
    stage_batches = []
    per_layer = len(configs.QWEN3_06B_PROJ)
    for layer in range(configs.QWEN3_06B_LAYERS):
        base = layer * per_layer
        item = lambda i: (mats[base + i][2], xs[base + i], ys[base + i])
        for group_ in ((0, 1, 2), (3,), (4, 5), (6,)):
            stage_batches.append(tensors.GemvBatch([item(i) for i in group_], 4, G))
    lm = (mats[-1][2], xs[-1], ys[-1])

    def dependent():
        for b in stage_batches:
            b()
        tensors.gemv(lm[0], lm[1], lm[2])
    dependent()
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        dependent()
    ms = timer.replay(g2)
    out["decode_dependent_stages_graph"] = {
        "launches": len(stage_batches) + 1, "per_token_us": round(ms * 1e3, 2),
        "GBps": round(set_bytes / ms / 1e6, 1), "projection_tok_per_s": round(1e3 / ms, 1)}
    log("dependent-stage graph: %.1f us" % (ms * 1e3))

    # The same decode step with its epilogues fused as a decoder layer runs
    # them: q|k|v as one GEMV over the three matrices stored as one [q; k; v]
    # matrix (they share x; the same bytes, one plain launch), o with the
    # residual add (y = r + W x), gate/up as one SiLU-gated launch, down with
    # the residual add; then the LM head.
    qkv_mats = []
    for layer in range(configs.QWEN3_06B_LAYERS):
        base = layer * per_layer
        parts = [mats[base + i][2] for i in (0, 1, 2)]
        qkv_mats.append(dict(parts[0], n=sum(p["n"] for p in parts),
                             w=torch.cat([p["w"] for p in parts]), scales=torch.cat([p["scales"] for p in parts]),
                             mins=torch.cat([p["mins"] for p in parts])))
    qkv_out = torch.empty(qkv_mats[0]["n"], dtype=torch.float32, device="cuda")
    resid = torch.zeros(configs.QWEN3_06B_PROJ[3][1], dtype=torch.float32, device="cuda")
    hbuf = torch.empty(configs.QWEN3_06B_PROJ[4][1], dtype=torch.float32, device="cuda")

    def dependent_fused():
        for layer in range(configs.QWEN3_06B_LAYERS):
            base = layer * per_layer
            tensors.gemv(qkv_mats[layer], xs[base], qkv_out)
            tensors.gemv_residual(mats[base + 3][2], xs[base + 3], resid, resid)
            tensors.gemv_swiglu(mats[base + 4][2], mats[base + 5][2], xs[base + 4], hbuf)
            tensors.gemv_residual(mats[base + 6][2], xs[base + 6], resid, resid)
        tensors.gemv(lm[0], lm[1], lm[2])
    dependent_fused()
    torch.cuda.synchronize()
    g3 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g3):
        dependent_fused()
    ms = timer.replay(g3)
    out["decode_dependent_fused_graph"] = {
        "launches": 4 * configs.QWEN3_06B_LAYERS + 1, "per_token_us": round(ms * 1e3, 2),
        "GBps": round(set_bytes / ms / 1e6, 1), "projection_tok_per_s": round(1e3 / ms, 1),
        "epilogues": "q|k|v one [q;k;v] matrix, o and down add the residual, gate/up write silu(g)*u"}
    log("dependent fused graph: %.1f us" % (ms * 1e3))
    if decode_graphs_only:
        return out

    # LM head alone, rotating device copies (CACHE_BUST_BYTES in all).
    name, n, k = configs.QWEN3_06B_LM_HEAD
    b = configs.gemv_bytes(n, k, 4)
    copies = device_copies(mats[-1][2], copies_for(b))
    yl = torch.empty(n, dtype=torch.float32, device="cuda")
    idx = [0]

    def lm_call():
        tensors.gemv(copies[idx[0] % len(copies)], xs[-1], yl)
        idx[0] += 1
    ms = timer(lm_call, reps=len(copies) * 4)
    out["lm_head_151936x1024_q4"] = {"us": round(ms * 1e3, 2), "GBps": round(b / ms / 1e6, 1),
                                     "pct_peak": round(100 * b / ms / 1e6 / HBM_PEAK_GBS, 1),
                                     "copies": len(copies)}
    del copies
    log("lm head: %.1f us" % (ms * 1e3))

    # Single 3072 x 1024 Q4 GEMV, rotating device copies.
    c = configs.SINGLE_Q4
    q = inputs.quantized_matrix(c["n"], c["k"], 4, G, key=(configs.CFG_SINGLE, 0, 0, 4))
    b = configs.gemv_bytes(c["n"], c["k"], 4)
    copies = device_copies(tensors.upload_matrix(q), copies_for(b))
    x = tensors.device_tensor(inputs.activation_rows(1, c["k"], key=(configs.CFG_SINGLE, 0, 0, 4))[0])
    y = torch.empty(c["n"], dtype=torch.float32, device="cuda")
    idx = [0]

    def single_call():
        tensors.gemv(copies[idx[0] % len(copies)], x, y)
        idx[0] += 1
    ms = timer(single_call, reps=len(copies))
    out["single_3072x1024_q4"] = {"us": round(ms * 1e3, 2), "GBps": round(b / ms / 1e6, 1),
                                  "pct_peak": round(100 * b / ms / 1e6 / HBM_PEAK_GBS, 2),
                                  "copies": len(copies)}
    del copies

    # Per-shape single launches of the Qwen3-0.6B projections: the 28 layers'
    # own matrices of each shape in turn, plus device copies of them until
    # the rotation exceeds CACHE_BUST_BYTES (one launch each,
    # graph-replayed).  At 0.6-1.8 MB a launch is too short to reach a
    # steady stream (it is dominated by its fixed start-up cost).
    per_shape = {}
    for pname, n, k in configs.QWEN3_06B_PROJ:
        own = [(d, x, y) for (layer, name, d), x, y in zip(mats, xs, ys) if name == pname]
        rounds = copies_for(len(own) * configs.gemv_bytes(n, k, 4))
        sel = [(cp, x, y) for r in range(rounds) for d, x, y in own
               for cp in ([d] if r == 0 else device_copies(d, 2)[1:])]
        jj = [0]

        def shape_call():
            d, x, y = sel[jj[0] % len(sel)]
            tensors.gemv(d, x, y)
            jj[0] += 1
        ms = timer(shape_call, reps=len(sel))
        b = configs.gemv_bytes(n, k, 4)
        per_shape[pname] = {"n": n, "k": k, "us": round(ms * 1e3, 2), "GBps": round(b / ms / 1e6, 1),
                            "pct_peak": round(100 * b / ms / 1e6 / HBM_PEAK_GBS, 2), "copies": len(sel)}
        del sel
    out["qwen3_0.6b_per_shape_q4"] = per_shape
    log("qwen3 per shape: " + ", ".join("%s %.2f us" % (k2, v["us"]) for k2, v in per_shape.items()))

    # Bit-width sweep on Llama-3.2-3B shapes (rotating device copies of each
    # matrix, CACHE_BUST_BYTES in all).
    sweep = {}
    for bits in configs.SWEEP_BITS:
        row = {}
        for j, (pname, n, k) in enumerate(configs.LLAMA32_3B_PROJ):
            if pname in ("k_proj", "o_proj", "up_proj"):
                continue  # same shapes as v, q and gate
            b = configs.gemv_bytes(n, k, bits)
            base = tensors.upload_matrix(inputs.quantized_matrix(n, k, bits, G, key=(configs.CFG_SWEEP, 0, j, bits)))
            cps = device_copies(base, copies_for(b))
            xv = tensors.device_tensor(inputs.activation_rows(1, k, key=(configs.CFG_SWEEP, 0, j, bits))[0])
            yv = torch.empty(n, dtype=torch.float32, device="cuda")
            ii = [0]

            def call():
                tensors.gemv(cps[ii[0] % len(cps)], xv, yv)
                ii[0] += 1
            ms = timer(call, reps=max(len(cps), 20))
            row[pname] = {"us": round(ms * 1e3, 2), "GBps": round(b / ms / 1e6, 1), "copies": len(cps)}
            del cps, base
        # Per-token projection time: 28 layers of q, k, v, o, gate, up, down
        # (k as v, o as q, up as gate: same shapes) plus the LM head, from the
        # per-launch times above.
        layer_us = 2 * row["q_proj"]["us"] + 2 * row["v_proj"]["us"] + 2 * row["gate_proj"]["us"] \
            + row["down_proj"]["us"]
        tok_us = configs.LLAMA32_3B_LAYERS * layer_us + row["lm_head"]["us"]
        row["per_token_projection_us"] = round(tok_us, 1)
        row["projection_tok_per_s"] = round(1e6 / tok_us, 1)
        sweep["q%d" % bits] = row
        log("sweep q%d: lm_head %.0f GB/s, %.0f us per token" % (bits, row["lm_head"]["GBps"], tok_us))
    out["llama3.2_3b_bit_sweep"] = sweep

    # Prefill GEMMs (Llama-3.2-1B shapes), Q4, then the same layer with fp16
    # weights through the same kernel family.
    for bits in (4, 16):
        out["prefill_llama3.2_1b_" + ("q4" if bits == 4 else "fp16")] = prefill_layers(
            torch, qmm, configs, inputs, tensors, timer, bits, configs.PREFILL_M)
    # 2048-token prefill, Q4, with fp32 and with fp16 output.
    out["prefill_llama3.2_1b_q4_pp2048"] = prefill_layers(
        torch, qmm, configs, inputs, tensors, timer, 4, (configs.PREFILL_M_LONG,))
    out["prefill_llama3.2_1b_q4_pp2048_fp16_out"] = prefill_layers(
        torch, qmm, configs, inputs, tensors, timer, 4, (configs.PREFILL_M_LONG,), out_fp16=True)

    # Fused gate/up projection with the SiLU-gated product vs two GEMV
    # launches (Q4, 8 rotating copies of the pair so the weights stream
    # from HBM).
    glu = {}
    for label, n, k in (("qwen3_0.6b_gate_up", 3072, 1024), ("llama3.2_3b_gate_up", 8192, 3072)):
        b = 2 * configs.weight_bytes(n, k, 4) + 2 * k + 4 * n
        dg0 = tensors.upload_matrix(inputs.quantized_matrix(n, k, 4, G, key=(configs.CFG_SWEEP, 90, 0, 0)))
        du0 = tensors.upload_matrix(inputs.quantized_matrix(n, k, 4, G, key=(configs.CFG_SWEEP, 90, 0, 1)))
        npair = copies_for(b)
        pairs = list(zip(device_copies(dg0, npair), device_copies(du0, npair)))
        xg = tensors.device_tensor(inputs.activation_rows(1, k, key=(configs.CFG_SWEEP, 90, k))[0])
        hg = torch.empty(n, dtype=torch.float32, device="cuda")
        yg2 = torch.empty(n, dtype=torch.float32, device="cuda")
        ii = [0]

        def fused():
            dg, du = pairs[ii[0] % npair]
            tensors.gemv_swiglu(dg, du, xg, hg)
            ii[0] += 1

        def separate():
            dg, du = pairs[ii[0] % npair]
            tensors.gemv(dg, xg, hg)
            tensors.gemv(du, xg, yg2)
            ii[0] += 1
        ms_f = timer(fused, reps=npair)
        ms_s = timer(separate, reps=npair)
        glu[label] = {"fused_us": round(ms_f * 1e3, 2), "two_gemvs_us": round(ms_s * 1e3, 2),
                      "fused_GBps": round(b / ms_f / 1e6, 1), "copies": npair}
        del pairs
        log("swiglu %s: fused %.1f us, two gemvs %.1f us" % (label, ms_f * 1e3, ms_s * 1e3))
    out["swiglu_fusion_q4"] = glu

    # Output projections with the residual add fused (y = r + W x, in place)
    # against the plain GEMV followed by a separate add launch.
    resid = {}
    for label, n, k in (("qwen3_0.6b_o_proj", 1024, 2048), ("llama3.2_3b_down", 3072, 8192)):
        nm = copies_for(configs.gemv_bytes(n, k, 4))
        mats = device_copies(tensors.upload_matrix(inputs.quantized_matrix(n, k, 4, G, key=(configs.CFG_SWEEP, 91, 0))),
                             nm)
        xr = tensors.device_tensor(inputs.activation_rows(1, k, key=(configs.CFG_SWEEP, 91, k))[0])
        hr = torch.zeros(n, dtype=torch.float32, device="cuda")
        yr = torch.empty(n, dtype=torch.float32, device="cuda")
        ii = [0]

        def fused_res():
            tensors.gemv_residual(mats[ii[0] % nm], xr, hr, hr)
            ii[0] += 1

        def gemv_then_add():
            tensors.gemv(mats[ii[0] % nm], xr, yr)
            hr.add_(yr)
            ii[0] += 1
        ms_f = timer(fused_res, reps=nm)
        ms_s = timer(gemv_then_add, reps=nm)
        resid[label] = {"fused_us": round(ms_f * 1e3, 2), "gemv_plus_add_us": round(ms_s * 1e3, 2),
                        "copies": nm}
        del mats
        log("residual %s: fused %.1f us, gemv + add %.1f us" % (label, ms_f * 1e3, ms_s * 1e3))
    out["residual_fusion_q4"] = resid

    # MoE expert projections (Qwen3-30B-A3B shapes).  Every timing loop
    # rotates over device copies of the expert stacks and over routings drawn
    # with different seeds, so the experts a call touches are not still
    # cached from the previous calls (at one token a call reads 7 MB per
    # projection; the loop reads more than CACHE_BUST_BYTES).
    moe = {}
    e, top = configs.MOE["n_experts"], configs.MOE["top_k"]
    n_stack = 6
    stacks = {}
    for j, (pname, n, k) in enumerate(configs.MOE_PROJ):
        base = tensors.upload_matrix(inputs.stacked_experts(e, n, k, 4, G, key=(configs.CFG_MOE, j)))
        stacks[pname] = device_copies(base, n_stack)
    for tokens in configs.MOE["tokens"]:
        n_route = 32 if tokens == 1 else 4
        routes = [inputs.routing(tokens, e, top, key=(configs.CFG_MOE, tokens) + ((r,) if r else ()))
                  for r in range(n_route)]
        p = tokens * top
        distinct = float(np.mean([(np.diff(r["offsets"]) > 0).sum() for r in routes]))
        off = [tensors.device_tensor(r["offsets"]) for r in routes]
        rows = [tensors.device_tensor(r["pair_token"]) for r in routes]
        pw = [tensors.device_tensor(r["pair_weight"]) for r in routes]
        pt64 = [rw.long() for rw in rows]
        combos = [(c, ri) for ri in range(n_route) for c in range(n_stack)]
        x_tok = tensors.device_tensor(inputs.activation_rows(tokens, 2048, key=(configs.CFG_MOE, tokens)))
        x_pair = tensors.device_tensor(inputs.activation_rows(p, 768, key=(configs.CFG_MOE, tokens, 9)))
        ii = [0]

        def rotating(fn):
            def call():
                c, ri = combos[ii[0] % len(combos)]
                fn(c, ri)
                ii[0] += 1
            return call
        row = {}
        tot_b, tot_ms = 0, 0.0
        for pname, n, k in configs.MOE_PROJ:
            yo = torch.empty((p, n), dtype=torch.float32, device="cuda")
            if pname == "down_proj":
                fn = rotating(lambda c, ri: tensors.moe(stacks["down_proj"][c], x_pair, None, off[ri], p, y=yo))
            else:
                fn = rotating(lambda c, ri, pname=pname: tensors.moe(stacks[pname][c], x_tok, rows[ri], off[ri],
                                                                     p, y=yo))
            ms = timer(fn, reps=len(combos))
            b = distinct * configs.weight_bytes(n, k, 4) + 2 * p * k + 4 * p * n
            row[pname] = {"us": round(ms * 1e3, 2), "GBps": round(b / ms / 1e6, 1)}
            tot_b += b
            tot_ms += ms
        # Gate and up fused with the SiLU-gated product (one launch), then down.
        ho = torch.empty((p, 768), dtype=torch.float32, device="cuda")
        ms_glu = timer(rotating(lambda c, ri: tensors.moe_swiglu(stacks["gate_proj"][c], stacks["up_proj"][c],
                                                                 x_tok, rows[ri], off[ri], p, h=ho)),
                       reps=len(combos))
        ms_fused = ms_glu + row["down_proj"]["us"] * 1e-3
        # Down projection with the routing-weighted combine into the token
        # rows (one launch), against the plain down projection followed by a
        # weighted scatter-add in torch.
        yc = torch.zeros((tokens, 2048), dtype=torch.float32, device="cuda")
        ms_cmb = timer(rotating(lambda c, ri: tensors.moe_combine(stacks["down_proj"][c], x_pair, None, off[ri],
                                                                  rows[ri], pw[ri], p, yc)),
                       reps=len(combos))
        yo_down = torch.empty((p, 2048), dtype=torch.float32, device="cuda")

        def down_then_scatter(c, ri):
            tensors.moe(stacks["down_proj"][c], x_pair, None, off[ri], p, y=yo_down)
            yc.index_add_(0, pt64[ri], yo_down * pw[ri][:, None])
        ms_scatter = timer(rotating(down_then_scatter), reps=len(combos))
        moe["t%d" % tokens] = {"distinct_experts": round(distinct, 1), "routings": n_route,
                               "stack_copies": n_stack, "us": round(tot_ms * 1e3, 2),
                               "GBps": round(tot_b / tot_ms / 1e6, 1), "proj": row,
                               "fused_gate_up_us": round(ms_glu * 1e3, 2),
                               "us_with_fused_gate_up": round(ms_fused * 1e3, 2),
                               "down_combine_fused_us": round(ms_cmb * 1e3, 2),
                               "down_then_scatter_add_us": round(ms_scatter * 1e3, 2),
                               "us_fully_fused": round((ms_glu + ms_cmb) * 1e3, 2)}
        log("moe T=%d: %.1f us (gate|up fused: %.1f us; + fused combine: %.1f us)"
            % (tokens, tot_ms * 1e3, ms_fused * 1e3, (ms_glu + ms_cmb) * 1e3))
    del stacks
    out["moe_qwen3_30b_a3b_q4"] = moe
    return out


def prefill_layers(torch, qmm, configs, inputs, tensors, timer, bits, ms_list, out_fp16=False):
    """Per-shape and per-layer times of the prefill GEMMs at each M (weights
    at `bits`: 4, or 16 for fp16; fp32 output, or fp16 with out_fp16), with
    the dense fp16 library matmul of the same shape timed beside them for
    context."""
    G = configs.GROUP
    pre = {}
    for m in ms_list:
        tot_flops, tot_ms, dense_ms = 0.0, 0.0, 0.0
        row = {}
        for j, (pname, n, k) in enumerate(configs.LLAMA32_1B_PROJ):
            q = inputs.quantized_matrix(n, k, bits, G, key=(configs.CFG_PREFILL, 0, j, bits))
            dq = tensors.upload_matrix(q)
            xm = tensors.device_tensor(inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, j, 4, m)))
            ym = torch.empty((m, n), dtype=torch.float16 if out_fp16 else torch.float32, device="cuda")
            need = qmm.qmm_gemm_workspace_bytes(m, n, k, bits, G)
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
            # Device-side copies of the same matrix, rotated so that the
            # weights come from HBM (CACHE_BUST_BYTES in all).
            wb = configs.weight_bytes(n, k, bits)
            ncp = copies_for(wb, cap=1024)
            cps = device_copies(dq, ncp)
            ii = [0]

            def call():
                tensors.gemm(cps[ii[0] % ncp], xm, ym, workspace=ws, out_fp16=out_fp16)
                ii[0] += 1
            ms = timer(call, reps=ncp)
            fl = 2.0 * m * n * k
            tf = fl / ms / 1e9
            pl = qmm.qmm_get_plan(1, m, n, k, bits, G, workspace_bytes=ws.numel())
            # Context only: dense fp16 matmul of the same shape through the
            # installed BLAS library (fp16 weights, fp16 output).
            wd = torch.randn((k, n), dtype=torch.float16, device="cuda")
            ms_dense = timer(lambda: torch.matmul(xm, wd), reps=20)
            row[pname] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
                          "pct_mfma": round(100 * tf / MFMA_FP16_PEAK_TFLOPS, 2),
                          "split_k": pl["split_k"], "tile_m": pl["tile_m"], "copies": ncp,
                          "dense_fp16_matmul_us": round(ms_dense * 1e3, 2)}
            del cps, wd
            tot_flops += fl
            tot_ms += ms
            dense_ms += ms_dense
        tf = tot_flops / tot_ms / 1e9
        pre["m%d" % m] = {"layer_us": round(tot_ms * 1e3, 2), "TFLOPs": round(tf, 1),
                          "pct_mfma": round(100 * tf / MFMA_FP16_PEAK_TFLOPS, 2),
                          "dense_fp16_matmul_layer_us": round(dense_ms * 1e3, 2), "shapes": row}
        msg = ""
        if not out_fp16:
            # The same layer with the projections that share their input
            # (q|k|v, gate|up) issued as grouped GEMMs: four dependent
            # launches per layer instead of seven.
            grouped = {}
            for gname, names in (("qkv", ("q_proj", "k_proj", "v_proj")), ("gate_up", ("gate_proj", "up_proj"))):
                sel = [(j, n, k) for j, (pname, n, k) in enumerate(configs.LLAMA32_1B_PROJ) if pname in names]
                k = sel[0][2]
                bases = [tensors.upload_matrix(inputs.quantized_matrix(n, k, bits, G, key=(configs.CFG_PREFILL, 0, j, bits)))
                         for j, n, _ in sel]
                wb = sum(configs.weight_bytes(n, k, bits) for _, n, _ in sel)
                ncp = copies_for(wb, cap=1024)
                sets = [bases] + [[device_copies(d, 2)[1] for d in bases] for _ in range(ncp - 1)]
                xg = tensors.device_tensor(inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, sel[0][0], 4, m)))
                ysg = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _, n, _ in sel]
                members = [(d["w"], d["scales"], d["mins"], y, d["n"]) for d, y in zip(bases, ysg)]
                need = qmm.qmm_gemm_grouped_workspace_bytes(members, m, k, bits, G)
                wsg = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
                gi = [0]

                def gcall():
                    tensors.gemm_grouped(sets[gi[0] % ncp], xg, ys=ysg, workspace=wsg)
                    gi[0] += 1
                ms_g = timer(gcall, reps=ncp)
                grouped[gname] = {"us": round(ms_g * 1e3, 2),
                                  "separate_us": round(sum(row[nm]["us"] for nm in names), 2)}
                del sets
            layer_g = (grouped["qkv"]["us"] + row["o_proj"]["us"] + grouped["gate_up"]["us"]
                       + row["down_proj"]["us"])
            tf_g = tot_flops / layer_g / 1e6
            pre["m%d" % m]["grouped"] = {"layer_us": round(layer_g, 2), "TFLOPs": round(tf_g, 1),
                                         "pct_mfma": round(100 * tf_g / MFMA_FP16_PEAK_TFLOPS, 2),
                                         "launch_groups": grouped}
            msg = "; grouped q|k|v, gate|up: layer %.1f us, %.1f TFLOP/s" % (layer_g, tf_g)
        log("prefill b%d m=%d%s: %.1f TFLOP/s (layer %.1f us, dense fp16 %.1f us)%s"
            % (bits, m, " fp16-out" if out_fp16 else "", tf, tot_ms * 1e3, dense_ms * 1e3, msg))
    return pre


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(np, configs, inputs, set_bytes):
    """The CPU oracle (C, fp64, OpenMP over rows) on the host cores, on a
    bounded sample of the decode set: layer 0's seven projections and the
    first 8192 rows of the LM head."""
    import oracle
    G = configs.GROUP
    work = []
    for j, (name, n, k) in enumerate(configs.QWEN3_06B_PROJ):
        key = (configs.CFG_DECODE_SET, 0, j, 4)
        work.append((inputs.quantized_matrix(n, k, 4, G, key=key), inputs.activation_rows(1, k, key=key)[0]))
    name, n, k = configs.QWEN3_06B_LM_HEAD
    key = (configs.CFG_DECODE_SET, configs.QWEN3_06B_LAYERS, 0, 4)
    q = inputs.quantized_matrix(n, k, 4, G, key=key)
    rows = 8192
    q = dict(q, w=q["w"][:rows], scales=q["scales"][:rows], mins=q["mins"][:rows], n=rows)
    work.append((q, inputs.activation_rows(1, k, key=key)[0]))
    b = sum(configs.gemv_bytes(q["n"], q["k"], 4) for q, _ in work)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for q, x in work:
            oracle.qmm(q["w"], q["scales"], q["mins"], x, q["n"], q["k"], 4, G)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0:  # about ten seconds of CPU work
            break
    gbs = reps * b / el / 1e9
    cores = oracle.threads()
    result = {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
              "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
              "sample": "layer 0's 7 Q4 projections + LM head rows 0..8191 (%d bytes), %d passes in %.1f s"
                        % (b, reps, el),
              "seconds_per_decode_set": round(set_bytes / (gbs * 1e9), 2)}
    # The same oracle on one thread, and on a prefill GEMM (all threads):
    # about five seconds each.
    try:
        oracle.set_threads(1)
        reps1, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            for q, x in work:
                oracle.qmm(q["w"], q["scales"], q["mins"], x, q["n"], q["k"], 4, G)
            reps1 += 1
        el1 = time.perf_counter() - t0
        result["single_thread"] = {"value": round(reps1 * b / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                   "sample": "the same sample, %d passes in %.1f s" % (reps1, el1)}
    finally:
        oracle.set_threads(cores)
    m = 128
    j = [p[0] for p in configs.LLAMA32_1B_PROJ].index("k_proj")
    _, n, k = configs.LLAMA32_1B_PROJ[j]
    q = inputs.quantized_matrix(n, k, 4, G, key=(configs.CFG_PREFILL, 0, j, 4))
    xm = inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, j, 4, m))
    reps2, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 5.0:
        oracle.qmm(q["w"], q["scales"], q["mins"], xm, n, k, 4, G)
        reps2 += 1
    el2 = time.perf_counter() - t0
    result["prefill"] = {"value": round(reps2 * 2.0 * m * n * k / el2 / 1e9, 3), "unit": "GFLOP/s",
                         "cores": cores,
                         "sample": "Llama-3.2-1B k_proj %dx%d, M = %d, Q4, %d calls in %.1f s"
                                   % (n, k, m, reps2, el2)}
    return result


if __name__ == "__main__":
    main()
