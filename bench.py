#!/usr/bin/env python3
"""Throughput of the MobileMoE MoE-FFN layer forward (eq. (*)) on one MI355X.

Default workload: the MobileMoE-S-shaped layer, prefill of 2048 tokens, INT4
group-32 weights with FP32 scales, per-token INT8 activations, 60 routed
experts (top-4) plus the shared expert.  One step = the seven library calls
(router/top-k, route/permute, activation quantisation, routed gate/up+SwiGLU,
routed down, shared expert, combine) over one batch of tokens already resident
in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--batch B]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
INT8_MFMA_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s_prefill")
    ap.add_argument("--batch", type=int, default=None, help="tokens per step (decode batch) override")
    ap.add_argument("--layers", type=int, default=None, help="decode stack depth override")
    ap.add_argument("--instances", type=int, default=0,
                    help="distinct weight sets rotated across steps (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="issue the calls eagerly instead of replaying graphs")
    ap.add_argument("--path", choices=("auto", "decode", "fused", "calls"), default="auto",
                    help="decode: the layer as one kernel launch (mm_moe_decode, 1..4 tokens, INT4); "
                         "fused: the one-call layer (mm_moe_forward, one stream, fewest launches); "
                         "calls: the seven calls with the activation quantiser and shared expert on "
                         "a second stream; auto: decode where it applies, else fused (measured "
                         "fastest on every workload)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    ap.add_argument("--op", choices=("layer", "attn_decode", "linear", "train_step", "block"), default="layer",
                    help="layer: the MoE-FFN layer (default); attn_decode: GQA decode attention "
                         "over an INT8 KV cache (--batch sequences, --context positions, --heads "
                         "query heads, 4 key/value heads); linear: the dense W4A8 projection "
                         "(--batch rows, --in-features, --out-features); train_step: one QAT "
                         "training step of the S layer's routed experts (--batch tokens)")
    ap.add_argument("--context", type=int, default=8192, help="attn_decode: cached positions per sequence")
    ap.add_argument("--heads", type=int, default=12, help="attn_decode: query heads (S: 12, M: 16, L: 20)")
    ap.add_argument("--in-features", type=int, default=768, help="linear: K")
    ap.add_argument("--out-features", type=int, default=768, help="linear: N")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches) and exit: the "
                         "reference for scaling HBM counters")
    return ap.parse_args()


def layer_work(w, T, counts=None):
    """Algorithmic work of one layer call: int8 ops per expert product and
    bytes the decode path must stream."""
    ops = {
        "router": 2 * T * w.E * w.d,
        "gateup": 2 * T * w.k * 2 * w.h * w.d,
        "down": 2 * T * w.k * w.d * w.h,
        "shared": 2 * T * 3 * w.d * w.hs,
    }
    wb = {"int4g32": 0.5 + 4 / 32, "bf16": 2.0, "f32": 4.0}[w.wfmt]
    B_r = 3 * w.d * w.h * wb
    B_s = 3 * w.d * w.hs * wb
    return ops, B_r, B_s


# Kernel chosen by the library for the routed expert products (mirrors the
# dispatch in csrc/api.hip and csrc/k_mfma.hip: weight-streaming up to 32
# routed rows (8 shared rows) when the reduction length fits, matrix cores
# beyond when K % 128 == 0, with two row tiles per wave once that still gives
# 4096 waves;
# BF16 weights always on the bf16 matrix cores).
GEMV_MAX_ROUTED, GEMV_MAX_DENSE = 32, 8  # csrc/launch.h kGemvMaxRowsRouted / kGemvMaxRowsDense


def kernel_of(w, T, gateup: bool):
    """(kernel name as rocprofv3 lists it, path) of the routed gate/up or down product."""
    rows, K = T * w.k, (w.d if gateup else w.h)
    gu = "true" if gateup else "false"
    if w.wfmt == "bf16":
        if rows <= 64 and K % 8 == 0 and K <= 2560 and (w.h % 4 == 0 if gateup else w.d % 8 == 0):
            return f"k_bf16_gemv<{gu}, false>", "weight-streaming"
        if rows >= 128 and (w.h % 64 == 0 if gateup else w.d % 128 == 0):
            return f"k_bf16_lds<{gu}, false>", "matrix-core, workgroup-tiled (LDS)"
        return f"k_bf16w<2, {gu}, false>", "matrix-core"
    if w.wfmt != "int4g32":
        return ("k_gateup_fp<false>" if gateup else "k_down_fp<false>"), "row-tile"
    if rows <= GEMV_MAX_ROUTED and K % 64 == 0 and K <= 2560:
        return f"k_gemv_i4<4, {gu}, false, false>", "weight-streaming"
    if rows > GEMV_MAX_ROUTED and K % 128 == 0:
        nsplit = w.h // 32 if gateup else w.d // 64
        mt = 2 if ((rows + 63) // 64 + min(w.E, rows)) * nsplit >= 4096 else 1
        return f"k_w4a8w<{mt}, {gu}, false, false>", "matrix-core"
    return ("k_gateup_i4<false>" if gateup else "k_down_i4<false>"), "row-tile"


def pair_kernel_of(w, T):
    """rocprofv3 name of the merged routed+shared gate/up kernel mm_moe_forward
    launches for this workload, or None when it takes another form (mirrors
    csrc/api.hip: neither side weight-streaming, both on the matrix cores)."""
    if w.wfmt != "int4g32" or not w.hs or w.d % 128:
        return None
    rows = T * w.k
    if rows <= GEMV_MAX_ROUTED or T <= GEMV_MAX_DENSE:
        return None
    r2 = ((rows + 63) // 64 + min(w.E, rows)) * (w.h // 32) >= 4096
    d2 = ((T + 63) // 64) * (w.hs // 32) >= 4096
    # two column pairs per wave once the one-pair waves would reach 4096
    waves = ((rows + 31) // 32 + min(w.E, rows)) * (w.h // 32) + ((T + 31) // 32) * (w.hs // 32)
    if not r2 and not d2 and waves >= 4096 and w.h % 64 == 0 and w.hs % 64 == 0:
        return "k_w4a8w_pair<1, 1, true, 4, 4, false>"
    # launches of at most 2048 one-pair waves keep the deep register ring
    deep = not r2 and not d2 and waves <= 2048
    return f"k_w4a8w_pair<{2 if r2 else 1}, {2 if d2 else 1}, true, 2, 2, {'true' if deep else 'false'}>"


def pair_gemv_kernel_of(w, T):
    """rocprofv3 name of the merged weight-streaming gate/up kernel
    mm_moe_forward launches for decode batches (routed rows <= 32, shared
    rows <= 8, reduction fits), or None."""
    if w.wfmt != "int4g32" or not w.hs:
        return None
    rows, K = T * w.k, w.d
    if rows <= GEMV_MAX_ROUTED and T <= GEMV_MAX_DENSE and K % 64 == 0 and K <= 2560:
        return "k_gemv_i4_pair<4, true, false>"
    return None


# Every library source: stored counter figures are valid only for the code
# they were taken on.
KERNEL_SOURCES = sorted(os.path.relpath(f, ROOT) for pat in ("*.hip", "*.h") for f in
                        __import__("glob").glob(os.path.join(ROOT, "sparse_moe_ffn_amd", "csrc", pat)))


ATTN_SOURCES = ["sparse_moe_ffn_amd/csrc/k_attn.hip", "sparse_moe_ffn_amd/csrc/common.h"]


def kernel_source_sha(sources=None):
    import hashlib
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str, summary: str = "traffic.md", sources=None, key=None):
    """HBM bytes per launch of `kernel` (or per step, kernel "step") on
    `workload` at `key` tokens per step from a committed rocprofv3 counter
    summary under profiles/, or None when there is none or the kernel sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha(sources)
    for line in open(path):
        if not line.startswith("traffic:"):
            continue
        kv = dict(p.split("=", 1) for p in line[len("traffic:"):].split() if "=" in p)
        if kv.get("workload") == workload and kv.get("kernel") == kernel.replace(" ", "") \
                and kv.get("source_sha256") == sha and (key is None or kv.get("tokens") == str(key)):
            return float(kv["bytes_per_launch"])
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens with replicated weights).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_moe_ffn_amd import binding as B
    from sparse_moe_ffn_amd import workloads as wl
    from sparse_moe_ffn_amd.layer import MoELayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones((n // 4,), dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return
    B.load()
    if args.op == "attn_decode":
        return bench_attn(args, dev)
    if args.op == "linear":
        return bench_linear(args, dev)
    if args.op == "train_step":
        return bench_train(args, dev)
    if args.op == "block":
        return bench_block(args, dev)
    w = wl.WORKLOADS[args.workload]
    if args.batch is not None:
        w = w.with_(T=args.batch)
    if args.layers is not None:
        w = w.with_(layers=args.layers)
    decode = w.mode == "decode"
    T = w.T

    # ---- weights: distinct layers (decode stack) or rotated instances (single layer)
    t0 = time.time()
    wb = {"int4g32": 0.625, "bf16": 2.0, "f32": 4.0}[w.wfmt]
    layer_bytes = (w.E * 3 * w.d * w.h + 3 * w.d * w.hs) * wb + w.E * w.d * 4
    if w.layers > 1:
        n_inst = w.layers
    elif args.instances > 0:
        n_inst = args.instances
    else:
        n_inst = int(min(16, max(1, math.ceil(1.15 * MALL_BYTES / layer_bytes))))
    layers = []
    for i in range(n_inst):
        lw = wl.layer_weights(w, layer=i)
        layers.append(MoELayer.from_workload(w, lw, device=dev))
        del lw
    for L in layers:
        L.buffers(T)
    print(f"[bench] {w.name}: T={T} layers/instances={n_inst} weights {n_inst * layer_bytes / 1e6:.0f} MB "
          f"setup {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    n_inputs = args.warmup + args.steps if decode else 1
    xs = [torch.from_numpy(wl.tokens(w, step=s)).to(dev) for s in range(n_inputs)]
    nxt = torch.empty((T, w.d), dtype=torch.float32, device=dev)

    one_launch = args.path in ("decode", "auto") and all(L.decode_supported(T) for L in layers)
    if args.path == "decode" and not one_launch:
        sys.exit(f"--path decode: no one-launch form for {w.name} at T={T}")
    fused = args.path in ("fused", "auto") or one_launch

    def fwd(L, src):
        if one_launch:
            return L.forward_decode(src)
        return L.forward_fused(src) if fused else L.forward(src)

    def layer_then_norm(L, src, dst):
        """One stack layer: dst = RMSNorm(layer(src)) (the combine writes it on the
        one-call path, a separate kernel on the seven-call path)."""
        if one_launch:
            L.forward_decode(src, y_norm=dst, norm_eps=1e-5)
        elif fused:
            L.forward_fused(src, y_norm=dst, norm_eps=1e-5)
        else:
            y = L.forward(src)
            B.rmsnorm_f32(T, w.d, 1e-5, y, dst)

    def eager_step(s: int):
        if decode:
            # RMSNorm between layers only (the last layer's y is the output);
            # a one-layer workload runs one of its rotated weight sets
            cur = xs[s % n_inputs]
            stack = layers if w.layers > 1 else [layers[s % n_inst]]
            for i, L in enumerate(stack):
                if i + 1 < len(stack):
                    layer_then_norm(L, cur, nxt)
                    cur = nxt
                else:
                    fwd(L, cur)
        else:
            fwd(layers[s % n_inst], xs[0])

    # The steps are replayed from HIP graphs: the W warm-up steps are recorded
    # into one graph and the K timed steps into another, replayed once each
    # (as a model's forward graph holds all of its layers, the per-replay
    # launch cost is paid once for the whole sequence, not once per step).
    # Prefill step s runs weight set s % n_inst; a decode step copies its
    # fresh input into the stack's input buffer, then runs the whole stack.
    if args.eager:
        def run_warmup():
            for s in range(args.warmup):
                eager_step(s)

        def run_timed():
            for s in range(args.warmup, args.warmup + args.steps):
                eager_step(s)
    else:
        xin = torch.empty((T, w.d), dtype=torch.float32, device=dev)
        for L in layers:
            L.buffers(T)

        def graph_step(s: int):
            if decode:
                xin.copy_(xs[s % n_inputs])
                cur = xin
                stack = layers if w.layers > 1 else [layers[s % n_inst]]
                for i, L in enumerate(stack):
                    if i + 1 < len(stack):
                        layer_then_norm(L, cur, nxt)
                        cur = nxt
                    else:
                        fwd(L, cur)
            else:
                fwd(layers[s % n_inst], xs[0])

        side = torch.cuda.Stream(device=dev)  # first (uncaptured) run of every launch
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for s in range(n_inst if (not decode or w.layers == 1) else 1):
                graph_step(s)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        def record(s0: int, n: int):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(s0, s0 + n):
                    graph_step(s)
            return g

        g_warm = record(0, args.warmup) if args.warmup else None
        g_timed = record(args.warmup, args.steps)

        def run_warmup():
            if g_warm is not None:
                g_warm.replay()

        def run_timed():
            g_timed.replay()

    run_warmup()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    run_timed()
    e1.record(st)
    e1.synchronize()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tok_s = T / (ms / 1e3)

    # ---- per-call durations: each call is recorded REPS times into a HIP
    # graph of its own and replayed between two HIP events on the stream it
    # runs on (kernel time plus the graph's dispatch gap, no host launch cost).
    calls = ["router", "route", "act_quant", "gateup", "down", "shared", "combine"]
    if w.wfmt != "int4g32":
        calls.remove("act_quant")
    if not w.hs:
        calls.remove("shared")
    x0 = xs[0]
    for L in layers:
        L.forward(x0)  # routing state for the expert calls
    torch.cuda.synchronize()
    REPS, REPLAYS = 10, 5

    def issue(c, L):
        if c == "router":
            L.router(x0, T)
        elif c == "route":
            L.route(T)
        elif c == "act_quant":
            L.act_quant(x0, T)
        elif c == "gateup":
            L.gateup(x0, T)
        elif c == "down":
            L.down(T)
        elif c == "shared":
            L.shared(x0, T)
        elif c == "combine":
            L.combine(T)

    per_call_us = {}
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(REPS):
                issue(c, layers[r % len(layers)])
        g.replay()
        torch.cuda.synchronize()
        e0c, e1c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0c.record(st)
        for _ in range(REPLAYS):
            g.replay()
        e1c.record(st)
        e1c.synchronize()
        per_call_us[c] = 1e3 * e0c.elapsed_time(e1c) / (REPS * REPLAYS)
        del g
    torch.cuda.synchronize()

    # ---- the layer's gate/up product stage inside the step (the largest
    # product: routed and shared gate/up with SwiGLU, one merged launch where
    # the one-call layer uses one): mm_moe_forward records HIP events around
    # it on its stream (mm_set_profile_events); the step runs eagerly with a
    # fresh event pair per layer call, so the figure is that stage's time in
    # the step's own context (the same launches a kernel trace of the step
    # shows).
    # On the one-launch path the stage is the whole layer: the events go
    # around each layer's single launch.
    stage_us = None
    if fused:
        pairs = []

        def timed_fwd(L, src, dst=None):
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            if one_launch:
                ev[0].record(st)
                L.forward_decode(src, y_norm=dst, norm_eps=1e-5)
                ev[1].record(st)
            else:
                B.set_profile_events(*ev)
                if dst is not None:
                    L.forward_fused(src, y_norm=dst, norm_eps=1e-5)
                else:
                    L.forward_fused(src)
            pairs.append(ev)

        for s in range(3):
            if decode:
                cur = xs[s % n_inputs]
                stack = layers if w.layers > 1 else [layers[s % n_inst]]
                for i, L in enumerate(stack):
                    if i + 1 < len(stack):
                        timed_fwd(L, cur, nxt)
                        cur = nxt
                    else:
                        timed_fwd(L, cur)
            else:
                timed_fwd(layers[s % n_inst], xs[0])
        B.set_profile_events(None, None)
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        stage_us = sum(times) / len(times)

    ops, B_r, B_s = layer_work(w, T)
    n_layers = w.layers if decode else 1
    # distinct routed experts each layer selected in its last call (decode bytes)
    distinct = [int(np.unique(L.idx.cpu().numpy()).size) for L in layers]
    n_distinct = distinct[0]
    layer_ops = ops["gateup"] + ops["down"] + ops["shared"]
    gu_ops = ops["gateup"] + ops["shared"] * 2 // 3  # shared gate/up: 2 of its 3 d x h_s products
    wb_r = B_r / (3 * w.d * w.h)  # bytes per weight
    if decode:
        # bytes the step must move: per layer the packed weights and scales of
        # the distinct selected experts, the shared expert's, the FP32 router,
        # and the token rows in and out
        per_layer = [u * B_r + B_s + 4 * w.E * w.d + 8 * T * w.d for u in distinct[:n_layers]]
        if w.layers == 1:
            per_layer = [sum(u * B_r for u in distinct) / len(distinct) + B_s + 4 * w.E * w.d
                         + 8 * T * w.d]
        step_bytes = sum(per_layer)
        achieved = step_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 5),
                "traffic": stored_traffic(w.name, "step", key=T),
                "scope": "whole step (every launch of the layer stack)",
                "algorithmic_bytes_per_step": int(step_bytes)}
        if stage_us and one_launch:
            lb = step_bytes / n_layers
            ka = lb / (stage_us * 1e-6) / 1e9
            roof["kernel"] = {"stage": "whole layer (one launch)", "kernel": "k_decode_fused",
                              "launch_us": round(stage_us, 3), "achieved": round(ka, 2),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ka / HBM_PEAK_GBS, 5),
                              "algorithmic_bytes_per_launch": int(lb),
                              "traffic": stored_traffic(w.name, "k_decode_fused", key=T),
                              "timing": "HIP events around each layer's launch inside eager steps"}
        elif stage_us:
            gu_bytes = n_distinct * 2 * w.h * w.d * wb_r + 2 * w.hs * w.d * wb_r
            ka = gu_bytes / (stage_us * 1e-6) / 1e9
            kind, path = kernel_of(w, T, True)
            kind = pair_gemv_kernel_of(w, T) or pair_kernel_of(w, T) or kind
            roof["kernel"] = {"stage": "gate/up (routed + shared)", "kernel": kind,
                              "launch_us": round(stage_us, 3), "achieved": round(ka, 2),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ka / HBM_PEAK_GBS, 5),
                              "algorithmic_bytes_per_launch": int(gu_bytes),
                              "traffic": stored_traffic(w.name, kind, key=T),
                              "timing": "HIP events around the stage inside eager steps"}
    else:
        peak = INT8_MFMA_PEAK_TOPS if w.wfmt == "int4g32" else (
            BF16_MFMA_PEAK_TFLOPS if w.wfmt == "bf16" else FP32_VALU_PEAK_TFLOPS)
        unit = "TOP/s" if w.wfmt == "int4g32" else "TFLOP/s"
        achieved = layer_ops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma" if w.wfmt != "f32" else "alu", "achieved": round(achieved, 3),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 5),
                "traffic": stored_traffic(w.name, "step", key=T),
                "scope": "whole step (router, count sort, quantisers, products, combine)",
                "algorithmic_ops_per_step": int(layer_ops)}
        if stage_us:
            ka = gu_ops / (stage_us * 1e-6) / 1e12
            kind = pair_kernel_of(w, T)
            kind = kind or kernel_of(w, T, True)[0]
            roof["kernel"] = {"stage": "gate/up (routed + shared)", "kernel": kind,
                              "launch_us": round(stage_us, 3), "achieved": round(ka, 3), "peak": peak,
                              "unit": unit, "frac": round(ka / peak, 5),
                              "algorithmic_ops_per_launch": int(gu_ops),
                              "traffic": stored_traffic(w.name, kind, key=T),
                              "timing": "HIP events around the stage inside eager steps"}

    # ---- CPU oracle on a bounded sample of the same workload: single thread
    # and all of this process's host cores.  Each figure is the slope between
    # two token counts, so the oracle's per-call weight quantisation (a fixed
    # cost per call) drops out.
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:
            ncpu = os.cpu_count() or 1
        cores = max(1, min(16, ncpu))
        model = "unknown"
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        lw = wl.layer_weights(w, layer=0)
        xall = wl.tokens(w, step=0)

        def run(n, threads):
            t1 = time.time()
            oracle.forward(xall[:n], lw.wr, lw.bias, lw.w_gu, lw.w_d, lw.ws_gu, lw.ws_d, k=w.k,
                           wfmt=w.wfmt, nthreads=threads)
            return time.time() - t1

        def rate(threads, budget):
            n1 = min(T, 8 if threads == 1 else 4 * threads)
            t1 = run(n1, threads)
            n2 = n1
            while n2 < T:
                n2 = min(T, max(2 * n2, int(n2 * budget / max(t1, 1e-3))))
                t2 = run(n2, threads)
                if t2 - t1 >= budget / 2 or n2 >= T:
                    break
            if n2 == n1:  # the whole workload in the first call
                return n1 / t1, n1, t1
            return (n2 - n1) / max(t2 - t1, 1e-9), n2, t2

        r1, n1s, t1s = rate(1, args.cpu_seconds / 3)
        rn, nns, tns = rate(cores, args.cpu_seconds / 3)
        per = n_layers
        cpu = {"value": round(rn / per, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "single_thread": round(r1 / per, 2), "cpu_model": model,
               "sample": f"{w.name}, one layer of the oracle (oracle.forward, the plain C++ evaluation of "
                         f"eq. (*)): rate = token-count slope between two calls (excludes the per-call "
                         f"weight quantisation); {cores} threads up to {nns} tokens ({tns:.1f} s), one "
                         f"thread up to {n1s} tokens ({t1s:.1f} s)"
                         + (f"; per-step rate = per-layer rate / {per} layers" if per > 1 else "")}

    out = {
        "metric": "MoE-layer tokens/s (prefill T=2048/8192, decode B=1-64) + % HBM/MFMA peak",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int4g32": "int8", "bf16": "bf16", "f32": "f32"}[w.wfmt],
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "tokens_per_step": T, "d_model": w.d,
                   "experts": w.E, "top_k": w.k, "hidden": w.h, "shared_hidden": w.hs,
                   "weights": w.wfmt, "layers": w.layers, "router_bias": w.bias,
                   "weight_sets_rotated": n_inst, "parallelism": "single GPU",
                   "path": ("mm_moe_decode (one launch per layer)" if one_launch else
                            "mm_moe_forward (one call)" if fused else
                            "seven calls, shared expert on a second stream")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_call_us": {c: round(v, 3) for c, v in per_call_us.items()},
        "distinct_experts_last_step": n_distinct,
    }
    print(json.dumps(out), flush=True)


def _time_graphs(issue, warmup: int, steps: int):
    """Warm-up steps recorded into one HIP graph and the timed steps into
    another; returns the mean ms per timed step (HIP events on the stream the
    calls run on)."""
    import torch
    st = torch.cuda.current_stream()
    gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw):
        for i in range(max(warmup, 1)):
            issue(i)
    with torch.cuda.graph(gt):
        for i in range(steps):
            issue(warmup + i)
    gw.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    gt.replay()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_attn(args, dev):
    """GQA decode attention of one new token per sequence over an INT8 KV cache
    (d_h = 64, 4 key/value heads): bytes of the cache read per second.  Caches
    of random codes and positive scales (seeded), enough of them rotated that
    every step reads HBM rather than the 256 MB MALL."""
    import torch
    from sparse_moe_ffn_amd import binding as B
    Bn, nh, nkv, T = args.batch or 32, args.heads, 4, args.context
    per = Bn * nkv * T * 136  # 64 + 64 code bytes and two FP32 scales per position and head
    n_inst = max(2, math.ceil(2.3 * MALL_BYTES / per))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    caches = []
    for _ in range(n_inst):
        kc = torch.randint(-127, 128, (Bn, nkv, T, 64), dtype=torch.int8, device=dev, generator=gen)
        vc = torch.randint(-127, 128, (Bn, nkv, T, 64), dtype=torch.int8, device=dev, generator=gen)
        ks = torch.rand((Bn, nkv, T), device=dev, generator=gen) * 0.04 + 1e-3
        vs = torch.rand((Bn, nkv, T), device=dev, generator=gen) * 0.04 + 1e-3
        caches.append((kc, vc, ks, vs))
    q = torch.randn((Bn, nh, 64), device=dev, generator=gen)
    lens = torch.full((Bn,), T, dtype=torch.int32, device=dev)
    wsb = B.attn_workspace_bytes(Bn, nkv, T)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
    out = torch.empty((Bn, nh, 64), dtype=torch.float32, device=dev)

    def issue(i):
        kc, vc, ks, vs = caches[i % n_inst]
        B.attn_decode_i8(Bn, nh, nkv, 64, T, T, lens, q, kc, vc, ks, vs, out, ws, wsb)

    ms = _time_graphs(issue, args.warmup, args.steps)
    nbytes = per + Bn * nh * 64 * 8  # cache + q and output
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        kc, vc, ks, vs = (t.cpu().numpy() for t in caches[0])
        qh = q.cpu().numpy()
        n = 1
        while True:
            t1 = time.time()
            oracle.attn_decode(qh[:n], kc[:n], vc[:n], ks[:n], vs[:n], T)
            dt = time.time() - t1
            if dt >= args.cpu_seconds / 4 or n >= Bn:
                break
            n = int(min(Bn, max(2 * n, n * args.cpu_seconds / 4 / max(dt, 1e-3))))
        cpu = {"value": round(n * nkv * T * 136 / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n} of the {Bn} sequences, {T} positions each, oracle.attn_decode "
                         f"(double, one thread), {dt:.1f}s"}
    out_line = {
        "metric": "decode attention over an INT8 KV cache: cache bytes read per second",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8 codes, f32 arithmetic",
        "data": "synthetic",
        "config": {"workload": "gqa_decode_attention", "sequences": Bn, "context": T,
                   "query_heads": nh, "kv_heads": nkv, "head_dim": 64, "caches_rotated": n_inst,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 5),
                     "traffic": stored_traffic(f"gqa_decode_attention_b{Bn}_h{nh}_t{T}",
                                               "k_attn_split+k_attn_merge",
                                               "gqa_decode_attention_kernels.md", ATTN_SOURCES),
                     "kernel": "k_attn_split + k_attn_merge (one mm_attn_decode_i8 call)",
                     "algorithmic_bytes_per_launch": nbytes, "launch_us": round(ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out_line), flush=True)


def bench_block(args, dev):
    """One decode step of a MobileMoE-S decoder block (RMSNorm, W4A8 q/k/v,
    INT8 KV append, GQA decode attention over `context` positions, W4A8 o,
    residual add + RMSNorm, the MoE-FFN layer, residual add) for a batch of
    sequences: tokens per second, and the step's algorithmic HBM bytes
    (projection weights, the KV cache read, the selected experts', shared
    expert's and router's weights, token rows) per second.  Distinct blocks
    (weights and caches) rotated past the 256 MB MALL; every step writes the
    new token at the cache's last position (the same work every step)."""
    import numpy as np
    import torch
    from sparse_moe_ffn_amd import workloads as wl
    from sparse_moe_ffn_amd.layer import DecoderBlock, MoELayer
    Bn, T = args.batch or 8, args.context
    w = wl.WORKLOADS["s_decode"].with_(T=Bn, layers=1)
    per = (w.E * 3 * w.d * w.h + 3 * w.d * w.hs) * 0.625 + Bn * 4 * T * 136
    n_inst = int(max(2, math.ceil(1.6 * MALL_BYTES / per)))  # a step touches about 3/4 of a block
    blocks = []
    for i in range(n_inst):
        lw = wl.layer_weights(w, layer=i)
        aw = wl.attn_weights(w, layer=i)
        moe = MoELayer.from_workload(w, lw, device=dev)
        blk = DecoderBlock(moe, aw.n_h, aw.n_kv, aw.wq, aw.wk, aw.wv, aw.wo, Bn, T)
        blk.load_context(*wl.kv_context(w, Bn, T, layer=i))
        blocks.append(blk)
    x = torch.from_numpy(wl.tokens(w, step=0)).to(dev)
    pos = torch.full((Bn,), T - 1, dtype=torch.int32, device=dev)
    lens = torch.full((Bn,), T, dtype=torch.int32, device=dev)
    for blk in blocks:  # buffers and workspaces exist before the graphs are recorded
        blk.decode(x, pos, lens, T)
    torch.cuda.synchronize()
    distinct = [len(np.unique(blk.moe.idx.cpu().numpy())) for blk in blocks]

    def issue(i):
        blocks[i % n_inst].decode(x, pos, lens, T)

    ms = _time_graphs(issue, args.warmup, args.steps)
    d, h, hs, qd, kd = w.d, w.h, w.hs, 12 * 64, 4 * 64
    proj = (2 * qd * d + 2 * kd * d) * 0.625
    kv = Bn * 4 * T * 136
    moe_b = float(np.mean(distinct)) * 3 * d * h * 0.625 + 3 * d * hs * 0.625 + 4 * w.E * d
    rows = 5 * Bn * d * 4
    nbytes = proj + kv + moe_b + rows
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        blk = blocks[0]
        lw, aw = wl.layer_weights(w, layer=0), wl.attn_weights(w, layer=0)
        kq, vq, ks, vs = wl.kv_context(w, Bn, T, layer=0)
        q4 = [oracle.quant_w4g32(m) for m in (aw.wq, aw.wk, aw.wv, aw.wo)]
        xh = x.cpu().numpy()
        f32 = np.float32

        def ora_step(n):
            a = oracle.rmsnorm(xh[:n], 1e-5).astype(f32)
            aq, sa = oracle.quant_act_i8(a)
            q, k, v = (oracle.linear_w4a8(aq, sa, *q4[j]).astype(f32) for j in range(3))
            kqq, kss = oracle.quant_act_i8(k.reshape(-1, 64))
            vqq, vss = oracle.quant_act_i8(v.reshape(-1, 64))
            kc, vc, ksc, vsc = kq[:n].copy(), vq[:n].copy(), ks[:n].copy(), vs[:n].copy()
            kc[:, :, T - 1] = kqq.reshape(n, 4, 64)
            vc[:, :, T - 1] = vqq.reshape(n, 4, 64)
            ksc[:, :, T - 1] = kss.reshape(n, 4)
            vsc[:, :, T - 1] = vss.reshape(n, 4)
            o = oracle.attn_decode(q.reshape(n, 12, 64), kc, vc, ksc, vsc, T).reshape(n, -1).astype(f32)
            oq, so = oracle.quant_act_i8(o)
            hh = xh[:n] + oracle.linear_w4a8(oq, so, *q4[3]).astype(f32)
            a2 = oracle.rmsnorm(hh, 1e-5).astype(f32)
            r = oracle.forward(a2, lw.wr, lw.bias, lw.w_gu, lw.w_d, lw.ws_gu, lw.ws_d, k=w.k,
                               wfmt="int4g32", nthreads=1)
            return hh + r.y.astype(f32)

        ora_step(1)  # the oracle's weight quantisation is per call; time the slope
        t1 = time.time()
        ora_step(1)
        d1 = time.time() - t1
        n = min(Bn, 8)
        t1 = time.time()
        ora_step(n)
        dn = time.time() - t1
        per_tok = (dn - d1) / (n - 1) if n > 1 and dn > d1 else dn / n
        cpu = {"value": round(1.0 / per_tok, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"the composed oracle block (the oracle's RMSNorm, INT8 quantiser, W4A8 "
                         f"linear, decode attention over {T} positions and layer forward) for 1 "
                         f"and {n} sequences, one thread; rate = token-count slope ({dn:.1f}s)"}
    out_line = {
        "metric": "decoder-block decode step (MobileMoE-S block): tokens per second",
        "value": round(Bn / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "s_decoder_block", "sequences": Bn, "context": T, "d_model": d,
                   "query_heads": 12, "kv_heads": 4, "head_dim": 64, "experts": w.E, "top_k": w.k,
                   "hidden": h, "shared_hidden": hs, "blocks_rotated": n_inst,
                   "parallelism": "single GPU",
                   "path": "DecoderBlock.decode (RMSNorm, 3 + 1 W4A8 projections, KV append, "
                           "mm_attn_decode_i8, mm_add_rmsnorm_f32 x 2, the MoE layer)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None,
                     "scope": "whole step", "algorithmic_bytes_per_step": int(nbytes),
                     "bytes": {"projections": int(proj), "kv_cache": int(kv), "moe_layer": int(moe_b),
                               "token_rows": int(rows)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out_line), flush=True)


def bench_linear(args, dev):
    """Dense W4A8 linear (eq. (6) INT4 weights, per-row INT8 activations), as
    in the projections around the MoE layer: int8 ops per second."""
    import numpy as np
    import torch
    from sparse_moe_ffn_amd import binding as B
    from sparse_moe_ffn_amd.layer import prepare_weight
    rows, K, N = args.batch or 2048, args.in_features, args.out_features
    g = np.random.default_rng(4321)
    n_inst = 9
    wts = [prepare_weight((g.standard_normal((N, K)) * 0.02).astype(np.float32), "int4g32", dev)
           for _ in range(n_inst)]
    x = torch.from_numpy(g.standard_normal((rows, K)).astype(np.float32)).to(dev)
    xq = torch.empty((rows, K), dtype=torch.int8, device=dev)
    sx = torch.empty((rows,), dtype=torch.float32, device=dev)
    B.act_quant_i8(rows, K, x, xq, sx)
    y = torch.empty((rows, N), dtype=torch.float32, device=dev)

    def issue(i):
        B.linear_w4a8(rows, K, N, xq, sx, wts[i % n_inst].c(), y)

    ms = _time_graphs(issue, args.warmup, args.steps)
    ops = 2.0 * rows * K * N
    tops = ops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        wq, wsc = oracle.quant_w4g32((g.standard_normal((N, K)) * 0.02).astype(np.float32))
        aq, sa = oracle.quant_act_i8(x.cpu().numpy())
        n = min(rows, 8)
        while True:
            t1 = time.time()
            oracle.linear_w4a8(aq[:n], sa[:n], wq, wsc)
            dt = time.time() - t1
            if dt >= args.cpu_seconds / 4 or n >= rows:
                break
            n = int(min(rows, max(2 * n, n * args.cpu_seconds / 4 / max(dt, 1e-3))))
        cpu = {"value": round(2.0 * n * K * N / dt / 1e12, 6), "unit": "TOP/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n} of the {rows} rows, oracle.linear_w4a8 (one thread), {dt:.1f}s"}
    out_line = {
        "metric": "dense W4A8 linear: int8 ops per second",
        "value": round(tops, 3), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "w4a8_linear", "rows": rows, "in_features": K, "out_features": N,
                   "weight_sets_rotated": n_inst, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if rows > 64 else "hbm",
                     "achieved": round(tops, 3) if rows > 64 else round(N * K * 0.625 / (ms * 1e-3) / 1e9, 2),
                     "peak": INT8_MFMA_PEAK_TOPS if rows > 64 else HBM_PEAK_GBS,
                     "unit": "TFLOP/s" if rows > 64 else "GB/s",
                     "frac": round(tops / INT8_MFMA_PEAK_TOPS, 5) if rows > 64
                     else round(N * K * 0.625 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                     "traffic": None, "kernel": "mm_linear_w4a8 (one launch)",
                     "launch_us": round(ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out_line), flush=True)


def bench_train(args, dev):
    """One QAT training step of the MobileMoE-S MoE-FFN layer (d = 768, 60
    routed experts of h = 384, top-4, shared expert of h_s = 1536): the FP32
    router with the pages' training gate (sigmoid, top-k renormalised, the
    balancing bias in the selection only), balancing-bias update, count
    sort, drop-and-pad at capacity factor 1.5, eq. (6) fake quantisation of
    the latent FP32 weights and of the input rows, row gathers, the grouped
    forward products of the routed and shared experts and the combine into
    y; then their backward, the token gradient (combine of the routed input
    gradients plus the shared one) through the input quantiser, the router
    backward with the z-loss, and the straight-through weight gradients.
    Inputs x and dy and the latent weights are seeded synthetic."""
    import numpy as np
    import torch
    from sparse_moe_ffn_amd import binding as B
    T, E, k, d, h, hs = args.batch or 2048, 60, 4, 768, 384, 1536
    Tk = T * k
    g = np.random.default_rng(777)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    idx_d = torch.empty((T, k), dtype=torch.int32, device=dev)
    wr = f32(g.standard_normal((E, d)) * 0.05)
    wgu = f32(g.standard_normal((E, 2 * h, d)) / np.sqrt(d))
    wd = f32(g.standard_normal((E, d, h)) / np.sqrt(h))
    sgu = f32(g.standard_normal((1, 2 * hs, d)) / np.sqrt(d))
    sd = f32(g.standard_normal((1, d, hs)) / np.sqrt(hs))
    topw = torch.empty((T, k), device=dev)
    x = f32(g.standard_normal((T, d)))
    dy = f32(g.standard_normal((T, d)))
    bias = torch.zeros((E,), device=dev)
    C = B.drop_pad_capacity(T, k, E)
    ds = B.desc(d, E, h, 0, k, gating=B.MM_GATE_SIGMOID_NORM | B.MM_GATE_BIAS_SELECT_ONLY)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((Tk,), dtype=torch.int32, device=dev)
    inv = torch.empty((Tk,), dtype=torch.int32, device=dev)
    nb = B.workspace_bytes(ds, T, B.MM_WS_ROUTE)
    rws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    buf = torch.empty((E * C,), dtype=torch.int32, device=dev)
    offc = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    permc = torch.empty((Tk,), dtype=torch.int32, device=dev)
    invc = torch.empty((Tk,), dtype=torch.int32, device=dev)
    wgu_b, wd_b, x_b = torch.empty_like(wgu), torch.empty_like(wd), torch.empty_like(x)
    xs = torch.empty((Tk, d), device=dev)
    dfs = torch.empty((Tk, d), device=dev)
    gu = torch.empty((Tk, 2 * h), device=dev)
    ab = torch.empty((Tk, h), device=dev)
    fo = torch.empty((Tk, d), device=dev)
    dxs = torch.empty((Tk, d), device=dev)
    dwgu, dwd = torch.empty_like(wgu), torch.empty_like(wd)
    gwgu, gwd = torch.empty_like(wgu), torch.empty_like(wd)
    wsb = max(B.expert_backward_workspace_bytes(Tk, h), B.expert_backward_workspace_bytes(T, hs))
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
    soff = torch.tensor([0, T], dtype=torch.int32, device=dev)
    sgu_b, sd_b = torch.empty_like(sgu), torch.empty_like(sd)
    s_gu = torch.empty((T, 2 * hs), device=dev)
    s_ab = torch.empty((T, hs), device=dev)
    s_f = torch.empty((T, d), device=dev)
    s_dx = torch.empty((T, d), device=dev)
    s_dgu, s_dd = torch.empty_like(sgu), torch.empty_like(sd)
    s_ggu, s_gd = torch.empty_like(sgu), torch.empty_like(sd)
    ones = torch.ones((T, k), device=dev)
    y = torch.empty((T, d), device=dev)
    dx_b, dx = torch.empty((T, d), device=dev), torch.empty((T, d), device=dev)
    dz = torch.empty((T, E), device=dev)
    dwr = torch.empty((E, d), device=dev)

    calls = {
        "router": lambda: B.router_topk(ds, T, x, wr, bias, idx_d, topw),
        "bias_update": lambda: B.bias_update(T, E, k, idx_d, 1e-3, bias),
        "route": lambda: B.route_permute(ds, T, idx_d, off, perm, inv, rws, nb),
        "drop_pad": lambda: B.drop_pad(T, E, k, C, idx_d, off, perm, inv, buf, offc, permc, invc),
        "fake_quant_w": lambda: (B.fake_quant(E * 2 * h, d, 4, 32, wgu, wgu_b),
                                 B.fake_quant(E * d, h, 4, 32, wd, wd_b),
                                 B.fake_quant(2 * hs, d, 4, 32, sgu, sgu_b),
                                 B.fake_quant(d, hs, 4, 32, sd, sd_b)),
        "fake_quant_x": lambda: B.fake_quant(T, d, 8, d, x, x_b),
        "gather": lambda: (B.gather_rows(Tk, d, k, permc, None, x_b, xs),
                           B.gather_rows(Tk, d, k, permc, topw, dy, dfs)),
        "forward": lambda: B.expert_train_forward_f32(E, d, h, Tk, offc, xs, wgu_b, wd_b, gu, ab, fo),
        "shared_forward": lambda: B.expert_train_forward_f32(1, d, hs, T, soff, x_b, sgu_b, sd_b, s_gu,
                                                             s_ab, s_f),
        "combine_y": lambda: B.combine(ds, T, fo, invc, topw, s_f, y),
        "backward": lambda: B.expert_backward_f32(E, d, h, Tk, offc, xs, wgu_b, wd_b, gu, ab, dfs, dxs,
                                                  dwgu, dwd, ws, wsb),
        "shared_backward": lambda: B.expert_backward_f32(1, d, hs, T, soff, x_b, sgu_b, sd_b, s_gu, s_ab,
                                                         dy, s_dx, s_dgu, s_dd, ws, wsb),
        "combine_dx": lambda: (B.combine(ds, T, dxs, invc, ones, s_dx, dx_b),
                               B.fake_quant(T, d, 8, d, x, None, dx_b, dx)),
        "router_backward": lambda: B.router_backward_f32(ds, T, x, wr, bias, idx_d, fo, invc, dy, 1e-4,
                                                         dz, dwr, dx),
        "ste_w": lambda: (B.fake_quant(E * 2 * h, d, 4, 32, wgu, None, dwgu, gwgu),
                          B.fake_quant(E * d, h, 4, 32, wd, None, dwd, gwd),
                          B.fake_quant(2 * hs, d, 4, 32, sgu, None, s_dgu, s_ggu),
                          B.fake_quant(d, hs, 4, 32, sd, None, s_dd, s_gd)),
    }

    def step(_i=0):
        for c in calls.values():
            c()

    ms = _time_graphs(step, args.warmup, args.steps)
    kept = int(offc[E].item())
    per_call = {}
    for name, c in calls.items():
        per_call[name] = round(1e3 * _time_graphs(lambda _i, c=c: c(), 1, 10), 3)
    flops_fwd = 6.0 * kept * h * d
    flops_bwd = 12.0 * kept * h * d
    flops_step = 18.0 * (kept * h + T * hs) * d
    bw_tf = flops_bwd / (per_call["backward"] * 1e-6) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # sample: the first expert's kept rows, forward and backward
        offs_h = offc.cpu().numpy()
        n_rows = int(offs_h[1])
        o = offs_h[:2].copy()
        xs_h, wg_h, wd_h = xs[:n_rows].cpu().numpy(), wgu_b[:1].cpu().numpy(), wd_b[:1].cpu().numpy()
        t1 = time.time()
        gu_o, _, _ = oracle.expert_train_forward(o, xs_h, wg_h, wd_h)
        oracle.expert_backward(o, xs_h, wg_h, wd_h, gu_o, dfs[:n_rows].cpu().numpy())
        dt = time.time() - t1
        cpu = {"value": round(n_rows / k / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"expert 0 ({n_rows} kept rows = {n_rows / k:.0f} token equivalents) forward + "
                         f"backward, oracle.expert_train_forward + expert_backward (double, one thread), "
                         f"{dt:.1f}s"}
    out = {
        "metric": "QAT training step of the MoE-FFN layer (router, routed + shared experts, forward + backward, drop-and-pad 1.5): tokens/s",
        "value": round(T / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (fake-quantised operands)",
        "data": "synthetic",
        "config": {"workload": "s_train_ffn", "tokens": T, "d_model": d, "experts": E, "top_k": k,
                   "hidden": h, "shared_hidden": hs, "capacity": C, "kept_rows": kept,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(bw_tf, 3), "peak": FP32_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bw_tf / FP32_MFMA_PEAK_TFLOPS, 5), "traffic": None,
                     "kernel": "k_gemm_f32 x4 + k_train_act_bwd (one mm_expert_backward_f32 call)",
                     "algorithmic_flops_per_launch": flops_bwd, "launch_us": per_call["backward"]},
        "cpu_baseline": cpu,
        "per_call_us": per_call,
        "forward_tflops": round(flops_fwd / (per_call["forward"] * 1e-6) / 1e12, 3),
        "step_matrix_tflops": round(flops_step / (ms * 1e-3) / 1e12, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
