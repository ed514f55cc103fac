#!/usr/bin/env python3
"""Benchmark of libmoedec on one MI355X: batch-1 MoE decode and the FP8 LM head.

One step is one Ling-shaped MoE layer at M = 1: top-8-of-512 routing (softmax
renormalised over the 8) and the 8 routed + 1 shared SwiGLU experts (MXFP4
weights, bf16 activations), run by moe_layer_mxfp4 as one kernel launch.  The steps cycle through
--layers distinct layers, each with its own 513 experts resident in HBM
(42 layers = 67.5 GB), so the 256 MB Infinity Cache cannot serve a repeated
expert.  Steps are captured into one HIP graph and replayed; HIP events on the
replay stream time exactly K steps.

Reported next to the headline (M = 1) figure, each measured the same way:
  * the same layers in the 4-token verify window (M = 4);
  * the two-call path (moe_route_topk, then moe_expert_ffn_mxfp4), and the
    FFN call alone on precomputed dispatch tables;
  * the LM head 157,184 x 2,560: one-off FP8 quantisation, FP8 GEMV at M = 1
    and 4, and the bf16 GEMV comparator;
  * the CPU oracle on a bounded sample of the same layers (cpu_baseline).

Bytes are algorithmic: the weights a step must read (codes + E8M0 scales of
the active experts, or of the whole LM head) plus its activations in and out.
GB/s = bytes / time, against MI355X's 8 TB/s HBM3E peak.

Only this script's cpu_baseline leg imports the oracle.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
EXPERT_BYTES_LING = 3 * (768 * 2560 // 2 + 768 * 2560 // 32)     # 3,133,440 B


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4200, help="timed MoE-layer steps (M = 1)")
    ap.add_argument("--warmup", type=int, default=420, help="untimed steps before timing")
    ap.add_argument("--layers", type=int, default=42, help="distinct layers the steps cycle through")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the LM-head measurements")
    ap.add_argument("--no-m4", action="store_true", help="skip the M = 4 measurement")
    ap.add_argument("--cpu-layers", type=int, default=3, help="layers in the CPU oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------
# Setup

def make_layers(m, synth, n_layers, dev):
    """Packed MXFP4 weights of n_layers Ling-shaped layers, generated on the device."""
    import torch
    import synth.device as sd
    shape = synth.LING
    layers = []
    for layer in range(n_layers):
        canon = sd.canonical_layer(0, layer, shape, dev)
        layers.append(m.MoELayerWeights.from_canonical(canon["gate"], canon["up"], canon["down"], shape.E))
        del canon
        if layer % 7 == 6 or layer == n_layers - 1:
            torch.cuda.synchronize()
            log(f"generated {layer + 1}/{n_layers} layers")
    return layers


def layer_inputs(synth, n_layers, M, dev):
    import numpy as np
    import torch
    shape = synth.LING
    xs, lgs = [], []
    for layer in range(n_layers):
        xb = synth.activations_bf16(0, layer, M, shape.H)
        lg = synth.logits_f32(0, layer, M, shape.E)
        xs.append(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev))
        lgs.append(torch.from_numpy(lg).to(dev))
    return xs, lgs


class Timer:
    """HIP events on torch's current stream, which is where the library
    launches (it is handed torch's current stream on every call)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn):
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)          # ms


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# ----------------------------------------------------------------------------
# MoE layer measurements

def moe_bench(m, torch, synth, layers, M, steps, warmup, dev):
    """Time K layer steps three ways: the fused layer call (routing + FFN in
    one launch; the headline), the two-call path (moe_route_topk then
    moe_expert_ffn_mxfp4) and the FFN call alone on precomputed tables."""
    n_layers = len(layers)
    shape = synth.LING
    k = shape.k
    xs, lgs = layer_inputs(synth, n_layers, M, dev)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    wts = torch.empty((M, k), dtype=torch.float32, device=dev)
    disp = [torch.zeros(m.DISPATCH_BYTES, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    ys = [torch.empty((M, shape.H), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    ws = m.make_ffn_workspace(M, k, shape.H, shape.I, dev)

    def fused_step(i):
        L = i % n_layers
        m.moe_layer(layers[L], xs[L], lgs[L], k, ws, y=ys[L], want_f32=False)

    def two_call_step(i):
        L = i % n_layers
        m.route_topk(lgs[L], k, ids=ids, weights=wts, dispatch=disp[L])
        m.expert_ffn(layers[L], xs[L], disp[L], k, ws, y=ys[L], want_f32=False)

    def ffn_only(i):
        L = i % n_layers
        m.expert_ffn(layers[L], xs[L], disp[L], k, ws, y=ys[L], want_f32=False)

    # one eager pass of each path: fills every layer's dispatch table, checks the calls work
    for i in range(n_layers):
        two_call_step(i)
        fused_step(i)
    torch.cuda.synchronize()
    n_slots = [m.decode_dispatch(d)["n_slots"] for d in disp]
    act_bytes = M * shape.E * 4 + 2 * M * shape.H * 2          # logits + x + y (bf16)
    bytes_per_layer = [s * EXPERT_BYTES_LING + act_bytes for s in n_slots]
    # steps cycle through the layers: average bytes over the steps actually run
    step_bytes = sum(bytes_per_layer[i % n_layers] for i in range(steps)) / steps

    t = Timer(torch)
    g_warm = capture(torch, lambda: [fused_step(i) for i in range(warmup)]) if warmup else None
    g_main = capture(torch, lambda: [fused_step(i) for i in range(steps)])
    g_two = capture(torch, lambda: [two_call_step(i) for i in range(steps)])
    g_ffn = capture(torch, lambda: [ffn_only(i) for i in range(steps)])
    if g_warm is not None:
        g_warm.replay()
    g_two.replay()
    g_ffn.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = t.run(g_main.replay)
    wall1 = time.perf_counter()
    ms_two = t.run(g_two.replay)
    ms_ffn = t.run(g_ffn.replay)
    ffn_bytes = step_bytes - M * shape.E * 4                   # no logits read
    res = {
        "M": M,
        "layers": n_layers,
        "steps": steps,
        "ms_total": ms,
        "wall_s": wall1 - wall0,
        "us_per_layer": 1e3 * ms / steps,
        "bytes_per_layer": step_bytes,
        "gbs": step_bytes / (1e6 * ms / steps),
        "two_call_us_per_layer": 1e3 * ms_two / steps,
        "two_call_gbs": step_bytes / (1e6 * ms_two / steps),
        "ffn_us": 1e3 * ms_ffn / steps,
        "ffn_bytes": ffn_bytes,
        "ffn_gbs": ffn_bytes / (1e6 * ms_ffn / steps),
        "mean_active_experts": sum(s - 1 for s in n_slots) / n_layers,
        "max_active_experts": max(s - 1 for s in n_slots),
    }
    res["frac_of_peak"] = res["gbs"] / PEAK_HBM_GBS
    res["two_call_frac_of_peak"] = res["two_call_gbs"] / PEAK_HBM_GBS
    res["ffn_frac_of_peak"] = res["ffn_gbs"] / PEAK_HBM_GBS
    del g_warm, g_main, g_two, g_ffn
    return res


# ----------------------------------------------------------------------------
# LM head measurements

def lmhead_bench(m, torch, synth, dev, reps=50):
    import numpy as np
    V, H = synth.LMHEAD_V, synth.LMHEAD_H
    log("generating LM-head weights", V, "x", H)
    wb = synth.lmhead_weight_bf16(0, V, H)
    w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev)
    del wb
    t = Timer(torch)
    head = m.lmhead_quant_fp8(w)
    torch.cuda.synchronize()
    g_q = capture(torch, lambda: [m.lmhead_quant_fp8(w) for _ in range(5)])
    ms_q = t.run(g_q.replay) / 5
    # the captured quantisations rewrote fresh buffers; keep the first head
    del g_q
    out = {"quant_us": 1e3 * ms_q,
           "quant_bytes": V * H * 2 + V * H + V * 4,
           }
    out["quant_gbs"] = out["quant_bytes"] / (1e6 * ms_q)
    for M in (1, 4):
        xb = synth.lmhead_x_bf16(0, M, H)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        lo = torch.empty((M, V), dtype=torch.float32, device=dev)
        m.lmhead_gemv_fp8(head, x, out=lo)
        m.lmhead_gemv_bf16(w, x, out=lo)
        g8 = capture(torch, lambda: [m.lmhead_gemv_fp8(head, x, out=lo) for _ in range(reps)])
        gb = capture(torch, lambda: [m.lmhead_gemv_bf16(w, x, out=lo) for _ in range(reps)])
        g8.replay()
        gb.replay()
        ms8 = t.run(g8.replay) / reps
        msb = t.run(gb.replay) / reps
        b8 = V * H + V * 4 + M * H * 2 + M * V * 4
        bb = V * H * 2 + M * H * 2 + M * V * 4
        out[f"fp8_m{M}_us"] = 1e3 * ms8
        out[f"fp8_m{M}_bytes"] = b8
        out[f"fp8_m{M}_gbs"] = b8 / (1e6 * ms8)
        out[f"fp8_m{M}_frac_of_peak"] = b8 / (1e6 * ms8) / PEAK_HBM_GBS
        out[f"bf16_m{M}_us"] = 1e3 * msb
        out[f"bf16_m{M}_gbs"] = bb / (1e6 * msb)
        out[f"bf16_m{M}_frac_of_peak"] = bb / (1e6 * msb) / PEAK_HBM_GBS
        del g8, gb
    del head, w
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)

def cpu_baseline(synth, n_layers):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:                     # pragma: no cover - threadpoolctl is installed
        limiter = None
    shape = synth.LING
    total_s = 0.0
    total_bytes = 0
    for layer in range(n_layers):
        xb = synth.activations_bf16(0, layer, 1, shape.H)
        lg = synth.logits_f32(0, layer, 1, shape.E)
        # input preparation, untimed: regenerate only the experts this layer routes to
        pre_ids, _ = oracle.route_topk(lg, shape.k)
        canon = {int(e): synth.mxfp4_expert(0, layer, int(e), shape) for e in list(pre_ids[0]) + [shape.E]}
        x = synth.bf16_values(xb).astype(np.float64)
        t0 = time.perf_counter()
        ids, w = oracle.route_topk(lg, shape.k)
        dense = {e: tuple(oracle.mxfp4_dequant(*canon[int(e)][n]) for n in ("gate", "up", "down"))
                 for e in list(ids[0]) + [shape.E]}
        oracle.moe_layer(x, ids, w, lambda e: dense[e], dense[shape.E])
        total_s += time.perf_counter() - t0
        total_bytes += (shape.k + 1) * EXPERT_BYTES_LING + shape.E * 4 + 2 * shape.H * 2
        log(f"oracle layer {layer}: {total_s:.2f} s so far")
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": total_bytes / (1e9 * total_s),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{n_layers} Ling-shaped MoE layers at M=1 (route + MXFP4 dequant of the 9 active "
                  f"experts + SwiGLU FFN in float64, numpy, BLAS limited to 1 thread): "
                  f"{1e6 * total_s / n_layers:.0f} us/layer",
        "us_per_layer": 1e6 * total_s / n_layers,
        "host_cores_available": len(os.sched_getaffinity(0)),
        "host_cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------

def copy_probe(torch, dev):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    t = Timer(torch)
    for _ in range(3):
        ms = t.run(lambda: b.copy_(a))
    print(json.dumps({"copy_probe_bytes_each_way": n, "ms": ms, "gbs": 2 * n / (1e6 * ms)}), flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(torch, dev)
        return 0
    import bit_moe_expert_topk_amd as m
    import synth

    log(f"device: {torch.cuda.get_device_name(0)}; layers {args.layers}, steps {args.steps}, warmup {args.warmup}")
    layers = make_layers(m, synth, args.layers, dev)
    r1 = moe_bench(m, torch, synth, layers, 1, args.steps, args.warmup, dev)
    log("M=1:", json.dumps(r1))
    r4 = None
    if not args.no_m4:
        r4 = moe_bench(m, torch, synth, layers, 4, args.steps, args.warmup, dev)
        log("M=4:", json.dumps(r4))
    del layers
    torch.cuda.empty_cache()
    lm = None
    if not args.no_lmhead:
        lm = lmhead_bench(m, torch, synth, dev)
        log("LM head:", json.dumps(lm))
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(synth, args.cpu_layers)
        log("cpu:", json.dumps(cpu))

    line = {
        "metric": "µs/MoE layer + achieved HBM GB/s (% of peak) at M=1 and M=4; LM-head GEMV GB/s",
        "value": round(r1["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1["us_per_layer"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4xbf16->f32",
        "data": "synthetic (seeded MXFP4 codes/E8M0 scales, N(0,1) bf16 activations and fp32 logits)",
        "config": {
            "workload": "Ling-shaped MoE layer decode, M=1: hidden 2560, 512 routed experts top-8 + 1 shared, "
                        "SwiGLU intermediate 768, MXFP4 experts, bf16 activations; "
                        f"steps cycle over {args.layers} layers resident in HBM",
            "M": 1,
            "layers_resident": args.layers,
        },
        "us_per_layer_m1": round(r1["us_per_layer"], 3),
        "frac_of_peak_m1": round(r1["frac_of_peak"], 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "moe_ffn_kernel (moe_layer_mxfp4: routing + routed/shared MXFP4 SwiGLU FFN, M=1)",
            "achieved": round(r1["gbs"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(r1["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": None,
            "bytes_per_launch": r1["bytes_per_layer"],
            "avg_launch_us": round(r1["us_per_layer"], 3),
        },
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "extra": {"m1": r1, "m4": r4, "lmhead": lm,
                  "cpu": cpu},
    }
    if r4 is not None:
        line["us_per_layer_m4"] = round(r4["us_per_layer"], 3)
        line["gbs_m4"] = round(r4["gbs"], 1)
        line["frac_of_peak_m4"] = round(r4["frac_of_peak"], 4)
    if lm is not None:
        line["lmhead_fp8_gbs_m1"] = round(lm["fp8_m1_gbs"], 1)
        line["lmhead_fp8_gbs_m4"] = round(lm["fp8_m4_gbs"], 1)
        line["lmhead_bf16_gbs_m1"] = round(lm["bf16_m1_gbs"], 1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
