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
  * the cold stack: passes over the layers in order on a residual stream
    (moe_layer_rmsnorm_mxfp4), each layer's input formed from the previous
    layer's output, as a HIP graph and eagerly;
  * the LM head 157,184 x 2,560: one-off FP8 quantisation, FP8 GEMV at M = 1
    and 4 (weight-only, and with dynamic per-token FP8 activations), and the
    bf16 GEMV comparator;
  * the many-token layer (moe_layer_mxfp4_prefill: a prefill chunk or a long
    verify window, grouped GEMM on bf16 matrix cores) on one layer's experts
    at T = 512 .. 32,768 tokens: µs per layer and algorithmic TFLOP/s against
    the 2.5 PFLOP/s dense bf16 peak;
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
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 (and fp4 x fp8) matrix peak
PREFILL_TOKENS = (512, 2048, 8192, 32768)
TRAFFIC_FILE = "moe_ffn_kernel_ling_m{M}_hbm_traffic.md"
COPY_PROBE_ELEMS = 1 << 28                 # float32: 1 GiB read and 1 GiB written
PMC_KERNEL = "moe_ffn_kernel"
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
    ap.add_argument("--no-fp8-shared", action="store_true", help="skip the FP8 shared-expert layer")
    ap.add_argument("--no-m4", action="store_true", help="skip the M = 4 measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the many-token (prefill) layer")
    ap.add_argument("--prefill-tokens", type=int, nargs="+", default=list(PREFILL_TOKENS),
                    help="token counts of the many-token layer measurement")
    ap.add_argument("--no-stack", action="store_true", help="skip the residual-stack measurement")
    ap.add_argument("--no-router", action="store_true", help="skip the router-logits measurement")
    ap.add_argument("--stack-passes", type=int, default=100, help="graph passes over the layers (stack)")
    ap.add_argument("--cpu-layers", type=int, default=3, help="layers in the CPU oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short eager run for rocprofv3 --pmc: a calibration copy of known size, "
                         "then fused layers of --pmc-m tokens")
    ap.add_argument("--pmc-m", type=int, default=1, choices=(1, 4), help="tokens per layer in --pmc-run")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --pmc-run (FETCH_SIZE, then WRITE_SIZE) "
                         "into the markdown file given by --traffic-out")
    ap.add_argument("--traffic-out", default=None,
                    help="default: profiles/" + TRAFFIC_FILE.format(M="<M>"))
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
    """Time K layer steps four ways: the fused layer call (routing + FFN in
    one launch; the headline), the two-call path (moe_route_topk then
    moe_expert_ffn_mxfp4), the FFN call alone on precomputed tables, and the
    fused layer with MXFP8 activations (moe_layer_mxfp4_a8, W4A8)."""
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

    def fused_a8(i):
        L = i % n_layers
        m.moe_layer(layers[L], xs[L], lgs[L], k, ws, y=ys[L], want_f32=False, act8=True)

    # one eager pass of each path: fills every layer's dispatch table, checks the calls work
    for i in range(n_layers):
        two_call_step(i)
        fused_a8(i)
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
    g_a8 = capture(torch, lambda: [fused_a8(i) for i in range(steps)])
    if g_warm is not None:
        g_warm.replay()
    g_two.replay()
    g_ffn.replay()
    g_a8.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = t.run(g_main.replay)
    wall1 = time.perf_counter()
    ms_two = t.run(g_two.replay)
    ms_ffn = t.run(g_ffn.replay)
    ms_a8 = t.run(g_a8.replay)
    m.check_ffn_workspace(ws)              # raises if a cross-block wait gave up
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
        "a8_us_per_layer": 1e3 * ms_a8 / steps,
        "mean_active_experts": sum(s - 1 for s in n_slots) / n_layers,
        "max_active_experts": max(s - 1 for s in n_slots),
    }
    res["frac_of_peak"] = res["gbs"] / PEAK_HBM_GBS
    res["two_call_frac_of_peak"] = res["two_call_gbs"] / PEAK_HBM_GBS
    res["ffn_frac_of_peak"] = res["ffn_gbs"] / PEAK_HBM_GBS
    del g_warm, g_main, g_two, g_ffn, g_a8
    return res


def shared_fp8_bench(m, torch, synth, layers, steps, dev):
    """The fused layer with its shared expert stored in FP8 (E4M3, float32 row
    scales; pack_shared_fp8 of seeded bf16 weights per layer) instead of MXFP4,
    the routed experts unchanged, at M = 1 and 4 (steps cycle over the layers)."""
    import numpy as np
    n_layers = len(layers)
    shape = synth.LING
    E, H, I, k = shape.E, shape.H, shape.I, shape.k
    s8 = m.shared_fp8_sizes(H, I)
    sh_bytes = s8.gu_codes + s8.gu_scales + s8.dn_codes + s8.dn_scales
    fp8_layers = []
    for L, W in enumerate(layers):
        g, u, d = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
                   for a in synth.shared_expert_bf16(0, L, H, I))
        sh8 = m.pack_shared_fp8(g, u, d)
        fp8_layers.append(m.MoELayerWeights(E, H, I, W.gu_codes, W.gu_scales, W.dn_codes, W.dn_scales,
                                            shared_fp8=sh8))
    torch.cuda.synchronize()
    t = Timer(torch)
    out = {"shared_bytes_fp8": sh_bytes, "shared_bytes_mxfp4": EXPERT_BYTES_LING}
    for M in (1, 4):
        xs, lgs = layer_inputs(synth, n_layers, M, dev)
        ws = m.make_ffn_workspace(M, k, H, I, dev)
        ys = [torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
        disp = [torch.zeros(m.DISPATCH_BYTES, dtype=torch.uint8, device=dev) for _ in range(n_layers)]

        def step(i):
            L = i % n_layers
            m.moe_layer(fp8_layers[L], xs[L], lgs[L], k, ws, y=ys[L], want_f32=False, dispatch=disp[L])

        for i in range(n_layers):
            step(i)
        torch.cuda.synchronize()
        n_routed = [m.decode_dispatch(dd)["n_slots"] - 1 for dd in disp]
        act = M * E * 4 + 2 * M * H * 2
        step_bytes = sum(n_routed[i % n_layers] * EXPERT_BYTES_LING + sh_bytes + act for i in range(steps)) / steps
        g_main = capture(torch, lambda: [step(i) for i in range(steps)])
        g_main.replay()
        ms = t.run(g_main.replay)
        m.check_ffn_workspace(ws)
        out[f"m{M}_us_per_layer"] = 1e3 * ms / steps
        out[f"m{M}_bytes_per_layer"] = step_bytes
        out[f"m{M}_gbs"] = step_bytes / (1e6 * ms / steps)
        del g_main
    del fp8_layers
    return out


def prefill_bench(m, torch, synth, layers, dev, tokens=PREFILL_TOKENS):
    """The many-token layer on layer 0's experts: T tokens of N(0,1) bf16
    activations with N(0,1) router logits, routed top-8 of 512 plus the shared
    expert.  Algorithmic flops per (token, expert) pair: 2 * (2 I H) for
    gate/up and 2 H I for down, over the T * (k + 1) pairs (the bf16 kernels
    carry h as two bf16 halves, so the down product runs twice on the
    matrix cores; that is not counted).  Each T is timed for both variants:
    bf16 activations (moe_layer_mxfp4_prefill) and MXFP8 activations
    (moe_layer_mxfp4_prefill_a8, keys suffixed _a8)."""
    shape = synth.LING
    E, H, I, k = shape.E, shape.H, shape.I, shape.k
    W = layers[0]
    t = Timer(torch)
    out = {}
    for T in tokens:
        x = torch.from_numpy(synth.activations_bf16(0, 0, T, H).view("int16")).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(synth.logits_f32(0, 0, T, E)).to(dev)
        ws = m.make_prefill_workspace(T, E, k, H, I, dev)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        counts = torch.empty(E + 1, dtype=torch.int32, device=dev)

        reps = max(5, min(50, 80000 // T))
        flops = T * (k + 1) * 6 * H * I
        r = {"reps": reps}
        for sfx, act8 in (("", False), ("_a8", True)):
            def call():
                m.moe_layer_prefill(W, x, lg, k, workspace=ws, y=y, want_f32=False, counts=counts, act8=act8)

            call()
            call()
            ms = t.run(lambda: [call() for _ in range(reps)])
            us = 1e3 * ms / reps
            active = int((counts[:E] > 0).sum().item()) + 1
            r.update({
                "us_per_layer" + sfx: us,
                "tflops" + sfx: flops / us / 1e6,
                "weight_gbs" + sfx: active * EXPERT_BYTES_LING / us / 1e3,
            })
        r["frac_of_bf16_peak"] = r["tflops"] / PEAK_BF16_TFLOPS
        r["frac_of_fp8_peak_a8"] = r["tflops_a8"] / PEAK_FP8_TFLOPS
        r["active_experts"] = active
        out[str(T)] = r
        del ws, x, lg, y
        torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# Cold stack: the layers in sequence on a residual stream

def stack_bench(m, torch, synth, layers, passes, eager_passes, dev):
    """Passes over all layers in order at M = 1, each layer on the residual
    stream, so every layer's input depends on the previous layer's output.
    Two forms: routed from pre-drawn logits (moe_layer_rmsnorm_mxfp4: x =
    bf16(RMSNorm(r)), r += MoE layer(x)), and routed from its own data
    (moe_layer_rmsnorm_router_mxfp4: the same with the router logits x W_router^T
    of each layer's own bf16 router [512][2560] in front).  Each is timed as a
    HIP graph of `passes` passes and eagerly (from Python)."""
    import numpy as np
    n_layers = len(layers)
    shape = synth.LING
    k = shape.k
    _, lgs = layer_inputs(synth, n_layers, 1, dev)
    wrs = [torch.from_numpy(synth.router_weight_bf16(0, L, shape.E, shape.H).view(np.int16))
           .view(torch.bfloat16).to(dev) for L in range(n_layers)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    r0 = torch.randn((1, shape.H), generator=gen, device=dev, dtype=torch.float32)
    bufs = [r0.clone(), torch.empty_like(r0)]
    lg_own = torch.empty((1, shape.E), dtype=torch.float32, device=dev)
    ws = m.make_ffn_workspace(1, k, shape.H, shape.I, dev)

    def pass_given():
        for L in range(n_layers):
            m.moe_layer_rmsnorm(layers[L], bufs[L % 2], lgs[L], k, ws, r_out=bufs[(L + 1) % 2])
        if n_layers % 2:
            bufs.reverse()

    def pass_routed():
        for L in range(n_layers):
            m.moe_layer_rmsnorm_router(layers[L], wrs[L], bufs[L % 2], k, ws, r_out=bufs[(L + 1) % 2],
                                       logits=lg_own)
        if n_layers % 2:
            bufs.reverse()

    t = Timer(torch)
    steps_g, steps_e = passes * n_layers, eager_passes * n_layers
    out = {"layers": n_layers, "passes_graph": passes, "passes_eager": eager_passes}
    for name, one_pass in (("", pass_given), ("routed_", pass_routed)):
        bufs[0].copy_(r0)
        one_pass()
        torch.cuda.synchronize()
        g = capture(torch, lambda: [one_pass() for _ in range(passes)])
        g.replay()
        ms_graph = t.run(g.replay)
        del g
        one_pass()
        ms_eager = t.run(lambda: [one_pass() for _ in range(eager_passes)])
        m.check_ffn_workspace(ws)
        layer_bytes = (shape.k + 1) * EXPERT_BYTES_LING + shape.E * 4 + 2 * shape.H * 4   # + r in, r out
        if name:
            layer_bytes += shape.E * shape.H * 2                                         # the router
        out.update({
            name + "us_per_layer_graph": 1e3 * ms_graph / steps_g,
            name + "us_per_layer_eager": 1e3 * ms_eager / steps_e,
            name + "us_per_pass_graph": 1e3 * ms_graph / passes,
            name + "bytes_per_layer": layer_bytes,
            name + "gbs_graph": layer_bytes * steps_g / (1e6 * ms_graph),
            name + "frac_of_peak_graph": layer_bytes * steps_g / (1e6 * ms_graph) / PEAK_HBM_GBS,
            name + "residual_finite": bool(torch.isfinite(bufs[0]).all().item()),
        })
    del wrs
    return out


def router_bench(m, torch, synth, layers, steps, dev, n_router=128):
    """The step before routing: router logits from x (moe_router_logits_bf16,
    bf16 W_router [512][2560], seeded N(0, 1/H)), alone over n_router distinct
    matrices (335 MB, beyond the Infinity Cache) at M = 1 and 4, and in front
    of the fused layer at M = 1 (router logits, then moe_layer_mxfp4 on them)."""
    shape = synth.LING
    E, H, k = shape.E, shape.H, shape.k
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    wrs = [(torch.randn((E, H), generator=gen, device=dev) * (1.0 / H ** 0.5)).to(torch.bfloat16)
           for _ in range(n_router)]
    t = Timer(torch)
    out = {"E": E, "H": H, "matrices": n_router, "bytes_per_call_m1": E * H * 2 + H * 2 + E * 4}
    for M in (1, 4):
        xs, _ = layer_inputs(synth, 4, M, dev)
        lg = torch.empty((M, E), dtype=torch.float32, device=dev)
        reps = 2 * n_router
        m.router_logits(wrs[0], xs[0], out=lg)
        g = capture(torch, lambda: [m.router_logits(wrs[i % n_router], xs[i % 4], out=lg) for i in range(reps)])
        g.replay()
        ms = t.run(g.replay)
        out[f"us_m{M}"] = 1e3 * ms / reps
        out[f"gbs_m{M}"] = (E * H * 2 + M * H * 2 + M * E * 4) / (1e3 * out[f"us_m{M}"])
        del g
    # router + fused layer, M = 1, cycling over the resident layers
    n_layers = len(layers)
    xs, _ = layer_inputs(synth, n_layers, 1, dev)
    lg = torch.empty((1, E), dtype=torch.float32, device=dev)
    ws = m.make_ffn_workspace(1, k, H, shape.I, dev)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)

    def step(i):
        L = i % n_layers
        m.router_logits(wrs[L % n_router], xs[L], out=lg)
        m.moe_layer(layers[L], xs[L], lg, k, ws, y=y, want_f32=False)

    step(0)
    g = capture(torch, lambda: [step(i) for i in range(steps)])
    g.replay()
    ms = t.run(g.replay)
    out["router_plus_layer_us_m1"] = 1e3 * ms / steps
    m.check_ffn_workspace(ws)
    del g, wrs
    torch.cuda.empty_cache()
    return out


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
        # the same head with dynamic per-token FP8 activations
        dyn = m.lmhead_dynamic_act(head)
        m.lmhead_gemv_fp8(dyn, x, out=lo)
        gd = capture(torch, lambda: [m.lmhead_gemv_fp8(dyn, x, out=lo) for _ in range(reps)])
        # greedy decode: FP8 GEMV with the argmax epilogue, logits not written
        aws = m.make_lmhead_workspace(V, M, dev)
        ids = torch.empty(M, dtype=torch.int32, device=dev)
        m.lmhead_argmax_fp8(head, x, workspace=aws, ids=ids)
        ga = capture(torch, lambda: [m.lmhead_argmax_fp8(head, x, workspace=aws, ids=ids) for _ in range(reps)])
        # sampled decode (temperature 0.6, top-p 0.95, top-k 29): logits written,
        # candidates and draw in the same launch
        u = torch.from_numpy(synth.sampling_uniforms(0, 0, M)).to(dev)
        m.lmhead_sample_fp8(head, x, u, 0.6, 0.95, 29, workspace=aws, ids=ids, logits=lo)
        gs = capture(torch, lambda: [m.lmhead_sample_fp8(head, x, u, 0.6, 0.95, 29, workspace=aws, ids=ids,
                                                         logits=lo) for _ in range(reps)])
        g8.replay()
        gb.replay()
        ga.replay()
        gs.replay()
        gd.replay()
        msd = t.run(gd.replay) / reps
        ms8 = t.run(g8.replay) / reps
        msb = t.run(gb.replay) / reps
        msa = t.run(ga.replay) / reps
        mss = t.run(gs.replay) / reps
        out[f"fp8_argmax_m{M}_us"] = 1e3 * msa
        out[f"fp8_argmax_m{M}_gbs"] = (V * H + V * 4 + M * H * 2) / (1e6 * msa)
        out[f"fp8_sample_m{M}_us"] = 1e3 * mss
        b8 = V * H + V * 4 + M * H * 2 + M * V * 4
        bb = V * H * 2 + M * H * 2 + M * V * 4
        out[f"fp8_dynact_m{M}_us"] = 1e3 * msd
        out[f"fp8_dynact_m{M}_gbs"] = b8 / (1e6 * msd)
        out[f"fp8_m{M}_us"] = 1e3 * ms8
        out[f"fp8_m{M}_bytes"] = b8
        out[f"fp8_m{M}_gbs"] = b8 / (1e6 * ms8)
        out[f"fp8_m{M}_frac_of_peak"] = b8 / (1e6 * ms8) / PEAK_HBM_GBS
        out[f"bf16_m{M}_us"] = 1e3 * msb
        out[f"bf16_m{M}_gbs"] = bb / (1e6 * msb)
        out[f"bf16_m{M}_frac_of_peak"] = bb / (1e6 * msb) / PEAK_HBM_GBS
        del g8, gb, ga, gs, gd
    del head, w
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded samples of the same workloads)
#
# The oracle functions run unchanged.  Each measurement runs jobs in worker
# processes (spawned, so they never inherit this process's GPU state), one
# BLAS thread each: the 1-thread setting runs its jobs one after another in a
# single worker; the all-cores setting runs one job per host core at once
# (whole layers, or row chunks of the LM head) and takes the wall time from
# the common start (a barrier after each worker has prepared its inputs) to
# the last finish.  Input preparation (drawing the synthetic weights, and
# quantising the LM-head sample) is never timed.

_CPU_BARRIER = None


def _cpu_worker_init(barrier):
    global _CPU_BARRIER
    _CPU_BARRIER = barrier
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:                     # pragma: no cover - threadpoolctl is installed
        pass


def _cpu_job(args):
    """One oracle job: ("moe", layer, M) = route + MXFP4 dequantisation of the
    layer's active experts + the float64 SwiGLU layer; ("lmhead", chunk, rows)
    = the FP8 LM-head GEMV on `rows` rows.  Returns (t0, t1, algorithmic bytes)."""
    import numpy as np
    import oracle
    import synth
    kind, idx, n = args
    if kind == "moe":
        shape = synth.LING
        M = n
        xb = synth.activations_bf16(0, idx, M, shape.H)
        lg = synth.logits_f32(0, idx, M, shape.E)
        pre_ids, _ = oracle.route_topk(lg, shape.k)
        active = sorted(set(int(e) for e in pre_ids.flatten()))
        canon = {e: synth.mxfp4_expert(0, idx, e, shape) for e in active + [shape.E]}
        x = synth.bf16_values(xb).astype(np.float64)
        nbytes = (len(active) + 1) * EXPERT_BYTES_LING + M * shape.E * 4 + 2 * M * shape.H * 2
        _CPU_BARRIER.wait()
        t0 = time.perf_counter()
        ids, w = oracle.route_topk(lg, shape.k)
        dense = {e: tuple(oracle.mxfp4_dequant(*canon[e][nm]) for nm in ("gate", "up", "down")) for e in canon}
        oracle.moe_layer(x, ids, w, lambda e: dense[int(e)], dense[shape.E])
        t1 = time.perf_counter()
    else:
        rows, H = n, synth.LMHEAD_H
        wb = synth.lmhead_weight_bf16(1000 + idx, rows, H)
        codes, scale = oracle.lmhead_quant_fp8(synth.bf16_values(wb))
        x = synth.bf16_values(synth.lmhead_x_bf16(0, 1, H)).astype(np.float64)
        nbytes = rows * H + rows * 4 + rows * 4 + H * 2 * rows / synth.LMHEAD_V
        _CPU_BARRIER.wait()
        t0 = time.perf_counter()
        oracle.lmhead_gemv_fp8(codes, scale, x)
        t1 = time.perf_counter()
    return t0, t1, nbytes


def _cpu_run(jobs, workers):
    """Run jobs in `workers` spawned processes; with one worker they run one
    after another.  Returns (algorithmic bytes / s, seconds timed, bytes)."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers)
    with ctx.Pool(workers, initializer=_cpu_worker_init, initargs=(barrier,)) as pool:
        res = pool.map(_cpu_job, jobs, chunksize=1)
    nbytes = sum(r[2] for r in res)
    if workers == 1:
        secs = sum(r[1] - r[0] for r in res)
    else:
        secs = max(r[1] for r in res) - min(r[0] for r in res)
    return nbytes / secs, secs, nbytes


def cpu_baseline(synth, n_layers):
    """The oracle on the host: Ling-shaped M = 1 layers (the headline workload),
    M = 4 layers and an FP8 LM-head row sample, each at 1 thread and at all
    host cores.  The headline figure is M = 1 at all cores."""
    cores = len(os.sched_getaffinity(0))
    lm_rows = 8192
    settings = {}
    plans = {
        "m1": ([("moe", L, 1) for L in range(n_layers)], [("moe", L, 1) for L in range(cores)]),
        "m4": ([("moe", 0, 4)], [("moe", L, 4) for L in range(cores)]),
        "lmhead_fp8_m1": ([("lmhead", 0, lm_rows)], [("lmhead", c, lm_rows) for c in range(cores)]),
    }
    for name, (one, many) in plans.items():
        for label, jobs, workers in (("1_thread", one, 1), ("all_cores", many, cores)):
            t0 = time.perf_counter()
            gbs, secs, nbytes = _cpu_run(jobs, workers)
            entry = {"gbs": gbs / 1e9, "seconds_timed": secs, "bytes": nbytes, "jobs": len(jobs),
                     "threads": workers, "wall_incl_setup_s": time.perf_counter() - t0}
            if name != "lmhead_fp8_m1":
                entry["us_per_layer"] = 1e6 * secs / (len(jobs) if workers == 1 else len(jobs) / workers)
            else:
                entry["us_per_token_full_head"] = 1e6 * (synth.LMHEAD_V * (synth.LMHEAD_H + 8)) / gbs
            settings[f"{name}_{label}"] = entry
            log(f"oracle {name} {label}: {entry}")
    head = settings["m1_all_cores"]
    return {
        "value": head["gbs"],
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{cores} Ling-shaped MoE layers at M=1 run at once, one per host core (route + MXFP4 "
                  f"dequant of the 9 active experts + SwiGLU FFN in float64, numpy, 1 BLAS thread each); "
                  f"{head['seconds_timed']:.2f} s wall; 1 thread: "
                  f"{settings['m1_1_thread']['gbs']:.4f} GB/s ({settings['m1_1_thread']['us_per_layer']:.0f} us/layer)",
        "settings": settings,
        "host_cores_available": cores,
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


# ----------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters

def kernel_source_hash():
    """Hash of what defines the measured kernel's code: its source file, the
    device headers it includes and the ABI header's structure definitions and
    constants that those files name (other entry points' declarations and
    structures do not count)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_moe_expert_topk_amd", "csrc")
    used = set()
    for name in ("ffn_mxfp4.hip", "device_common.h", "route_device.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            text = f.read()
        h.update(name.encode() + b"\0" + text)
        used.update(re.findall(r"MOEDEC_\w+|moedec_\w+", text.decode()))
    with open(os.path.join(ROOT, "include", "moedec.h")) as f:
        header = f.read()
    for block in re.findall(r"typedef struct[^}]*\}[^;]*;", header):
        name = re.search(r"\}\s*(\w+)\s*;", block).group(1)
        if name in used:
            h.update(block.encode() + b"\0")
    for name, value in sorted(re.findall(r"#define (MOEDEC_\w+)\s+([^\n/]*)", header)):
        if name in used:
            h.update(f"{name}={value.strip()}".encode() + b"\0")
    return h.hexdigest()[:16]


def pmc_run(m, torch, synth, dev, M=1, n_layers=8, passes=2):
    """Dispatches for the counter runs: three float32 copies of COPY_PROBE_ELEMS
    elements (an elementwise kernel with known bytes), then `passes` eager
    passes of the fused layer (M tokens) over n_layers layers."""
    a = torch.ones(COPY_PROBE_ELEMS, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b
    layers = make_layers(m, synth, n_layers, dev)
    k = synth.LING.k
    xs, lgs = layer_inputs(synth, n_layers, M, dev)
    ws = m.make_ffn_workspace(M, k, synth.LING.H, synth.LING.I, dev)
    y = torch.empty((M, synth.LING.H), dtype=torch.bfloat16, device=dev)
    for _ in range(passes):
        for L in range(n_layers):
            m.moe_layer(layers[L], xs[L], lgs[L], k, ws, y=y, want_f32=False)
    torch.cuda.synchronize()
    m.check_ffn_workspace(ws)
    log(f"pmc run: {passes} x {n_layers} fused M={M} layers")


def algorithmic_layer_bytes(synth, M, n_layers=8):
    """Bytes a fused layer must move, per layer of the counter run: every
    active expert's packed bytes once (the distinct top-k experts of the M
    tokens, plus the shared expert), the logits, x and y.  The expert count
    comes from the same seeded logits (top-k by value; ties have probability
    zero for these inputs)."""
    import numpy as np
    shape = synth.LING
    out = []
    for layer in range(n_layers):
        lg = synth.logits_f32(0, layer, M, shape.E)
        active = np.unique(np.argsort(-lg, axis=1, kind="stable")[:, :shape.k])
        out.append((len(active) + 1) * EXPERT_BYTES_LING + M * shape.E * 4 + 2 * M * shape.H * 2)
    return out


def _counter_rows(run_dir, counter):
    """(kernel name, value) per dispatch from a rocprofv3 csv counter file."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, fn)) as f:
                    for r in csv.DictReader(f):
                        if r.get("Counter_Name") == counter:
                            rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_summary(fetch_dir, write_dir, out_path, M):
    """Per-dispatch HBM bytes of the fused layer kernel (M tokens): FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by bytes / counter of the
    calibration copy, against the algorithmic bytes of the same layers."""
    import statistics
    import synth
    copy_bytes = COPY_PROBE_ELEMS * 4
    res = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(run_dir, counter)
        cal = [v for name, v in rows if "elementwise" in name.lower() and v * 1024 > copy_bytes / 2]
        ker = [v for name, v in rows if PMC_KERNEL in name]
        if not cal or not ker:
            raise SystemExit(f"{counter}: no calibration ({len(cal)}) or kernel ({len(ker)}) dispatches in {run_dir}")
        factor = copy_bytes / (1024 * statistics.median(cal))
        res[counter] = {"kib_per_dispatch": statistics.mean(ker), "dispatches": len(ker),
                        "calibration_kib": statistics.median(cal), "factor": factor,
                        "bytes_per_dispatch": 1024 * statistics.mean(ker) * factor}
    total = res["FETCH_SIZE"]["bytes_per_dispatch"] + res["WRITE_SIZE"]["bytes_per_dispatch"]
    algo = statistics.mean(algorithmic_layer_bytes(synth, M))
    summary = {"kernel": f"{PMC_KERNEL} (fused M={M} Ling layer)", "M": M, "source_hash": kernel_source_hash(),
               "fetch_bytes": round(res["FETCH_SIZE"]["bytes_per_dispatch"]),
               "write_bytes": round(res["WRITE_SIZE"]["bytes_per_dispatch"]),
               "traffic_bytes": round(total), "algorithmic_bytes": round(algo),
               "traffic_over_algorithmic": round(total / algo, 4)}
    def rel(d):
        d = os.path.abspath(d)
        return os.path.relpath(d, ROOT) if d.startswith(ROOT + os.sep) else d

    fetch_dir, write_dir = rel(fetch_dir), rel(write_dir)
    lines = [
        f"# HBM traffic of the fused MoE layer kernel, Ling-shaped layer, M = {M}",
        "",
        "Commands (R = the repository root on the GPU host; the profiler runs from /tmp):",
        "",
        "```",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d R/{fetch_dir} -o run -- python3 R/bench.py --pmc-run --pmc-m {M}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d R/{write_dir} -o run -- python3 R/bench.py --pmc-run --pmc-m {M}",
        f"python3 bench.py --traffic-from {fetch_dir} {write_dir} --pmc-m {M} --traffic-out <this file>",
        "```",
        "",
        "Calibration: an elementwise float32 copy of 2^28 elements (1 GiB read, 1 GiB written);",
        "factor = known bytes / counter bytes.",
        "",
        "| counter | KiB per dispatch (mean) | dispatches | calibration KiB | factor | bytes per dispatch |",
        "|---|---|---|---|---|---|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        lines.append(f"| {c} | {r['kib_per_dispatch']:.1f} | {r['dispatches']} | {r['calibration_kib']:.0f} | "
                     f"{r['factor']:.4f} | {r['bytes_per_dispatch']:.0f} |")
    lines += ["",
              f"Algorithmic bytes per launch (mean over the {len(algorithmic_layer_bytes(synth, M))} layers): "
              f"(distinct active experts + 1 shared) x {EXPERT_BYTES_LING} B + logits + x + y = {algo:.0f} B; "
              f"measured / algorithmic = {total / algo:.4f}.", "",
              "```json", json.dumps(summary), "```", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(summary), flush=True)


def stored_traffic(M=1):
    """Traffic bytes per launch from the committed counter summary for M tokens,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(M=M))
    try:
        with open(path) as f:
            text = f.read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        summary = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if summary.get("source_hash") != kernel_source_hash():
        return None
    return summary


def main(argv=None):
    args = parse_args(argv)
    if args.traffic_from:
        out = args.traffic_out or os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(M=args.pmc_m))
        traffic_summary(args.traffic_from[0], args.traffic_from[1], out, args.pmc_m)
        return 0
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
    if args.pmc_run:
        pmc_run(m, torch, synth, dev, M=args.pmc_m)
        return 0

    log(f"device: {torch.cuda.get_device_name(0)}; layers {args.layers}, steps {args.steps}, warmup {args.warmup}")
    layers = make_layers(m, synth, args.layers, dev)
    r1 = moe_bench(m, torch, synth, layers, 1, args.steps, args.warmup, dev)
    log("M=1:", json.dumps(r1))
    r4 = None
    if not args.no_m4:
        r4 = moe_bench(m, torch, synth, layers, 4, args.steps, args.warmup, dev)
        log("M=4:", json.dumps(r4))
    sh8 = None
    if not args.no_fp8_shared:
        sh8 = shared_fp8_bench(m, torch, synth, layers, args.steps, dev)
        log("FP8 shared:", json.dumps(sh8))
    stack = None
    if not args.no_stack:
        stack = stack_bench(m, torch, synth, layers, args.stack_passes, max(1, args.stack_passes // 10), dev)
        log("stack:", json.dumps(stack))
    router = None
    if not args.no_router:
        router = router_bench(m, torch, synth, layers, min(args.steps, 2100), dev)
        log("router:", json.dumps(router))
    pf = None
    if not args.no_prefill:
        pf = prefill_bench(m, torch, synth, layers, dev, tuple(args.prefill_tokens))
        log("prefill:", json.dumps(pf))
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

    traffic = stored_traffic(1)
    traffic4 = stored_traffic(4)
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
            "traffic": None if traffic is None else traffic["traffic_bytes"],
            "traffic_fetch_write": None if traffic is None else [traffic["fetch_bytes"], traffic["write_bytes"]],
            "bytes_per_launch": r1["bytes_per_layer"],
            "avg_launch_us": round(r1["us_per_layer"], 3),
        },
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        "traffic_m4": None if traffic4 is None else {k: traffic4[k] for k in (
            "fetch_bytes", "write_bytes", "traffic_bytes", "algorithmic_bytes", "traffic_over_algorithmic")},
        "extra": {"m1": r1, "m4": r4, "stack": stack, "router": router, "lmhead": lm, "fp8_shared": sh8,
                  "prefill": pf, "cpu": cpu},
    }
    if router is not None:
        line["router_us_m1"] = round(router["us_m1"], 3)
        line["router_plus_layer_us_m1"] = round(router["router_plus_layer_us_m1"], 3)
    line["a8_us_per_layer_m1"] = round(r1["a8_us_per_layer"], 3)
    if r4 is not None:
        line["a8_us_per_layer_m4"] = round(r4["a8_us_per_layer"], 3)
        line["us_per_layer_m4"] = round(r4["us_per_layer"], 3)
        line["gbs_m4"] = round(r4["gbs"], 1)
        line["frac_of_peak_m4"] = round(r4["frac_of_peak"], 4)
    if stack is not None:
        line["stack_us_per_layer_graph"] = round(stack["us_per_layer_graph"], 3)
        line["stack_us_per_layer_eager"] = round(stack["us_per_layer_eager"], 3)
        line["stack_norm_router_layer_us_graph"] = round(stack["routed_us_per_layer_graph"], 3)
    if sh8 is not None:
        line["fp8_shared_us_per_layer_m1"] = round(sh8["m1_us_per_layer"], 3)
        line["fp8_shared_us_per_layer_m4"] = round(sh8["m4_us_per_layer"], 3)
    if pf is not None:
        for T, r in pf.items():
            line[f"prefill_us_t{T}"] = round(r["us_per_layer"], 1)
            line[f"prefill_tflops_t{T}"] = round(r["tflops"], 1)
            line[f"prefill_a8_us_t{T}"] = round(r["us_per_layer_a8"], 1)
            line[f"prefill_a8_tflops_t{T}"] = round(r["tflops_a8"], 1)
    if lm is not None:
        line["lmhead_fp8_gbs_m1"] = round(lm["fp8_m1_gbs"], 1)
        line["lmhead_fp8_argmax_us_m1"] = round(lm["fp8_argmax_m1_us"], 2)
        line["lmhead_fp8_sample_us_m1"] = round(lm["fp8_sample_m1_us"], 2)
        line["lmhead_fp8_sample_us_m4"] = round(lm["fp8_sample_m4_us"], 2)
        line["lmhead_fp8_gbs_m4"] = round(lm["fp8_m4_gbs"], 1)
        line["lmhead_fp8_dynact_gbs_m1"] = round(lm["fp8_dynact_m1_gbs"], 1)
        line["lmhead_fp8_dynact_gbs_m4"] = round(lm["fp8_dynact_m4_gbs"], 1)
        line["lmhead_bf16_gbs_m1"] = round(lm["bf16_m1_gbs"], 1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
