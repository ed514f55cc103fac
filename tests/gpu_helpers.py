"""Shared helpers of the GPU parity tests: tolerances and reference runs.

Tolerances (applied per token):
  * float32 accumulators (y before rounding, logits): max|gpu - ref| <=
    1e-5 * max|ref|, ref the float64 oracle;
  * bf16 outputs: the kernel's bf16 equals the round-to-nearest-even of its
    own float32 accumulator, and max|gpu - ref_bf16| <= 1e-2 * rms(ref_bf16),
    where a one-ulp difference is accepted when the float64 value lies within
    1e-5 * max|ref| of the midpoint between the two bf16 neighbours (either
    rounding is then correct);
  * indices and dispatch tables bit-exact; routing weights within 1e-6.
"""

import sys

import numpy as np
import torch

import oracle
import synth

ACC_RTOL = 1e-5
BF16_RMS_TOL = 1e-2
W_ATOL = 1e-6


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_of(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_acc(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    for m in range(ref.shape[0]):
        scale = np.max(np.abs(ref[m]))
        err = np.max(np.abs(gpu[m] - ref[m]))
        assert err <= ACC_RTOL * scale, f"{what} token {m}: max err {err:.3e} > {ACC_RTOL} * {scale:.3e}"


def check_bf16(gpu_bits, gpu_f32, ref, what):
    # (1) bf16 is the nearest-even rounding of the kernel's own float32 sum
    own = torch.from_numpy(np.ascontiguousarray(gpu_f32, np.float32)).to(torch.bfloat16)
    own = own.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gpu_bits, own, err_msg=f"{what}: bf16 is not RNE of y_f32")
    # (2) against the oracle's bf16 rounding of the float64 result
    ref = np.asarray(ref, np.float64)
    ref_b = oracle.bf16_round(ref)
    gpu_v = oracle.formats.bf16_from_bits(gpu_bits)
    for m in range(ref.shape[0]):
        tol_mid = ACC_RTOL * np.max(np.abs(ref[m]))
        rms = np.sqrt(np.mean(ref_b ** 2))
        d = gpu_v[m] != ref_b[m]
        if d.any():
            lo = np.minimum(gpu_v[m][d], ref_b[m][d])
            hi = np.maximum(gpu_v[m][d], ref_b[m][d])
            mid = (lo + hi) / 2
            r = oracle.bf16_round(mid)
            adjacent = (r == lo) | (r == hi)          # no bf16 value strictly between
            excused = adjacent & (np.abs(ref[m][d] - mid) <= tol_mid)
            bad = ~excused
            if bad.any():
                err = np.max(np.abs(gpu_v[m][d][bad] - ref_b[m][d][bad]))
                assert err <= BF16_RMS_TOL * rms, f"{what} token {m}: bf16 err {err:.3e} > 1e-2 rms {rms:.3e}"


def dense_expert(layer_canon, e):
    """float64 dense (gate, up, down) of expert e from canonical numpy arrays."""
    return tuple(oracle.mxfp4_dequant(layer_canon[n][0][e], layer_canon[n][1][e])
                 for n in ("gate", "up", "down"))


def oracle_layer(x_bits, logits, k, expert_fn, shared):
    x = synth.bf16_values(x_bits).astype(np.float64)
    ids, w = oracle.route_topk(logits, k)
    y = oracle.moe_layer(x, ids, w, expert_fn, shared)
    return ids, w, y
