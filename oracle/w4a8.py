"""W4A8: the routed and shared experts with MXFP4 weights and 8-bit activations.

What the pages fix: the measured baseline serves this model in the cookbook's
W4A8 configuration (4-bit weights, 8-bit activations) [news §boundary: the
baseline is the W4A8 default], and the routed experts' 4-bit weights are MXFP4
[ic §three scalpels].

Readings where the pages are silent:
  * "A8" is MXFP8 [MX §5.2, §6.3]: E4M3 elements sharing one E8M0 scale per
    32 consecutive values along the reduction axis -- the activations take the
    weights' block format, with 8-bit elements;
  * a block's scale is X = 2^(floor(log2(max |v|)) - 8) (8 = the exponent of
    E4M3's largest normal, 448), its exponent clamped to [-127, 127]; an
    all-zero block has X = 2^-127; each element is v / X rounded to the nearest
    E4M3 value, ties to even, saturating at +-448 (v / X is exact: X is a power
    of two);
  * both GEMM inputs are quantised: x (per token, along H) before gate/up and
    h = silu(g) * u (per (token, expert) pair, along I) before down; products
    of the dequantised values accumulate in full precision; the layer output
    and its combine order are moe_layer's.

Parity status: mxfp8_quantize is pinned (tests/test_oracle_w4a8.py) by
hand-worked blocks (scale choice, rounding of a midpoint to the even code,
saturation above 448 X, an all-zero block), by blocks whose values already lie
on the grid (lossless), by scaling a block by 2^j (same codes, scale shifted)
and by torch's float8_e4m3fn cast for the element rounding; moe_layer_w4a8 by a
closed-form layer (constant weights and activations, hand-computed MXFP8 of h)
and by x = 0 giving 0.
"""

import numpy as np

from .formats import e4m3_encode_rne_sat, e4m3_value

MX_BLOCK = 32
E4M3_EMAX = 8


def mxfp8_quantize(v):
    """MXFP8 (E4M3 elements, E8M0 block scales) of the last axis of v.

    v      float array [..., K], K a multiple of 32
    returns codes uint8 [..., K], scale bytes uint8 [..., K/32] (2^(b-127))
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    q = blocks / np.ldexp(1.0, e)[..., None]        # exact: X is a power of two
    codes = e4m3_encode_rne_sat(q.astype(np.float32)).reshape(v.shape)
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def mxfp8_dequant(codes, scales):
    """Values of MXFP8 codes [..., K] with scale bytes [..., K/32]."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.int64)
    vals = e4m3_value(c).reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (vals * np.ldexp(1.0, s - 127)[..., None]).reshape(c.shape)


def mxfp8_round(v):
    """v rounded to MXFP8 and back (the dequantised values)."""
    return mxfp8_dequant(*mxfp8_quantize(v))


def w4a8_h(wg, wu, x_q):
    """h = silu(W_gate x_q) * (W_up x_q) of one expert for rows of x_q (the
    dequantised MXFP8 activations), float64 [n][I], before its own MXFP8."""
    g = x_q @ wg.T
    u = x_q @ wu.T
    with np.errstate(over="ignore"):        # exp(-g) = inf for g << 0 gives silu = -0, as it should
        return g / (1.0 + np.exp(-g)) * u


def moe_layer_w4a8(x, ids, w, expert_weights, shared_weights, tokens=None):
    """The MoE layer with MXFP8 activations into both products, float64.

    Same arguments and combine order as moe_layer_by_expert: per token
    y = sum_j w[t][j] * W_down_j mxfp8(h_j) + W_down_s mxfp8(h_s), with
    h = silu(W_gate mxfp8(x)) * (W_up mxfp8(x)).
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    x_q = mxfp8_round(x[tokens])
    k = ids.shape[1]
    terms = np.zeros((len(tokens), k, x.shape[1]))
    for e in sorted(set(int(v) for v in ids[tokens].flatten())):
        rows, slots = np.nonzero(ids[tokens] == e)
        wg, wu, wd = expert_weights(e)
        terms[rows, slots] = mxfp8_round(w4a8_h(wg, wu, x_q[rows])) @ wd.T
    wg, wu, wd = shared_weights
    shared = mxfp8_round(w4a8_h(wg, wu, x_q)) @ wd.T
    y = np.zeros((len(tokens), x.shape[1]))
    for i, t in enumerate(tokens):
        for j in range(k):
            y[i] += w[t, j] * terms[i, j]
        y[i] += shared[i]
    return y
