"""The shared expert stored in FP8: E4M3 codes with one float32 scale per
output row, built once from bf16 weights -- the scheme of the LM head applied
to the shared expert's three projections.

What the pages fix: shared projections keep a higher-precision format than
the MXFP4 routed experts [ic §three scalpels]; a dynamic FP8 configuration
applied when a layer is built halves what bf16 weights cost to read [card
method #2; news §where the speed comes from].

Readings where the pages are silent:
  * "FP8" is OCP E4M3 (FN) with one float32 scale per output row, s = absmax /
    448 (1 for an all-zero row), q = E4M3 nearest-even, saturating, of fl32(W
    / s) -- exactly the LM head's quantiser (lmhead_quant_fp8), applied to
    W_gate [I][H], W_up [I][H] and W_down [H][I] row by row;
  * the expert computes with the dequantised weights s_row * e4m3(q): h =
    silu(W_gate x) * (W_up x), y = W_down h, as every other expert; x stays
    bf16.

Parity status: the quantiser is the LM head's (pinned there).  Dequantisation
is pinned by hand-worked codes and scales; a shared expert whose weights are
already of the form e4m3 value * 2^k per row quantises without loss, so its
FP8 layer equals the layer on the bf16 weights; and a row scaled by a power of
two keeps its codes and scales its scale (tests/test_oracle_shared_fp8.py).
"""

import numpy as np

from .formats import e4m3_value
from .lmhead import lmhead_quant_fp8


def quant_fp8_rows(w):
    """Per-row E4M3 quantisation of a bf16-exact matrix: (codes uint8 [R][K],
    scale float32 [R]); the LM head's rule."""
    return lmhead_quant_fp8(w)


def dequant_fp8_rows(codes, scale):
    """Dense float64 matrix scale[r] * e4m3(codes[r, k])."""
    return e4m3_value(np.asarray(codes, dtype=np.uint8)) * np.asarray(scale, np.float64)[:, None]


def shared_fp8_dense(gate_bf16, up_bf16, down_bf16):
    """The FP8 shared expert's dense weights (w_gate, w_up, w_down), float64,
    from its bf16-exact source matrices: quantise each row, dequantise."""
    return tuple(dequant_fp8_rows(*quant_fp8_rows(w)) for w in (gate_bf16, up_bf16, down_bf16))
