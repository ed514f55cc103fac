"""LM head: online FP8 weight quantisation and the per-token vocabulary GEMV.

What the pages fix: the vocabulary projection is 157,184 x 2,560 and its whole
weight block is read for every generated token; the checkpoint keeps it in
bf16, and a dynamic FP8 configuration applied only when the LM head is built
halves what each token reads [news §where the speed comes from; card §method
#2; ic §three scalpels].

Readings where the pages are silent:
  * "FP8" is OCP E4M3 (FN) with one float32 scale per output row (per-row
    absmax), computed once when the head is built; activations stay bf16;
  * per row v: a_v = max_k |W[v,k]|, s_v = fl32(a_v / 448) (s_v = 1 when
    a_v = 0), q[v,k] = E4M3 round-to-nearest-even, saturating, of
    fl32(W[v,k] / s_v) -- the float32 divisions are those the quantiser
    performs, so that codes can be compared bit for bit;
  * logits[m, v] = s_v * sum_k x[m,k] * e4m3(q[v,k]), no bias, no soft-cap,
    float32 out; the bf16 comparator is logits = W x.

Parity status: quantisation pinned (tests/test_oracle_lmhead.py) by rows whose
absmax is 448 (scale exactly 1, codes equal to the direct E4M3 encoding), an
all-zero row, the per-element error bound of E4M3, and torch's float8_e4m3fn
cast for in-range values; the GEMVs by one-hot activations selecting a single
column times its row scale (orientation and scale) and x = 0; the greedy
argmax by hand-worked rows with ties and signed zeros and by a library sort.
"""

import numpy as np

from .formats import e4m3_encode_rne_sat, e4m3_value

E4M3_MAX = np.float32(448.0)


def lmhead_quant_fp8(w):
    """Per-row FP8 quantisation of a bf16 weight matrix.

    w  [V][H] bf16-exact values (any float dtype)
    returns codes uint8 [V][H], row_scale float32 [V]
    """
    w32 = np.asarray(w, dtype=np.float32)          # bf16 -> float32 is exact
    a = np.max(np.abs(w32), axis=1)                # exact
    s = a / E4M3_MAX                               # float32 IEEE division
    s = np.where(a == 0, np.float32(1.0), s).astype(np.float32)
    q = w32 / s[:, None]                           # float32 IEEE division
    return e4m3_encode_rne_sat(q), s


def lmhead_gemv_fp8(codes, row_scale, x):
    """logits [M][V] float64 = row_scale[v] * sum_k x[m,k] * e4m3(codes[v,k])."""
    wq = e4m3_value(np.asarray(codes, dtype=np.uint8))       # [V][H] float64
    x = np.asarray(x, dtype=np.float64)                       # [M][H]
    s = np.asarray(row_scale, dtype=np.float64)               # [V]
    return (x @ wq.T) * s[None, :]


def lmhead_argmax(logits):
    """Greedy token of each row of logits [M][V]: the index of the largest
    logit, the lowest such index on ties (+0.0 equals -0.0); int64 [M].
    Greedy choice is the temperature-0 case of the sampling the pages' decode
    step runs on these logits [card results]."""
    logits = np.asarray(logits, dtype=np.float64)
    return np.argmax(logits, axis=1).astype(np.int64)     # first index of the maximum


def lmhead_gemv_bf16(w, x):
    """logits [M][V] float64 = x W^T with bf16-exact W [V][H] and x [M][H]."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return x @ w.T
