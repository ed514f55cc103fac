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

Dynamic FP8 activations (the other half of a dynamic FP8 configuration: the
activations quantised per token when the layer runs, as the weights were per
row when it was built).  Reading: each token row x[m] gets the weights' rule,
t_m = fl32(max_k |x[m,k]| / 448) (1 for a zero row), p[m,k] = E4M3
nearest-even, saturating, of fl32(x[m,k] / t_m); then logits[m, v] =
s_v * t_m * sum_k e4m3(p[m,k]) * e4m3(q[v,k]).

Sampling (the decode step's draw on these logits; the pages give the settings
only -- temperature 0.6, top-p 0.95, top-k 29 [card results]).  Readings:
  * candidates: the top_k logits of the row, ordered by (logit desc, index
    asc), the order the greedy argmax uses;
  * probabilities: softmax of logit / temperature over the candidates
    (temperature > 0);
  * nucleus: the shortest prefix of the candidates whose cumulative
    probability reaches top_p (at least one token);
  * draw: the nucleus renormalised to sum 1; with a uniform u in [0, 1) the
    token is the first nucleus entry whose cumulative renormalised
    probability exceeds u (the inverse of the cumulative distribution).
    u is an input: both sides take it from synth's counter-based generator.

Parity status: quantisation pinned (tests/test_oracle_lmhead.py) by rows whose
absmax is 448 (scale exactly 1, codes equal to the direct E4M3 encoding), an
all-zero row, the per-element error bound of E4M3, and torch's float8_e4m3fn
cast for in-range values; the GEMVs by one-hot activations selecting a single
column times its row scale (orientation and scale) and x = 0; the greedy
argmax by hand-worked rows with ties and signed zeros and by a library sort;
the dynamic-activation GEMV by activations that are already E4M3 values times
a per-token power of two with absmax 448 * 2^j (quantised without loss, so the
logits equal the weight-only GEMV's), by a hand-worked two-element case, by x =
0 and by scaling a token by a power of two (same codes, logits scaled); the
sampling by hand-worked distributions (inverse-CDF boundaries, nucleus cut,
top-k cut, temperature), the top_k = 1 and vanishing-temperature limits
(argmax), and by the interval each token's draws occupy, which equals its
renormalised probability computed by an independent loop.
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


def lmhead_gemv_fp8_dynact(codes, row_scale, x):
    """logits [M][V] float64 with dynamic per-token FP8 activations:
    row_scale[v] * t[m] * sum_k e4m3(p[m,k]) * e4m3(codes[v,k]), where (p, t)
    is the weights' per-row quantisation applied to each token row of x."""
    p, t = lmhead_quant_fp8(x)
    xq = e4m3_value(p) * np.asarray(t, dtype=np.float64)[:, None]
    return lmhead_gemv_fp8(codes, row_scale, xq)


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


def lmhead_sample(logits, u, temperature, top_p, top_k):
    """Sampled token of each row of logits [M][V] (float64 arithmetic), int64 [M].

    u [M] uniforms in [0, 1); temperature > 0; 0 < top_p <= 1; top_k >= 1.
    Follows the readings in the module docstring: top_k candidates by
    (logit desc, index asc), softmax of logit / temperature over them, the
    shortest prefix reaching top_p, renormalised, inverse-CDF draw at u.
    """
    logits = np.asarray(logits, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    assert temperature > 0 and 0 < top_p <= 1 and top_k >= 1
    out = np.empty(logits.shape[0], dtype=np.int64)
    for m in range(logits.shape[0]):
        row = logits[m]
        idx = np.arange(row.shape[0])
        order = np.lexsort((idx, -row))                    # logit desc, then index asc
        cand = order[:min(top_k, row.shape[0])]
        z = row[cand] / temperature
        p = np.exp(z - z[0])                               # z[0] is the largest
        p = p / p.sum()
        cum = np.cumsum(p)
        n_keep = int(np.searchsorted(cum, top_p, side="left")) + 1   # first cum >= top_p
        n_keep = min(n_keep, cand.shape[0])
        q = p[:n_keep] / cum[n_keep - 1]
        cq = np.cumsum(q)
        j = int(np.searchsorted(cq, u[m], side="right"))   # first cq > u
        out[m] = cand[min(j, n_keep - 1)]
    return out
