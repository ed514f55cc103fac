"""Routed + shared SwiGLU expert FFN of one MoE layer, and the RMSNorm step
that carries the residual between stacked layers.

What the pages fix: the layer has 512 routed experts (8 active per token) and
one shared expert, expert intermediate size 768, hidden size 2,560 (the LM
head is 157,184 x 2,560) [card §background, §method #1, #2; ic §three
scalpels].  Routed expert weights are MXFP4 [ic §three scalpels].

Readings where the pages are silent:
  * expert FFN is SwiGLU: h = silu(W_gate x) * (W_up x), out = W_down h, with
    silu(g) = g / (1 + exp(-g)); h is not rounded between the two products;
  * the shared expert has the routed experts' shape and format and weight 1;
  * activations are bf16 (weight-only MXFP4); the layer output is the sum in
    full precision, rounded once to bf16 at the end;
  * stacked layers: x_{l+1} = bf16(RMSNorm(r_l)), r_{l+1} = r_l + y_l, with
    gamma = 1, eps = 1e-6.

Parity status: pinned (tests/test_oracle_moe.py) by a dense brute force that
sums every expert under a routing mask in a different loop order, by k = E
giving the dense softmax mixture, by x = 0 giving y = 0 exactly, and by a
hand-computed closed-form layer (constant codes, known silu value).
rmsnorm: pinned by a hand-computed constant vector and scale invariance.
moe_layer_by_expert: pinned against moe_layer (to float64 rounding) on tiny
shapes, including an expert every token chose, ragged token counts and a token
subset (tests/test_oracle_moe.py).
"""

import numpy as np


def expert_ffn(w_gate, w_up, w_down, x):
    """One SwiGLU expert in float64.

    w_gate, w_up  [I][H] dense float64;  w_down [H][I];  x [H] float64
    """
    g = w_gate @ x
    u = w_up @ x
    h = g / (1.0 + np.exp(-g)) * u
    return w_down @ h


def moe_layer(x, ids, w, expert_weights, shared_weights):
    """MoE layer output for M tokens, float64, unrounded.

    x               [M][H] values (bf16-exact activations as float64)
    ids, w          [M][k] routing from route_topk
    expert_weights  callable e -> (w_gate, w_up, w_down) dense float64
    shared_weights  (w_gate, w_up, w_down) of the shared expert
    y[m] = sum_j w[m][j] * FFN(ids[m][j], x[m]) + FFN(shared, x[m])
    """
    x = np.asarray(x, dtype=np.float64)
    m_tokens = x.shape[0]
    y = np.zeros_like(x)
    for m in range(m_tokens):
        for j in range(ids.shape[1]):
            wg, wu, wd = expert_weights(int(ids[m, j]))
            y[m] += w[m, j] * expert_ffn(wg, wu, wd, x[m])
        y[m] += expert_ffn(*shared_weights, x[m])
    return y


def moe_layer_by_expert(x, ids, w, expert_weights, shared_weights, tokens=None):
    """moe_layer's sum evaluated expert by expert, for many tokens.

    Each active expert's dense weights are formed once and applied to all the
    tokens that chose it (one matrix product per expert); each token's terms
    are then added in moe_layer's order: w[t][0] * FFN_0 + ... + w[t][k-1] *
    FFN_{k-1}, then the shared expert.  Only the float64 rounding of the
    products may differ from moe_layer.

    tokens  optional ascending token indices; only their rows are evaluated
            (the returned array has one row per listed token)
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    k = ids.shape[1]
    terms = np.zeros((len(tokens), k, x.shape[1]))
    for e in sorted(set(int(v) for v in ids[tokens].flatten())):
        rows, slots = np.nonzero(ids[tokens] == e)
        wg, wu, wd = expert_weights(e)
        xs = x[tokens[rows]]                      # [n][H]
        g = xs @ wg.T
        u = xs @ wu.T
        h = g / (1.0 + np.exp(-g)) * u
        terms[rows, slots] = h @ wd.T
    wg, wu, wd = shared_weights
    xs = x[tokens]
    g = xs @ wg.T
    u = xs @ wu.T
    shared = (g / (1.0 + np.exp(-g)) * u) @ wd.T
    y = np.zeros((len(tokens), x.shape[1]))
    for i, t in enumerate(tokens):
        for j in range(k):
            y[i] += w[t, j] * terms[i, j]
        y[i] += shared[i]
    return y


def rmsnorm(r, eps=1e-6):
    """RMSNorm with unit gain along the last axis, float64."""
    r = np.asarray(r, dtype=np.float64)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return r / np.sqrt(ms + eps)
