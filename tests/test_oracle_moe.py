"""Pins of the oracle's MoE layer: a dense brute force over all experts under
a routing mask (different loop order), k = E, x = 0, and a closed-form layer."""

import math

import numpy as np
import pytest

import oracle
import synth


def _dense_experts(shape, seed=0, layer=0):
    lay = synth.mxfp4_layer(seed, layer, shape)
    deq = {}
    for name in ("gate", "up", "down"):
        codes, scales = lay[name]
        deq[name] = np.stack([oracle.mxfp4_dequant(codes[e], scales[e]) for e in range(shape.E + 1)])
    return deq


def _brute_force(x, ids, w, deq, n_exp):
    """Sum over every routed expert, masked by a dense [M][E] weight matrix,
    tokens batched per expert; the shared expert added last."""
    m_tokens = x.shape[0]
    dense_w = np.zeros((m_tokens, n_exp))
    for m in range(m_tokens):
        for j in range(ids.shape[1]):
            dense_w[m, ids[m, j]] += w[m, j]
    y = np.zeros_like(x)
    for e in list(range(n_exp)) + [n_exp]:
        g = x @ deq["gate"][e].T           # [M][I]
        u = x @ deq["up"][e].T
        h = g * (1.0 / (1.0 + np.exp(-g))) * u
        out = h @ deq["down"][e].T         # [M][H]
        coef = np.ones(m_tokens) if e == n_exp else dense_w[:, e]
        y += coef[:, None] * out
    return y


@pytest.mark.parametrize("m_tokens", [1, 3, 4])
def test_moe_matches_dense_brute_force(m_tokens):
    shape = synth.TINY
    deq = _dense_experts(shape)
    wl = synth.Workload("t", shape, m_tokens, router_matrix=True)
    xb, lg = synth.moe_inputs(wl)
    x = synth.bf16_values(xb).astype(np.float64)
    ids, w = oracle.route_topk(lg, shape.k)
    y = oracle.moe_layer(x, ids, w, lambda e: (deq["gate"][e], deq["up"][e], deq["down"][e]),
                         (deq["gate"][shape.E], deq["up"][shape.E], deq["down"][shape.E]))
    ref = _brute_force(x, ids, w, deq, shape.E)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_k_equals_e_is_dense_softmax_mixture():
    shape = synth.TINY
    deq = _dense_experts(shape)
    xb, lg = synth.moe_inputs(synth.Workload("t", shape, 2, router_matrix=True))
    x = synth.bf16_values(xb).astype(np.float64)
    ids, w = oracle.route_topk(lg, shape.E)
    y = oracle.moe_layer(x, ids, w, lambda e: (deq["gate"][e], deq["up"][e], deq["down"][e]),
                         (deq["gate"][shape.E], deq["up"][shape.E], deq["down"][shape.E]))
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = np.zeros_like(x)
    for e in range(shape.E + 1):
        g = x @ deq["gate"][e].T
        u = x @ deq["up"][e].T
        out = (g / (1 + np.exp(-g)) * u) @ deq["down"][e].T
        ref += (p[:, e:e + 1] if e < shape.E else 1.0) * out
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_zero_input_gives_zero():
    shape = synth.TINY
    deq = _dense_experts(shape)
    x = np.zeros((1, shape.H))
    ids = np.array([[3, 9]])
    w = np.array([[0.7, 0.3]])
    y = oracle.moe_layer(x, ids, w, lambda e: (deq["gate"][e], deq["up"][e], deq["down"][e]),
                         (deq["gate"][shape.E], deq["up"][shape.E], deq["down"][shape.E]))
    assert (y == 0).all()


def test_moe_closed_form_constant_layer():
    # H = 64, I = 32, two routed experts + shared, k = 1.  Expert 0 codes all
    # 0x22 (every element 1.0), expert 1 all 0x44 (2.0), shared 0x22 with scale
    # 2^-1.  x = 1/64 everywhere.  Token routes to expert 1 with weight 1.
    H, I = 64, 32
    def const(byte, scale_code, n, k):
        return oracle.mxfp4_dequant(np.full((n, k // 2), byte, np.uint8),
                                    np.full((n, k // 32), scale_code, np.uint8))
    experts = {0: tuple(const(0x22, 127, *s) for s in ((I, H), (I, H), (H, I))),
               1: tuple(const(0x44, 127, *s) for s in ((I, H), (I, H), (H, I)))}
    shared = tuple(const(0x22, 126, *s) for s in ((I, H), (I, H), (H, I)))
    x = np.full((1, H), 1.0 / 64)
    ids, w = oracle.route_topk(np.float32([[0.0, 1.0]]), 1)
    assert ids.tolist() == [[1]] and w.tolist() == [[1.0]]
    y = oracle.moe_layer(x, ids, w, lambda e: experts[e], shared)
    # expert 1: g = u = 64 * 2 / 64 = 2, h = silu(2) * 2, y_n = 32 * 2 * h
    h1 = 2.0 / (1.0 + math.exp(-2.0)) * 2.0
    # shared: g = u = 64 * 0.5 / 64 = 0.5, h = silu(0.5) * 0.5, y_n = 32 * 0.5 * h
    hs = 0.5 / (1.0 + math.exp(-0.5)) * 0.5
    want = 64.0 * h1 + 16.0 * hs
    assert abs(want - 227.9738892871453) < 1e-12
    np.testing.assert_allclose(y[0], want, rtol=1e-15)


def test_rmsnorm_hand_worked():
    r = np.array([[3.0, -4.0, 0.0, 0.0]])     # mean square 25/4, rms 2.5
    np.testing.assert_allclose(oracle.rmsnorm(r, eps=0.0), [[1.2, -1.6, 0.0, 0.0]], rtol=1e-15)
    # eps inside the square root: 25/4 + 3/4 = 7, so the result is r / sqrt(7)
    # (eps outside the root, 3/sqrt(6.25) + 0.75, or dropped, 3/2.5, both differ)
    s7 = np.sqrt(7.0)
    np.testing.assert_allclose(oracle.rmsnorm(r, eps=0.75), [[3.0 / s7, -4.0 / s7, 0.0, 0.0]], rtol=1e-15)
    # eps dominating a tiny vector: r = 1e-3 * [1, 1], eps = 3e-6 -> r / sqrt(1e-6 + 3e-6) = r / 2e-3
    np.testing.assert_allclose(oracle.rmsnorm(np.array([[1e-3, -1e-3]]), eps=3e-6), [[0.5, -0.5]], rtol=1e-13)
    r2 = np.random.default_rng(1).standard_normal((2, 64))
    np.testing.assert_allclose(oracle.rmsnorm(r2 * 7.0, eps=0.0), oracle.rmsnorm(r2, eps=0.0), rtol=1e-13)


def test_library_selftest_cases_agree_with_the_oracle():
    """The start-up self-test inside the library (moedec_selftest) expects
    closed forms written from the mathematics; the oracle, computing the same
    cases from their definitions, must agree: routing of {1.5, 0.5, 1.5, -1}
    with k = 2 is ids {0, 2} with weights {0.5, 0.5}; an MXFP4 layer whose
    every gate/up weight is code 2 (1.0) at scale 2^0 and every down weight is
    code 2 at scale 2^-5, with x = 2^-6 over H = 64 and I = 32, gives
    2 / (1 + e^-1) on every output; the FP8 codes of {448, -2, 1, 0.5, 0} and
    of a row of 0.25 are {0x7E, 0xC0, 0x38, 0x30, 0x00} and 0x7E."""
    ids, w = oracle.route_topk(np.float32([[1.5, 0.5, 1.5, -1.0]]), 2)
    np.testing.assert_array_equal(ids, [[0, 2]])
    np.testing.assert_array_equal(w, [[0.5, 0.5]])
    H, I = 64, 32
    gate = oracle.mxfp4_dequant(np.full((I, H // 2), 0x22, np.uint8), np.full((I, H // 32), 127, np.uint8))
    down = oracle.mxfp4_dequant(np.full((H, I // 2), 0x22, np.uint8), np.full((H, I // 32), 122, np.uint8))
    x = np.full((1, H), 2.0 ** -6)
    y = oracle.moe_layer(x, ids, w, lambda e: (gate, gate, down), (gate, gate, down))
    np.testing.assert_allclose(y, 2.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    row0 = np.array([448.0, -2.0, 1.0, 0.5] + [0.0] * 12)
    codes, scale = oracle.lmhead_quant_fp8(np.stack([row0, np.full(16, 0.25)]))
    np.testing.assert_array_equal(codes[0, :5], [0x7E, 0xC0, 0x38, 0x30, 0x00])
    assert (codes[0, 4:] == 0).all() and (codes[1] == 0x7E).all() and scale[0] == 1.0
    logits = oracle.lmhead_gemv_fp8(codes, scale, np.eye(16)[1:2])
    np.testing.assert_allclose(logits, [[-2.0, 0.25]], rtol=1e-6)
    assert oracle.lmhead_argmax(logits)[0] == 1


@pytest.mark.parametrize("m_tokens,forced", [(37, False), (64, True)])
def test_by_expert_equals_moe_layer(m_tokens, forced):
    """The expert-by-expert evaluation equals the per-token definition up to
    float64 rounding: ragged token counts, and a case where every token chose
    expert 5 (one expert multiplying the whole batch)."""
    shape = synth.TINY
    deq = _dense_experts(shape)
    xb, lg = synth.moe_inputs(synth.Workload("t", shape, m_tokens, router_matrix=True))
    if forced:
        lg = lg.copy()
        lg[:, 5] = 100.0
    x = synth.bf16_values(xb).astype(np.float64)
    ids, w = oracle.route_topk(lg, shape.k)
    if forced:
        assert (ids[:, 0] == 5).all()
    fn = lambda e: (deq["gate"][e], deq["up"][e], deq["down"][e])
    shared = (deq["gate"][shape.E], deq["up"][shape.E], deq["down"][shape.E])
    ref = oracle.moe_layer(x, ids, w, fn, shared)
    y = oracle.moe_layer_by_expert(x, ids, w, fn, shared)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    sub = np.array([0, 3, m_tokens - 1])
    ys = oracle.moe_layer_by_expert(x, ids, w, fn, shared, tokens=sub)
    assert np.max(np.abs(ys - ref[sub])) <= 1e-12 * np.max(np.abs(ref))
