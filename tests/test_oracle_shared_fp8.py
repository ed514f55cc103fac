"""Pins of the FP8 shared expert's oracle (oracle/shared_fp8.py) against
hand-worked values and against the bf16 layer where FP8 is lossless."""

import numpy as np

import oracle
import synth


def test_dequant_hand_worked():
    # E4M3: 0x38 = 1.0, 0x3C = 1.5, 0x7E = 448, 0xB8 = -1.0, 0x01 = 2^-9 (smallest subnormal),
    # 0x08 = 2^-6 (smallest normal), 0x00 = 0
    codes = np.array([[0x38, 0x3C, 0x7E, 0xB8], [0x01, 0x08, 0x00, 0x80]], dtype=np.uint8)
    scale = np.array([0.5, 4.0], dtype=np.float32)
    want = np.array([[0.5, 0.75, 224.0, -0.5], [2.0 ** -7, 2.0 ** -4, 0.0, 0.0]])
    np.testing.assert_array_equal(oracle.dequant_fp8_rows(codes, scale), want)


def _fp8_exact_rows(rng, rows, cols):
    """Rows of e4m3 values times a per-row power of two, each with one entry of
    magnitude 448 * 2^k (so that s = 2^k exactly and W / s is the code's value)."""
    codes = rng.integers(0, 0x7F, size=(rows, cols), dtype=np.uint8)      # no NaN (0x7F)
    codes[codes == 0x7F] = 0x7E
    codes |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E                                                    # absmax 448
    k = rng.integers(-12, -4, size=rows)
    vals = oracle.e4m3_value(codes) * np.ldexp(1.0, k)[:, None]
    bits = synth.bf16_bits_from_f32(vals.astype(np.float32))
    assert np.array_equal(synth.bf16_values(bits).astype(np.float64), vals)   # bf16-exact
    return bits, codes, np.ldexp(1.0, k).astype(np.float32)


def test_quantisation_of_fp8_exact_rows_is_lossless():
    rng = np.random.default_rng(3)
    bits, codes, scale = _fp8_exact_rows(rng, 24, 96)
    q, s = oracle.quant_fp8_rows(synth.bf16_values(bits))
    np.testing.assert_array_equal(s, scale)
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(oracle.dequant_fp8_rows(q, s), synth.bf16_values(bits).astype(np.float64))


def test_fp8_shared_layer_equals_bf16_layer_when_lossless():
    """A layer whose shared expert is FP8-exact: the FP8 shared expert's layer
    output equals the one computed on the bf16 weights (float64, no rounding
    in between)."""
    rng = np.random.default_rng(4)
    H, I, E, k = 64, 32, 4, 2
    g, _, _ = _fp8_exact_rows(rng, I, H)
    u, _, _ = _fp8_exact_rows(rng, I, H)
    d, _, _ = _fp8_exact_rows(rng, H, I)
    dense_sh = tuple(synth.bf16_values(b).astype(np.float64) for b in (g, u, d))
    fp8_sh = oracle.shared_fp8_dense(*(synth.bf16_values(b) for b in (g, u, d)))
    for a, b in zip(fp8_sh, dense_sh):
        np.testing.assert_array_equal(a, b)
    routed = [tuple(rng.standard_normal(sh) * 0.1 for sh in ((I, H), (I, H), (H, I))) for _ in range(E)]
    x = synth.bf16_values(synth.activations_bf16(0, 0, 2, H)).astype(np.float64)
    ids, w = oracle.route_topk(rng.standard_normal((2, E)), k)
    y_fp8 = oracle.moe_layer(x, ids, w, lambda e: routed[e], fp8_sh)
    y_bf16 = oracle.moe_layer(x, ids, w, lambda e: routed[e], dense_sh)
    np.testing.assert_array_equal(y_fp8, y_bf16)


def test_power_of_two_row_scaling_keeps_codes():
    """Scaling a row by 2^j scales its FP8 scale by 2^j and keeps every code
    (division by the scale is exact in float32 up to the same rounding)."""
    rng = np.random.default_rng(5)
    w = synth.bf16_values(synth.bf16_bits_from_f32(rng.standard_normal((8, 40)).astype(np.float32) * 0.03))
    q, s = oracle.quant_fp8_rows(w)
    q2, s2 = oracle.quant_fp8_rows(w * np.float32(2.0 ** -5))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s * np.float32(2.0 ** -5))


def test_shared_expert_generator():
    g, u, d = synth.shared_expert_bf16(0, 0, 256, 64)
    assert g.shape == (64, 256) and u.shape == (64, 256) and d.shape == (256, 64)
    assert g.dtype == np.uint16
    gv = synth.bf16_values(g)
    assert abs(gv.std() * np.sqrt(256) - 1.0) < 0.05
    assert not np.array_equal(g, u)
    g2, _, _ = synth.shared_expert_bf16(0, 0, 256, 64)
    np.testing.assert_array_equal(g, g2)
