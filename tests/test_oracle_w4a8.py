"""Pins of the W4A8 oracle: MXFP8 quantisation by hand-worked blocks, lossless
grid values, power-of-two scaling and torch's E4M3 cast; the W4A8 layer by a
closed-form constant layer and x = 0."""

import math

import numpy as np
import torch

import oracle
from oracle import w4a8


def test_mxfp8_hand_worked_block():
    # amax 3 -> floor(log2 3) - 8 = -7: X = 2^-7, scale byte 120.
    # 1 -> 128 (0x70); 3 -> 384 (0x7C); -0.40625 -> -52 (0xE5);
    # 0.53125 -> 68, the midpoint of 64 (even code 0x68) and 72 (0x69): 0x68.
    v = np.zeros((1, 32))
    v[0, :4] = [1.0, 3.0, -0.40625, 0.53125]
    codes, scales = w4a8.mxfp8_quantize(v)
    assert scales.tolist() == [[120]]
    assert codes[0, :5].tolist() == [0x70, 0x7C, 0xE5, 0x68, 0x00]
    np.testing.assert_array_equal(w4a8.mxfp8_dequant(codes, scales)[0, :4], [1.0, 3.0, -0.40625, 0.5])


def test_mxfp8_saturates_and_zero_block():
    # amax 480: floor(log2 480) = 8 -> X = 1; 480 and 460 saturate to 448 (0x7E); the
    # second block is all zero: scale byte 0, codes 0.
    v = np.zeros((1, 64))
    v[0, 0] = 480.0
    v[0, 1] = -460.0
    v[0, 2] = 100.0
    codes, scales = w4a8.mxfp8_quantize(v)
    assert scales.tolist() == [[127, 0]]
    assert codes[0, :3].tolist() == [0x7E, 0xFE, 0x6C] and (codes[0, 32:] == 0).all()


def test_mxfp8_grid_values_are_lossless_and_scaling_shifts_the_scale():
    rng = np.random.default_rng(61)
    vals = oracle.formats.e4m3_value(rng.integers(0, 0x7F, size=(5, 64)))
    vals *= np.where(rng.random((5, 64)) < 0.5, -1.0, 1.0)
    vals[:, 3] = 448.0
    vals[:, 40] = -288.0                      # on the grid; amax in [256, 448] keeps the scale exponent
    for j in (-20, 0, 7):
        v = vals * 2.0 ** j
        codes, scales = w4a8.mxfp8_quantize(v)
        assert (scales.astype(int) == 127 + j).all()
        np.testing.assert_array_equal(w4a8.mxfp8_dequant(codes, scales), v)
    rnd = rng.standard_normal((4, 96)) * 3.0
    c0, s0 = w4a8.mxfp8_quantize(rnd)
    c1, s1 = w4a8.mxfp8_quantize(rnd * 2.0 ** -9)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0.astype(int) - 9, s1.astype(int))


def test_mxfp8_element_rounding_matches_torch_cast():
    rng = np.random.default_rng(62)
    v = (rng.standard_normal((64, 32)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(np.float32)
    codes, scales = w4a8.mxfp8_quantize(v)
    q = v / np.ldexp(1.0, scales.astype(np.int64) - 127)
    ok = (np.abs(q) <= 448).all(axis=1)          # torch's cast does not saturate
    assert ok.sum() > 40
    ref = torch.from_numpy(q[ok].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[ok], ref)


def _const(byte, scale_code, n, k):
    return oracle.mxfp4_dequant(np.full((n, k // 2), byte, np.uint8), np.full((n, k // 32), scale_code, np.uint8))


def test_w4a8_closed_form_constant_layer():
    # H = 64, I = 32; every gate/up weight 1.0, every down weight 2^-5; x = 2^-6
    # (MXFP8 exact: X = 2^-14, x / X = 256).  g = u = 64 * 2^-6 = 1, h = silu(1) =
    # 0.7310586; its block: X = 2^-9, h / X = 374.30 -> 384, so h_q = 0.75.
    # y_n = 32 * 2^-5 * 0.75 = 0.75 for the routed expert (weight 1) plus the
    # same for the shared expert: 1.5 (the unquantised layer gives 1.4621).
    H, I = 64, 32
    ex = (_const(0x22, 127, I, H), _const(0x22, 127, I, H), _const(0x22, 122, H, I))
    x = np.full((1, H), 2.0 ** -6)
    ids, w = oracle.route_topk(np.float32([[0.0, 1.0]]), 1)
    y = w4a8.moe_layer_w4a8(x, ids, w, lambda e: ex, ex)
    np.testing.assert_array_equal(y, np.full((1, H), 1.5))
    y_plain = oracle.moe_layer(x, ids, w, lambda e: ex, ex)
    np.testing.assert_allclose(y_plain, 2.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)


def test_w4a8_zero_input():
    H, I = 64, 32
    ex = (_const(0x35, 125, I, H), _const(0x2A, 126, I, H), _const(0x47, 120, H, I))
    y = w4a8.moe_layer_w4a8(np.zeros((2, H)), np.array([[1], [0]]), np.array([[1.0], [1.0]]),
                            lambda e: ex, ex)
    assert (y == 0).all()
