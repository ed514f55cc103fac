"""Pins of the oracle's LM-head quantiser and GEMVs."""

import numpy as np
import torch

import oracle
import synth


def _bf16(v):
    return synth.bf16_values(synth.bf16_bits_from_f32(np.asarray(v, np.float32)))


def test_quant_absmax_448_row_has_unit_scale():
    row = _bf16([448.0, -3.0, 1.0625, 0.5, -448.0, 100.0, 7.0, 0.0])
    codes, s = oracle.lmhead_quant_fp8(row[None, :])
    assert s[0] == np.float32(1.0)
    np.testing.assert_array_equal(codes[0], oracle.e4m3_encode_rne_sat(row))
    assert codes[0, 0] == 0x7E and codes[0, 4] == 0xFE and codes[0, 2] == 0x38


def test_quant_zero_row():
    codes, s = oracle.lmhead_quant_fp8(np.zeros((1, 64), np.float32))
    assert s[0] == 1.0 and (codes == 0).all()


def test_quant_scale_is_float32_division():
    w = synth.bf16_values(synth.lmhead_weight_bf16(0, 64, 256, n_rows=64))
    codes, s = oracle.lmhead_quant_fp8(w)
    a = np.abs(w).max(axis=1)
    np.testing.assert_array_equal(s, (a / np.float32(448)).astype(np.float32))
    assert s.dtype == np.float32
    # the largest element of each row lands on (or next to) the top code 448
    top = np.abs(oracle.e4m3_value(codes)).max(axis=1)
    assert (top == 448.0).all()


def test_quant_matches_torch_cast_and_error_bound():
    w = synth.bf16_values(synth.lmhead_weight_bf16(0, 256, 512, n_rows=256))
    codes, s = oracle.lmhead_quant_fp8(w)
    q = (w / s[:, None]).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    deq = oracle.e4m3_value(codes) * s[:, None].astype(np.float64)
    err = np.abs(deq - w)
    normal = np.abs(q) >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * np.abs(w[normal]) * (1 + 1e-6)).all()
    assert (err[~normal] <= 2.0 ** -10 * np.broadcast_to(s[:, None], w.shape)[~normal] * (1 + 1e-6)).all()


def test_gemv_fp8_one_hot_orientation_and_scale():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(6, 40), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11            # no NaN codes
    s = np.float32([0.5, 2.0, 0.25, 4.0, 1.0, 8.0])
    for k in (0, 13, 39):
        x = np.zeros((1, 40))
        x[0, k] = 1.0
        got = oracle.lmhead_gemv_fp8(codes, s, x)
        assert got.shape == (1, 6)
        for v in range(6):
            assert got[0, v] == oracle.e4m3_value(codes[v, k]) * s[v]
    assert (oracle.lmhead_gemv_fp8(codes, s, np.zeros((2, 40))) == 0).all()


def test_gemv_bf16_one_hot_orientation():
    w = synth.bf16_values(synth.lmhead_weight_bf16(1, 5, 64, n_rows=5)).astype(np.float64)
    x = np.zeros((2, 64))
    x[0, 3] = 1.0
    x[1, 63] = -2.0
    got = oracle.lmhead_gemv_bf16(w, x)
    np.testing.assert_array_equal(got[0], w[:, 3])
    np.testing.assert_array_equal(got[1], -2.0 * w[:, 63])


def test_argmax_hand_worked_ties_and_signed_zeros():
    lg = np.array([[0.5, 2.0, -1.0, 2.0],        # tie at the top: the lower index, 1
                   [-0.0, 0.0, -3.0, -2.0],      # +0 and -0 are equal: index 0
                   [-5.0, -4.0, -4.5, -7.0],     # all negative: index 1
                   [1.0, 1.0, 1.0, 1.0]])        # all equal: index 0
    np.testing.assert_array_equal(oracle.lmhead_argmax(lg), [1, 0, 1, 0])


def test_argmax_matches_a_stable_sort():
    rng = np.random.default_rng(21)
    lg = rng.integers(-3, 4, size=(6, 50)).astype(np.float64)      # many ties
    order = [np.lexsort((np.arange(50), -row))[0] for row in lg]   # largest, then lowest index
    np.testing.assert_array_equal(oracle.lmhead_argmax(lg), order)
