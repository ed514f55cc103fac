"""Pins of the oracle's number formats against the OCP definitions, hand-worked
fixtures and torch's own decoders/casts (library routines)."""

import math

import numpy as np
import torch

import oracle
from oracle import formats


def test_e2m1_all_16_codes_match_mx_table(golden):
    table = golden("e2m1_values.json")["values"]
    got = oracle.e2m1_value(np.arange(16))
    for code, want in table.items():
        v = got[int(code)]
        assert v == want, (code, v, want)
        assert math.copysign(1.0, v) == math.copysign(1.0, want), code  # -0.0 for code 8


def test_e8m0_all_codes_match_torch_decoder():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = oracle.e8m0_value(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_mxfp4_packing_hand_worked(golden):
    fx = golden("mxfp4_handworked.json")
    codes = np.frombuffer(bytes.fromhex(fx["codes_hex"] + fx["codes_hex_block1"]), dtype=np.uint8)
    codes = codes.reshape(1, 32)
    scales = np.array([fx["scales"]], dtype=np.uint8)
    dense = oracle.mxfp4_dequant(codes, scales)
    assert dense.shape == (1, 64)
    want = np.zeros(64)
    for k, v in fx["nonzero_expected"].items():
        want[int(k)] = v
    np.testing.assert_array_equal(dense[0], want)
    assert math.copysign(1.0, dense[0, 6]) == -1.0   # code 8 is -0.0


def test_mxfp4_one_hot_picks_scaled_element():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    scales = rng.integers(120, 130, size=(3, 4), dtype=np.uint8)
    dense = oracle.mxfp4_dequant(codes, scales)
    for n in range(3):
        for k in (0, 1, 31, 32, 77, 127):
            byte = int(codes[n, k // 2])
            nib = byte & 15 if k % 2 == 0 else byte >> 4
            x = np.zeros(128)
            x[k] = 1.0
            assert dense[n] @ x == oracle.e2m1_value(nib) * 2.0 ** (int(scales[n, k // 32]) - 127)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_value(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and set(np.flatnonzero(nan)) == {127, 255}
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_fixture(golden):
    fx = golden("e4m3_cases.json")
    for code, want in fx["decode"].items():
        v = oracle.e4m3_value(int(code))
        assert v == want and math.copysign(1, v) == math.copysign(1, want), code
    for code in fx["decode_nan"]:
        assert np.isnan(oracle.e4m3_value(code))


def test_e4m3_encode_fixture(golden):
    fx = golden("e4m3_cases.json")
    for value, code, why in fx["encode"]:
        got = int(oracle.e4m3_encode_rne_sat(np.float32(value)))
        assert got == code, (value, got, code, why)


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (127, 255)], dtype=np.uint8)
    vals = oracle.e4m3_value(codes).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode_rne_sat(vals), codes)


def test_e4m3_encode_all_midpoints_go_to_even_code():
    pos = oracle.e4m3_value(np.arange(127))
    for c in range(126):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2       # exact in float32
        want = c if c % 2 == 0 else c + 1
        assert int(oracle.e4m3_encode_rne_sat(mid)) == want
        assert int(oracle.e4m3_encode_rne_sat(-mid)) == want | 0x80


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode_rne_sat(v), ref)


def test_e4m3_error_bound():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(50000) * 50).astype(np.float32)
    v = np.clip(v, -448, 448)
    q = oracle.e4m3_value(oracle.e4m3_encode_rne_sat(v))
    a = np.abs(v.astype(np.float64))
    normal = a >= 2.0 ** -6
    assert (np.abs(q - v)[normal] <= 2.0 ** -4 * a[normal]).all()
    assert (np.abs(q - v)[~normal] <= 2.0 ** -10).all()


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(100000) * s for s in (1e-20, 1e-3, 1, 1e3, 1e20)])
    v = v.astype(np.float32)
    # exact ties: 1 + 2^-8 (to 1.0), 1 + 3*2^-8 (to 1 + 2^-6)
    v = np.concatenate([v, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0])])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert got[-4] == 1.0 and got[-3] == 1 + 2 ** -6


def test_bf16_round_from_float64_is_single_rounding():
    # 1 + 2^-8 + 2^-40 is above the midpoint in float64 but rounds to the
    # midpoint in float32; a direct float64 -> bf16 rounding must go up.
    y = np.array([1 + 2.0 ** -8 + 2.0 ** -40])
    assert oracle.bf16_round(y)[0] == 1 + 2.0 ** -7


def test_bf16_bits_roundtrip():
    vals = np.array([1.0, -2.5, 0.0, 3.140625])
    bits = oracle.bf16_bits(vals)
    np.testing.assert_array_equal(formats.bf16_from_bits(bits), vals)
    assert bits[0] == 0x3F80
