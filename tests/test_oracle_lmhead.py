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


# ---------------------------------------------------------------- sampling

LN1234 = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))       # softmax (T = 1): 0.1, 0.2, 0.3, 0.4


def _sample(lg, u, t=1.0, p=1.0, k=4):
    return int(oracle.lmhead_sample(lg, np.array([u]), t, p, k)[0])


def test_sample_inverse_cdf_hand_worked():
    # candidates in order 3, 2, 1, 0 with probabilities 0.4, 0.3, 0.2, 0.1:
    # cumulative 0.4, 0.7, 0.9, 1.0
    for u, tok in ((0.0, 3), (0.39, 3), (0.41, 2), (0.69, 2), (0.71, 1), (0.89, 1), (0.91, 0), (0.999, 0)):
        assert _sample(LN1234, u) == tok, u


def test_sample_nucleus_and_top_k_cuts():
    # top_p 0.65: the prefix 0.4 + 0.3 reaches it; renormalised 4/7, 3/7
    assert _sample(LN1234, 0.5, p=0.65) == 3
    assert _sample(LN1234, 0.58, p=0.65) == 2
    assert _sample(LN1234, 0.999, p=0.65) == 2
    # top_p 0.35: the first token alone reaches it
    for u in (0.0, 0.5, 0.999):
        assert _sample(LN1234, u, p=0.35) == 3
    # top_k 2 with top_p 1: the same two tokens, 4/7 and 3/7
    assert _sample(LN1234, 0.5, k=2) == 3
    assert _sample(LN1234, 0.58, k=2) == 2
    assert _sample(LN1234, 0.999, k=2) == 2


def test_sample_temperature():
    # T = 0.5 squares the probabilities: 16, 9, 4, 1 over 30 -> cumulative 16/30, 25/30, 29/30
    assert _sample(LN1234, 0.5, t=0.5) == 3
    assert _sample(LN1234, 0.55, t=0.5) == 2
    assert _sample(LN1234, 0.84, t=0.5) == 1
    assert _sample(LN1234, 0.97, t=0.5) == 0
    # T = 2 takes square roots: 2, 1.732, 1.414, 1 over their sum 6.146 ->
    # cumulative 0.3254, 0.6072, 0.8373
    assert _sample(LN1234, 0.32, t=2.0) == 3
    assert _sample(LN1234, 0.33, t=2.0) == 2
    assert _sample(LN1234, 0.60, t=2.0) == 2
    assert _sample(LN1234, 0.61, t=2.0) == 1
    assert _sample(LN1234, 0.84, t=2.0) == 0


def test_sample_limits_reduce_to_argmax():
    rng = np.random.default_rng(5)
    lg = rng.normal(size=(5, 40))
    am = oracle.lmhead_argmax(lg)
    for u in (0.0, 0.3, 0.999):
        uu = np.full(5, u)
        np.testing.assert_array_equal(oracle.lmhead_sample(lg, uu, 0.6, 0.95, 1), am)        # top_k = 1
        np.testing.assert_array_equal(oracle.lmhead_sample(lg, uu, 1e-6, 0.95, 29), am)     # T -> 0
        np.testing.assert_array_equal(oracle.lmhead_sample(lg, uu, 1.0, 1e-9, 29), am)      # top_p -> 0


def test_sample_ties_follow_index_order():
    eq = np.array([[1.0, 1.0, 1.0, 1.0]])            # 0.25 each, candidates 0, 1, 2, 3
    for u, tok in ((0.1, 0), (0.3, 1), (0.6, 2), (0.8, 3)):
        assert _sample(eq, u) == tok
    sz = np.array([[-0.0, 0.0, -1.0]])               # +0 and -0 tie: index 0 first
    assert _sample(sz, 0.0, k=3) == 0


def _expected_distribution(row, t, top_p, top_k):
    """The renormalised nucleus written as a plain loop: (token, probability)
    pairs in candidate order."""
    cand = sorted(range(len(row)), key=lambda i: (-row[i], i))[:top_k]
    w = [np.exp((row[i] - row[cand[0]]) / t) for i in cand]
    tot = sum(w)
    keep, acc = [], 0.0
    for i, wi in zip(cand, w):
        keep.append((i, wi / tot))
        acc += wi / tot
        if acc >= top_p:
            break
    s = sum(q for _, q in keep)
    return [(i, q / s) for i, q in keep]


def test_sample_draw_intervals_match_probabilities():
    """Each token's draws form one interval of u whose length is its
    renormalised probability: scan u on a grid and compare with the loop."""
    rng = np.random.default_rng(11)
    grid = (np.arange(200000) + 0.5) / 200000
    for trial in range(4):
        row = rng.normal(size=30) * 2
        t, top_p, top_k = [(0.6, 0.95, 29), (1.0, 0.5, 10), (0.3, 0.99, 5), (2.0, 0.9, 30)][trial]
        toks = oracle.lmhead_sample(np.repeat(row[None, :], grid.shape[0], axis=0), grid, t, top_p, top_k)
        dist = _expected_distribution(row, t, top_p, top_k)
        # tokens appear in candidate order, each over one run of u
        runs = [toks[0]] + [b for a, b in zip(toks[:-1], toks[1:]) if a != b]
        assert runs == [i for i, _ in dist]
        for i, q in dist:
            assert abs(np.mean(toks == i) - q) < 2e-5, (trial, i)


def test_sampling_uniforms_are_in_range_and_counter_based():
    u = synth.sampling_uniforms(3, 7, 4)
    assert u.dtype == np.float32 and ((u >= 0) & (u < 1)).all()
    np.testing.assert_array_equal(u, synth.sampling_uniforms(3, 7, 4))
    assert not np.array_equal(u, synth.sampling_uniforms(3, 8, 4))
    # u * 2^24 is the top 24 bits of the stream's outputs
    st = synth.stream_state(3, synth.SAMPLING_STREAM_BASE + 7)
    words = synth.splitmix_outputs(st, np.arange(4, dtype=np.uint64))
    np.testing.assert_array_equal((u.astype(np.float64) * (1 << 24)).astype(np.uint64), words >> np.uint64(40))


def test_dynact_lossless_activations_equal_weight_only_gemv():
    """Token rows that are E4M3 values times 2^j with absmax 448 * 2^j quantise
    without loss (t = 2^j exactly), so the dynamic-activation logits equal the
    weight-only FP8 logits bit for bit."""
    rng = np.random.default_rng(31)
    w = rng.standard_normal((40, 64)).astype(np.float32)
    codes, s = oracle.lmhead_quant_fp8(w)
    vals = oracle.formats.e4m3_value(rng.integers(0, 0x7F, size=(3, 64)))
    vals *= np.where(rng.random((3, 64)) < 0.5, -1.0, 1.0)
    vals[:, 5] = 448.0
    x = vals * np.array([[2.0 ** -3], [1.0], [2.0 ** 4]])
    p, t = oracle.lmhead_quant_fp8(x)
    np.testing.assert_array_equal(t, np.float32([2.0 ** -3, 1.0, 2.0 ** 4]))
    np.testing.assert_array_equal(oracle.lmhead_gemv_fp8_dynact(codes, s, x),
                                  oracle.lmhead_gemv_fp8(codes, s, x))


def test_dynact_hand_worked():
    # W = [1, 2]: s_w = fl32(2/448), codes 224 -> 0x76, 448 -> 0x7E.
    # x = [3, -1]: t = fl32(3/448), x / t = [448, -149.33] -> codes 0x7E, 0xF1 (-144).
    # sum of code products 224*448 + 448*(-144) = 35840.
    codes, s = oracle.lmhead_quant_fp8(np.float32([[1.0, 2.0]]))
    assert codes.tolist() == [[0x76, 0x7E]]
    x = np.float32([[3.0, -1.0]])
    p, t = oracle.lmhead_quant_fp8(x)
    assert p.tolist() == [[0x7E, 0xF1]]
    want = 35840.0 * float(np.float32(2.0) / np.float32(448.0)) * float(np.float32(3.0) / np.float32(448.0))
    np.testing.assert_allclose(oracle.lmhead_gemv_fp8_dynact(codes, s, x), [[want]], rtol=1e-15)
    assert abs(want - 15.0 / 14.0) < 1e-6      # the quantised x is [3, -0.964]


def test_dynact_zero_and_power_of_two_scaling():
    rng = np.random.default_rng(32)
    w = rng.standard_normal((20, 32)).astype(np.float32)
    codes, s = oracle.lmhead_quant_fp8(w)
    assert (oracle.lmhead_gemv_fp8_dynact(codes, s, np.zeros((2, 32))) == 0).all()
    x = synth.bf16_values(synth.bf16_bits_from_f32(rng.standard_normal((2, 32)).astype(np.float32)))
    base = oracle.lmhead_gemv_fp8_dynact(codes, s, x)
    for j in (-5, 3):
        np.testing.assert_array_equal(oracle.lmhead_quant_fp8(x * 2.0 ** j)[0], oracle.lmhead_quant_fp8(x)[0])
        np.testing.assert_array_equal(oracle.lmhead_gemv_fp8_dynact(codes, s, x * 2.0 ** j), base * 2.0 ** j)
