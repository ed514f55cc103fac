"""The shared input generator: SplitMix64 known answers and layout."""

import numpy as np

import synth


def test_splitmix64_published_known_answers():
    # First outputs of SplitMix64 seeded with 0.
    out = synth.splitmix_outputs(0, np.arange(3))
    assert [int(v) for v in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_hash_bytes_little_endian_and_offsets():
    st = synth.stream_state(0, 5)
    full = synth.hash_bytes(st, 64)
    w0 = int(synth.splitmix_outputs(st, 0))
    assert full[:8].tolist() == [(w0 >> (8 * i)) & 0xFF for i in range(8)]
    for start, n in ((3, 20), (8, 8), (17, 40)):
        np.testing.assert_array_equal(synth.hash_bytes(st, n, start=start), full[start:start + n])


def test_scale_codes_range_and_offsets():
    st = synth.stream_state(0, 9)
    sc = synth.hash_scale_codes(st, 50000, 117, 121)
    assert sc.min() == 117 and sc.max() == 121
    counts = np.bincount(sc - 117)
    assert (np.abs(counts - 10000) < 500).all()
    np.testing.assert_array_equal(synth.hash_scale_codes(st, 10, 117, 121, start=100), sc[100:110])


def test_code_bytes_uniform():
    b = synth.hash_bytes(synth.stream_state(0, 11), 1 << 18)
    counts = np.bincount(b, minlength=256)
    assert (np.abs(counts - 1024) < 200).all()


def test_expert_streams_are_distinct_and_deterministic():
    a = synth.mxfp4_expert(0, 0, 3, synth.TINY)
    b = synth.mxfp4_expert(0, 0, 3, synth.TINY)
    c = synth.mxfp4_expert(0, 0, 4, synth.TINY)
    for name in ("gate", "up", "down"):
        np.testing.assert_array_equal(a[name][0], b[name][0])
        assert not np.array_equal(a[name][0], c[name][0])
    assert a["gate"][0].shape == (64, 128) and a["gate"][1].shape == (64, 8)
    assert a["down"][0].shape == (256, 32) and a["down"][1].shape == (256, 2)
