"""CPU checks of the arithmetic the FP8 quantiser kernel relies on.

The kernel (lmhead.hip) computes each code from fl32(|W| / s) without a
division per element, and encodes E4M3 with integer operations instead of a
table search.  Both are restated here in C, built with gcc at test time, and
checked on the CPU:

  * the quotient: q0 = W*y with y = fl32(1/s), r = fma(-q0, s, W),
    q = fma(r, y, q0) (Markstein's correction with the exact remainder) equals
    the IEEE float32 quotient W / s wherever either is at least 2^-14, and is
    never more than one float32 step above 448 (so it needs no clamp), for
    every bf16 W in [0, a] and every bf16 absmax a whose scale
    s = fl32(a / 448) is at least 2^-90.  Scaling W and a by the same power of
    two scales the quotient exactly while everything stays normal, so the
    mantissas of a (all 128) at the lowest, a middle and the highest exponent
    of that range cover the cases; every W below a is taken.
  * the encoding: the branch-free E4M3 magnitude code equals the oracle's
    search over the E4M3 value table at every code value, every midpoint
    between neighbouring codes and the float32 values either side of them,
    around the subnormal/normal boundary, at saturation and on random inputs.
"""

import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

/* E4M3 magnitude code of a non-negative float: the kernel's integer form. */
uint32_t e4m3_mag_code(float q) {
    const uint32_t b = bits(q);
    const uint32_t nrm = (b + (0x7FFFFu - (120u << 23)) + ((b >> 20) & 1u)) >> 20;
    const uint32_t sub = bits(q + 16384.0f) - 0x46800000u;
    const uint32_t c = b >= 0x3C800000u ? nrm : sub;
    return c < 0x7Eu ? c : 0x7Eu;
}

void encode_many(const float* q, uint8_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = (uint8_t)e4m3_mag_code(q[i]);
}

/* For each absmax (bf16 bits), every bf16 magnitude W <= a: counts the W whose
   corrected quotient differs from W / s where either is >= 2^-14 or exceeds
   448 by more than one step, and the pairs checked.  Returns -1 if a scale falls outside [2^-90, FLT_MAX]. */
long quotient_mismatches(const uint16_t* amax_bits, long n_a, long* checked) {
    long bad = 0, n = 0;
    for (long i = 0; i < n_a; ++i) {
        const float a = f32((uint32_t)amax_bits[i] << 16);
        const float s = a / 448.0f;
        if (!(s >= 0x1p-90f) || !(s <= 0x1.fffffep127f)) return -1;
        const float y = 1.0f / s;
        for (uint32_t wb = 0; wb <= amax_bits[i]; ++wb) {
            const float w = f32(wb << 16);
            const float q = w / s;
            const float q0 = w * y;
            const float r = fmaf(-q0, s, w);
            const float q1 = fmaf(r, y, q0);
            ++n;
            if (bits(q1) != bits(q) && (q >= 0x1p-14f || q1 >= 0x1p-14f)) ++bad;
            if (q1 > 0x1.c00002p+8f) ++bad;        /* above 448 + one step: would need a clamp */
        }
    }
    *checked = n;
    return bad;
}
"""


@pytest.fixture(scope="module")
def arith():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp(prefix="quant_arith_")
    src, lib = os.path.join(d, "a.c"), os.path.join(d, "a.so")
    with open(src, "w") as fh:
        fh.write(C_SRC)
    # ISO C, no contraction: every operation rounds exactly as written
    subprocess.run([gcc, "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", lib, src, "-lm"], check=True)
    so = ctypes.CDLL(lib)
    so.encode_many.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
    so.quotient_mismatches.argtypes = [ctypes.c_void_p, ctypes.c_long,
                                       ctypes.POINTER(ctypes.c_long)]
    so.quotient_mismatches.restype = ctypes.c_long
    yield so
    shutil.rmtree(d)


def _encode(so, q):
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape, dtype=np.uint8)
    so.encode_many(q.ctypes.data, out.ctypes.data, q.size)
    return out


def test_encoder_matches_oracle(arith):
    vals = oracle.formats.e4m3_value(np.arange(0x7F)).astype(np.float64)   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [464.0, 480.0, 1e4, 2.0 ** 127, 2.0 ** -6, 2.0 ** -10, 2.0 ** -9]])
    pts32 = pts.astype(np.float32)
    assert np.all(pts32.astype(np.float64) == pts)                  # every point is a float32
    near = np.concatenate([pts32, np.nextafter(pts32, np.float32(0)), np.nextafter(pts32, np.float32(np.inf))])
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.uniform(0, 500, 1 << 20), np.exp2(rng.uniform(-40, 10, 1 << 20))])
    q = np.concatenate([near, rand.astype(np.float32), np.float32([0.0, np.inf])])
    got = _encode(arith, q)
    want = oracle.formats.e4m3_encode_rne_sat(q)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(q[i]), int(got[i]), int(want[i])) for i in bad[:8]]
    assert _encode(arith, np.float32([np.nan]))[0] == 0x7E             # NaN saturates too


def test_corrected_quotient_matches_division(arith):
    mant = np.arange(128, dtype=np.uint16)
    # lowest bf16 exponent whose scale a/448 is >= 2^-90 for every mantissa: 2^-81
    exps = np.array([127 - 81, 127, 254], dtype=np.uint16)
    amax = (exps[:, None] << 7 | mant[None, :]).ravel()
    amax = amax[amax < 0x7F80]                                       # finite
    checked = ctypes.c_long(0)
    bad = arith.quotient_mismatches(amax.ctypes.data, amax.size, ctypes.byref(checked))
    assert bad == 0
    assert checked.value > 3 * 128 * 16000


def test_quotient_check_sees_a_wrong_correction(arith):
    """The check is not vacuous: the uncorrected product W*y differs from the
    quotient on many pairs, and a scale below the range is refused."""
    so = arith
    src = C_SRC.replace("const float q1 = fmaf(r, y, q0);", "const float q1 = q0; (void)r;")
    d = tempfile.mkdtemp(prefix="quant_arith_neg_")
    try:
        with open(os.path.join(d, "b.c"), "w") as fh:
            fh.write(src)
        lib = os.path.join(d, "b.so")
        subprocess.run([shutil.which("gcc"), "-std=c11", "-O2", "-ffp-contract=off", "-fPIC",
                        "-shared", "-o", lib, os.path.join(d, "b.c"), "-lm"], check=True)
        neg = ctypes.CDLL(lib)
        neg.quotient_mismatches.argtypes = so.quotient_mismatches.argtypes
        neg.quotient_mismatches.restype = ctypes.c_long
        amax = (np.uint16(127) << 7 | np.arange(128, dtype=np.uint16)).astype(np.uint16)
        n = ctypes.c_long(0)
        assert neg.quotient_mismatches(amax.ctypes.data, amax.size, ctypes.byref(n)) > 0
        tiny = np.uint16([(127 - 100) << 7])
        assert so.quotient_mismatches(tiny.ctypes.data, 1, ctypes.byref(n)) == -1
    finally:
        shutil.rmtree(d)
