"""GPU parity of the W4A8 many-token layer (moe_layer_mxfp4_prefill_a8: MXFP8
activations into both products on the block-scaled fp4 x fp8 matrix
instruction) against the oracle (oracle.w4a8), through the C ABI.

The layer quantises twice, so its parity is checked stage by stage on what the
call leaves in its workspace (moe_prefill_workspace_layout):
  routing   ids and per-expert counts bit-exact, weights within 1e-6;
  x         MXFP8 codes and scale bytes of x bit-exact (x is bf16: v / X is
            exact and both sides round it to nearest even);
  h         MXFP8 of h = silu(W_gate x_q) * (W_up x_q): an element may land
            on the neighbouring E4M3 value, or a block on the neighbouring
            scale, only where the oracle's float64 value lies within the
            kernel's arithmetic error of that rounding boundary (a midpoint
            between adjacent codes, or a power of two for the block maximum);
  y         the down product and combine of the kernel's own h codes within
            that arithmetic error; y_bf16 is the nearest-even rounding of the
            kernel's y_f32.
The arithmetic error: the block-scaled fp4 x fp8 instruction does not return
the exact sum when its products span many binades (an in-bounds probe with
E4M3 exponents over the whole range, checked against exact sums on the host,
gave at most 2^-13.4 and in RMS 2^-15.6 of the products' absolute sum per 64-k
step, and exact results when the exponents span six binades).  The bound used
is HW_REL = 2^-11 of sum_k |a_k b_k| per output (four times the worst seen),
plus float32 accumulation; over every checked output the RMS of error / bound
base must also stay below 2^-14, which a systematic mistake (a wrong block
scale, a dropped block) breaks.
End to end, the oracle's moe_layer_w4a8 is compared as a sanity bound only
(its h may differ by the boundary cases above)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import w4a8
from gpu_helpers import W_ATOL, bf16_tensor, bits_of, dense_expert, say

pytestmark = pytest.mark.gpu

MID = synth.MoEShape(H=512, I=256, E=32, k=4, scale_lo=127 - 9, scale_hi=127 - 5)
ODD = synth.MoEShape(H=320, I=96, E=24, k=3, scale_lo=127 - 8, scale_hi=127 - 5)

# the block-scaled instruction's error bound and its RMS ceiling, relative to
# sum_k |a_k b_k|; float32 accumulation relative to the largest magnitude
HW_REL = 2.0 ** -11
HW_RMS = 2.0 ** -14
F32_REL = 1e-5
# end-to-end bound against moe_layer_w4a8 (boundary flips of h allowed)
E2E_REL = 2e-2

_GRID = np.unique(oracle.e4m3_value(np.arange(256, dtype=np.uint8)))
_GRID = _GRID[np.isfinite(_GRID)]


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


def _small_layer(m, shape, seed=0, layer=0):
    lay = synth.mxfp4_layer(seed, layer, shape)
    dev = {n: tuple(torch.from_numpy(a).cuda() for a in lay[n]) for n in lay}
    W = m.MoELayerWeights.from_canonical(dev["gate"], dev["up"], dev["down"], shape.E)
    dense = {e: dense_expert(lay, e) for e in range(shape.E + 1)}
    return W, (lambda e: dense[e]), dense[shape.E]


def _run(m, W, x_bits, logits, k):
    T = x_bits.shape[0]
    ws = m.make_prefill_workspace(T, W.E, k, W.H, W.I, "cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    counts = torch.full((W.E + 1,), -1, dtype=torch.int32, device="cuda")
    y, y32 = m.moe_layer_prefill(W, bf16_tensor(x_bits), torch.from_numpy(logits).cuda(), k, workspace=ws,
                                 ids=ids, topk_w=tw, counts=counts, act8=True)
    torch.cuda.synchronize()
    lay = m.prefill_workspace_layout(T, W.E, k, W.H, W.I)
    P = T * (k + 1)

    def region(off, n, dt=torch.uint8):
        return ws[off:off + n * torch.tensor([], dtype=dt).element_size()].view(dt).cpu().numpy()

    sb, sbi = lay["x_scale_stride"], lay["h_scale_stride"]
    inter = {
        "pos": region(lay["pos"], T * k, torch.int32).reshape(T, k),
        "x8": region(lay["x_codes"], T * W.H).reshape(T, W.H),
        "xs": region(lay["x_scales"], T * sb).reshape(T, sb)[:, :W.H // 32],
        "h8": region(lay["h_codes"], P * W.I).reshape(P, W.I),
        "hs": region(lay["h_scales"], P * sbi).reshape(P, sbi)[:, :W.I // 32],
    }
    return (ids.cpu().numpy(), tw.cpu().numpy(), counts.cpu().numpy(), bits_of(y), y32.cpu().numpy(), inter)


def check_mxfp8_near(codes, scales, h_ref, tol, what):
    """GPU MXFP8 (codes [n][K], scale bytes [n][K/32]) of values whose float64
    reference is h_ref [n][K], computed with an absolute error of at most tol
    [n][K]: equal except at rounding boundaries within tol."""
    n, K = h_ref.shape
    rc, rs = w4a8.mxfp8_quantize(h_ref)
    blk = h_ref.reshape(n, K // 32, 32)
    tb = tol.reshape(n, K // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    # scale bytes: only where the block maximum is within tol of a power of two
    ds = scales != rs
    if ds.any():
        a = amax[ds]
        gap = np.abs(a - np.exp2(np.round(np.log2(a))))
        near = gap <= np.max(tb[ds], axis=-1) + F32_REL * a
        assert near.all(), f"{what}: {int((~near).sum())} block scales differ away from a power of two"
    # elements of blocks with the same scale: rounding is monotone, so the
    # kernel's value lies between the roundings of h_ref - tol and h_ref + tol
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    vg = oracle.e4m3_value(codes).reshape(n, K // 32, 32)
    vr = oracle.e4m3_value(rc).reshape(n, K // 32, 32)
    d = ~ds[..., None] & (vg != vr)
    if d.any():
        Xb = np.broadcast_to(X, vg.shape)[d]
        t = tb[d] + F32_REL * np.broadcast_to(amax[..., None], vg.shape)[d]
        lo = oracle.e4m3_value(oracle.e4m3_encode_rne_sat(((blk[d] - t) / Xb).astype(np.float32)))
        hi = oracle.e4m3_value(oracle.e4m3_encode_rne_sat(((blk[d] + t) / Xb).astype(np.float32)))
        ok = (lo <= vg[d]) & (vg[d] <= hi)
        assert ok.all(), (f"{what}: {int((~ok).sum())} h codes outside the rounding of h +- tol, "
                          f"e.g. q={blk[d][~ok][:4] / Xb[~ok][:4]} gpu={vg[d][~ok][:4]} ref={vr[d][~ok][:4]}")
    # blocks on another scale: each value within half a step (or the
    # saturation of the lower scale) of h, plus tol
    if ds.any():
        e = np.abs(vg * X - blk)[ds]
        Xd = np.ldexp(1.0, scales[ds].astype(np.int64) - 127)[..., None]
        bound = (np.abs(blk[ds]) * 2.0 ** -4 + Xd * 2.0 ** -10 + tb[ds] + F32_REL * amax[ds][..., None]
                 + np.maximum(np.abs(blk[ds]) - 448.0 * Xd, 0.0))
        assert (e <= bound).all(), f"{what}: values of re-scaled blocks off by more than half a step"
    return int(d.sum()), int(ds.sum()), d.size, ds.size


def check_hw(gpu, ref, base, what):
    """gpu within HW_REL * base + F32_REL * max|ref| of ref per element, and
    the RMS of (gpu - ref) / base below HW_RMS."""
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    lim = HW_REL * base + F32_REL * np.max(np.abs(ref), axis=-1, keepdims=True)
    assert (err <= lim).all(), (f"{what}: {int((err > lim).sum())} outputs beyond the bound, worst "
                                f"{np.max(err / lim):.2f} x")
    rms = np.sqrt(np.mean((err / np.maximum(base, 1e-300)) ** 2))
    assert rms <= HW_RMS, f"{what}: RMS error {rms:.3g} of the products' absolute sum > {HW_RMS:.3g}"
    return rms


def _check(m, W, x_bits, logits, k, expert_fn, shared, what, tokens=None):
    T = x_bits.shape[0]
    say(what, "T", T, "k", k)
    ids, tw, counts, yb, y32, it = _run(m, W, x_bits, logits, k)
    ref_ids, ref_w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids, ref_ids, err_msg=f"{what}: expert ids")
    assert np.max(np.abs(tw - ref_w)) <= W_ATOL, f"{what}: routing weights"
    groups = oracle.expert_groups(ref_ids, W.E)
    np.testing.assert_array_equal(counts, [len(g) for g in groups], err_msg=f"{what}: group counts")

    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    # x: bit-exact MXFP8 on every token (on the sampled tokens and the first
    # 2,048 beyond 20 M values, to bound the oracle's time)
    rows_x = (np.arange(T) if T * W.H <= 20_000_000
              else np.unique(np.concatenate([sel, np.arange(min(T, 2048))])))
    x = synth.bf16_values(x_bits[rows_x]).astype(np.float64)
    xc, xsb = w4a8.mxfp8_quantize(x)
    np.testing.assert_array_equal(it["xs"][rows_x], xsb, err_msg=f"{what}: x scale bytes")
    np.testing.assert_array_equal(it["x8"][rows_x], xc, err_msg=f"{what}: x codes")
    x_q_rows = w4a8.mxfp8_dequant(xc, xsb)
    row_of = {int(t): i for i, t in enumerate(rows_x)}
    # h of every pair of the selected tokens, then y from the kernel's own h
    flips = rescaled = n_el = n_blk = 0
    y_ref = np.zeros((len(sel), W.H))
    by_expert = {}
    for i, t in enumerate(sel):
        for j in range(k):
            by_expert.setdefault(int(ref_ids[t, j]), []).append((i, t, j, int(it["pos"][t, j])))
        by_expert.setdefault(W.E, []).append((i, t, -1, T * k + t))
    y_base = np.zeros((len(sel), W.H))
    for e, items in sorted(by_expert.items()):
        wg, wu, wd = expert_fn(e) if e < W.E else shared
        rows = np.array([p for _, _, _, p in items])
        toks = np.array([t for _, t, _, _ in items])
        xq = x_q_rows[[row_of[int(t)] for t in toks]]
        g, u = xq @ wg.T, xq @ wu.T
        with np.errstate(over="ignore"):
            silu = g / (1.0 + np.exp(-g))
        h_ref = silu * u
        # propagate the instruction's error bound on g and u into h:
        # |silu'| <= 1.1 everywhere
        g_tol = HW_REL * (np.abs(xq) @ np.abs(wg).T)
        u_tol = HW_REL * (np.abs(xq) @ np.abs(wu).T)
        h_tol = 1.1 * np.abs(u) * g_tol + np.abs(silu) * u_tol + 1.1 * g_tol * u_tol
        f, r, ne, nb = check_mxfp8_near(it["h8"][rows], it["hs"][rows], h_ref, h_tol, f"{what}: h of expert {e}")
        flips, rescaled, n_el, n_blk = flips + f, rescaled + r, n_el + ne, n_blk + nb
        hq = w4a8.mxfp8_dequant(it["h8"][rows], it["hs"][rows])
        yp, yb1 = hq @ wd.T, np.abs(hq) @ np.abs(wd).T
        for (i, t, j, _), v, b in zip(items, yp, yb1):
            wt = ref_w[t, j] if j >= 0 else 1.0
            y_ref[i] += wt * v
            y_base[i] += abs(wt) * b
    # boundary cases stay rare (each is individually within the bound above)
    assert flips <= 0.05 * n_el and rescaled <= 0.05 * n_blk, f"{what}: {flips} flips, {rescaled} re-scaled blocks"
    rms = check_hw(y32[sel], y_ref, y_base, f"{what}: y from the kernel's h")
    say(what, "h boundary flips", flips, "re-scaled blocks", rescaled, "y rms err / base", f"{rms:.3g}")
    own = torch.from_numpy(np.ascontiguousarray(y32, np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(yb, own.view(torch.int16).numpy().view(np.uint16),
                                  err_msg=f"{what}: bf16 is not RNE of y_f32")
    return ids, ref_w, y32, sel, x


def _check_e2e(y32, x, ids, w, expert_fn, shared, sel, what):
    ref = w4a8.moe_layer_w4a8(x, ids, w, expert_fn, shared, tokens=sel)
    for i in range(len(sel)):
        scale = np.max(np.abs(ref[i]))
        err = np.max(np.abs(y32[sel[i]] - ref[i]))
        assert err <= E2E_REL * scale, f"{what} token {sel[i]}: end-to-end err {err:.3e} vs {scale:.3e}"


@pytest.mark.parametrize("T", [1, 8, 37, 200, 600])
def test_prefill_a8_tiny(m, T):
    """hidden 256 (two 128-k chunks), I 64 (one chunk of down, half padding);
    T = 200 and 600 give 64- and 128-token tiles."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    xb = synth.activations_bf16(1, 0, T, shape.H)
    ids, w, y32, sel, x = _check(m, W, xb, synth.router_logits_f32(1, xb, shape.E), shape.k, fn, sh,
                                 f"a8 tiny T={T}")
    _check_e2e(y32, x, ids, w, fn, sh, sel, f"a8 tiny T={T}")


@pytest.mark.parametrize("T", [300, 700])
def test_prefill_a8_mid(m, T):
    W, fn, sh = _small_layer(m, MID, seed=2)
    xb = synth.activations_bf16(2, 0, T, MID.H)
    ids, w, y32, sel, x = _check(m, W, xb, synth.logits_f32(2, 0, T, MID.E), MID.k, fn, sh, f"a8 mid T={T}")
    _check_e2e(y32, x, ids, w, fn, sh, sel, f"a8 mid T={T}")


def test_prefill_a8_odd_shape(m):
    """H = 320: 10 MX blocks of x, the last 128-k chunk half padding; I = 96:
    3 blocks of h, a partial row block."""
    W, fn, sh = _small_layer(m, ODD, seed=3)
    xb = synth.activations_bf16(3, 0, 129, ODD.H)
    _check(m, W, xb, synth.logits_f32(3, 0, 129, ODD.E), ODD.k, fn, sh, "a8 odd H=320 I=96 T=129")


def test_prefill_a8_max_k(m):
    """k = 32 of 64 experts (the largest k): 33 pairs per token."""
    shape = synth.MoEShape(H=256, I=64, E=64, k=32, scale_lo=127 - 8, scale_hi=127 - 5)
    W, fn, sh = _small_layer(m, shape, seed=11)
    xb = synth.activations_bf16(11, 0, 100, shape.H)
    _check(m, W, xb, synth.logits_f32(11, 0, 100, shape.E), shape.k, fn, sh, "a8 k=32 of 64")


def test_prefill_a8_skewed_and_zero_blocks(m):
    """Every token picks experts 3 and 5 (1000 rows each); some tokens have
    all-zero MX blocks of x (scale byte 0) and one token is zero throughout."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = 1000
    xb = synth.activations_bf16(4, 0, T, shape.H).copy()
    xb[::7, 32:96] = 0
    xb[5] = 0
    lg = synth.logits_f32(4, 0, T, shape.E).copy()
    lg[:, 3] += 50.0
    lg[:, 5] += 40.0
    _check(m, W, xb, lg, shape.k, fn, sh, "a8 skewed")


def test_prefill_a8_wide_range(m):
    """Activations spanning many binades within a block (x ~ N(0,1) times
    2^U(-12, 12) per element): small values land on E4M3 subnormals or 0."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = 96
    xb = synth.activations_bf16(8, 0, T, shape.H)
    v = synth.bf16_values(xb).astype(np.float32)
    g = np.random.default_rng(8).uniform(-12, 12, v.shape)
    xb = synth.bf16_bits_from_f32((v * np.exp2(np.round(g))).astype(np.float32))
    _check(m, W, xb, synth.logits_f32(8, 0, T, shape.E), shape.k, fn, sh, "a8 wide range")


def test_prefill_a8_max_tokens(m):
    """T = MOEDEC_MAX_PREFILL_T (65,536) on the tiny shape; h and y sampled."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = m._lib.MOEDEC_MAX_PREFILL_T
    xb = synth.activations_bf16(9, 0, T, shape.H)
    tokens = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(9).choice(T, 30, replace=False)]))
    _check(m, W, xb, synth.logits_f32(9, 0, T, shape.E), shape.k, fn, sh, f"a8 tiny T={T}", tokens=tokens)


def test_prefill_a8_repeatable(m):
    W, fn, sh = _small_layer(m, MID, seed=6)
    xb = synth.activations_bf16(6, 0, 700, MID.H)
    lg = synth.logits_f32(6, 0, 700, MID.E)
    a = _run(m, W, xb, lg, MID.k)
    b = _run(m, W, xb, lg, MID.k)
    np.testing.assert_array_equal(a[3], b[3])
    np.testing.assert_array_equal(a[4], b[4])


@pytest.fixture(scope="module")
def ling_layer(m):
    import synth.device as sd
    say("generate Ling layer on device")
    lay = sd.canonical_layer(0, 0, synth.LING, "cuda")
    W = m.MoELayerWeights.from_canonical(lay["gate"], lay["up"], lay["down"], synth.LING.E)
    torch.cuda.synchronize()
    del lay
    return W


def _ling_expert(e):
    return dense_expert({n: (c[None], s[None]) for n, (c, s) in
                         synth.mxfp4_expert(0, 0, e, synth.LING).items()}, 0)


@pytest.mark.parametrize("T,n_sample", [(64, 3), (4096, 3), (32768, 3)])
def test_prefill_a8_ling(m, ling_layer, T, n_sample):
    """Ling-shaped layer (hidden 2560, 512 experts top-8 + shared, I 768):
    routing, counts and x's MXFP8 on every token; h and y on the first, last
    and a few seeded tokens; T = 32,768 is the largest token count the bench
    times."""
    xb = synth.activations_bf16(7, 0, T, synth.LING.H)
    lg = synth.logits_f32(7, 0, T, synth.LING.E)
    rng = np.random.default_rng(T)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample, replace=False)]))
    _check(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), f"a8 ling T={T}", tokens=tokens)
