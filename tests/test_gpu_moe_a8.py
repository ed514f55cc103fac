"""GPU parity of the W4A8 fused decode layer (moe_layer_mxfp4_a8: MXFP8 x
and h) against the oracle (oracle.w4a8), through the C ABI, stage by stage:
  routing   ids bit-exact against oracle.route_topk;
  h         the float32 h the kernel leaves in its workspace
            (moe_ffn_workspace_layout) for each (slot, token) against the
            oracle's silu(W_gate x_q) * (W_up x_q) from x's MXFP8 (exact on both
            sides) within the float32 accumulator tolerance;
  y         y_f32 against the oracle's MXFP8 rounding, down products and
            combine applied to the kernel's own h within the same tolerance
            (the kernel's products of E2M1 x 2^k weights and MXFP8 values are
            exact; they accumulate in float32); y_bf16 the nearest-even
            rounding of y_f32;
  end to end, against moe_layer_w4a8 within 2 % of the token's largest output
            (h may round across an MXFP8 boundary there: a sanity bound)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import w4a8
from gpu_helpers import bf16_tensor, bits_of, check_acc, dense_expert, say

pytestmark = pytest.mark.gpu

E2E_REL = 2e-2

@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


def _host_case(m, shape, M, seed=0):
    lay = synth.mxfp4_layer(seed, 0, shape)
    dev = {n: tuple(torch.from_numpy(a).cuda() for a in lay[n]) for n in lay}
    W = m.MoELayerWeights.from_canonical(dev["gate"], dev["up"], dev["down"], shape.E)
    xb = synth.activations_bf16(seed, 0, M, shape.H)
    lg = synth.router_logits_f32(seed, xb, shape.E)
    dense = {e: dense_expert(lay, e) for e in range(shape.E + 1)}
    return W, xb, lg, (lambda e: dense[e]), dense[shape.E]


def _check(m, W, xb, lg, k, expert_fn, shared, what):
    M = xb.shape[0]
    say(what, "M", M)
    ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    disp = torch.zeros(m.DISPATCH_BYTES, dtype=torch.uint8, device="cuda")
    y, y32 = m.moe_layer(W, bf16_tensor(xb), torch.from_numpy(lg).cuda(), k, ws, ids=ids, dispatch=disp,
                         act8=True)
    torch.cuda.synchronize()
    assert m.check_ffn_workspace(ws) == 0
    ref_ids, ref_w = oracle.route_topk(lg, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids, err_msg=f"{what}: expert ids")
    d = m.decode_dispatch(disp)
    hg = m.ffn_workspace_h(ws, M, k, W.H, W.I).cpu().numpy().astype(np.float64)
    x = synth.bf16_values(xb).astype(np.float64)
    x_q = w4a8.mxfp8_round(x)
    # h per (slot, token) against the oracle; y from the kernel's own h
    y_ref = np.zeros((M, W.H))
    # workspace slot 0 is the shared expert (the table's last entry), slot
    # s >= 1 the table's routed entry s - 1
    for s in range(d["n_slots"]):
        e = W.E if s == 0 else int(d["expert"][s - 1])
        mask = (1 << M) - 1 if s == 0 else int(d["token_mask"][s - 1])
        wg, wu, wd = expert_fn(e) if e < W.E else shared
        for t in range(M):
            if not (mask >> t) & 1:
                continue
            h_ref = w4a8.w4a8_h(wg, wu, x_q[t:t + 1])[0]
            check_acc(hg[s, t][None], h_ref[None], f"{what}: h of slot {s} (expert {e}) token {t}")
            wt = 1.0 if e == W.E else float(ref_w[t][list(ref_ids[t]).index(e)])
            y_ref[t] += wt * (wd @ w4a8.mxfp8_round(hg[s, t][None])[0])
    check_acc(y32.cpu().numpy(), y_ref, f"{what}: y from the kernel's h")
    own = y32.cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits_of(y), own, err_msg=f"{what}: bf16 is not RNE of y_f32")
    # end to end (sanity bound)
    ref = w4a8.moe_layer_w4a8(x, ref_ids, ref_w, expert_fn, shared)
    err = np.max(np.abs(y32.cpu().numpy() - ref), axis=1)
    assert (err <= E2E_REL * np.max(np.abs(ref), axis=1)).all(), f"{what}: end to end {err}"


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_a8_tiny(m, M):
    W, xb, lg, fn, sh = _host_case(m, synth.TINY, M)
    _check(m, W, xb, lg, synth.TINY.k, fn, sh, f"a8 tiny M={M}")


@pytest.mark.parametrize("H,I,E,k,M", [(320, 96, 24, 3, 4), (192, 160, 8, 3, 2), (64, 32, 3, 3, 1)])
def test_a8_ragged(m, H, I, E, k, M):
    """Block counts that are not multiples of four (padded MX blocks of x
    and h), a partial last group of pairs."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=127 - 8, scale_hi=127 - 5)
    W, xb, lg, fn, sh = _host_case(m, shape, M, seed=3)
    _check(m, W, xb, lg, k, fn, sh, f"a8 ragged H={H} I={I} M={M}")


@pytest.mark.parametrize("H,I,E,k,M", [(1024, 64, 8, 2, 3), (2048, 128, 8, 3, 2), (4096, 64, 16, 4, 4),
                                       (4096, 2048, 4, 2, 1)])
def test_a8_wide_hidden(m, H, I, E, k, M):
    """Hidden sizes that select the other chunk-pair counts per wave (2, 4, 8)
    and the largest intermediate size."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=127 - 9, scale_hi=127 - 5)
    W, xb, lg, fn, sh = _host_case(m, shape, M, seed=4)
    _check(m, W, xb, lg, k, fn, sh, f"a8 H={H} I={I} M={M}")


def test_a8_zero_and_wide_blocks(m):
    """A token of zeros (every block scale 2^-127) and a token whose blocks
    span 2^+-10 (E4M3 subnormals and zeros after quantisation)."""
    shape = synth.TINY
    W, xb, lg, fn, sh = _host_case(m, shape, 2, seed=5)
    xb = xb.copy()
    xb[0] = 0
    v = synth.bf16_values(xb[1:2]).astype(np.float32)
    sc = np.exp2(np.round(np.random.default_rng(5).uniform(-10, 10, v.shape)))
    xb[1:2] = synth.bf16_bits_from_f32((v * sc).astype(np.float32))
    _check(m, W, xb, lg, shape.k, fn, sh, "a8 zero and wide blocks")


@pytest.fixture(scope="module")
def ling_layer(m):
    import synth.device as sd
    say("generate Ling layer on device")
    lay = sd.canonical_layer(0, 0, synth.LING, "cuda")
    W = m.MoELayerWeights.from_canonical(lay["gate"], lay["up"], lay["down"], synth.LING.E)
    torch.cuda.synchronize()
    del lay
    return W


def _ling_expert(e, cache={}):
    if e not in cache:
        cache[e] = dense_expert({n: (c[None], s[None]) for n, (c, s) in
                                 synth.mxfp4_expert(0, 0, e, synth.LING).items()}, 0)
    return cache[e]


@pytest.mark.parametrize("M,seed", [(1, 0), (1, 1), (2, 2), (3, 3), (4, 4)])
def test_a8_ling(m, ling_layer, M, seed):
    """The Ling-shaped layer (hidden 2560, 512 experts top-8 + shared, I 768)
    at M = 1..4 (the one-token block-per-unit grid and the persistent grid)."""
    xb = synth.activations_bf16(seed, 0, M, synth.LING.H)
    lg = synth.logits_f32(seed, 0, M, synth.LING.E)
    _check(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), f"a8 ling M={M} seed={seed}")
