"""GPU parity of the many-token MoE layer (moe_layer_mxfp4_prefill, grouped
GEMM on bf16 matrix cores) against the float64 oracle, through the C ABI:
routing and per-expert token counts bit-exact, routing weights within 1e-6,
y_f32 within the float32-accumulator tolerance, y_bf16 within the bf16 rule
(gpu_helpers).  Small shapes are checked on every token; the Ling-shaped layer
on sampled tokens, which the oracle evaluates one expert at a time."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import W_ATOL, bf16_tensor, bits_of, check_acc, check_bf16, dense_expert, say

pytestmark = pytest.mark.gpu

MID = synth.MoEShape(H=512, I=256, E=32, k=4, scale_lo=127 - 9, scale_hi=127 - 5)
# H = 320: 10 MX blocks (not a multiple of 4) and a partial 128-row block of
# outputs; I = 96: 3 MX blocks and a partial 128-row block of h.
ODD = synth.MoEShape(H=320, I=96, E=24, k=3, scale_lo=127 - 8, scale_hi=127 - 5)


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


def _run(m, W, x_bits, logits, k, workspace=None):
    T = x_bits.shape[0]
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    counts = torch.full((W.E + 1,), -1, dtype=torch.int32, device="cuda")
    y, y32 = m.moe_layer_prefill(W, bf16_tensor(x_bits), torch.from_numpy(logits).cuda(), k,
                                 workspace=workspace, ids=ids, topk_w=tw, counts=counts)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), tw.cpu().numpy(), counts.cpu().numpy(), bits_of(y), y32.cpu().numpy()


def _check(m, W, x_bits, logits, k, expert_fn, shared, what, tokens=None, workspace=None):
    T = x_bits.shape[0]
    say(what, "T", T, "k", k)
    ids, tw, counts, yb, y32 = _run(m, W, x_bits, logits, k, workspace)
    ref_ids, ref_w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids, ref_ids, err_msg=f"{what}: expert ids")
    assert np.max(np.abs(tw - ref_w)) <= W_ATOL, f"{what}: routing weights"
    groups = oracle.expert_groups(ref_ids, W.E)
    np.testing.assert_array_equal(counts, [len(g) for g in groups], err_msg=f"{what}: group counts")
    x = synth.bf16_values(x_bits).astype(np.float64)
    ref = oracle.moe_layer_by_expert(x, ref_ids, ref_w, expert_fn, shared, tokens=tokens)
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    check_acc(y32[sel], ref, what)
    check_bf16(yb[sel], y32[sel], ref, what)
    return yb, y32


@pytest.mark.parametrize("T", [1, 8, 37, 200, 600])
def test_prefill_tiny(m, T):
    """hidden 256, 16 experts top-2, I 64 (one 128-k chunk of down, half of it
    padding); T = 200 and 600 give 64- and 128-token tiles."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    xb = synth.activations_bf16(1, 0, T, shape.H)
    _check(m, W, xb, synth.router_logits_f32(1, xb, shape.E), shape.k, fn, sh, f"prefill tiny T={T}")


@pytest.mark.parametrize("T", [300, 700])
def test_prefill_mid(m, T):
    """Two 128-row blocks of h, four of outputs, several tiles per expert."""
    W, fn, sh = _small_layer(m, MID, seed=2)
    xb = synth.activations_bf16(2, 0, T, MID.H)
    _check(m, W, xb, synth.logits_f32(2, 0, T, MID.E), MID.k, fn, sh, f"prefill mid T={T}")


def test_prefill_odd_shape(m):
    W, fn, sh = _small_layer(m, ODD, seed=3)
    xb = synth.activations_bf16(3, 0, 129, ODD.H)
    _check(m, W, xb, synth.logits_f32(3, 0, 129, ODD.E), ODD.k, fn, sh, "prefill odd H=320 I=96 T=129")


def test_prefill_max_k(m):
    """k = 32 of 64 experts (the largest k): 33 pairs per token."""
    shape = synth.MoEShape(H=256, I=64, E=64, k=32, scale_lo=127 - 8, scale_hi=127 - 5)
    W, fn, sh = _small_layer(m, shape, seed=11)
    xb = synth.activations_bf16(11, 0, 100, shape.H)
    _check(m, W, xb, synth.logits_f32(11, 0, 100, shape.E), shape.k, fn, sh, "prefill k=32 of 64")


def test_prefill_skewed_routing_and_idle_experts(m):
    """Every token picks experts 3 and 5 (1000 rows each: eight 128-token tiles
    and a ragged one); the other 14 experts get no token at all."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = 1000
    xb = synth.activations_bf16(4, 0, T, shape.H)
    lg = synth.logits_f32(4, 0, T, shape.E).copy()
    lg[:, 3] += 50.0
    lg[:, 5] += 40.0
    _check(m, W, xb, lg, shape.k, fn, sh, "prefill skewed")


def test_prefill_max_tokens(m):
    """T = MOEDEC_MAX_PREFILL_T (65,536) on the tiny shape: 8,192 tokens per
    expert on average; routing and counts on every token, outputs sampled."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = m._lib.MOEDEC_MAX_PREFILL_T
    xb = synth.activations_bf16(9, 0, T, shape.H)
    tokens = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(9).choice(T, 30, replace=False)]))
    _check(m, W, xb, synth.logits_f32(9, 0, T, shape.E), shape.k, fn, sh, f"prefill tiny T={T}", tokens=tokens)


def test_prefill_chunk_tails_and_reuse(m):
    """Counting runs over chunks of the token-major routed pairs (at most 64
    chunks of at least 2,048 pairs).  T = 65,535 on the tiny shape (k = 2):
    64 chunks of 2,048 pairs, the last one 2,046; the first 30,000 tokens all
    pick experts 3 and 5, so the early chunks' counts differ from the late
    ones'.  Tokens at chunk edges (1,024 tokens per chunk) are sampled.  Then
    T = 3,001 (three chunks, a ragged last) on the same workspace, in full."""
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    T = 65535
    ws = m.make_prefill_workspace(T, shape.E, shape.k, shape.H, shape.I, "cuda")
    xb = synth.activations_bf16(12, 0, T, shape.H)
    lg = synth.logits_f32(12, 0, T, shape.E).copy()
    lg[:30000, 3] += 50.0
    lg[:30000, 5] += 40.0
    edges = [c * 1024 + d for c in (1, 2, 29, 30, 63) for d in (-1, 0)]
    tokens = np.unique(np.concatenate([[0, 29999, 30000, T - 2, T - 1], edges,
                                       np.random.default_rng(12).choice(T, 20, replace=False)]))
    _check(m, W, xb, lg, shape.k, fn, sh, f"prefill chunk tails T={T}", tokens=tokens, workspace=ws)
    xb2 = synth.activations_bf16(13, 0, 3001, shape.H)
    _check(m, W, xb2, synth.logits_f32(13, 0, 3001, shape.E), shape.k, fn, sh, "prefill T=3001 after T=65535",
           workspace=ws)


def test_prefill_zero_input(m):
    shape = synth.TINY
    W, fn, sh = _small_layer(m, shape)
    xb = np.zeros((70, shape.H), np.uint16)
    _, _, _, yb, y32 = _run(m, W, xb, synth.logits_f32(5, 0, 70, shape.E), shape.k)
    assert (y32 == 0).all() and (yb == 0).all()


def test_prefill_repeatable_and_workspace_reuse(m):
    """Rows inside an expert's group follow LDS-atomic arrival order; the
    outputs must not depend on it: two calls on one workspace give identical bits, and
    a smaller call after a larger one on the same workspace is still correct."""
    W, fn, sh = _small_layer(m, MID, seed=6)
    ws = m.make_prefill_workspace(700, MID.E, MID.k, MID.H, MID.I, "cuda")
    xb = synth.activations_bf16(6, 0, 700, MID.H)
    lg = synth.logits_f32(6, 0, 700, MID.E)
    a = _run(m, W, xb, lg, MID.k, ws)
    b = _run(m, W, xb, lg, MID.k, ws)
    np.testing.assert_array_equal(a[3], b[3])
    np.testing.assert_array_equal(a[4], b[4])
    _check(m, W, xb[:90], lg[:90], MID.k, fn, sh, "prefill mid T=90 after T=700", workspace=ws)


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


@pytest.mark.parametrize("T,n_sample", [(64, 4), (256, 4), (4096, 3), (32768, 3)])
def test_prefill_ling(m, ling_layer, T, n_sample):
    """Ling-shaped layer (hidden 2560, 512 experts top-8 + shared, I 768):
    routing and counts on every token, outputs on the first, last and a few
    seeded tokens; T = 32,768 is the largest token count the bench times."""
    xb = synth.activations_bf16(7, 0, T, synth.LING.H)
    lg = synth.logits_f32(7, 0, T, synth.LING.E)
    rng = np.random.default_rng(T)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample, replace=False)]))
    _check(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), f"prefill ling T={T}",
           tokens=tokens)
