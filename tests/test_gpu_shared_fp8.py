"""GPU parity of the FP8 shared expert (E4M3, one float32 scale per row):
its packing against the documented layout of the oracle's codes, and the
fused layer with it -- one token and several, ragged shapes, the Ling shape,
the residual form and the router chain -- against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import bf16_tensor, bits_of, check_acc, check_bf16, dense_expert, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


def _layout_rows(codes, n_units, n_chunks):
    """The documented lane layout of row-major codes [16 * n_units][K]:
    [unit][chunk][64 lanes][16], lane l = row 16 unit + (l & 15), values
    64 chunk + 16 (l >> 4) .. + 15, zero past K."""
    R, K = codes.shape
    padded = np.zeros((R, 64 * n_chunks), dtype=np.uint8)
    padded[:, :K] = codes
    out = padded.reshape(n_units, 16, n_chunks, 4, 16)            # [unit][row][chunk][quarter][b]
    return out.transpose(0, 2, 3, 1, 4).reshape(n_units, n_chunks, 64, 16)


def _expected_pack(g_bits, u_bits, d_bits):
    I, H = g_bits.shape
    kh8, ki8 = 2 * ((H // 32 + 3) // 4), 2 * ((I // 32 + 3) // 4)
    qg, sg = oracle.quant_fp8_rows(synth.bf16_values(g_bits))
    qu, su = oracle.quant_fp8_rows(synth.bf16_values(u_bits))
    qd, sd = oracle.quant_fp8_rows(synth.bf16_values(d_bits))
    gu = np.stack([_layout_rows(qg, I // 16, kh8), _layout_rows(qu, I // 16, kh8)], axis=2)   # [u][c][2][64][16]
    dn = _layout_rows(qd, H // 16, ki8)
    return gu.reshape(-1), np.concatenate([sg, su]), dn.reshape(-1), sd


@pytest.mark.parametrize("H,I", [(256, 64), (192, 96), (2560, 768)])
def test_pack_matches_documented_layout(m, H, I):
    """Codes and scales bit for bit against the oracle's per-row E4M3 rule
    laid out as documented, including an all-zero row, a row of -0.0 and a
    row whose absmax is negative."""
    say("pack shared fp8", H, I)
    g, u, d = synth.shared_expert_bf16(2, 0, H, I)
    g[3] = 0
    u[5] = 0x8000
    d[7, 1] = synth.bf16_bits_from_f32(np.float32([-1.5]))[0]
    gu_c, gu_s, dn_c, dn_s = m.pack_shared_fp8(bf16_tensor(g), bf16_tensor(u), bf16_tensor(d))
    torch.cuda.synchronize()
    e_gu, e_gs, e_dn, e_ds = _expected_pack(g, u, d)
    np.testing.assert_array_equal(gu_s.cpu().numpy(), e_gs)
    np.testing.assert_array_equal(dn_s.cpu().numpy(), e_ds)
    np.testing.assert_array_equal(gu_c.cpu().numpy(), e_gu)
    np.testing.assert_array_equal(dn_c.cpu().numpy(), e_dn)


def _fp8_layer(m, shape, seed=0, layer=0):
    """Routed MXFP4 experts of a host-generated layer and an FP8 shared expert
    from bf16 weights; returns (weights, expert_fn, dense shared)."""
    lay = synth.mxfp4_layer(seed, layer, shape)
    E = shape.E
    dev = {n: tuple(torch.from_numpy(a[:E]).cuda() for a in lay[n]) for n in lay}
    gu_c, gu_s = m.pack_gateup(dev["gate"][0], dev["gate"][1], dev["up"][0], dev["up"][1])
    dn_c, dn_s = m.pack_down(dev["down"][0], dev["down"][1])
    g, u, d = synth.shared_expert_bf16(seed, layer, shape.H, shape.I)
    sh8 = m.pack_shared_fp8(bf16_tensor(g), bf16_tensor(u), bf16_tensor(d))
    W = m.MoELayerWeights(E, shape.H, shape.I, gu_c, gu_s, dn_c, dn_s, shared_fp8=sh8)
    dense = {e: dense_expert(lay, e) for e in range(E)}
    shared = oracle.shared_fp8_dense(synth.bf16_values(g), synth.bf16_values(u), synth.bf16_values(d))
    return W, (lambda e: dense[e]), shared


def _check_layer(m, W, x_bits, logits, k, expert_fn, shared, what):
    say("fp8 shared", what)
    x = bf16_tensor(x_bits)
    M = x.shape[0]
    ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    y, y32 = m.moe_layer(W, x, torch.from_numpy(logits).cuda(), k, ws, ids=ids)
    torch.cuda.synchronize()
    assert m.check_ffn_workspace(ws) == 0
    ref_ids, _, ref_y = oracle_layer(x_bits, logits, k, expert_fn, shared)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    y32 = y32.cpu().numpy()
    check_acc(y32, ref_y, what)
    check_bf16(bits_of(y), y32, ref_y, what)
    return y32


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_fp8_shared_tiny(m, M):
    shape = synth.TINY
    W, ef, sh = _fp8_layer(m, shape, seed=3)
    xb = synth.activations_bf16(3, 0, M, shape.H)
    _check_layer(m, W, xb, synth.router_logits_f32(3, xb, shape.E), shape.k, ef, sh, f"tiny M={M}")


@pytest.mark.parametrize("H,I,E,k,M", [(192, 96, 8, 3, 2), (320, 160, 5, 2, 4), (64, 32, 3, 3, 1),
                                       (1536, 768, 20, 16, 1), (1024, 768, 20, 16, 4)])
def test_fp8_shared_ragged_and_grid_forms(m, H, I, E, k, M):
    """Chunk counts not a multiple of four (zero padding in both layouts), a
    shared slot alone in its group, and the one-token grid of a block per
    unit."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=127 - 8, scale_hi=127 - 4)
    W, ef, sh = _fp8_layer(m, shape, seed=H + M)
    xb = synth.activations_bf16(H, 0, M, H)
    _check_layer(m, W, xb, synth.router_logits_f32(H, xb, E), k, ef, sh, f"H={H} I={I} E={E} k={k} M={M}")


def test_fp8_shared_zero_input_is_exact_zero(m):
    W, ef, sh = _fp8_layer(m, synth.TINY, seed=4)
    xb = np.zeros((2, synth.TINY.H), dtype=np.uint16)
    y32 = _check_layer(m, W, xb, synth.logits_f32(4, 0, 2, synth.TINY.E), synth.TINY.k, ef, sh, "x = 0")
    assert not y32.any()


@pytest.fixture(scope="module")
def ling_fp8(m):
    """The Ling layer's 512 routed MXFP4 experts (device-generated) with an FP8
    shared expert of the Ling shape."""
    import synth.device as sd
    say("generate Ling layer on device (FP8 shared)")
    lay = sd.canonical_layer(0, 0, synth.LING, "cuda")
    E, H, I = synth.LING.E, synth.LING.H, synth.LING.I
    gu_c, gu_s = m.pack_gateup(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1])
    dn_c, dn_s = m.pack_down(lay["down"][0], lay["down"][1])
    del lay
    g, u, d = synth.shared_expert_bf16(0, 0, H, I)
    sh8 = m.pack_shared_fp8(bf16_tensor(g), bf16_tensor(u), bf16_tensor(d))
    W = m.MoELayerWeights(E, H, I, gu_c, gu_s, dn_c, dn_s, shared_fp8=sh8)
    torch.cuda.synchronize()
    shared = oracle.shared_fp8_dense(synth.bf16_values(g), synth.bf16_values(u), synth.bf16_values(d))
    return W, shared


def _ling_expert(e, cache={}):
    if e not in cache:
        cache[e] = dense_expert({n: (c[None], s[None]) for n, (c, s) in
                                 synth.mxfp4_expert(0, 0, e, synth.LING).items()}, 0)
    return cache[e]


@pytest.mark.parametrize("name", ["ling_m1", "ling_m4"])
def test_fp8_shared_ling(m, ling_fp8, name):
    W, shared = ling_fp8
    xb, lg = synth.moe_inputs(synth.WORKLOADS[name])
    _check_layer(m, W, xb, lg, 8, _ling_expert, shared, name)


def test_fp8_shared_residual_and_router_chain(m, ling_fp8):
    """The residual form and the router chain on the Ling layer with the FP8
    shared expert: y equals the fused layer on the exported x bit for bit and
    the oracle within tolerance; r advances by exactly y."""
    W, shared = ling_fp8
    H, E = synth.LING.H, synth.LING.E
    r0 = np.random.default_rng(12).standard_normal((2, H)).astype(np.float32)
    r = torch.from_numpy(r0).cuda()
    wr_bits = synth.router_weight_bf16(3, 0, E, H)
    ws = m.make_ffn_workspace(2, 8, H, synth.LING.I, "cuda")
    x_out = torch.empty((2, H), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((2, H), dtype=torch.float32, device="cuda")
    say("fp8 shared router chain ling M=2")
    r_out, lg = m.moe_layer_rmsnorm_router(W, bf16_tensor(wr_bits), r, 8, ws, x_out=x_out, y_f32=y32)
    _, y_plain = m.moe_layer(W, x_out, lg, 8, ws)
    torch.cuda.synchronize()
    assert m.check_ffn_workspace(ws) == 0
    y_h = y32.cpu().numpy()
    np.testing.assert_array_equal(y_h, y_plain.cpu().numpy())
    np.testing.assert_array_equal(r_out.cpu().numpy(), r0 + y_h)
    _, _, ref_y = oracle_layer(bits_of(x_out), lg.cpu().numpy(), 8, _ling_expert, shared)
    check_acc(y_h, ref_y, "fp8 shared router chain")
