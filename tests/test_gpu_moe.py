"""GPU parity of routing, MXFP4 packing and the routed + shared expert FFN
against the float64 oracle, through the C ABI (via the ctypes binding)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (ACC_RTOL, W_ATOL, bf16_tensor, bits_of, check_acc, check_bf16, dense_expert,
                         oracle_layer, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


# ---------------------------------------------------------------- routing

def _check_route(m, logits, k):
    say("route", logits.shape, "k", k)
    ids, w, disp = m.route_topk(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    assert np.max(np.abs(w.cpu().numpy() - ref_w)) <= W_ATOL
    d = m.decode_dispatch(disp)
    experts, masks, weights = oracle.dispatch_table(ref_ids, ref_w, logits.shape[1])
    assert d["n_slots"] == len(experts) and d["M"] == logits.shape[0]
    np.testing.assert_array_equal(d["expert"], experts)
    np.testing.assert_array_equal(d["token_mask"], masks)
    assert np.max(np.abs(d["weight"][:, :logits.shape[0]] - weights)) <= W_ATOL
    raw = d["raw"]
    for s in range(d["n_slots"], m.MAX_SLOTS):          # unused entries are zero
        assert raw.expert[s] == 0 and raw.token_mask[s] == 0
    return ids, w, disp


@pytest.mark.parametrize("name", ["tiny_m1", "ling_m1", "ling_m4"])
def test_route_workloads(m, name):
    wl = synth.WORKLOADS[name]
    _, lg = synth.moe_inputs(wl)
    _check_route(m, lg, wl.shape.k)


@pytest.mark.parametrize("seed", range(3))
def test_route_ling_m4_seeds(m, seed):
    _check_route(m, synth.logits_f32(seed, 7, 4, 512), 8)


@pytest.mark.parametrize("seed", range(4))
def test_route_tie_heavy(m, seed):
    rng = np.random.default_rng(100 + seed)
    lg = rng.choice(np.float32([-1.0, 0.0, -0.0, 1.0, 0.5]), size=(4, 512))
    for k in (1, 8, 32):
        _check_route(m, lg, k)


def test_route_all_equal_and_signed_zeros(m):
    lg = np.zeros((4, 64), np.float32)
    lg[1] = -0.0
    lg[2, ::2] = -0.0
    _check_route(m, lg, 16)


@pytest.mark.parametrize("M,E,k", [(1, 1, 1), (2, 16, 16), (3, 100, 7), (4, 1024, 32), (4, 1000, 32),
                                   (1, 65, 1), (4, 512, 1)])
def test_route_shapes(m, M, E, k):
    lg = synth.logits_f32(3, E, M, E) * np.float32(4.0)
    _check_route(m, lg, k)


# ---------------------------------------------------------------- packing

PAD_SCALE = 127


def _lanes(a, n_units, kb4):
    """[n][rows][kb4*4][...] -> [n][rows/16][kb4][64][...] with lane l = row
    16u + (l & 15), MX block 4c + (l >> 4)."""
    n = a.shape[0]
    tail = a.shape[3:]
    a = a.reshape((n, n_units, 16, kb4, 4) + tail)
    a = a.transpose((0, 1, 3, 4, 2) + tuple(range(5, 5 + len(tail))))
    return np.ascontiguousarray(a).reshape((n, n_units, kb4, 64) + tail)


def _pad_blocks(codes, scales, kb4):
    n, rows, half_k = codes.shape
    kb = 2 * half_k // 32
    c = np.zeros((n, rows, kb4 * 4, 16), np.uint8)
    c[:, :, :kb] = codes.reshape(n, rows, kb, 16)
    s = np.full((n, rows, kb4 * 4), PAD_SCALE, np.uint8)
    s[:, :, :kb] = scales
    return c, s


def np_pack_gateup(gc, gs, uc, us):
    n, I, hh = gc.shape
    kb4 = (2 * hh // 32 + 3) // 4
    gcp, gsp = _pad_blocks(gc, gs, kb4)
    ucp, usp = _pad_blocks(uc, us, kb4)
    codes = np.stack([_lanes(gcp, I // 16, kb4), _lanes(ucp, I // 16, kb4)], axis=3)
    scales = np.stack([_lanes(gsp, I // 16, kb4), _lanes(usp, I // 16, kb4)], axis=-1)
    return codes.reshape(-1), scales.reshape(-1)


def np_pack_down(dc, ds):
    n, H, hi = dc.shape
    kb4 = (2 * hi // 32 + 3) // 4
    dcp, dsp = _pad_blocks(dc, ds, kb4)
    return _lanes(dcp, H // 16, kb4).reshape(-1), _lanes(dsp, H // 16, kb4).reshape(-1)


@pytest.mark.parametrize("H,I,E", [(256, 64, 4), (192, 96, 3), (2560, 768, 2)])
def test_pack_is_the_documented_permutation(m, H, I, E):
    say("pack", H, I, E)
    shape = synth.MoEShape(H=H, I=I, E=E, k=1, scale_lo=110, scale_hi=140)
    lay = synth.mxfp4_layer(5, 0, shape)
    dev = {n: tuple(torch.from_numpy(a).cuda() for a in lay[n]) for n in lay}
    gu_c, gu_s = m.pack_gateup(dev["gate"][0], dev["gate"][1], dev["up"][0], dev["up"][1])
    dn_c, dn_s = m.pack_down(dev["down"][0], dev["down"][1])
    torch.cuda.synchronize()
    ec, es = np_pack_gateup(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1])
    np.testing.assert_array_equal(gu_c.cpu().numpy(), ec)
    np.testing.assert_array_equal(gu_s.cpu().numpy(), es)
    dc, ds = np_pack_down(lay["down"][0], lay["down"][1])
    np.testing.assert_array_equal(dn_c.cpu().numpy(), dc)
    np.testing.assert_array_equal(dn_s.cpu().numpy(), ds)


def test_device_generator_matches_host_twin(m):
    import synth.device as sd
    say("synth device twin")
    shape = synth.LING
    lay = sd.canonical_layer(0, 3, shape, "cuda", n_experts=shape.E + 1)
    torch.cuda.synchronize()
    for e in (0, 17, 511, 512):
        host = synth.mxfp4_expert(0, 3, e, shape)
        for name in ("gate", "up", "down"):
            np.testing.assert_array_equal(lay[name][0][e].cpu().numpy(), host[name][0])
            np.testing.assert_array_equal(lay[name][1][e].cpu().numpy(), host[name][1])


# ---------------------------------------------------------------- router logits

def _check_route_from_router(ids, w, ref_logits, k, what):
    """Selection from the kernel's float32 logits against the float64 oracle
    logits.  The two differ by float32 rounding, so where two logits that
    decide the selection or its order lie within 2 * tol of each other either
    outcome is correct; there only validity is required.  Elsewhere the ids
    must equal the oracle's, and the weights its softmax over the chosen."""
    E = ref_logits.shape[1]
    for m in range(ref_logits.shape[0]):
        L = ref_logits[m]
        tol = ACC_RTOL * np.max(np.abs(L))
        g = ids[m].astype(np.int64)
        assert len(set(g.tolist())) == k, f"{what} token {m}: repeated ids"
        chosen = np.zeros(E, dtype=bool)
        chosen[g] = True
        if k < E:
            assert L[g].min() >= L[~chosen].max() - 2 * tol, f"{what} token {m}: not a top-{k}"
        assert np.all(L[g][:-1] >= L[g][1:] - 2 * tol), f"{what} token {m}: order"
        order = np.lexsort((np.arange(E), -L))
        top = L[order[:min(k + 1, E)]]
        if np.all(np.abs(np.diff(top)) > 2 * tol):
            np.testing.assert_array_equal(g, order[:k], err_msg=f"{what} token {m}")
        p = np.exp(L[g] - L[g].max())
        np.testing.assert_allclose(w[m], p / p.sum(), rtol=0, atol=1e-5, err_msg=f"{what} token {m}")


@pytest.mark.parametrize("E,H,k,M", [(512, 2560, 8, 1), (512, 2560, 8, 4), (16, 256, 2, 3), (1000, 72, 32, 2)])
def test_router_logits_and_route_from_x(m, E, H, k, M):
    """Router GEMV (bf16 W_router [E][H] ~ N(0, 1/H), x ~ N(0, 1)) within the
    float32-accumulator tolerance of the oracle, and the experts chosen from
    those logits under the near-tie rule."""
    say(f"router E={E} H={H} k={k} M={M}")
    wr_bits = synth.router_weight_bf16(0, 0, E, H)
    x_bits = synth.activations_bf16(0, 0, M, H)
    lg = m.router_logits(bf16_tensor(wr_bits), bf16_tensor(x_bits))
    ids, w, _ = m.route_topk(lg, k)
    torch.cuda.synchronize()
    ref = oracle.router_logits(synth.bf16_values(wr_bits), synth.bf16_values(x_bits))
    check_acc(lg.cpu().numpy(), ref, f"router logits E={E} H={H} M={M}")
    # routing on the kernel's own float32 logits is bit-exact against the oracle's
    ref_ids, ref_w = oracle.route_topk(lg.cpu().numpy(), k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    _check_route_from_router(ids.cpu().numpy(), w.cpu().numpy(), ref, k, f"route from x E={E} M={M}")


# ---------------------------------------------------------------- FFN

def _host_layer_case(m, shape, M, seed=0, layer=0, logits=None, x_bits=None, k=None):
    k = shape.k if k is None else k
    lay = synth.mxfp4_layer(seed, layer, shape)
    dev = {n: tuple(torch.from_numpy(a).cuda() for a in lay[n]) for n in lay}
    W = m.MoELayerWeights.from_canonical(dev["gate"], dev["up"], dev["down"], shape.E)
    if x_bits is None:
        x_bits = synth.activations_bf16(seed, layer, M, shape.H)
    if logits is None:
        logits = synth.router_logits_f32(seed, x_bits, shape.E)
    dense = {e: dense_expert(lay, e) for e in range(shape.E + 1)}
    return W, x_bits, logits, (lambda e: dense[e]), dense[shape.E], k


def _run_ffn(m, W, x_bits, logits, k, ws=None):
    x = bf16_tensor(x_bits)
    ids, w, disp = m.route_topk(torch.from_numpy(logits).cuda(), k)
    if ws is None:
        ws = m.make_ffn_workspace(x.shape[0], k, W.H, W.I, "cuda")
    y, y32 = m.expert_ffn(W, x, disp, k, ws)
    torch.cuda.synchronize()
    assert m.check_ffn_workspace(ws) == 0          # no cross-block wait gave up
    return ids.cpu().numpy(), bits_of(y), y32.cpu().numpy(), disp


def _check_case(m, W, x_bits, logits, k, expert_fn, shared, what):
    say(what)
    ids, yb, y32, _ = _run_ffn(m, W, x_bits, logits, k)
    ref_ids, _, ref_y = oracle_layer(x_bits, logits, k, expert_fn, shared)
    np.testing.assert_array_equal(ids, ref_ids)
    check_acc(y32, ref_y, what)
    check_bf16(yb, y32, ref_y, what)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_ffn_tiny(m, M):
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, M)
    _check_case(m, W, xb, lg, k, ef, sh, f"tiny M={M}")


def test_ffn_tiny_k_equals_e(m):
    W, xb, lg, ef, sh, _ = _host_layer_case(m, synth.TINY, 4)
    _check_case(m, W, xb, lg, synth.TINY.E, ef, sh, "tiny M=4 k=E")


def test_ffn_tiny_k1(m):
    W, xb, lg, ef, sh, _ = _host_layer_case(m, synth.TINY, 3)
    _check_case(m, W, xb, lg, 1, ef, sh, "tiny M=3 k=1")


@pytest.mark.parametrize("H,I,E,k,M", [(192, 96, 8, 3, 2), (320, 160, 5, 2, 4), (64, 32, 3, 3, 1)])
def test_ffn_ragged_block_counts(m, H, I, E, k, M):
    """Block counts that are not multiples of 4 exercise the scale padding."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=119, scale_hi=123)
    W, xb, lg, ef, sh, k = _host_layer_case(m, shape, M, seed=2)
    _check_case(m, W, xb, lg, k, ef, sh, f"ragged H={H} I={I} E={E} k={k} M={M}")


def test_ffn_dispatch_with_invalid_entries(m):
    """Table entries with an expert id outside [0, E) or an empty token mask
    contribute nothing: the result equals the oracle over the valid entries,
    and is bit-identical to the same table with those entries left out."""
    say("dispatch with invalid entries")
    M = 3
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, M, seed=3, k=4)
    x = bf16_tensor(xb)
    _, _, disp = m.route_topk(torch.from_numpy(lg).cuda(), k)
    d = m.decode_dispatch(disp)
    n = d["n_slots"]
    routed = [(int(d["expert"][i]), int(d["token_mask"][i]), d["weight"][i].copy()) for i in range(n - 1)]
    shared_entry = (int(d["expert"][n - 1]), int(d["token_mask"][n - 1]), d["weight"][n - 1].copy())
    assert len(routed) >= 4
    bad = {0: (-1, routed[0][1]), 2: (synth.TINY.E + 7, routed[2][1]), 3: (routed[3][0], 0)}
    with_bad = [(bad[i][0], bad[i][1], wt) if i in bad else (e, mk, wt) for i, (e, mk, wt) in enumerate(routed)]
    valid = [ent for i, ent in enumerate(routed) if i not in bad]

    def table(entries):
        t = m.Dispatch()
        rows = entries + [shared_entry]
        t.n_slots = len(rows)
        t.M = M
        for i, (e, mk, wt) in enumerate(rows):
            t.expert[i] = e
            t.token_mask[i] = mk
            for j in range(m.MAX_M):
                t.weight[i][j] = float(wt[j]) if j < len(wt) else 0.0
        return torch.frombuffer(bytearray(bytes(t)), dtype=torch.uint8).cuda()

    ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
    y_bad, y32_bad = m.expert_ffn(W, x, table(with_bad), k, ws)
    y_ok, y32_ok = m.expert_ffn(W, x, table(valid), k, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(y_bad), bits_of(y_ok))
    np.testing.assert_array_equal(y32_bad.cpu().numpy(), y32_ok.cpu().numpy())
    # oracle over the valid entries: per token, the experts whose mask has its bit
    ids = np.zeros((M, len(valid)), np.int64)
    w = np.zeros((M, len(valid)), np.float64)
    for j, (e, mk, wt) in enumerate(valid):
        for t in range(M):
            ids[t, j] = e
            w[t, j] = float(wt[t]) if (mk >> t) & 1 else 0.0
    ref = oracle.moe_layer(synth.bf16_values(xb).astype(np.float64), ids, w, ef, sh)
    check_acc(y32_ok.cpu().numpy(), ref, "valid entries only")


def test_ffn_zero_input_is_exact_zero(m):
    W, _, lg, _, _, k = _host_layer_case(m, synth.TINY, 2)
    xb = np.zeros((2, synth.TINY.H), np.uint16)
    _, yb, y32, _ = _run_ffn(m, W, xb, lg, k)
    assert (y32 == 0).all() and (yb == 0).all()


def test_ffn_workspace_reuse_is_deterministic(m):
    """Back-to-back calls on one workspace (the tickets reset themselves),
    with a different M in between, give bit-identical results."""
    say("workspace reuse")
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, 4)
    ws = m.make_ffn_workspace(4, k, W.H, W.I, "cuda")
    a = _run_ffn(m, W, xb, lg, k, ws)
    _run_ffn(m, W, xb[:1], lg[:1], k, ws)
    b = _run_ffn(m, W, xb, lg, k, ws)
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])


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


@pytest.mark.parametrize("name", ["ling_m1", "ling_m4"])
def test_ffn_ling(m, ling_layer, name):
    wl = synth.WORKLOADS[name]
    xb, lg = synth.moe_inputs(wl)
    _check_case(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), name)


@pytest.mark.parametrize("seed", [1, 2])
def test_ffn_ling_m4_more_seeds(m, ling_layer, seed):
    xb = synth.activations_bf16(seed, 0, 4, synth.LING.H)
    lg = synth.logits_f32(seed, 0, 4, synth.LING.E)
    _check_case(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), f"ling M=4 seed {seed}")


def test_ffn_ling_shared_tokens_overlap(m, ling_layer):
    """Four tokens routed to the same 8 experts: each expert serves all four."""
    xb = synth.activations_bf16(9, 0, 4, synth.LING.H)
    lg = np.repeat(synth.logits_f32(9, 0, 1, synth.LING.E), 4, axis=0)
    lg[1:, :] += np.float32(0.0)
    _check_case(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), "ling M=4 same experts")


# ---------------------------------------------------------------- fused layer (routing in the FFN launch)

def _run_fused(m, W, x_bits, logits, k, ws=None):
    x = bf16_tensor(x_bits)
    lg = torch.from_numpy(logits).cuda()
    M = x.shape[0]
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((M, k), dtype=torch.float32, device="cuda")
    disp = torch.zeros(m.DISPATCH_BYTES, dtype=torch.uint8, device="cuda")
    if ws is None:
        ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
    y, y32 = m.moe_layer(W, x, lg, k, ws, ids=ids, topk_w=wts, dispatch=disp)
    torch.cuda.synchronize()
    assert m.check_ffn_workspace(ws) == 0          # no cross-block wait gave up
    return ids.cpu().numpy(), wts.cpu().numpy(), disp, bits_of(y), y32.cpu().numpy()


def _check_fused(m, W, x_bits, logits, k, expert_fn, shared, what):
    say("fused", what)
    ids, wts, disp, yb, y32 = _run_fused(m, W, x_bits, logits, k)
    # routing outputs equal those of the separate routing call, bit for bit
    r_ids, r_w, r_disp = m.route_topk(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids, r_ids.cpu().numpy())
    np.testing.assert_array_equal(wts.view(np.uint32), r_w.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(disp.cpu().numpy(), r_disp.cpu().numpy())
    # the layer output equals the two-call path bit for bit, and the oracle within tolerance
    _, yb2, y322, _ = _run_ffn(m, W, x_bits, logits, k)
    np.testing.assert_array_equal(y32.view(np.uint32), y322.view(np.uint32))
    np.testing.assert_array_equal(yb, yb2)
    ref_ids, _, ref_y = oracle_layer(x_bits, logits, k, expert_fn, shared)
    np.testing.assert_array_equal(ids, ref_ids)
    check_acc(y32, ref_y, what)
    check_bf16(yb, y32, ref_y, what)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_fused_tiny(m, M):
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, M)
    _check_fused(m, W, xb, lg, k, ef, sh, f"tiny M={M}")


@pytest.mark.parametrize("H,I,E,k,M", [(192, 96, 8, 3, 2), (320, 160, 5, 2, 4), (64, 32, 3, 3, 1),
                                       (4096, 64, 40, 32, 4)])
def test_fused_ragged_and_extreme(m, H, I, E, k, M):
    """Ragged block counts, and the largest hidden size with k = 32 at M = 4
    (129 slots, many slot groups)."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=119, scale_hi=123)
    W, xb, lg, ef, sh, k = _host_layer_case(m, shape, M, seed=4)
    _check_fused(m, W, xb, lg, k, ef, sh, f"fused H={H} I={I} E={E} k={k} M={M}")


@pytest.mark.parametrize("M", [1, 2, 4])
def test_fused_largest_intermediate(m, M):
    """I = 2048, the largest supported intermediate size (64 MX blocks per down
    row, the widest h staging and the smallest slot groups the LDS allows)."""
    shape = synth.MoEShape(H=64, I=2048, E=6, k=2, scale_lo=119, scale_hi=123)
    W, xb, lg, ef, sh, k = _host_layer_case(m, shape, M, seed=9)
    _check_fused(m, W, xb, lg, k, ef, sh, f"fused H=64 I=2048 M={M}")


@pytest.mark.parametrize("H,I,E,k", [(256, 768, 40, 32), (1536, 768, 20, 16), (1024, 768, 20, 16)])
def test_fused_one_token_grid_forms(m, H, I, E, k):
    """One token: the kernel gives every work unit a block of its own when the
    units fit four blocks per CU, and otherwise walks them with the persistent
    three-block grid.  On a 256-CU MI355X the first two shapes (1,584 + 240 and
    816 + 288 units) take the persistent form and the last (816 + 192 = 1,008)
    the block-per-unit form at its limit; both forms must match the oracle."""
    shape = synth.MoEShape(H=H, I=I, E=E, k=k, scale_lo=119, scale_hi=123)
    W, xb, lg, ef, sh, k = _host_layer_case(m, shape, 1, seed=5)
    _check_fused(m, W, xb, lg, k, ef, sh, f"fused one token H={H} I={I} E={E} k={k}")


def test_fused_tie_heavy_routing(m):
    W, xb, _, ef, sh, k = _host_layer_case(m, synth.TINY, 4)
    rng = np.random.default_rng(7)
    lg = rng.choice(np.float32([-1.0, 0.0, -0.0, 1.0]), size=(4, synth.TINY.E))
    _check_fused(m, W, xb, lg, k, ef, sh, "tiny M=4 tied logits")


@pytest.mark.parametrize("name", ["ling_m1", "ling_m4"])
def test_fused_ling(m, ling_layer, name):
    wl = synth.WORKLOADS[name]
    xb, lg = synth.moe_inputs(wl)
    _check_fused(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E), f"fused {name}")


@pytest.mark.parametrize("M,seed", [(1, 1), (1, 2), (2, 0), (3, 0), (2, 3), (3, 4)])
def test_fused_ling_more_tokens_and_seeds(m, ling_layer, M, seed):
    """The Ling-shaped layer at every window size the verify path takes (M = 2
    and 3 besides the headline 1 and 4) and on further seeds."""
    xb = synth.activations_bf16(seed, 0, M, synth.LING.H)
    lg = synth.logits_f32(seed, 0, M, synth.LING.E)
    _check_fused(m, ling_layer, xb, lg, 8, _ling_expert, _ling_expert(synth.LING.E),
                 f"fused ling M={M} seed {seed}")


# ------------------------------------------------------- residual stack

def _check_rmsnorm_x(x_bits, r, eps, what):
    """x = bf16(RMSNorm(r)): equal to the float64 value rounded to nearest even,
    except where that value lies within 1e-5 (relative) of the midpoint between
    two bf16 neighbours, where either rounding is accepted."""
    xr = oracle.rmsnorm(np.asarray(r, np.float64), eps=eps)
    want = oracle.bf16_bits(oracle.bf16_round(xr))
    got = np.asarray(x_bits, np.uint16)
    bad = got != want
    if bad.any():
        gv = synth.bf16_values(got[bad]).astype(np.float64)
        wv = synth.bf16_values(want[bad]).astype(np.float64)
        mid = (gv + wv) / 2
        ok = np.abs(xr[bad] - mid) <= 1e-5 * np.abs(xr[bad])
        assert ok.all(), f"{what}: {int((~ok).sum())} x values differ from bf16(RMSNorm(r))"


def _residual_stack(m, layers, r0, logits_per_layer, k, expert_fns, shareds, what, eps=1e-6):
    M, H = r0.shape
    W0 = layers[0]
    ws = m.make_ffn_workspace(M, k, W0.H, W0.I, "cuda")
    r = torch.from_numpy(r0).cuda()
    for L, W in enumerate(layers):
        say(f"{what} layer {L}")
        lg = torch.from_numpy(logits_per_layer[L]).cuda()
        x_out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        y32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
        r_out = m.moe_layer_rmsnorm(W, r, lg, k, ws, eps=eps, x_out=x_out, y_f32=y32)
        torch.cuda.synchronize()
        assert m.check_ffn_workspace(ws) == 0
        r_in_h, r_out_h, y_h = r.cpu().numpy(), r_out.cpu().numpy(), y32.cpu().numpy()
        xb = bits_of(x_out)
        _check_rmsnorm_x(xb, r_in_h, eps, f"{what} layer {L}")
        # the same kernel on the same x without the residual: bit-identical y
        _, y32_plain = m.moe_layer(W, x_out, lg, k, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y_h, y32_plain.cpu().numpy())
        _, _, ref_y = oracle_layer(xb, logits_per_layer[L], k, expert_fns[L], shareds[L])
        check_acc(y_h, ref_y, f"{what} layer {L}")
        np.testing.assert_array_equal(r_out_h, r_in_h + y_h)        # float32 sum, exact
        r = r_out


@pytest.mark.parametrize("M,scale,eps", [(1, 3.0, 1e-6), (3, 3.0, 1e-6), (1, 1e-3, 1e-6), (3, 1e-3, 2e-6),
                                         (2, 1.0, 0.5)])
def test_residual_stack_tiny(m, M, scale, eps):
    """Three layers with their own weights and logits: every layer's x is
    bf16(RMSNorm(r)), its y matches the oracle on that x, and r advances by y.
    With r of about 1e-3 (mean square about 1e-6) or eps = 0.5 the epsilon
    moves x far beyond the tolerance, so its place in the norm is checked."""
    shape = synth.TINY
    layers, efs, shs, lgs = [], [], [], []
    for L in range(3):
        W, _, _, ef, sh, k = _host_layer_case(m, shape, M, seed=5, layer=L,
                                              logits=synth.logits_f32(5, L, M, shape.E))
        layers.append(W)
        efs.append(ef)
        shs.append(sh)
        lgs.append(synth.logits_f32(5, L, M, shape.E))
    r0 = (np.random.default_rng(7).standard_normal((M, shape.H)) * scale).astype(np.float32)
    _residual_stack(m, layers, r0, lgs, k, efs, shs, f"residual tiny M={M} scale={scale} eps={eps}", eps=eps)


def test_residual_layer_ling_m1(m, ling_layer):
    wl = synth.WORKLOADS["ling_m1"]
    _, lg = synth.moe_inputs(wl)
    r0 = np.random.default_rng(8).standard_normal((1, synth.LING.H)).astype(np.float32)
    _residual_stack(m, [ling_layer], r0, [lg], 8, [_ling_expert], [_ling_expert(synth.LING.E)],
                    "residual ling M=1")


def _router_chain_stack(m, layers, routers, r0, k, expert_fns, shareds, what, eps=1e-6):
    """Layers routed from their own data (moe_layer_rmsnorm_router): per
    layer, x = bf16(RMSNorm(r)); the router logits equal the router GEMV on
    that exported x bit for bit (so the router and the layer used one x) and
    the float64 oracle's within the float32 tolerance; the experts chosen are
    a valid top-k of the oracle logits under the near-tie rule; y equals the
    layer on (x, logits) bit for bit and the oracle within tolerance; r
    advances by exactly y."""
    M, H = r0.shape
    W0 = layers[0]
    ws = m.make_ffn_workspace(M, k, W0.H, W0.I, "cuda")
    r = torch.from_numpy(r0).cuda()
    for L, (W, wr_bits) in enumerate(zip(layers, routers)):
        say(f"{what} layer {L}")
        wr = bf16_tensor(wr_bits)
        x_out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        y32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
        r_out, lg = m.moe_layer_rmsnorm_router(W, wr, r, k, ws, eps=eps, x_out=x_out, y_f32=y32)
        lg_plain = m.router_logits(wr, x_out)
        ids, w, _ = m.route_topk(lg, k)
        _, y32_plain = m.moe_layer(W, x_out, lg, k, ws)
        torch.cuda.synchronize()
        assert m.check_ffn_workspace(ws) == 0
        r_in_h, r_out_h, y_h, lg_h = r.cpu().numpy(), r_out.cpu().numpy(), y32.cpu().numpy(), lg.cpu().numpy()
        xb = bits_of(x_out)
        _check_rmsnorm_x(xb, r_in_h, eps, f"{what} layer {L}")
        np.testing.assert_array_equal(lg_h.view(np.uint32), lg_plain.cpu().numpy().view(np.uint32))
        ref_lg = oracle.router_logits(synth.bf16_values(wr_bits), synth.bf16_values(xb))
        check_acc(lg_h, ref_lg, f"{what} layer {L} router logits")
        _check_route_from_router(ids.cpu().numpy(), w.cpu().numpy(), ref_lg, k, f"{what} layer {L}")
        np.testing.assert_array_equal(y_h, y32_plain.cpu().numpy())
        _, _, ref_y = oracle_layer(xb, lg_h, k, expert_fns[L], shareds[L])
        check_acc(y_h, ref_y, f"{what} layer {L}")
        np.testing.assert_array_equal(r_out_h, r_in_h + y_h)
        r = r_out


@pytest.mark.parametrize("M,scale,eps", [(1, 3.0, 1e-6), (4, 3.0, 1e-6), (3, 1e-3, 2e-6), (2, 1.0, 0.5)])
def test_router_chain_stack_tiny(m, M, scale, eps):
    """Three tiny layers, each with its own router, routed from the residual
    stream alone."""
    shape = synth.TINY
    layers, efs, shs, wrs = [], [], [], []
    for L in range(3):
        W, _, _, ef, sh, k = _host_layer_case(m, shape, M, seed=6, layer=L,
                                              logits=synth.logits_f32(6, L, M, shape.E))
        layers.append(W)
        efs.append(ef)
        shs.append(sh)
        wrs.append(synth.router_weight_bf16(6, L, shape.E, shape.H))
    r0 = (np.random.default_rng(9).standard_normal((M, shape.H)) * scale).astype(np.float32)
    _router_chain_stack(m, layers, wrs, r0, k, efs, shs, f"router chain tiny M={M} scale={scale}", eps=eps)


@pytest.mark.parametrize("M", [1, 4])
def test_router_chain_ling(m, ling_layer, M):
    """The Ling-shaped layer (512 experts, top-8, H = 2560) behind a 512 x 2560
    router, two steps on the residual stream."""
    wrs = [synth.router_weight_bf16(1, L, synth.LING.E, synth.LING.H) for L in range(2)]
    r0 = np.random.default_rng(10 + M).standard_normal((M, synth.LING.H)).astype(np.float32)
    ef = [_ling_expert] * 2
    sh = [_ling_expert(synth.LING.E)] * 2
    _router_chain_stack(m, [ling_layer, ling_layer], wrs, r0, 8, ef, sh, f"router chain ling M={M}")


def test_paths_share_one_workspace(m):
    """The fused and two-call paths alternate on one workspace with different
    M; every call still matches the oracle (launch generations stay in step)."""
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, 4)
    ws = m.make_ffn_workspace(4, k, W.H, W.I, "cuda")
    for M, fused in ((4, True), (1, False), (2, True), (4, False), (3, True)):
        say("shared workspace", M, fused)
        xs, ls = xb[:M].copy(), lg[:M].copy()
        if fused:
            _, _, _, yb, y32 = _run_fused(m, W, xs, ls, k, ws)
        else:
            _, yb, y32, _ = _run_ffn(m, W, xs, ls, k, ws)
        _, _, ref_y = oracle_layer(xs, ls, k, ef, sh)
        check_acc(y32, ref_y, f"shared ws M={M} fused={fused}")


def test_workspace_status_stays_clear(m):
    """No wait in any call gave up: moe_ffn_workspace_status reports a clear
    workspace after fused and two-call runs back to back."""
    W, xb, lg, ef, sh, k = _host_layer_case(m, synth.TINY, 2)
    ws = m.make_ffn_workspace(2, k, W.H, W.I, "cuda")
    for _ in range(3):
        _run_fused(m, W, xb, lg, k, ws)
        _run_ffn(m, W, xb, lg, k, ws)
    flags = np.zeros(1, np.uint32)
    assert m.lib.moe_ffn_workspace_status(m._ptr(ws), ws.numel(), flags.ctypes.data_as(
        __import__("ctypes").POINTER(__import__("ctypes").c_uint32)), m._stream(ws)) == 0
    assert flags[0] == 0


def test_selftest_passes(m):
    """The library's start-up check (closed-form routing, MXFP4 layer and FP8
    head cases) passes on the device, twice on the same scratch."""
    say("selftest")
    m.selftest()
    m.selftest()


@pytest.mark.parametrize("M", [1, 4])
def test_graph_replays_match_eager(m, M):
    """The fused layer captured in a HIP graph (as the benchmark runs it):
    every replay, with eager calls and synchronisations between replays,
    gives the eager result bit for bit (workspace generations advance per
    launch, so replays must not see stale tags)."""
    say(f"graph replays M={M}")
    W, xb, lg, _, _, k = _host_layer_case(m, synth.TINY, M)
    x = bf16_tensor(xb)
    lgt = torch.from_numpy(lg).cuda()
    ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
    y_e, y32_e = m.moe_layer(W, x, lgt, k, ws)
    torch.cuda.synchronize()
    ref_b, ref_f = bits_of(y_e), y32_e.cpu().numpy().view(np.uint32)
    y = torch.empty_like(y_e)
    y32 = torch.empty_like(y32_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):                      # several launches in one graph
            m.moe_layer(W, x, lgt, k, ws, y=y, y_f32=y32)
    for _ in range(4):
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(y), ref_b)
        np.testing.assert_array_equal(y32.cpu().numpy().view(np.uint32), ref_f)
        yb2, _ = m.moe_layer(W, x, lgt, k, ws)  # eager work between replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(yb2), ref_b)
    assert m.check_ffn_workspace(ws) == 0
