"""GPU parity of the LM-head FP8 quantiser and both GEMVs against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import bf16_tensor, check_acc, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


def _weights(V, H, seed=0):
    return synth.lmhead_weight_bf16(seed, V, H)


def _check_quant(m, w_bits, rows=None):
    w = bf16_tensor(w_bits)
    head = m.lmhead_quant_fp8(w)
    torch.cuda.synchronize()
    codes = head.codes.cpu().numpy()
    scale = head.row_scale.cpu().numpy()
    sel = np.arange(w_bits.shape[0]) if rows is None else rows
    ref_c, ref_s = oracle.lmhead_quant_fp8(synth.bf16_values(w_bits[sel]))
    np.testing.assert_array_equal(scale[sel], ref_s)
    np.testing.assert_array_equal(codes[sel], ref_c)
    assert head.desc.magic == m.LMHEAD_MAGIC and head.desc.V == w_bits.shape[0]
    return head


@pytest.mark.parametrize("V,H", [(300, 2560), (77, 256), (129, 4096), (5, 16), (33, 8192)])
def test_quant_small(m, V, H):
    say("quant", V, H)
    wb = _weights(V, H, seed=V)
    wb[0] = 0                                   # all-zero row -> scale 1, codes 0
    wb[1, :] = synth.bf16_bits_from_f32(np.float32([-(2.0 ** -20)] * H))   # tiny negative row
    wb[2, 3] = synth.bf16_bits_from_f32(np.float32([-3.0]))[0]            # negative absmax
    # scale below 2^-90: the kernel divides element by element for this row
    rng = np.random.default_rng(V)
    wb[3] = synth.bf16_bits_from_f32((rng.standard_normal(H) * 2.0 ** -100).astype(np.float32))
    # bf16 subnormals (and -0.0) beside normal values: quotients far below code 0x01
    wb[4, :4] = [0x0001, 0x8003, 0x007F, 0x8000]
    _check_quant(m, wb)


def _check_gemv(m, head_or_w, x_bits, ref, what, fp8=True):
    say(what)
    x = bf16_tensor(x_bits)
    out = m.lmhead_gemv_fp8(head_or_w, x) if fp8 else m.lmhead_gemv_bf16(head_or_w, x)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("V,H", [(300, 2560), (77, 256), (129, 4096), (5, 16)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gemv_small(m, V, H, M):
    wb = _weights(V, H, seed=V + 1)
    head = _check_quant(m, wb)
    xb = synth.lmhead_x_bf16(M, M, H)
    x = synth.bf16_values(xb).astype(np.float64)
    got = _check_gemv(m, head, xb, None, f"gemv fp8 V={V} H={H} M={M}")
    ref = oracle.lmhead_gemv_fp8(head.codes.cpu().numpy(), head.row_scale.cpu().numpy(), x)
    check_acc(got, ref, f"fp8 gemv V={V} H={H} M={M}")
    gotb = _check_gemv(m, bf16_tensor(wb), xb, None, f"gemv bf16 V={V} H={H} M={M}", fp8=False)
    refb = oracle.lmhead_gemv_bf16(synth.bf16_values(wb), x)
    check_acc(gotb, refb, f"bf16 gemv V={V} H={H} M={M}")


@pytest.fixture(scope="module")
def full_head(m):
    say("full-size LM head weights")
    wb = _weights(synth.LMHEAD_V, synth.LMHEAD_H)
    return wb


# activations of the full-size checks: (seed, M)
FULL_X = {"gemv_m1": (0, 1), "gemv_m4": (0, 4), "argmax_m1": (5, 1), "argmax_m4": (5, 4)}


def _oracle_rows(args):
    """Oracle codes, scales and float64 logits (FP8 and bf16) for one row chunk."""
    w_chunk, xs = args
    vals = synth.bf16_values(w_chunk)
    codes, scale = oracle.lmhead_quant_fp8(vals)
    fp8 = oracle.lmhead_gemv_fp8(codes, scale, xs)
    bf = oracle.lmhead_gemv_bf16(vals, xs)
    return codes, scale, fp8, bf


@pytest.fixture(scope="module")
def full_oracle(full_head):
    """The oracle over all 157,184 rows, in row chunks spread over host threads
    (numpy releases the interpreter lock in these loops): codes, row scales,
    and float64 logits of every FULL_X activation for both heads."""
    import concurrent.futures as cf
    import os
    say("full-size oracle (all rows, chunked)")
    H = synth.LMHEAD_H
    xs_bits = {k: synth.lmhead_x_bf16(seed, M, H) for k, (seed, M) in FULL_X.items()}
    xs = np.concatenate([synth.bf16_values(xs_bits[k]).astype(np.float64) for k in FULL_X])
    V = full_head.shape[0]
    step = 8192
    chunks = [(full_head[r:r + step], xs) for r in range(0, V, step)]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(_oracle_rows, chunks))
    codes = np.concatenate([p[0] for p in parts])
    scale = np.concatenate([p[1] for p in parts])
    fp8 = np.concatenate([p[2] for p in parts], axis=1)
    bf = np.concatenate([p[3] for p in parts], axis=1)
    out = {"codes": codes, "scale": scale, "x_bits": xs_bits}
    row = 0
    for k, (_, M) in FULL_X.items():
        out["fp8_" + k] = fp8[row:row + M]
        out["bf16_" + k] = bf[row:row + M]
        row += M
    say("full-size oracle done")
    return out


def test_full_size_quant_and_gemv(m, full_head, full_oracle):
    """157,184 x 2,560: quantise on the GPU and compare every row bit for bit,
    then the FP8 and bf16 GEMVs at M = 1 and 4 on every logit."""
    say("full quant")
    w_dev = bf16_tensor(full_head)
    head = m.lmhead_quant_fp8(w_dev)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(head.row_scale.cpu().numpy(), full_oracle["scale"])
    np.testing.assert_array_equal(head.codes.cpu().numpy(), full_oracle["codes"])
    for key in ("gemv_m1", "gemv_m4"):
        xb = full_oracle["x_bits"][key]
        M = xb.shape[0]
        got = _check_gemv(m, head, xb, None, f"full fp8 gemv M={M}")
        check_acc(got, full_oracle["fp8_" + key], f"full fp8 M={M}")
        gotb = _check_gemv(m, w_dev, xb, None, f"full bf16 gemv M={M}", fp8=False)
        check_acc(gotb, full_oracle["bf16_" + key], f"full bf16 M={M}")


def _check_argmax(m, head, xb, what, ref_logits=None):
    """Greedy ids: equal to the argmax (lowest index on ties) of the kernel's
    own float32 logits, which the epilogue leaves unchanged; with float64
    oracle logits, equal to their argmax unless the top two lie within the
    float32-accumulator tolerance of each other (then either is correct)."""
    say("argmax", what)
    x = bf16_tensor(xb)
    M = x.shape[0]
    lg_plain = m.lmhead_gemv_fp8(head, x)
    lg = torch.empty_like(lg_plain)
    ids = m.lmhead_argmax_fp8(head, x, logits=lg)
    ids_only = m.lmhead_argmax_fp8(head, x)                  # logits not written
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    np.testing.assert_array_equal(lg_np.view(np.uint32), lg_plain.cpu().numpy().view(np.uint32))
    got = ids.cpu().numpy()
    np.testing.assert_array_equal(got, ids_only.cpu().numpy())
    np.testing.assert_array_equal(got, oracle.lmhead_argmax(lg_np), err_msg=what)
    if ref_logits is not None:
        for mm in range(M):
            r = ref_logits[mm]
            tol = 1e-5 * np.max(np.abs(r))
            top2 = np.sort(r)[-2:]
            if top2[1] - top2[0] > 2 * tol:
                assert got[mm] == int(np.argmax(r)), f"{what} token {mm}"
            else:
                assert r[got[mm]] >= top2[1] - 2 * tol, f"{what} token {mm}: not a near-maximum"


@pytest.mark.parametrize("V,H", [(300, 2560), (77, 256), (129, 4096), (5, 16), (4097, 64)])
@pytest.mark.parametrize("M", [1, 4])
def test_argmax_small(m, V, H, M):
    wb = _weights(V, H, seed=V + 2)
    head = _check_quant(m, wb)
    xb = synth.lmhead_x_bf16(M + 7, M, H)
    ref = oracle.lmhead_gemv_fp8(head.codes.cpu().numpy(), head.row_scale.cpu().numpy(),
                                 synth.bf16_values(xb).astype(np.float64))
    _check_argmax(m, head, xb, f"V={V} H={H} M={M}", ref)


def test_argmax_exact_tie_takes_the_lower_row(m):
    """Two identical rows hold the largest logit (identical codes and scales give
    bit-identical sums): the lower row wins, across waves as within one."""
    V, H = 700, 256
    wb = _weights(V, H, seed=3)
    xb = synth.lmhead_x_bf16(9, 2, H)
    sign = np.sign(synth.bf16_values(xb[0])).astype(np.float32)
    big = synth.bf16_bits_from_f32(0.05 * sign)
    for row in (650, 37, 41):                    # rows in different waves (32 rows per wave)
        wb[row] = big
    head = _check_quant(m, wb)
    ids = m.lmhead_argmax_fp8(head, bf16_tensor(xb))
    torch.cuda.synchronize()
    assert int(ids.cpu().numpy()[0]) == 37
    _check_argmax(m, head, xb, "tie rows 37/41/650")


def test_argmax_full_size(m, full_head, full_oracle):
    """157,184 x 2,560 at M = 1 and 4: the epilogue's ids against the argmax of
    the kernel's own logits, and against the float64 oracle logits of all rows
    (near-ties within the float32 tolerance excepted)."""
    head = m.lmhead_quant_fp8(bf16_tensor(full_head))
    for key in ("argmax_m1", "argmax_m4"):
        xb = full_oracle["x_bits"][key]
        _check_argmax(m, head, xb, f"full M={xb.shape[0]}", full_oracle["fp8_" + key])


def test_argmax_graph_replays(m):
    """The greedy epilogue captured in a HIP graph: every replay (with eager
    calls between) gives the eager ids."""
    wb = _weights(3000, 256, seed=8)
    head = m.lmhead_quant_fp8(bf16_tensor(wb))
    x = bf16_tensor(synth.lmhead_x_bf16(3, 4, 256))
    ref = m.lmhead_argmax_fp8(head, x).cpu().numpy()
    ws = m.make_lmhead_workspace(3000, 4, "cuda")
    ids = torch.empty(4, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.lmhead_argmax_fp8(head, x, workspace=ws, ids=ids)
    for _ in range(3):
        ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy(), ref)
        np.testing.assert_array_equal(m.lmhead_argmax_fp8(head, x).cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# Sampling epilogue (lmhead_gemv_fp8_sample)

SETTINGS = [(0.6, 0.95, 29), (1.0, 1.0, 32), (0.6, 0.5, 5), (2.0, 0.9, 17), (0.3, 0.99, 2)]
DELTA = 1e-5      # float32 softmax + scan against float64: decisions this close to a boundary may go either way


def _sample_ok(row, u, T, p, k, tok):
    """The sampled token is the oracle's draw on the same float32 logits, or,
    when u or the nucleus cut lies within DELTA of a boundary of the
    cumulative distribution, the draw at a perturbed u or top_p (the kernel's
    float32 softmax and scan may land on either side).  Returns (ok, exact)."""
    row = np.asarray(row, np.float64)[None, :]
    ref = int(oracle.lmhead_sample(row, [u], T, p, k)[0])
    if tok == ref:
        return True, True
    for du in (-DELTA, 0.0, DELTA):
        for dp in (-DELTA, 0.0, DELTA):
            uu = min(max(u + du, 0.0), np.nextafter(1.0, 0.0))
            pp = min(max(p + dp, 1e-9), 1.0)
            if int(oracle.lmhead_sample(row, [uu], T, pp, k)[0]) == tok:
                return True, False
    return False, False


def _check_sample(m, head, xb, u, T, p, k, what):
    """Kernel ids against the oracle's draw on the kernel's own logits (which
    must equal the plain GEMV's bit for bit); returns the number of draws that
    needed the boundary allowance."""
    x = bf16_tensor(xb)
    M = x.shape[0]
    u_dev = torch.from_numpy(np.asarray(u, np.float32)).cuda()
    ids, lg = m.lmhead_sample_fp8(head, x, u_dev, T, p, k)
    ids_only, none = m.lmhead_sample_fp8(head, x, u_dev, T, p, k, want_logits=False)
    plain = m.lmhead_gemv_fp8(head, x)
    torch.cuda.synchronize()
    assert none is None
    lg_np = lg.cpu().numpy()
    np.testing.assert_array_equal(lg_np.view(np.uint32), plain.cpu().numpy().view(np.uint32))
    got = ids.cpu().numpy()
    np.testing.assert_array_equal(got, ids_only.cpu().numpy())
    loose = 0
    for mm in range(M):
        ok, exact = _sample_ok(lg_np[mm], float(u[mm]), T, p, k, int(got[mm]))
        assert ok, f"{what} token {mm}: kernel {got[mm]}, oracle " \
                   f"{oracle.lmhead_sample(lg_np[mm:mm + 1].astype(np.float64), u[mm:mm + 1], T, p, k)}"
        loose += not exact
    return loose


@pytest.mark.parametrize("V,H", [(300, 2560), (77, 256), (4097, 64), (33, 16), (1100, 128)])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_sample_small(m, V, H, M):
    """Several vocabulary sizes (one wave, a ragged last wave, many blocks)
    and every setting, at uniforms from the counter-based stream."""
    wb = _weights(V, H, seed=V + 11)
    head = _check_quant(m, wb)
    loose = 0
    for i, (T, p, k) in enumerate(SETTINGS):
        k = min(k, V)
        say("sample", V, H, M, T, p, k)
        xb = synth.lmhead_x_bf16(100 + i, M, H)
        loose += _check_sample(m, head, xb, synth.sampling_uniforms(V, i, M), T, p, k,
                               f"V={V} H={H} M={M} T={T} p={p} k={k}")
    assert loose <= 1


def test_sample_tiny_vocabulary_all_candidates(m):
    """V = 5 < top_k bound: the candidates are every row (one wave holds
    them all); a grid of uniforms visits every token with top_p = 1."""
    V, H = 5, 64
    wb = _weights(V, H, seed=41)
    head = _check_quant(m, wb)
    xb = synth.lmhead_x_bf16(41, 4, H)
    seen = set()
    for j in range(32):
        u = (np.arange(4, dtype=np.float32) + 4 * j) / 128.0
        _check_sample(m, head, xb, u, 3.0, 1.0, 5, f"tiny grid {j}")
        ids, _ = m.lmhead_sample_fp8(head, bf16_tensor(xb), torch.from_numpy(u).cuda(), 3.0, 1.0, 5)
        seen.update(int(t) for t in ids.cpu().numpy())
    assert seen == set(range(V))


def test_sample_frequencies_follow_the_nucleus(m):
    """Fixed logits, uniforms on a fine grid: how often each token is drawn
    equals its renormalised nucleus probability times the grid size, up to
    the two grid points at each interval's ends."""
    V, H, M = 2000, 256, 4
    wb = _weights(V, H, seed=12)
    head = _check_quant(m, wb)
    xb = synth.lmhead_x_bf16(12, M, H)
    x = bf16_tensor(xb)
    T, p, k, n = 0.6, 0.95, 29, 512
    counts = [dict() for _ in range(M)]
    lg_np = None
    for j in range(n):
        u = np.full(M, (j + 0.5) / n, np.float32)
        ids, lg = m.lmhead_sample_fp8(head, x, torch.from_numpy(u).cuda(), T, p, k)
        for mm, t in enumerate(ids.cpu().numpy()):
            counts[mm][int(t)] = counts[mm].get(int(t), 0) + 1
        lg_np = lg.cpu().numpy()
    for mm in range(M):
        row = lg_np[mm].astype(np.float64)
        order = np.lexsort((np.arange(V), -row))[:k]
        z = row[order] / T
        pr = np.exp(z - z[0])
        pr /= pr.sum()
        cum = np.cumsum(pr)
        n_keep = min(int(np.searchsorted(cum, p, side="left")) + 1, k)
        q = pr[:n_keep] / cum[n_keep - 1]
        for i in range(n_keep):
            assert abs(counts[mm].get(int(order[i]), 0) - q[i] * n) <= 2, f"token {mm} cand {i}"
        assert sum(counts[mm].values()) == n
        assert set(counts[mm]) <= set(int(t) for t in order[:n_keep])


def test_sample_candidates_clustered_and_tied(m):
    """The top logits packed into one wave's rows (stage A must keep that
    wave), and an exact tie straddling the top_k cut (identical rows: the
    lower row is a candidate, the higher one is not)."""
    V, H = 3000, 256
    wb = _weights(V, H, seed=21)
    xb = synth.lmhead_x_bf16(21, 2, H)
    sign = np.sign(synth.bf16_values(xb[0])).astype(np.float32)
    for i, row in enumerate(range(640, 671)):            # 31 of one wave's 32 rows, graded
        wb[row] = synth.bf16_bits_from_f32((0.02 + 0.0005 * i) * sign)
    tie = synth.bf16_bits_from_f32(0.0195 * sign)
    wb[2999] = tie                                        # ties with row 5 for the last place
    wb[5] = tie
    head = _check_quant(m, wb)
    x = bf16_tensor(xb)
    lg = m.lmhead_gemv_fp8(head, x).cpu().numpy()
    assert lg[0, 5] == lg[0, 2999]
    top = np.lexsort((np.arange(V), -lg[0].astype(np.float64)))[:33]
    assert set(range(640, 671)) == set(top[:31])
    k = 32                                                # row 5 is the last candidate, row 2999 the first one cut
    assert top[31] == 5 and top[32] == 2999
    hits = set()
    for j in range(64):
        u = np.float32([(j + 0.5) / 64, 0.999])
        _check_sample(m, head, xb, u, 50.0, 1.0, k, f"cluster/tie grid {j}")
        ids, _ = m.lmhead_sample_fp8(head, x, torch.from_numpy(u).cuda(), 50.0, 1.0, k)
        hits.add(int(ids.cpu().numpy()[0]))
    assert 5 in hits and 2999 not in hits and hits <= set(int(t) for t in top[:k])


def test_sample_greedy_limits(m):
    """top_k = 1, and a vanishing temperature, give the greedy token."""
    V, H, M = 5000, 512, 4
    wb = _weights(V, H, seed=31)
    head = _check_quant(m, wb)
    x = bf16_tensor(synth.lmhead_x_bf16(31, M, H))
    greedy = m.lmhead_argmax_fp8(head, x).cpu().numpy()
    u = torch.from_numpy(synth.sampling_uniforms(31, 0, M)).cuda()
    for T, p, k in ((0.6, 0.95, 1), (1e-6, 0.95, 29), (1.0, 1e-6, 32)):
        ids, _ = m.lmhead_sample_fp8(head, x, u, T, p, k)
        np.testing.assert_array_equal(ids.cpu().numpy(), greedy, err_msg=f"T={T} p={p} k={k}")


def test_sample_full_size(m, full_head):
    """157,184 x 2,560 at M = 1 and 4 with the pages' settings: several decode
    steps of uniforms, each draw against the oracle on the kernel's logits."""
    head = m.lmhead_quant_fp8(bf16_tensor(full_head))
    loose = 0
    for M in (1, 4):
        for step in range(4):
            xb = synth.lmhead_x_bf16(50 + step, M, synth.LMHEAD_H)
            say("full sample", M, step)
            loose += _check_sample(m, head, xb, synth.sampling_uniforms(0, step, M), 0.6, 0.95, 29,
                                   f"full M={M} step={step}")
    assert loose <= 1


def test_sample_graph_replays_and_shared_workspace(m):
    """Sampling captured in a HIP graph: new uniforms written into the
    captured tensor before each replay give the eager draw; greedy and
    sampling calls share one workspace in between."""
    V, H, M = 3000, 256, 4
    wb = _weights(V, H, seed=9)
    head = m.lmhead_quant_fp8(bf16_tensor(wb))
    x = bf16_tensor(synth.lmhead_x_bf16(4, M, H))
    ws = m.make_lmhead_workspace(V, M, "cuda")
    u = torch.zeros(M, dtype=torch.float32, device="cuda")
    ids = torch.empty(M, dtype=torch.int32, device="cuda")
    lg = torch.empty((M, V), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.lmhead_sample_fp8(head, x, u, 0.6, 0.95, 29, workspace=ws, ids=ids, logits=lg)
    for step in range(4):
        u.copy_(torch.from_numpy(synth.sampling_uniforms(9, step, M)))
        ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        ref, _ = m.lmhead_sample_fp8(head, x, u.clone(), 0.6, 0.95, 29)
        np.testing.assert_array_equal(ids.cpu().numpy(), ref.cpu().numpy())
        greedy = m.lmhead_argmax_fp8(head, x, workspace=ws).cpu().numpy()
        np.testing.assert_array_equal(greedy, m.lmhead_argmax_fp8(head, x).cpu().numpy())


# ---------------------------------------------------------------- dynamic FP8 activations

def _dynact_ref(head, x_bits):
    return oracle.lmhead_gemv_fp8_dynact(head.codes.cpu().numpy(), head.row_scale.cpu().numpy(),
                                         synth.bf16_values(x_bits))


@pytest.mark.parametrize("V,H", [(300, 2560), (77, 256), (129, 4096), (5, 16)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_dynact_gemv_small(m, V, H, M):
    """Per-token FP8 activations (the weights' rule per token row) against
    the oracle: an all-zero token (scale 1), a token of tiny values (scale far
    below 2^-90: the division path), a token whose absmax is negative."""
    wb = _weights(V, H, seed=V + 21)
    head = m.lmhead_dynamic_act(_check_quant(m, wb))
    assert head.desc.format == m.FMT_E4M3FN_ROWSCALE_F32_DYNACT
    xb = synth.lmhead_x_bf16(M + 40, M, H)
    if M >= 2:
        xb[1] = 0
    if M >= 3:
        rng = np.random.default_rng(V)
        xb[2] = synth.bf16_bits_from_f32((rng.standard_normal(H) * 2.0 ** -110).astype(np.float32))
    if M >= 4:
        xb[3, 7] = synth.bf16_bits_from_f32(np.float32([-50.0]))[0]
    got = _check_gemv(m, head, xb, None, f"dynact gemv V={V} H={H} M={M}")
    check_acc(got, _dynact_ref(head, xb), f"dynact gemv V={V} H={H} M={M}")
    if M >= 2:
        assert (got[1] == 0).all()


def test_dynact_full_size(m, full_head, full_oracle):
    """157,184 x 2,560 with dynamic activations at M = 1 and 4 (every logit),
    the greedy token and a sampled token from the same head."""
    say("full dynact head")
    head = m.lmhead_dynamic_act(m.lmhead_quant_fp8(bf16_tensor(full_head)))
    torch.cuda.synchronize()
    for key in ("gemv_m1", "gemv_m4"):
        xb = full_oracle["x_bits"][key]
        M = xb.shape[0]
        ref = oracle.lmhead_gemv_fp8_dynact(full_oracle["codes"], full_oracle["scale"], synth.bf16_values(xb))
        got = _check_gemv(m, head, xb, None, f"full dynact gemv M={M}")
        check_acc(got, ref, f"full dynact M={M}")
        _check_argmax(m, head, xb, f"full dynact argmax M={M}", ref_logits=ref)
    xb = full_oracle["x_bits"]["gemv_m4"]
    loose = _check_sample(m, head, xb, synth.sampling_uniforms(synth.LMHEAD_V, 7, 4), 0.6, 0.95, 29,
                          "full dynact sample")
    assert loose <= 1


@pytest.mark.parametrize("M", [1, 4])
def test_dynact_argmax_and_sample_small(m, M):
    V, H = 4097, 64
    head = m.lmhead_dynamic_act(_check_quant(m, _weights(V, H, seed=91)))
    xb = synth.lmhead_x_bf16(92, M, H)
    _check_argmax(m, head, xb, f"dynact argmax M={M}", ref_logits=_dynact_ref(head, xb))
    loose = 0
    for i, (T, p, k) in enumerate(SETTINGS):
        loose += _check_sample(m, head, synth.lmhead_x_bf16(93 + i, M, H), synth.sampling_uniforms(V, 50 + i, M),
                               T, p, min(k, V), f"dynact sample M={M} T={T} p={p} k={k}")
    assert loose <= 1
