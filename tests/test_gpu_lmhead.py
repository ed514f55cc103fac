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


def _sample_rows(V, n=384, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(8), rng.choice(V, n, replace=False), np.arange(V - 8, V)])
    return np.unique(rows)


def test_full_size_quant_and_gemv(m, full_head):
    """157,184 x 2,560: quantise on the GPU, compare sampled rows bit for bit,
    then the FP8 and bf16 GEMVs at M = 1 and 4 on sampled logits."""
    V, H = synth.LMHEAD_V, synth.LMHEAD_H
    rows = _sample_rows(V)
    say("full quant")
    head = _check_quant(m, full_head, rows)
    codes = head.codes[torch.from_numpy(rows).cuda()].cpu().numpy()
    scale = head.row_scale.cpu().numpy()[rows]
    w_dev = bf16_tensor(full_head)
    for M in (1, 4):
        xb = synth.lmhead_x_bf16(0, M, H)
        x = synth.bf16_values(xb).astype(np.float64)
        got = _check_gemv(m, head, xb, None, f"full fp8 gemv M={M}")[:, rows]
        check_acc(got, oracle.lmhead_gemv_fp8(codes, scale, x), f"full fp8 M={M}")
        gotb = _check_gemv(m, w_dev, xb, None, f"full bf16 gemv M={M}", fp8=False)[:, rows]
        check_acc(gotb, oracle.lmhead_gemv_bf16(synth.bf16_values(full_head[rows]), x), f"full bf16 M={M}")


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


def test_argmax_full_size(m, full_head):
    """157,184 x 2,560 at M = 1 and 4: the epilogue's ids against the argmax of
    the kernel's own logits."""
    head = m.lmhead_quant_fp8(bf16_tensor(full_head))
    for M in (1, 4):
        _check_argmax(m, head, synth.lmhead_x_bf16(5, M, synth.LMHEAD_H), f"full M={M}")


def test_argmax_graph_replays(m):
    """The greedy epilogue captured in a HIP graph: every replay (with eager
    calls between) gives the eager ids."""
    wb = _weights(3000, 256, seed=8)
    head = m.lmhead_quant_fp8(bf16_tensor(wb))
    x = bf16_tensor(synth.lmhead_x_bf16(3, 4, 256))
    ref = m.lmhead_argmax_fp8(head, x).cpu().numpy()
    ws = torch.empty(m.lib.lmhead_argmax_workspace_bytes(3000, 4), dtype=torch.uint8, device="cuda")
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
