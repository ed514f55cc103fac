"""The entry point that allocates nothing (moe_layer_mxfp4_noalloc), through
the C ABI: its results equal moe_layer_mxfp4's with a caller workspace, bit
for bit, on two calls in a row -- a Ling-shaped layer at M = 4, then the same
layer at M = 1 (smaller input, same scratch) -- and on a tiny layer after
them; the scratch's status stays clear."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import bf16_tensor, bits_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_moe_expert_topk_amd as m
    return m


def _both(m, W, xb, lg, k):
    """(ids, weights, y bits, y_f32) from the workspace call and the no-alloc
    call on the same inputs."""
    x = bf16_tensor(xb)
    lgt = torch.from_numpy(lg).cuda()
    M = x.shape[0]
    out = []
    for noalloc in (False, True):
        ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
        wts = torch.zeros((M, k), dtype=torch.float32, device="cuda")
        disp = torch.zeros(m.DISPATCH_BYTES, dtype=torch.uint8, device="cuda")
        y = torch.empty((M, W.H), dtype=torch.bfloat16, device="cuda")
        y32 = torch.empty((M, W.H), dtype=torch.float32, device="cuda")
        if noalloc:
            st = m.lib.moe_layer_mxfp4_noalloc(ctypes.byref(W.desc), m._ptr(x), m._ptr(lgt), M, k, m._ptr(ids),
                                               m._ptr(wts), m._ptr(disp), m._ptr(y), m._ptr(y32), m._stream(x))
            assert st == 0, m.lib.moedec_last_error()
        else:
            ws = m.make_ffn_workspace(M, k, W.H, W.I, "cuda")
            m.moe_layer(W, x, lgt, k, ws, y=y, y_f32=y32, ids=ids, topk_w=wts, dispatch=disp)
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), wts.cpu().numpy(), disp.cpu().numpy(), bits_of(y),
                    y32.cpu().numpy().view(np.uint32)))
        if noalloc:
            assert m.check_ffn_workspace(None) == 0
        else:
            assert m.check_ffn_workspace(ws) == 0
    for a, b in zip(out[0], out[1]):
        np.testing.assert_array_equal(a, b)


def test_noalloc_matches_workspace_call(m):
    import synth.device as sd
    say("no-alloc: Ling layer on device")
    shape = synth.LING
    lay = sd.canonical_layer(0, 0, shape, "cuda")
    W = m.MoELayerWeights.from_canonical(lay["gate"], lay["up"], lay["down"], shape.E)
    torch.cuda.synchronize()
    del lay
    for M in (4, 1):                                   # second call: a smaller input
        say(f"no-alloc Ling M={M}")
        xb = synth.activations_bf16(0, 0, M, shape.H)
        lg = synth.logits_f32(0, 0, M, shape.E)
        _both(m, W, xb, lg, shape.k)
    say("no-alloc tiny M=2")
    t = synth.TINY
    lay = synth.mxfp4_layer(0, 0, t)
    d = {n: tuple(torch.from_numpy(a).cuda() for a in lay[n]) for n in lay}
    Wt = m.MoELayerWeights.from_canonical(d["gate"], d["up"], d["down"], t.E)
    xb = synth.activations_bf16(0, 0, 2, t.H)
    _both(m, Wt, xb, synth.router_logits_f32(0, xb, t.E), t.k)


def test_noalloc_refuses_oversized_shapes(m):
    """A shape whose workspace exceeds the scratch is refused before launch."""
    W = m.MoEWeights(m.MOE_MAGIC, 512, 4096, 2048, *([1 << 20] * 8))
    FAKE = ctypes.c_void_p(1 << 20)
    assert m.lib.moe_layer_mxfp4_noalloc(ctypes.byref(W), FAKE, FAKE, 4, 32, None, None, None, FAKE,
                                         None, None) == -5
