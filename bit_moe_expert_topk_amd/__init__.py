"""libmoedec Python binding: batch-1 MoE decode (top-k routing, MXFP4 routed +
shared SwiGLU experts, M = 1..4 tokens) and an online-FP8 LM head on gfx950.

Thin torch-tensor wrappers over the C ABI in include/moedec.h: they check
dtypes/devices, allocate outputs with torch when none are given, and pass raw
pointers plus torch's current HIP stream.  All computation happens in the
library's HIP kernels; there is no CPU fallback.
"""

import ctypes

import torch

from . import _lib
from ._lib import (Dispatch, LMHeadFP8Desc, MoEWeights, MXFP4Sizes, MAX_E, MAX_K, MAX_M,
                   MAX_SLOTS, MOE_MAGIC, MOE_MAGIC_SHARED_FP8, LMHEAD_MAGIC, FMT_E4M3FN_ROWSCALE_F32,
                   FMT_E4M3FN_ROWSCALE_F32_DYNACT)

lib = _lib.lib
LIB_PATH = _lib.LIB_PATH
DISPATCH_BYTES = ctypes.sizeof(Dispatch)


class MoedecError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libmoedec status {status}: {message}")
        self.status = status


def _check(status):
    if status != 0:
        msg = lib.moedec_status_string(status).decode()
        detail = lib.moedec_last_error().decode()
        raise MoedecError(status, f"{msg}: {detail}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


# --------------------------------------------------------------------------
# Routing

def route_topk(logits, k, ids=None, weights=None, dispatch=None):
    """Top-k routing of [M][E] float32 logits -> (ids [M][k] int32,
    weights [M][k] float32, dispatch uint8[DISPATCH_BYTES])."""
    _need(logits, torch.float32, "logits", 2)
    m_tokens, n_exp = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty((m_tokens, k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((m_tokens, k), dtype=torch.float32, device=dev)
    if dispatch is None:
        dispatch = torch.empty(DISPATCH_BYTES, dtype=torch.uint8, device=dev)
    _check(lib.moe_route_topk(_ptr(logits), m_tokens, n_exp, k, _ptr(ids), _ptr(weights),
                              _ptr(dispatch), _stream(logits)))
    return ids, weights, dispatch


def decode_dispatch(dispatch):
    """Host copy of a device dispatch table as a dict of python/numpy values."""
    import numpy as np
    raw = bytes(dispatch.detach().cpu().numpy().tobytes())
    d = Dispatch.from_buffer_copy(raw)
    n = d.n_slots
    return {
        "n_slots": n,
        "M": d.M,
        "expert": np.array(d.expert[:n], dtype=np.int32),
        "token_mask": np.array(d.token_mask[:n], dtype=np.uint32),
        "weight": np.array([list(d.weight[i]) for i in range(n)], dtype=np.float32),
        "raw": d,
    }


# --------------------------------------------------------------------------
# MXFP4 experts

def packed_sizes(H, I):
    out = MXFP4Sizes()
    _check(lib.moedec_mxfp4_packed_sizes(H, I, ctypes.byref(out)))
    return out


def pack_gateup(gate_codes, gate_scales, up_codes, up_scales, out_codes=None, out_scales=None):
    """Pack canonical gate/up MXFP4 matrices [n][I][H/2], [n][I][H/32]."""
    for t, n in ((gate_codes, "gate_codes"), (gate_scales, "gate_scales"),
                 (up_codes, "up_codes"), (up_scales, "up_scales")):
        _need(t, torch.uint8, n, 3)
    n_exp, I, half_h = gate_codes.shape
    H = 2 * half_h
    sz = packed_sizes(H, I)
    if out_codes is None:
        out_codes = torch.empty(n_exp * sz.gu_codes, dtype=torch.uint8, device=gate_codes.device)
    if out_scales is None:
        out_scales = torch.empty(n_exp * sz.gu_scales, dtype=torch.uint8, device=gate_codes.device)
    _check(lib.moe_pack_gateup_mxfp4(_ptr(gate_codes), _ptr(gate_scales), _ptr(up_codes),
                                     _ptr(up_scales), n_exp, H, I, _ptr(out_codes),
                                     _ptr(out_scales), _stream(gate_codes)))
    return out_codes, out_scales


def pack_down(down_codes, down_scales, out_codes=None, out_scales=None):
    """Pack canonical down MXFP4 matrices [n][H][I/2], [n][H][I/32]."""
    _need(down_codes, torch.uint8, "down_codes", 3)
    _need(down_scales, torch.uint8, "down_scales", 3)
    n_exp, H, half_i = down_codes.shape
    I = 2 * half_i
    sz = packed_sizes(H, I)
    if out_codes is None:
        out_codes = torch.empty(n_exp * sz.dn_codes, dtype=torch.uint8, device=down_codes.device)
    if out_scales is None:
        out_scales = torch.empty(n_exp * sz.dn_scales, dtype=torch.uint8, device=down_codes.device)
    _check(lib.moe_pack_down_mxfp4(_ptr(down_codes), _ptr(down_scales), n_exp, H, I,
                                   _ptr(out_codes), _ptr(out_scales), _stream(down_codes)))
    return out_codes, out_scales


class MoELayerWeights:
    """Packed weights of one MoE layer: E routed MXFP4 experts + 1 shared.

    The four packed arrays hold E+1 consecutive MXFP4 experts; the last one is
    the shared expert -- unless shared_fp8 (the four tensors of
    pack_shared_fp8) is given, which then is the shared expert (the arrays
    need only E experts).  Tensors are kept alive by this object.
    """

    def __init__(self, E, H, I, gu_codes, gu_scales, dn_codes, dn_scales, shared_fp8=None):
        self.E, self.H, self.I = E, H, I
        self.sizes = packed_sizes(H, I)
        sz = self.sizes
        n_mx = E if shared_fp8 is not None else E + 1
        for t, per in ((gu_codes, sz.gu_codes), (gu_scales, sz.gu_scales),
                       (dn_codes, sz.dn_codes), (dn_scales, sz.dn_scales)):
            _need(t, torch.uint8, "packed weights")
            if t.numel() < n_mx * per:
                raise ValueError(f"packed array has {t.numel()} bytes, need {n_mx * per}")
        self.gu_codes, self.gu_scales = gu_codes, gu_scales
        self.dn_codes, self.dn_scales = dn_codes, dn_scales
        self.shared_fp8 = shared_fp8
        base = lambda t: t.data_ptr()
        if shared_fp8 is None:
            magic = MOE_MAGIC
            shared = (base(gu_codes) + E * sz.gu_codes, base(gu_scales) + E * sz.gu_scales,
                      base(dn_codes) + E * sz.dn_codes, base(dn_scales) + E * sz.dn_scales)
        else:
            s8 = shared_fp8_sizes(H, I)
            sgc, sgs, sdc, sds = shared_fp8
            for t, dt, n in ((sgc, torch.uint8, s8.gu_codes), (sgs, torch.float32, s8.gu_scales // 4),
                             (sdc, torch.uint8, s8.dn_codes), (sds, torch.float32, s8.dn_scales // 4)):
                _need(t, dt, "FP8 shared expert")
                if t.numel() != n:
                    raise ValueError(f"FP8 shared expert array has {t.numel()} elements, need {n}")
            magic = MOE_MAGIC_SHARED_FP8
            shared = (base(sgc), base(sgs), base(sdc), base(sds))
        self.desc = MoEWeights(magic, E, H, I, base(gu_codes), base(gu_scales), base(dn_codes),
                               base(dn_scales), *shared)

    @classmethod
    def from_canonical(cls, gate, up, down, E):
        """gate/up/down: (codes, scales) uint8 device tensors with E+1 experts
        stacked on dim 0 (index E = shared expert)."""
        gu_c, gu_s = pack_gateup(gate[0], gate[1], up[0], up[1])
        dn_c, dn_s = pack_down(down[0], down[1])
        H = 2 * gate[0].shape[2]
        I = gate[0].shape[1]
        return cls(E, H, I, gu_c, gu_s, dn_c, dn_s)


def shared_fp8_sizes(H, I):
    out = MXFP4Sizes()
    _check(lib.moedec_shared_fp8_packed_sizes(H, I, ctypes.byref(out)))
    return out


def pack_shared_fp8(gate, up, down):
    """Quantise a shared expert's bf16 W_gate, W_up [I][H] and W_down [H][I] to
    E4M3 with a float32 scale per row, in the FP8 streaming layout: returns
    (gu_codes uint8, gu_scales float32 [2I], dn_codes uint8, dn_scales float32 [H])."""
    for t, n in ((gate, "gate"), (up, "up"), (down, "down")):
        _need(t, torch.bfloat16, n, 2)
    I, H = gate.shape
    if tuple(up.shape) != (I, H) or tuple(down.shape) != (H, I):
        raise ValueError("gate, up must be [I][H] and down [H][I]")
    sz = shared_fp8_sizes(H, I)
    dev = gate.device
    gu_c = torch.empty(sz.gu_codes, dtype=torch.uint8, device=dev)
    gu_s = torch.empty(2 * I, dtype=torch.float32, device=dev)
    dn_c = torch.empty(sz.dn_codes, dtype=torch.uint8, device=dev)
    dn_s = torch.empty(H, dtype=torch.float32, device=dev)
    _check(lib.moe_pack_shared_fp8(_ptr(gate), _ptr(up), _ptr(down), H, I, _ptr(gu_c), _ptr(gu_s), _ptr(dn_c),
                                   _ptr(dn_s), _stream(gate)))
    return gu_c, gu_s, dn_c, dn_s


def ffn_workspace_bytes(M, k_max, H, I):
    return lib.moe_ffn_workspace_bytes(M, k_max, H, I)


def make_ffn_workspace(M, k_max, H, I, device):
    """Zero-filled workspace for expert_ffn (zero fill is required once)."""
    n = ffn_workspace_bytes(M, k_max, H, I)
    if n == 0:
        raise ValueError("unsupported workspace shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def expert_ffn(weights, x, dispatch, k_max, workspace, y=None, y_f32=None, want_f32=True):
    """Routed + shared expert FFN.  x: [M][H] bfloat16.  Returns (y bf16, y_f32 or None)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(dispatch, torch.uint8, "dispatch", 1)
    _need(workspace, torch.uint8, "workspace", 1)
    m_tokens, hidden = x.shape
    if y is None:
        y = torch.empty((m_tokens, hidden), dtype=torch.bfloat16, device=x.device)
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((m_tokens, hidden), dtype=torch.float32, device=x.device)
    _check(lib.moe_expert_ffn_mxfp4(ctypes.byref(weights.desc), _ptr(x), m_tokens, _ptr(dispatch),
                                    k_max, _ptr(y), _ptr(y_f32), _ptr(workspace),
                                    workspace.numel(), _stream(x)))
    return y, y_f32


def moe_layer(weights, x, logits, k, workspace, y=None, y_f32=None, want_f32=True,
              ids=None, topk_w=None, dispatch=None, act8=False):
    """Routing and expert FFN in one launch.  x: [M][H] bfloat16, logits [M][E]
    float32.  Returns (y bf16, y_f32 or None); ids / topk_w / dispatch are
    filled when given (device tensors as route_topk returns them).  act8 =
    True runs the W4A8 variant (moe_layer_mxfp4_a8: MXFP8 x and h)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(logits, torch.float32, "logits", 2)
    _need(workspace, torch.uint8, "workspace", 1)
    m_tokens, hidden = x.shape
    if logits.shape[0] != m_tokens or logits.shape[1] != weights.E:
        raise ValueError(f"logits must be [{m_tokens}][{weights.E}], got {tuple(logits.shape)}")
    for t, dt, n in ((ids, torch.int32, "ids"), (topk_w, torch.float32, "topk_w"),
                     (dispatch, torch.uint8, "dispatch")):
        if t is not None:
            _need(t, dt, n)
    if y is None:
        y = torch.empty((m_tokens, hidden), dtype=torch.bfloat16, device=x.device)
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((m_tokens, hidden), dtype=torch.float32, device=x.device)
    fn = lib.moe_layer_mxfp4_a8 if act8 else lib.moe_layer_mxfp4
    _check(fn(ctypes.byref(weights.desc), _ptr(x), _ptr(logits), m_tokens, k, _ptr(ids), _ptr(topk_w),
              _ptr(dispatch), _ptr(y), _ptr(y_f32), _ptr(workspace), workspace.numel(), _stream(x)))
    return y, y_f32


def prefill_workspace_bytes(T, E, k, H, I):
    n = lib.moe_prefill_workspace_bytes(T, E, k, H, I)
    if n == 0:
        raise ValueError(f"no many-token workspace for T={T} E={E} k={k} H={H} I={I}")
    return n


def make_prefill_workspace(T, E, k, H, I, device):
    """Workspace of moe_layer_prefill (no initial contents needed)."""
    return torch.empty(prefill_workspace_bytes(T, E, k, H, I), dtype=torch.uint8, device=device)


def ffn_workspace_h(workspace, M, k, H, I):
    """float32 h [M * k + 1][M][I] (slot-major, the call's dispatch order)
    that the last FFN / fused-layer call left in `workspace`
    (moe_ffn_workspace_layout); valid for each slot's own tokens."""
    out = _lib.FfnLayout()
    _check(lib.moe_ffn_workspace_layout(M, k, H, I, ctypes.byref(out)))
    n = out.max_slots * M * I
    words = workspace[out.h_words:out.h_words + 8 * n].view(torch.int32).reshape(n, 2)[:, 0]
    return words.view(torch.float32).reshape(out.max_slots, M, I)


def prefill_workspace_layout(T, E, k, H, I):
    """Byte offsets of the many-token intermediates in the workspace
    (moe_prefill_workspace_layout), as a dict."""
    out = _lib.PrefillLayout()
    _check(lib.moe_prefill_workspace_layout(T, E, k, H, I, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in _lib.PrefillLayout._fields_}


def moe_layer_prefill(weights, x, logits, k, workspace=None, y=None, y_f32=None, want_f32=True,
                      ids=None, topk_w=None, counts=None, act8=False):
    """The layer for many tokens (moe_layer_mxfp4_prefill): x [T][H] bfloat16,
    logits [T][E] float32.  Returns (y bf16, y_f32 or None); ids [T][k],
    topk_w [T][k] and counts [E + 1] (int32, tokens per expert, then T) are
    filled when given.  act8 = True runs the W4A8 variant
    (moe_layer_mxfp4_prefill_a8: MXFP8 activations into both products)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(logits, torch.float32, "logits", 2)
    t_tokens, hidden = x.shape
    if logits.shape[0] != t_tokens or logits.shape[1] != weights.E:
        raise ValueError(f"logits must be [{t_tokens}][{weights.E}], got {tuple(logits.shape)}")
    for t, dt, n in ((ids, torch.int32, "ids"), (topk_w, torch.float32, "topk_w"),
                     (counts, torch.int32, "counts")):
        if t is not None:
            _need(t, dt, n)
    if workspace is None:
        workspace = make_prefill_workspace(t_tokens, weights.E, k, weights.H, weights.I, x.device)
    _need(workspace, torch.uint8, "workspace", 1)
    if y is None:
        y = torch.empty((t_tokens, hidden), dtype=torch.bfloat16, device=x.device)
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((t_tokens, hidden), dtype=torch.float32, device=x.device)
    fn = lib.moe_layer_mxfp4_prefill_a8 if act8 else lib.moe_layer_mxfp4_prefill
    _check(fn(ctypes.byref(weights.desc), _ptr(x), _ptr(logits), t_tokens, k, _ptr(ids), _ptr(topk_w),
              _ptr(counts), _ptr(y), _ptr(y_f32), _ptr(workspace), workspace.numel(), _stream(x)))
    return y, y_f32


def check_ffn_workspace(workspace=None, device=None):
    """Wait for the stream and raise MoedecError (MOEDEC_ERR_TIMEOUT) when a
    cross-block wait of any FFN call on `workspace` gave up since the last
    check (those results are invalid; the library has cleared the workspace).
    workspace=None checks the no-alloc scratch of `device` (default: current)."""
    flags = ctypes.c_uint32(0)
    if workspace is None:
        dev = torch.device("cuda") if device is None else torch.device(device)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        _check(lib.moe_ffn_workspace_status(None, 0, ctypes.byref(flags), stream))
    else:
        _need(workspace, torch.uint8, "workspace", 1)
        _check(lib.moe_ffn_workspace_status(_ptr(workspace), workspace.numel(), ctypes.byref(flags),
                                            _stream(workspace)))
    return int(flags.value)


def moe_layer_noalloc(weights, x, logits, k, y=None, y_f32=None, want_f32=True, ids=None, topk_w=None,
                      dispatch=None):
    """moe_layer without a workspace argument (moe_layer_mxfp4_noalloc): the
    library's per-device scratch array serves as the workspace."""
    _need(x, torch.bfloat16, "x", 2)
    _need(logits, torch.float32, "logits", 2)
    m_tokens, hidden = x.shape
    if logits.shape[0] != m_tokens or logits.shape[1] != weights.E:
        raise ValueError(f"logits must be [{m_tokens}][{weights.E}], got {tuple(logits.shape)}")
    for t, dt, n in ((ids, torch.int32, "ids"), (topk_w, torch.float32, "topk_w"),
                     (dispatch, torch.uint8, "dispatch")):
        if t is not None:
            _need(t, dt, n)
    if y is None:
        y = torch.empty((m_tokens, hidden), dtype=torch.bfloat16, device=x.device)
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((m_tokens, hidden), dtype=torch.float32, device=x.device)
    _check(lib.moe_layer_mxfp4_noalloc(ctypes.byref(weights.desc), _ptr(x), _ptr(logits), m_tokens, k,
                                       _ptr(ids), _ptr(topk_w), _ptr(dispatch), _ptr(y), _ptr(y_f32),
                                       _stream(x)))
    return y, y_f32


def moe_layer_rmsnorm(weights, r_in, logits, k, workspace, r_out=None, eps=1e-6, x_out=None,
                      y_f32=None):
    """One layer on the residual stream, in one launch: x = bf16(RMSNorm(r_in)),
    y = MoE layer(x), r_out = r_in + y.  r_in: [M][H] float32 (not modified),
    logits [M][E] float32.  Returns r_out; x_out (bf16) and y_f32 are filled
    when given."""
    _need(r_in, torch.float32, "r_in", 2)
    _need(logits, torch.float32, "logits", 2)
    _need(workspace, torch.uint8, "workspace", 1)
    m_tokens, hidden = r_in.shape
    if logits.shape[0] != m_tokens or logits.shape[1] != weights.E:
        raise ValueError(f"logits must be [{m_tokens}][{weights.E}], got {tuple(logits.shape)}")
    if r_out is None:
        r_out = torch.empty_like(r_in)
    _need(r_out, torch.float32, "r_out", 2)
    if x_out is not None:
        _need(x_out, torch.bfloat16, "x_out", 2)
    if y_f32 is not None:
        _need(y_f32, torch.float32, "y_f32", 2)
    _check(lib.moe_layer_rmsnorm_mxfp4(ctypes.byref(weights.desc), _ptr(r_in), _ptr(logits), m_tokens, k,
                                       float(eps), _ptr(r_out), _ptr(x_out), _ptr(y_f32),
                                       _ptr(workspace), workspace.numel(), _stream(r_in)))
    return r_out


def moe_layer_rmsnorm_router(weights, w_router, r_in, k, workspace, r_out=None, eps=1e-6, logits=None,
                             x_out=None, y_f32=None):
    """One layer on the residual stream with its router in front, in two
    launches: x = bf16(RMSNorm(r_in)), logits = x W_router^T, then the layer of
    moe_layer_rmsnorm on those logits.  w_router: [E][H] bfloat16.  Returns
    (r_out, logits); x_out (bf16) and y_f32 are filled when given."""
    _need(r_in, torch.float32, "r_in", 2)
    _need(w_router, torch.bfloat16, "w_router", 2)
    _need(workspace, torch.uint8, "workspace", 1)
    m_tokens, hidden = r_in.shape
    if tuple(w_router.shape) != (weights.E, weights.H) or hidden != weights.H:
        raise ValueError(f"w_router must be [{weights.E}][{weights.H}] and r_in [M][{weights.H}]")
    if logits is None:
        logits = torch.empty((m_tokens, weights.E), dtype=torch.float32, device=r_in.device)
    _need(logits, torch.float32, "logits", 2)
    if tuple(logits.shape) != (m_tokens, weights.E):
        raise ValueError(f"logits must be [{m_tokens}][{weights.E}], got {tuple(logits.shape)}")
    if r_out is None:
        r_out = torch.empty_like(r_in)
    _need(r_out, torch.float32, "r_out", 2)
    if x_out is not None:
        _need(x_out, torch.bfloat16, "x_out", 2)
    if y_f32 is not None:
        _need(y_f32, torch.float32, "y_f32", 2)
    _check(lib.moe_layer_rmsnorm_router_mxfp4(ctypes.byref(weights.desc), _ptr(w_router), _ptr(r_in), m_tokens,
                                              k, float(eps), _ptr(logits), _ptr(r_out), _ptr(x_out),
                                              _ptr(y_f32), _ptr(workspace), workspace.numel(), _stream(r_in)))
    return r_out, logits


# --------------------------------------------------------------------------
# LM head

class LMHeadFP8:
    """An FP8 LM head: E4M3 codes [V][H] + float32 row scales [V], carried
    with a typed descriptor so the codes cannot be consumed as bf16."""

    def __init__(self, codes, row_scale, desc):
        self.codes, self.row_scale, self.desc = codes, row_scale, desc
        self.V, self.H = codes.shape


def lmhead_dynamic_act(head):
    """The same FP8 head with dynamic per-token FP8 activations
    (MOEDEC_FMT_E4M3FN_ROWSCALE_F32_DYNACT): shares the codes and scales."""
    desc = LMHeadFP8Desc()
    ctypes.memmove(ctypes.byref(desc), ctypes.byref(head.desc), ctypes.sizeof(LMHeadFP8Desc))
    desc.format = FMT_E4M3FN_ROWSCALE_F32_DYNACT
    return LMHeadFP8(head.codes, head.row_scale, desc)


def lmhead_quant_fp8(w_bf16):
    _need(w_bf16, torch.bfloat16, "w_bf16", 2)
    V, H = w_bf16.shape
    codes = torch.empty((V, H), dtype=torch.uint8, device=w_bf16.device)
    row_scale = torch.empty(V, dtype=torch.float32, device=w_bf16.device)
    desc = LMHeadFP8Desc()
    _check(lib.lmhead_quant_fp8(_ptr(w_bf16), V, H, _ptr(codes), _ptr(row_scale),
                                ctypes.byref(desc), _stream(w_bf16)))
    return LMHeadFP8(codes, row_scale, desc)


def lmhead_gemv_fp8(head, x, out=None):
    _need(x, torch.bfloat16, "x", 2)
    m_tokens = x.shape[0]
    if out is None:
        out = torch.empty((m_tokens, head.V), dtype=torch.float32, device=x.device)
    _check(lib.lmhead_gemv_fp8(ctypes.byref(head.desc), _ptr(x), m_tokens, _ptr(out), _stream(x)))
    return out


def make_lmhead_workspace(V, m_tokens, device):
    """Zero-filled workspace for lmhead_argmax_fp8 / lmhead_sample_fp8 of one
    head (per-block launch counts and the published keys; every call leaves it
    ready for the next)."""
    need = lib.lmhead_argmax_workspace_bytes(V, m_tokens)
    if need == 0:
        raise MoedecError(-3, f"no LM-head workspace for V={V}, M={m_tokens}")
    return torch.zeros(need, dtype=torch.uint8, device=device)


def lmhead_argmax_fp8(head, x, workspace=None, ids=None, logits=None):
    """Greedy token ids [M] int32 from the FP8 head (lmhead_gemv_fp8_argmax);
    logits [M][V] float32 are written too when a tensor is given.  A workspace
    passed in must come from make_lmhead_workspace (zero-filled once)."""
    _need(x, torch.bfloat16, "x", 2)
    m_tokens = x.shape[0]
    if workspace is None:
        workspace = make_lmhead_workspace(head.V, m_tokens, x.device)
    _need(workspace, torch.uint8, "workspace", 1)
    if ids is None:
        ids = torch.empty(m_tokens, dtype=torch.int32, device=x.device)
    _need(ids, torch.int32, "ids", 1)
    if logits is not None:
        _need(logits, torch.float32, "logits", 2)
    if ids.numel() != m_tokens or (logits is not None and tuple(logits.shape) != (m_tokens, head.V)):
        raise ValueError(f"ids [{m_tokens}] and logits [{m_tokens}][{head.V}] needed")
    _check(lib.lmhead_gemv_fp8_argmax(ctypes.byref(head.desc), _ptr(x), m_tokens, _ptr(logits), _ptr(ids),
                                      _ptr(workspace), workspace.numel(), _stream(x)))
    return ids


def lmhead_sample_fp8(head, x, u, temperature=0.6, top_p=0.95, top_k=29, workspace=None, ids=None,
                      logits=None, want_logits=True):
    """Sampled token ids [M] int32 from the FP8 head (lmhead_gemv_fp8_sample):
    top_k candidates, softmax at `temperature`, the top_p nucleus, drawn at the
    uniforms u [M] float32 (device).  Returns (ids, logits [M][V] float32, or
    None when want_logits is false and no logits tensor is given)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(u, torch.float32, "u", 1)
    m_tokens = x.shape[0]
    if workspace is None:
        workspace = make_lmhead_workspace(head.V, m_tokens, x.device)
    _need(workspace, torch.uint8, "workspace", 1)
    if ids is None:
        ids = torch.empty(m_tokens, dtype=torch.int32, device=x.device)
    if logits is None and want_logits:
        logits = torch.empty((m_tokens, head.V), dtype=torch.float32, device=x.device)
    if logits is not None:
        _need(logits, torch.float32, "logits", 2)
        if tuple(logits.shape) != (m_tokens, head.V):
            raise ValueError(f"logits [{m_tokens}][{head.V}] needed")
    _need(ids, torch.int32, "ids", 1)
    if u.numel() != m_tokens or ids.numel() != m_tokens:
        raise ValueError(f"u [{m_tokens}] and ids [{m_tokens}] needed")
    _check(lib.lmhead_gemv_fp8_sample(ctypes.byref(head.desc), _ptr(x), m_tokens, float(temperature),
                                      float(top_p), int(top_k), _ptr(u), _ptr(logits), _ptr(ids),
                                      _ptr(workspace), workspace.numel(), _stream(x)))
    return ids, logits


def selftest(device="cuda"):
    """moedec_selftest on the current stream of `device`: closed-form cases
    through routing, the fused MXFP4 layer and the FP8 head; raises on a
    mismatch."""
    scratch = torch.empty(lib.moedec_selftest_bytes() + 256, dtype=torch.uint8, device=device)
    off = (-scratch.data_ptr()) % 256
    buf = scratch[off:off + lib.moedec_selftest_bytes()]
    _check(lib.moedec_selftest(_ptr(buf), buf.numel(), _stream(buf)))


def router_logits(w_router, x, out=None):
    """logits [M][E] float32 = x W_router^T (moe_router_logits_bf16)."""
    _need(w_router, torch.bfloat16, "w_router", 2)
    _need(x, torch.bfloat16, "x", 2)
    E, H = w_router.shape
    m_tokens = x.shape[0]
    if out is None:
        out = torch.empty((m_tokens, E), dtype=torch.float32, device=x.device)
    _check(lib.moe_router_logits_bf16(_ptr(w_router), E, H, _ptr(x), m_tokens, _ptr(out), _stream(x)))
    return out


def lmhead_gemv_bf16(w_bf16, x, out=None):
    _need(w_bf16, torch.bfloat16, "w_bf16", 2)
    _need(x, torch.bfloat16, "x", 2)
    V, H = w_bf16.shape
    m_tokens = x.shape[0]
    if out is None:
        out = torch.empty((m_tokens, V), dtype=torch.float32, device=x.device)
    _check(lib.lmhead_gemv_bf16(_ptr(w_bf16), V, H, _ptr(x), m_tokens, _ptr(out), _stream(x)))
    return out
