"""The C ABI boundary without a GPU: the library loads, exports every function
include/moedec.h declares, and rejects bad arguments on the host with the
documented status codes before touching a device."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moedec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def m():
    import bit_moe_expert_topk_amd as m
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("moe_route_topk", "moe_expert_ffn_mxfp4", "moe_layer_mxfp4", "moe_layer_rmsnorm_mxfp4",
                 "lmhead_quant_fp8", "lmhead_gemv_fp8",
                 "lmhead_gemv_bf16", "lmhead_gemv_fp8_argmax", "lmhead_gemv_fp8_sample", "moe_router_logits_bf16", "moe_pack_gateup_mxfp4", "moe_pack_down_mxfp4",
                 "moe_ffn_workspace_bytes", "moedec_mxfp4_packed_sizes", "moedec_status_string",
                 "moedec_last_error", "moedec_abi_version", "moe_ffn_workspace_status",
                 "moe_layer_mxfp4_noalloc", "moe_layer_rmsnorm_router_mxfp4",
                 "moe_pack_shared_fp8", "moedec_shared_fp8_packed_sizes",
                 "moe_layer_mxfp4_prefill", "moe_prefill_workspace_bytes", "moe_layer_mxfp4_prefill_a8",
                 "moe_prefill_workspace_layout", "moe_layer_mxfp4_a8", "moe_ffn_workspace_layout"):
        assert want in names


def test_library_exports_every_declared_symbol(m):
    raw = ctypes.CDLL(m.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    # and the binding declares a signature for each of them
    from bit_moe_expert_topk_amd import _lib
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_status_strings_and_version(m):
    assert m.lib.moedec_abi_version() == 1
    for code, text in ((0, b"ok"), (-1, b"null pointer"), (-4, b"descriptor format mismatch"),
                       (-7, b"device is not gfx950"), (-99, b"unknown status")):
        assert m.lib.moedec_status_string(code) == text


def test_struct_sizes_match_header(m):
    assert ctypes.sizeof(m.Dispatch) == 8 + 129 * 4 * 2 + 129 * 4 * 4
    assert ctypes.sizeof(m.MoEWeights) == 16 + 8 * 8
    assert ctypes.sizeof(m.LMHeadFP8Desc) == 16 + 16


FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced on these paths
ODD = ctypes.c_void_p((1 << 20) + 2)


def test_route_argument_checks(m):
    L = m.lib
    assert L.moe_route_topk(None, 1, 512, 8, FAKE, FAKE, FAKE, None) == -1
    assert L.moe_route_topk(FAKE, 1, 512, 8, None, None, None, None) == -1
    assert L.moe_route_topk(FAKE, 0, 512, 8, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_route_topk(FAKE, 5, 512, 8, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_route_topk(FAKE, 1, 1025, 8, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_route_topk(FAKE, 1, 16, 17, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_route_topk(FAKE, 1, 512, 33, FAKE, FAKE, FAKE, None) == -3
    assert L.moe_route_topk(ODD, 1, 512, 8, FAKE, FAKE, FAKE, None) == -2
    assert L.moe_route_topk(FAKE, 1, 512, 8, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 4), None) == -2
    # the message belongs to the call just made
    assert L.moe_route_topk(FAKE, 1, 512, 33, FAKE, FAKE, FAKE, None) == -3
    assert b"k=33" in L.moedec_last_error()


def test_argmax_workspace_and_argument_checks(m):
    """Workspace = 2,048 per-block 4-byte launch counts, then 8-byte keys per
    token: 2,048 block slots, 8,192 wave slots (the most 2^18 rows need at 32
    rows per wave and 4 waves per block) and one per row."""
    L = m.lib
    for M in (1, 4):
        assert L.lmhead_argmax_workspace_bytes(157184, M) == 8192 + (2048 + 8192 + 157184) * M * 8
    assert L.lmhead_argmax_workspace_bytes(0, 1) == 0 and L.lmhead_argmax_workspace_bytes(10, 5) == 0
    assert L.lmhead_argmax_workspace_bytes((1 << 18) + 1, 1) == 0
    assert L.lmhead_argmax_workspace_bytes(1 << 18, 1) > 0
    desc = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, 157184, 2560, FAKE, FAKE)
    ws = L.lmhead_argmax_workspace_bytes(157184, 1)
    assert L.lmhead_gemv_fp8_argmax(None, FAKE, 1, None, FAKE, FAKE, ws, None) == -1
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(desc), FAKE, 1, None, None, FAKE, ws, None) == -1
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(desc), FAKE, 5, None, FAKE, FAKE, ws, None) == -3
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(desc), FAKE, 1, None, FAKE, FAKE, ws - 8, None) == -5
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(desc), FAKE, 1, None, ODD, FAKE, ws, None) == -2
    bad = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, 7, 157184, 2560, FAKE, FAKE)
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(bad), FAKE, 1, None, FAKE, FAKE, ws, None) == -4
    huge = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, (1 << 18) + 1, 2560, FAKE, FAKE)
    assert L.lmhead_gemv_fp8_argmax(ctypes.byref(huge), FAKE, 1, None, FAKE, FAKE, 1 << 40, None) == -3


def test_sample_argument_checks(m):
    """The sampling call rejects its settings on the host before any device
    work: temperature <= 0 or not finite, top_p outside (0, 1], top_k outside
    1..min(32, V); u is required (logits are optional)."""
    L = m.lib
    desc = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, 157184, 2560, FAKE, FAKE)
    ws = L.lmhead_argmax_workspace_bytes(157184, 1)
    d = ctypes.byref(desc)

    def call(T=0.6, p=0.95, k=29, u=FAKE, logits=FAKE, ids=FAKE, wsb=ws, head=d, M=1):
        return L.lmhead_gemv_fp8_sample(head, FAKE, M, T, p, k, u, logits, ids, FAKE, wsb, None)

    ARG = m._lib.MOEDEC_ERR_ARG
    assert call(T=0.0) == ARG and b"temperature" in L.moedec_last_error()
    assert call(T=-1.0) == ARG and call(T=float("inf")) == ARG and call(T=float("nan")) == ARG
    assert call(p=0.0) == ARG and call(p=1.0000001) == ARG and call(p=float("nan")) == ARG
    assert call(k=0) == ARG and call(k=33) == ARG
    assert b"top_k=33" in L.moedec_last_error()
    small = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, 5, 2560, FAKE, FAKE)
    assert call(k=6, head=ctypes.byref(small), wsb=L.lmhead_argmax_workspace_bytes(5, 1)) == ARG
    assert call(u=None) == -1 and call(ids=None) == -1
    assert call(u=ODD) == -2
    assert call(M=5) == -3 and call(wsb=ws - 8) == -5
    assert L.moedec_status_string(ARG) == b"argument out of range"


def test_selftest_argument_checks(m):
    L = m.lib
    n = L.moedec_selftest_bytes()
    assert n > 0 and n % 256 == 0
    assert L.moedec_selftest(None, n, None) == -1
    assert L.moedec_selftest(ctypes.c_void_p((1 << 20) + 16), n, None) == -2
    assert L.moedec_selftest(FAKE, n - 256, None) == -5
    assert L.moedec_status_string(-8) == b"self-test mismatch"


def test_router_argument_checks(m):
    L = m.lib
    assert L.moe_router_logits_bf16(None, 512, 2560, FAKE, 1, FAKE, None) == -1
    assert L.moe_router_logits_bf16(FAKE, 512, 2560, FAKE, 0, FAKE, None) == -3
    assert L.moe_router_logits_bf16(FAKE, 512, 2560, FAKE, 5, FAKE, None) == -3
    assert L.moe_router_logits_bf16(FAKE, 0, 2560, FAKE, 1, FAKE, None) == -3
    assert L.moe_router_logits_bf16(FAKE, 1025, 2560, FAKE, 1, FAKE, None) == -3
    assert L.moe_router_logits_bf16(FAKE, 512, 2564, FAKE, 1, FAKE, None) == -3
    assert L.moe_router_logits_bf16(FAKE, 512, 8192, FAKE, 1, FAKE, None) == -3
    assert L.moe_router_logits_bf16(ODD, 512, 2560, FAKE, 1, FAKE, None) == -2


def test_valid_arguments_without_gpu_report_device(m):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert m.lib.moe_route_topk(FAKE, 1, 512, 8, FAKE, FAKE, FAKE, None) == -7
    assert b"device" in m.lib.moedec_last_error()


def test_packed_sizes(m):
    s = m.packed_sizes(2560, 768)
    # Ling-shaped expert: packing adds no padding (80 and 24 blocks are multiples of 4)
    assert (s.gu_codes, s.gu_scales, s.dn_codes, s.dn_scales) == (1966080, 122880, 983040, 61440)
    assert s.gu_codes + s.gu_scales + s.dn_codes + s.dn_scales == 3133440
    # tiny expert: 2 MX blocks along I are padded to 4 in the down stream
    t = m.packed_sizes(256, 64)
    assert (t.gu_codes, t.gu_scales, t.dn_codes, t.dn_scales) == (16384, 1024, 16384, 1024)
    out = m.MXFP4Sizes()
    for H, I in ((2560, 48), (96, 64), (32, 64), (256, 0), (4160, 64), (256, 2080)):
        assert m.lib.moedec_mxfp4_packed_sizes(H, I, ctypes.byref(out)) == -3


def test_pack_argument_checks(m):
    L = m.lib
    assert L.moe_pack_gateup_mxfp4(FAKE, FAKE, None, FAKE, 3, 256, 64, FAKE, FAKE, None) == -1
    assert L.moe_pack_gateup_mxfp4(FAKE, FAKE, FAKE, FAKE, 0, 256, 64, FAKE, FAKE, None) == -3
    assert L.moe_pack_gateup_mxfp4(ODD, FAKE, FAKE, FAKE, 3, 256, 64, FAKE, FAKE, None) == -2
    assert L.moe_pack_down_mxfp4(FAKE, FAKE, 3, 200, 64, FAKE, FAKE, None) == -3


def _weights(m, **kw):
    w = m.MoEWeights(m.MOE_MAGIC, 512, 2560, 768, *([1 << 20] * 8))
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def test_ffn_argument_checks(m):
    L = m.lib
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    assert ws > 0 and m.ffn_workspace_bytes(5, 8, 2560, 768) == 0
    call = lambda w, x=FAKE, M=1, k=8, n=ws: L.moe_expert_ffn_mxfp4(
        ctypes.byref(w), x, M, FAKE, k, FAKE, None, FAKE, n, None)
    assert L.moe_expert_ffn_mxfp4(None, FAKE, 1, FAKE, 8, FAKE, None, FAKE, ws, None) == -1
    assert call(_weights(m, magic=0x12345678)) == -4
    assert call(_weights(m, sh_dn_scales=None)) == -1
    assert call(_weights(m), x=None) == -1
    assert call(_weights(m), M=0) == -3
    assert call(_weights(m), k=0) == -3
    assert call(_weights(m, H=2500)) == -3
    assert call(_weights(m, E=4), k=8) == -3
    assert call(_weights(m, gu_codes=(1 << 20) + 4)) == -2
    assert call(_weights(m), x=ODD) == -2
    assert call(_weights(m), x=ctypes.c_void_p((1 << 20) + 4)) == -2      # x needs 16 bytes
    assert call(_weights(m, I=4096)) == -3
    assert call(_weights(m, H=8192)) == -3
    assert call(_weights(m), n=ws - 1) == -5


def test_fused_layer_argument_checks(m):
    L = m.lib
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    call = lambda w, lg=FAKE, M=1, k=8, n=ws, disp=None: L.moe_layer_mxfp4(
        ctypes.byref(w), FAKE, lg, M, k, None, None, disp, FAKE, None, FAKE, n, None)
    assert call(_weights(m), lg=None) == -1
    assert call(_weights(m, magic=1)) == -4
    assert call(_weights(m), k=33) == -3
    assert call(_weights(m), M=5) == -3
    assert call(_weights(m), lg=ODD) == -2
    assert call(_weights(m), disp=ctypes.c_void_p((1 << 20) + 8)) == -2
    assert call(_weights(m), n=ws - 1) == -5


def test_residual_layer_argument_checks(m):
    L = m.lib
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    far = ctypes.c_void_p(1 << 24)

    def call(w, r_in=FAKE, r_out=far, lg=FAKE, eps=1e-6, x=None, M=1, k=8, n=ws):
        return L.moe_layer_rmsnorm_mxfp4(ctypes.byref(w), r_in, lg, M, k, eps, r_out, x, None, FAKE, n, None)

    assert call(_weights(m), r_in=None) == -1
    assert call(_weights(m), r_out=None) == -1
    assert call(_weights(m), lg=None) == -1
    assert call(_weights(m, magic=1)) == -4
    assert call(_weights(m), eps=-1.0) == -3
    assert call(_weights(m), eps=float("nan")) == -3
    assert call(_weights(m), r_out=ctypes.c_void_p((1 << 20) + 4096)) == -3     # overlaps r_in
    assert call(_weights(m), r_out=ctypes.c_void_p((1 << 24) + 4)) == -2
    assert call(_weights(m), x=ctypes.c_void_p((1 << 22) + 8)) == -2
    assert call(_weights(m), M=5) == -3
    assert call(_weights(m), n=ws - 1) == -5


def test_shared_fp8_sizes_and_argument_checks(m):
    """FP8 shared expert: packed sizes (16 codes per 16-byte lane, chunks of
    64 values per row, twice the MXFP4 chunk counts), pack argument checks,
    and descriptor rules -- the fused layer takes the FP8 magic, the
    dispatch-table FFN refuses it, and its float32 scales must be 4-byte
    aligned."""
    L = m.lib
    sz = m.shared_fp8_sizes(2560, 768)
    assert sz.gu_codes == 768 // 16 * 40 * 2 * 1024 == 2 * 768 * 2560
    assert sz.dn_codes == 2560 // 16 * 12 * 1024 == 2560 * 768
    assert sz.gu_scales == 2 * 768 * 4 and sz.dn_scales == 2560 * 4
    ragged = m.shared_fp8_sizes(192, 96)               # 6 and 3 MX blocks: chunk counts padded to 4 and 2
    assert ragged.gu_codes == 96 // 16 * 4 * 2 * 1024 and ragged.dn_codes == 192 // 16 * 2 * 1024
    out = m.MXFP4Sizes()
    assert L.moedec_shared_fp8_packed_sizes(100, 768, ctypes.byref(out)) == -3
    args = [FAKE, FAKE, FAKE, 2560, 768, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(args); bad[0] = None
    assert L.moe_pack_shared_fp8(*bad) == -1
    bad = list(args); bad[5] = ctypes.c_void_p((1 << 20) + 8)
    assert L.moe_pack_shared_fp8(*bad) == -2
    bad = list(args); bad[6] = ctypes.c_void_p((1 << 20) + 2)
    assert L.moe_pack_shared_fp8(*bad) == -2
    bad = list(args); bad[3] = 2500
    assert L.moe_pack_shared_fp8(*bad) == -3
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    w8 = _weights(m, magic=m.MOE_MAGIC_SHARED_FP8)
    assert L.moe_expert_ffn_mxfp4(ctypes.byref(w8), FAKE, 1, FAKE, 8, FAKE, None, FAKE, ws, None) == -4
    assert b"MXFP4 shared" in L.moedec_last_error()
    w8.sh_dn_scales = (1 << 20) + 2
    assert L.moe_layer_mxfp4(ctypes.byref(w8), FAKE, FAKE, 1, 8, None, None, None, FAKE, None, FAKE, ws,
                             None) == -2
    assert L.moe_layer_mxfp4(ctypes.byref(_weights(m, magic=0x4D4F4539)), FAKE, FAKE, 1, 8, None, None, None,
                             FAKE, None, FAKE, ws, None) == -4


def test_router_chain_argument_checks(m):
    """The layer with its router in front checks what the residual layer
    checks, plus the router matrix, before any device work."""
    L = m.lib
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    far = ctypes.c_void_p(1 << 24)

    def call(w, wr=FAKE, r_in=FAKE, r_out=far, lg=FAKE, eps=1e-6, M=1, k=8, n=ws):
        return L.moe_layer_rmsnorm_router_mxfp4(ctypes.byref(w), wr, r_in, M, k, eps, lg, r_out, None, None,
                                                FAKE, n, None)

    assert call(_weights(m), wr=None) == -1 and b"w_router" in L.moedec_last_error()
    assert call(_weights(m), wr=ctypes.c_void_p((1 << 20) + 8)) == -2
    assert call(_weights(m), r_in=None) == -1
    assert call(_weights(m), lg=None) == -1
    assert call(_weights(m, magic=1)) == -4
    assert call(_weights(m), eps=2.0) == -3
    assert call(_weights(m), r_out=ctypes.c_void_p((1 << 20) + 4096)) == -3     # overlaps r_in
    assert call(_weights(m), M=0) == -3 and call(_weights(m), k=0) == -3
    assert call(_weights(m), n=ws - 1) == -5


def test_lmhead_descriptor_guards_format(m):
    """FP8 codes must never be consumed as bf16 (or vice versa): the GEMV takes a
    typed descriptor and rejects one whose magic/format tag is wrong."""
    L = m.lib
    good = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, 157184, 2560, 1 << 20, 1 << 20)
    wrong_magic = m.LMHeadFP8Desc(0, m.FMT_E4M3FN_ROWSCALE_F32, 157184, 2560, 1 << 20, 1 << 20)
    wrong_fmt = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, 3, 157184, 2560, 1 << 20, 1 << 20)
    dyn = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32_DYNACT, 157184, 2560, 1 << 20, 1 << 20)
    assert L.lmhead_gemv_fp8(ctypes.byref(dyn), FAKE, 5, FAKE, None) == -3      # format accepted, M checked
    assert L.lmhead_gemv_fp8(ctypes.byref(wrong_magic), FAKE, 1, FAKE, None) == -4
    assert L.lmhead_gemv_fp8(ctypes.byref(wrong_fmt), FAKE, 1, FAKE, None) == -4
    assert L.lmhead_gemv_fp8(None, FAKE, 1, FAKE, None) == -1
    assert L.lmhead_gemv_fp8(ctypes.byref(good), FAKE, 5, FAKE, None) == -3
    bad_h = m.LMHeadFP8Desc(m.LMHEAD_MAGIC, m.FMT_E4M3FN_ROWSCALE_F32, 10, 4100, 1 << 20, 1 << 20)
    assert L.lmhead_gemv_fp8(ctypes.byref(bad_h), FAKE, 1, FAKE, None) == -3
    assert L.lmhead_quant_fp8(FAKE, 10, 2561, FAKE, FAKE, None, None) == -3
    assert L.lmhead_quant_fp8(ODD, 10, 2560, FAKE, FAKE, None, None) == -2
    assert L.lmhead_gemv_bf16(FAKE, 10, 2560, FAKE, 0, FAKE, None) == -3
    assert L.lmhead_gemv_bf16(FAKE, 10, 2560, None, 1, FAKE, None) == -1


def test_workspace_status_and_noalloc_argument_checks(m):
    """The status call and the no-alloc layer reject bad arguments on the host,
    before any device work: a workspace too small to hold the status word, a
    misaligned one, a NULL weights descriptor, and a shape whose workspace
    exceeds the 4 MiB no-alloc scratch."""
    L = m.lib
    FAKE = ctypes.c_void_p(1 << 20)
    flags = ctypes.c_uint32(7)
    assert L.moe_ffn_workspace_status(FAKE, 64, ctypes.byref(flags), None) == m._lib.MOEDEC_ERR_WORKSPACE
    assert flags.value == 0
    assert b"status word" in L.moedec_last_error()
    assert L.moe_ffn_workspace_status(ctypes.c_void_p((1 << 20) + 8), 1 << 20, None, None) == -2
    assert L.moe_layer_mxfp4_noalloc(None, FAKE, FAKE, 1, 8, None, None, None, FAKE, None, None) == -1
    w = m.MoEWeights(m.MOE_MAGIC, 512, 4096, 2048, *([1 << 20] * 8))
    # M = 4, k = 32 at H 4096, I 2048: a workspace far beyond 4 MiB
    assert L.moe_layer_mxfp4_noalloc(ctypes.byref(w), FAKE, FAKE, 4, 32, None, None, None, FAKE, None, None) == -5
    assert b"no-alloc limit" in L.moedec_last_error()
    assert m.lib.moedec_status_string(-9) != b"unknown status"


def test_prefill_workspace_and_argument_checks(m):
    L = m.lib
    for T, E, k, H, I in ((8192, 512, 8, 2560, 768), (1, 16, 2, 256, 64), (37, 16, 2, 256, 64)):
        n = L.moe_prefill_workspace_bytes(T, E, k, H, I)
        pairs = T * (k + 1)
        body = pairs * (4 * H + 4 * I)                    # y_pair float32 + h as two bf16
        x8 = T * H + T * (H // 32 + 4)                     # MXFP8 x of the W4A8 call
        chunks = 2 * 64 * E * 4                            # per-chunk expert counts and first rows
        assert body <= n <= (body + pairs * 4 + 3 * T * k * 4 + (2 * (E + 2) * 4) + ((pairs // 32 + E + 1) * 8)
                             + x8 + chunks + 4096)
    assert L.moe_prefill_workspace_bytes(0, 512, 8, 2560, 768) == 0
    assert L.moe_prefill_workspace_bytes(m._lib.MOEDEC_MAX_PREFILL_T + 1, 512, 8, 2560, 768) == 0
    assert L.moe_prefill_workspace_bytes(64, 512, 33, 2560, 768) == 0
    assert L.moe_prefill_workspace_bytes(64, 512, 8, 2560 + 32, 768) == 0
    ws = L.moe_prefill_workspace_bytes(64, 512, 8, 2560, 768)
    for fn in (L.moe_layer_mxfp4_prefill, L.moe_layer_mxfp4_prefill_a8):
        _prefill_argument_checks(m, fn, ws)


def test_a8_layer_argument_checks(m):
    """moe_layer_mxfp4_a8 checks as moe_layer_mxfp4 and refuses an FP8 shared
    expert (before touching the device)."""
    L = m.lib
    ws = m.ffn_workspace_bytes(1, 8, 2560, 768)
    call = lambda w, lg=FAKE, k=8, n=ws: L.moe_layer_mxfp4_a8(
        ctypes.byref(w), FAKE, lg, 1, k, None, None, None, FAKE, None, FAKE, n, None)
    assert call(_weights(m, magic=m._lib.MOE_MAGIC_SHARED_FP8)) == -4
    assert call(_weights(m, magic=0x12345678)) == -4
    assert call(_weights(m), lg=None) == -1
    assert call(_weights(m), k=33) == -3
    assert call(_weights(m), n=ws - 1) == -5


def _prefill_argument_checks(m, fn, ws):
    call = lambda w, lg=FAKE, T=64, k=8, n=ws, work=FAKE, y32=None: fn(
        ctypes.byref(w), FAKE, lg, T, k, None, None, None, FAKE, y32, work, n, None)
    assert call(_weights(m), lg=None) == -1
    assert call(_weights(m, magic=1)) == -4
    assert call(_weights(m, magic=m._lib.MOE_MAGIC_SHARED_FP8)) == -4
    assert call(_weights(m), k=33) == -3
    assert call(_weights(m, dn_scales=(1 << 20) + 2)) == -2
    assert call(_weights(m), T=0) == -3
    assert call(_weights(m), T=m._lib.MOEDEC_MAX_PREFILL_T + 1) == -3
    assert call(_weights(m), lg=ODD) == -2
    assert call(_weights(m), y32=ctypes.c_void_p((1 << 20) + 8)) == -2
    assert call(_weights(m), work=ctypes.c_void_p((1 << 20) + 16)) == -2
    assert call(_weights(m), work=None) == -1
    assert call(_weights(m), n=ws - 1) == -5


def test_prefill_workspace_layout(m):
    """The layout query: regions inside the workspace, disjoint, aligned, with
    the scale strides of 128-value chunks; errors for NULL and bad shapes."""
    L = m.lib
    out = m._lib.PrefillLayout()
    assert L.moe_prefill_workspace_layout(64, 512, 8, 2560, 768, None) == -1
    assert L.moe_prefill_workspace_layout(0, 512, 8, 2560, 768, ctypes.byref(out)) == -3
    assert L.moe_prefill_workspace_layout(64, 512, 8, 2560 + 32, 768, ctypes.byref(out)) == -3
    for T, E, k, H, I in ((8192, 512, 8, 2560, 768), (1, 16, 2, 256, 64), (129, 24, 3, 320, 96),
                          (m._lib.MOEDEC_MAX_PREFILL_T, 1024, 32, 4096, 2048)):
        lay = m.prefill_workspace_layout(T, E, k, H, I)
        assert lay["total_bytes"] == L.moe_prefill_workspace_bytes(T, E, k, H, I)
        sb, sbi = lay["x_scale_stride"], lay["h_scale_stride"]
        assert sb == 4 * -(-H // 128) and sbi == 4 * -(-I // 128)
        P = T * (k + 1)
        regions = sorted([(lay["pos"], T * k * 4), (lay["y_pair"], P * H * 4), (lay["x_codes"], T * H),
                          (lay["x_scales"], T * sb), (lay["h_codes"], P * I), (lay["h_scales"], P * sbi)])
        for (a, n), (b, _) in zip(regions, regions[1:]):
            assert a + n <= b
        assert regions[-1][0] + regions[-1][1] <= lay["total_bytes"]
        assert all(off % 256 == 0 for off, _ in regions)


def test_ffn_workspace_layout(m):
    L = m.lib
    out = m._lib.FfnLayout()
    assert L.moe_ffn_workspace_layout(1, 8, 2560, 768, None) == -1
    assert L.moe_ffn_workspace_layout(5, 8, 2560, 768, ctypes.byref(out)) == -3
    for M, k, H, I in ((1, 8, 2560, 768), (4, 8, 2560, 768), (4, 32, 4096, 2048), (2, 3, 320, 96)):
        assert L.moe_ffn_workspace_layout(M, k, H, I, ctypes.byref(out)) == 0
        assert out.total_bytes == L.moe_ffn_workspace_bytes(M, k, H, I)
        assert out.max_slots == M * k + 1 and out.M == M
        assert out.h_words % 256 == 0
        assert out.h_words + 8 * out.max_slots * M * I <= out.total_bytes
