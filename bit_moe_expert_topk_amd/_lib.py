"""ctypes declarations of libmoedec's C ABI (include/moedec.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmoedec.so.  Importing this module loads the library and raises if it has
not been built -- there is no fallback.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoedec.so")

MOEDEC_OK = 0
MOEDEC_ERR_NULL = -1
MOEDEC_ERR_ALIGN = -2
MOEDEC_ERR_SHAPE = -3
MOEDEC_ERR_FORMAT = -4
MOEDEC_ERR_WORKSPACE = -5
MOEDEC_ERR_LAUNCH = -6
MOEDEC_ERR_DEVICE = -7
MOEDEC_ERR_SELFTEST = -8
MOEDEC_ERR_TIMEOUT = -9
MOEDEC_ERR_ARG = -10
MOEDEC_MAX_SAMPLE_K = 32
MOEDEC_MAX_EPILOGUE_V = 1 << 18
MOEDEC_MAX_PREFILL_T = 65536

MAX_M = 4
MAX_K = 32
MAX_E = 1024
MAX_SLOTS = MAX_M * MAX_K + 1

MOE_MAGIC = 0x4D4F4534
MOE_MAGIC_SHARED_FP8 = 0x4D4F4538
LMHEAD_MAGIC = 0x4C4D4838
FMT_E4M3FN_ROWSCALE_F32 = 1
FMT_E4M3FN_ROWSCALE_F32_DYNACT = 2

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_size_t = ctypes.c_size_t
c_float = ctypes.c_float
c_uint32 = ctypes.c_uint32
c_int32 = ctypes.c_int32


class Dispatch(ctypes.Structure):
    _fields_ = [
        ("n_slots", c_int32),
        ("M", c_int32),
        ("expert", c_int32 * MAX_SLOTS),
        ("token_mask", c_uint32 * MAX_SLOTS),
        ("weight", (ctypes.c_float * MAX_M) * MAX_SLOTS),
    ]


class MXFP4Sizes(ctypes.Structure):
    _fields_ = [("gu_codes", c_size_t), ("gu_scales", c_size_t),
                ("dn_codes", c_size_t), ("dn_scales", c_size_t)]


class MoEWeights(ctypes.Structure):
    _fields_ = [
        ("magic", c_uint32), ("E", c_int32), ("H", c_int32), ("I", c_int32),
        ("gu_codes", c_void_p), ("gu_scales", c_void_p),
        ("dn_codes", c_void_p), ("dn_scales", c_void_p),
        ("sh_gu_codes", c_void_p), ("sh_gu_scales", c_void_p),
        ("sh_dn_codes", c_void_p), ("sh_dn_scales", c_void_p),
    ]


class FfnLayout(ctypes.Structure):
    """moedec_ffn_layout: where an FFN call leaves each (slot, token)'s h."""
    _fields_ = [("total_bytes", ctypes.c_uint64), ("h_words", ctypes.c_uint64), ("max_slots", ctypes.c_int32),
                ("M", ctypes.c_int32)]


class PrefillLayout(ctypes.Structure):
    """moedec_prefill_layout: byte offsets of the many-token intermediates."""
    _fields_ = [("total_bytes", ctypes.c_uint64), ("pos", ctypes.c_uint64), ("y_pair", ctypes.c_uint64),
                ("x_codes", ctypes.c_uint64), ("x_scales", ctypes.c_uint64), ("h_codes", ctypes.c_uint64),
                ("h_scales", ctypes.c_uint64), ("x_scale_stride", ctypes.c_int32),
                ("h_scale_stride", ctypes.c_int32)]


class LMHeadFP8Desc(ctypes.Structure):
    _fields_ = [
        ("magic", c_uint32), ("format", c_uint32), ("V", c_int32), ("H", c_int32),
        ("codes", c_void_p), ("row_scale", c_void_p),
    ]


# name -> (restype, argtypes); mirrors include/moedec.h
SIGNATURES = {
    "moedec_abi_version": (c_int, []),
    "moedec_status_string": (ctypes.c_char_p, [c_int]),
    "moedec_last_error": (ctypes.c_char_p, []),
    "moe_route_topk": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moedec_selftest_bytes": (c_size_t, []),
    "moedec_selftest": (c_int, [c_void_p, c_size_t, c_void_p]),
    "lmhead_argmax_workspace_bytes": (c_size_t, [c_int, c_int]),
    "lmhead_gemv_fp8_argmax": (c_int, [ctypes.POINTER(LMHeadFP8Desc), c_void_p, c_int, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "lmhead_gemv_fp8_sample": (c_int, [ctypes.POINTER(LMHeadFP8Desc), c_void_p, c_int, c_float, c_float, c_int,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_router_logits_bf16": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p]),
    "moedec_mxfp4_packed_sizes": (c_int, [c_int, c_int, ctypes.POINTER(MXFP4Sizes)]),
    "moe_pack_gateup_mxfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p]),
    "moe_pack_down_mxfp4": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "moedec_shared_fp8_packed_sizes": (c_int, [c_int, c_int, ctypes.POINTER(MXFP4Sizes)]),
    "moe_pack_shared_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
    "moe_ffn_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "moe_ffn_workspace_layout": (c_int, [c_int, c_int, c_int, c_int, ctypes.POINTER(FfnLayout)]),
    "moe_expert_ffn_mxfp4": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_int, c_void_p, c_int,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_layer_mxfp4": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_layer_mxfp4_a8": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_layer_rmsnorm_mxfp4": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int,
                                        ctypes.c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                        c_void_p]),
    "moe_layer_rmsnorm_router_mxfp4": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int,
                                               ctypes.c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_size_t, c_void_p]),
    "moe_prefill_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_layer_mxfp4_prefill": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_layer_mxfp4_prefill_a8": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                           c_void_p]),
    "moe_prefill_workspace_layout": (c_int, [c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(PrefillLayout)]),
    "moe_ffn_workspace_status": (c_int, [c_void_p, c_size_t, ctypes.POINTER(c_uint32), c_void_p]),
    "moe_layer_mxfp4_noalloc": (c_int, [ctypes.POINTER(MoEWeights), c_void_p, c_void_p, c_int, c_int, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "lmhead_quant_fp8": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p,
                                 ctypes.POINTER(LMHeadFP8Desc), c_void_p]),
    "lmhead_gemv_fp8": (c_int, [ctypes.POINTER(LMHeadFP8Desc), c_void_p, c_int, c_void_p, c_void_p]),
    "lmhead_gemv_bf16": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p]),
}


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
            "or python bit_moe_expert_topk_amd/build.py)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()
