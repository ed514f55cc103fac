"""Device-side filling of MXFP4 layers with the synth SplitMix64 streams.

Wraps synth/libmoedec_synth.so (synth/fill.hip), the device twin of
synth.hash_bytes / synth.hash_scale_codes: the bytes it writes are the bytes
the host functions return for the same (seed, layer, expert, matrix, part).
"""

import ctypes
import os

import torch

from . import MAT_DOWN, MAT_GATE, MAT_UP, PART_CODES, PART_SCALES

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoedec_synth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run the build first")
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.synth_fill_mxfp4.restype = ctypes.c_int
        _lib.synth_fill_mxfp4.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_ulonglong, ctypes.c_ulonglong, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return _lib


def fill(dst, n_experts, bytes_per_expert, seed, layer, expert0, matrix, part, lo=0, hi=255):
    lib = _load()
    assert dst.dtype == torch.uint8 and dst.is_cuda and dst.numel() >= n_experts * bytes_per_expert
    st = lib.synth_fill_mxfp4(ctypes.c_void_p(dst.data_ptr()), n_experts, bytes_per_expert, seed,
                              layer, expert0, matrix, part, lo, hi,
                              ctypes.c_void_p(torch.cuda.current_stream(dst.device).cuda_stream))
    if st != 0:
        raise RuntimeError(f"synth_fill_mxfp4 failed with {st}")


def canonical_layer(seed, layer, shape, device, n_experts=None):
    """Canonical MXFP4 tensors of a whole layer (E routed + shared = E+1
    experts) generated on the device: dict name -> (codes, scales) with
    codes [E+1][N][K/2] and scales [E+1][N][K/32]."""
    n = shape.E + 1 if n_experts is None else n_experts
    H, I = shape.H, shape.I
    out = {}
    for name, mat, (rows, cols) in (("gate", MAT_GATE, (I, H)), ("up", MAT_UP, (I, H)),
                                    ("down", MAT_DOWN, (H, I))):
        codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((n, rows, cols // 32), dtype=torch.uint8, device=device)
        fill(codes, n, rows * cols // 2, seed, layer, 0, mat, PART_CODES)
        fill(scales, n, rows * cols // 32, seed, layer, 0, mat, PART_SCALES,
             shape.scale_lo, shape.scale_hi)
        out[name] = (codes, scales)
    return out
