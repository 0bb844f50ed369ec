"""ctypes loader for libsvdq.so (the C ABI declared in include/svdq.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvdq.so")

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/svdq.h
SIGNATURES = {
    "svdq_last_error": (ctypes.c_char_p, []),
    "svdq_version": (ctypes.c_char_p, []),
    "svdq_smooth_inputs": (c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp, c_int,
                                   c_vp, c_i64, c_vp, c_i64, c_vp]),
    "svdq_check_smoothing": (c_int, [c_i64, c_i64, c_i64, c_i64, c_i64, c_vp]),
    "svdq_check_rank": (c_int, [c_i64, c_i64, c_i64]),
    "svdq_split_weight": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_i64, c_vp, c_vp, c_vp]),
    "svdq_fake_quantize_workspace": (c_sz, [c_i64, c_i64]),
    "svdq_fake_quantize": (c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_i64, c_vp, c_vp, c_sz,
                                   c_vp]),
    "svdq_prepared_layout": (c_int, [c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_i64)]),
    "svdq_prepare": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "svdq_workspace_bytes": (c_int, [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_sz)]),
    "svdq_linear": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_i64, c_vp,
                            c_sz, c_vp]),
    "svdq_linear_bias": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp,
                                 c_i64, c_vp, c_sz, c_vp]),
    "svdq_linear_noalloc": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_i64,
                                    c_vp]),
    "svdq_quantize_activations": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_int, c_int, c_int, c_vp, c_i64, c_vp,
                                          c_i64, c_vp, c_vp, c_sz, c_vp]),
    "svdq_prepare_gpu_workspace_bytes": (c_int, [c_i64, c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "svdq_prepare_gpu": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp,
                                 c_vp, c_sz, c_vp]),
    "svdq_prepare_two_level": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, ctypes.c_float, c_int, c_vp, c_vp,
                                       c_vp, c_vp]),
    "svdq_prepare_linear": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "svdq_calibrate_workspace_bytes": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "svdq_calibrate_scale": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_int, ctypes.c_double, c_vp, c_vp,
                                     c_sz, c_vp]),
    "svdq_profile_begin": (c_int, [c_int, ctypes.c_uint]),
    "svdq_profile_begin_sampled": (c_int, [c_int, ctypes.c_uint, c_int]),
    "svdq_profile_end": (c_int, [ctypes.POINTER(ctypes.c_float), c_int, ctypes.POINTER(c_int)]),
    "svdq_ceiling": (c_int, [c_int, ctypes.c_int64, c_vp, ctypes.c_size_t, c_vp, ctypes.c_size_t, c_vp,
                             ctypes.POINTER(ctypes.c_double)]),
}
NSTAGES = 4
STAGE_NAMES = ("amax", "act_quant_down", "down_reduce", "gemm")

SVDQ_OK, SVDQ_EINVAL, SVDQ_EDTYPE, SVDQ_EUNSUPPORTED, SVDQ_EHIP = 0, 1, 2, 3, 4
SVDQ_F32, SVDQ_BF16, SVDQ_F64 = 0, 1, 2
SVDQ_FMT_INT, SVDQ_FMT_MX = 0, 1
SEC_SCALE, SEC_RCODES, SEC_RSCALES, SEC_L1T, SEC_L2T, SEC_RECIP, SEC_GLOBAL, SEC_END = 0, 1, 2, 3, 4, 5, 6, 7
NSEC = 8
NOALLOC_SCRATCH_BYTES = 16 << 20  # SVDQ_NOALLOC_SCRATCH_BYTES

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libsvdq.so once; raise LibraryMissing if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is missing: build it with `python -m rank_bit_residual_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    """Map a non-zero svdq_status to a Python exception (EINVAL -> ValueError)."""
    if status == SVDQ_OK:
        return
    msg = load().svdq_last_error().decode()
    if status == SVDQ_EINVAL:
        raise ValueError(msg)
    if status == SVDQ_EDTYPE:
        raise TypeError(msg)
    raise RuntimeError(f"svdq status {status}: {msg}")
