"""The C ABI library loads without a GPU and exports every function include/svdq.h declares."""
import ctypes
import os
import re

import pytest

from rank_bit_residual_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "svdq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_page_calls():
    names = declared_functions()
    for required in ("svdq_smooth_inputs", "svdq_split_weight", "svdq_fake_quantize", "svdq_linear"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert set(declared_functions()) <= set(_lib.SIGNATURES)


def test_host_calls_report_errors_without_a_gpu():
    lib = _lib.load()
    assert lib.svdq_check_rank(4, 3, 4) == _lib.SVDQ_EINVAL
    assert b"rank" in lib.svdq_last_error()
    assert lib.svdq_check_rank(4, 3, 3) == _lib.SVDQ_OK
    assert lib.svdq_last_error() == b""
    off = (ctypes.c_int64 * _lib.NSEC)()
    assert lib.svdq_prepared_layout(64, 48, 8, _lib.SVDQ_FMT_MX, 3, _lib.SVDQ_BF16, off) == _lib.SVDQ_EINVAL
    assert lib.svdq_prepared_layout(64, 48, 8, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_F64, off) == _lib.SVDQ_EDTYPE
    assert lib.svdq_prepared_layout(64, 48, 8, _lib.SVDQ_FMT_INT, 9, _lib.SVDQ_F32, off) == _lib.SVDQ_EINVAL
    assert lib.svdq_prepared_layout(64, 48, 8, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_F32, off) == _lib.SVDQ_OK
    assert all(v % 256 == 0 for v in off)
    ws = ctypes.c_size_t()
    assert lib.svdq_workspace_bytes(16, 64, 48, 8, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_F32, ctypes.byref(ws)) == 0
    assert ws.value > 0
    assert lib.svdq_calibrate_workspace_bytes(0, 64, ctypes.byref(ws)) == _lib.SVDQ_EINVAL
    assert lib.svdq_calibrate_workspace_bytes(4096, 3072, ctypes.byref(ws)) == 0 and ws.value % 256 == 0
    assert lib.svdq_calibrate_scale(None, 4, 4, 4, None, 4, 4, _lib.SVDQ_F32, 0.5, None, None, 0, None) == _lib.SVDQ_EINVAL
    assert lib.svdq_calibrate_scale(None, 4, 4, 4, None, 4, 4, _lib.SVDQ_F64, 0.5, None, None, 0, None) == _lib.SVDQ_EDTYPE
    # profiling session: argument errors are reported before any HIP call
    assert lib.svdq_profile_begin(0, 8) == _lib.SVDQ_EINVAL
    assert lib.svdq_profile_begin(4, 0) == _lib.SVDQ_EINVAL
    assert lib.svdq_profile_begin(4, 16) == _lib.SVDQ_EINVAL
    assert b"stage_mask" in lib.svdq_last_error()
    assert lib.svdq_profile_begin_sampled(4, 8, 0) == _lib.SVDQ_EINVAL
    assert b"every" in lib.svdq_last_error()
    n = ctypes.c_int()
    assert lib.svdq_profile_end(None, 0, ctypes.byref(n)) == _lib.SVDQ_EINVAL  # no open session
    # ceiling probes: an unknown kind or a NULL buffer is refused before any HIP call
    work = ctypes.c_double()
    assert lib.svdq_ceiling(3, 1, None, 0, None, 0, None, ctypes.byref(work)) == _lib.SVDQ_EINVAL
    assert b"kind" in lib.svdq_last_error()
    assert lib.svdq_ceiling(0, 1, None, 0, None, 0, None, ctypes.byref(work)) == _lib.SVDQ_EINVAL


def test_int_shapes_beyond_exact_int32_accumulation_are_refused():
    """INT residual products accumulate in int32 on the matrix cores; shapes where
    Kp * max|code product| could reach 2^31 (4-bit codes enter the int8 MFMAs as 16 c) are
    refused with EUNSUPPORTED by preparation and the operator; MX (fp32 accumulation) and the
    size query are unaffected."""
    lib = _lib.load()
    off = (ctypes.c_int64 * _lib.NSEC)()
    # 4 bits: 256 * 7^2 = 12544 per product; 171008 * 12544 < 2^31 <= 171264 * 12544
    assert lib.svdq_prepared_layout(171008, 64, 0, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_BF16, off) == _lib.SVDQ_OK
    assert lib.svdq_prepared_layout(171009, 64, 0, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_BF16, off) == _lib.SVDQ_EUNSUPPORTED
    assert b"int32" in lib.svdq_last_error()
    # 8 bits (int8 codes as they are): 127^2 = 16129 per product
    assert lib.svdq_prepared_layout(133120, 64, 0, _lib.SVDQ_FMT_INT, 8, _lib.SVDQ_F32, off) == _lib.SVDQ_OK
    assert lib.svdq_prepared_layout(133121, 64, 0, _lib.SVDQ_FMT_INT, 8, _lib.SVDQ_F32, off) == _lib.SVDQ_EUNSUPPORTED
    # 2 bits and MXFP4 are far from the bound
    assert lib.svdq_prepared_layout(1 << 20, 64, 0, _lib.SVDQ_FMT_INT, 2, _lib.SVDQ_F32, off) == _lib.SVDQ_OK
    assert lib.svdq_prepared_layout(1 << 20, 64, 0, _lib.SVDQ_FMT_MX, 4, _lib.SVDQ_BF16, off) == _lib.SVDQ_OK
    # the operator refuses before touching any buffer; the size query still answers
    assert lib.svdq_linear(None, 16, 200000, 200000, None, 64, 0, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_BF16,
                           None, 64, None, 0, None) == _lib.SVDQ_EUNSUPPORTED
    ws = ctypes.c_size_t()
    assert lib.svdq_workspace_bytes(16, 200000, 64, 0, _lib.SVDQ_FMT_INT, 4, _lib.SVDQ_BF16, ctypes.byref(ws)) == 0
