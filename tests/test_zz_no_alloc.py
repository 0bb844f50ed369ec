"""svdq_linear_noalloc (the entry point for callers that cannot allocate device memory)
against svdq_linear, through the C ABI: the same kernels on the library's own scratch must
give the caller-workspace call's output bit for bit. Two calls in a row on the shared
scratch, the second with a smaller input, so the second runs over what the first left there;
and a shape whose workspace exceeds the scratch is refused before any work is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import rank_bit_residual_amd as R
from rank_bit_residual_amd import _lib
from workloads import smoothing_scale

pytestmark = pytest.mark.gpu

FMT = {"int": _lib.SVDQ_FMT_INT, "mx": _lib.SVDQ_FMT_MX}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(x, p):
    lib = _lib.load()
    y = torch.empty((x.shape[0], p.N), dtype=x.dtype, device=x.device)
    st = lib.svdq_linear_noalloc(ctypes.c_void_p(x.data_ptr()), x.shape[0], p.M, x.stride(0),
                                 ctypes.c_void_p(p.blob.data_ptr()), p.N, p.rank, FMT[p.fmt], p.bits,
                                 _lib.SVDQ_BF16 if x.dtype == torch.bfloat16 else _lib.SVDQ_F32,
                                 ctypes.c_void_p(y.data_ptr()), y.stride(0),
                                 ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream))
    _lib.check(st)
    return y


def _with_workspace(x, p):
    """svdq_linear with a caller workspace (filled with a non-zero pattern)."""
    lib = _lib.load()
    y = torch.empty((x.shape[0], p.N), dtype=x.dtype, device=x.device)
    wsb = R.workspace_bytes(x.shape[0], p)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=x.device)
    st = lib.svdq_linear(ctypes.c_void_p(x.data_ptr()), x.shape[0], p.M, x.stride(0),
                         ctypes.c_void_p(p.blob.data_ptr()), p.N, p.rank, FMT[p.fmt], p.bits,
                         _lib.SVDQ_BF16 if x.dtype == torch.bfloat16 else _lib.SVDQ_F32,
                         ctypes.c_void_p(y.data_ptr()), y.stride(0), ctypes.c_void_p(ws.data_ptr()), wsb,
                         ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream))
    _lib.check(st)
    return y


@pytest.mark.parametrize("fmt,bits,dtype,M,N,rank,B1,B2", [
    ("mx", 4, torch.bfloat16, 3072, 3072, 32, 2048, 16),   # large-batch kernel, then the decode kernel
    ("int", 4, torch.bfloat16, 4096, 1024, 32, 256, 40),   # max pre-pass + INT4 kernel, twice
    ("int", 8, torch.float32, 640, 300, 16, 300, 7),       # general kernel, float32 io
])
def test_noalloc_matches_workspace_call(fmt, bits, dtype, M, N, rank, B1, B2):
    dev = _dev()
    rng = np.random.default_rng(M + N + B1)
    x = rng.standard_t(3, (B1, M)).astype(np.float32)
    w = (0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)))
    w = w.astype(np.float32)
    s = smoothing_scale(x, w, 0.25)
    p = R.prepare(torch.from_numpy(w).to(dtype), torch.from_numpy(s), rank, bits, fmt, device=dev)
    xg = torch.from_numpy(x).to(dtype).to(dev)
    for B in (B1, B2):  # the second call is smaller and reuses the scratch the first wrote
        xb = xg[:B].contiguous()
        got = _noalloc(xb, p)
        want = _with_workspace(xb, p)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"B={B}: no-alloc output differs from svdq_linear"


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """An MXFP4 bf16 shape of 8192 x 8192 needs ~35 MB of workspace, above the 16 MiB scratch:
    EINVAL with a message naming the maximum, and nothing is launched."""
    _dev()
    lib = _lib.load()
    need = ctypes.c_size_t()
    _lib.check(lib.svdq_workspace_bytes(8192, 8192, 8192, 32, _lib.SVDQ_FMT_MX, 4, _lib.SVDQ_BF16,
                                        ctypes.byref(need)))
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.svdq_linear_noalloc(None, 8192, 8192, 8192, None, 8192, 32, _lib.SVDQ_FMT_MX, 4, _lib.SVDQ_BF16, None,
                                 8192, None)
    assert st == _lib.SVDQ_EINVAL
    assert "maximum" in lib.svdq_last_error().decode()
