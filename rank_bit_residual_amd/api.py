"""Python binding of libsvdq with the exercise page's function names.

"SVDQuant Smoothing, Low-rank and Residual Quantization" ("Functions / Return
requirements") defines smooth_inputs, split_weight, svdquant_linear and fake_quantize;
this module exposes them on GPU tensors (float32 or bfloat16), plus the prepared-weight
form of the operator (prepare + linear) that the per-call hot path uses.

Only argument marshalling happens here: validation that needs Python types (rank must be
an int), dtype/stride bookkeeping, output and workspace allocation through torch, and the
current HIP stream. Every arithmetic step runs in libsvdq (HIP kernels for device calls,
C++ for the one-time host preparation). There is no CPU fallback: device calls raise if
the library is not built or the tensors are not on a GPU.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.SVDQ_F32, torch.bfloat16: L.SVDQ_BF16, torch.float64: L.SVDQ_F64}
_FMT = {"int": L.SVDQ_FMT_INT, "mx": L.SVDQ_FMT_MX}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _fmt_code(fmt: str) -> int:
    if fmt not in _FMT:
        raise ValueError(f"fmt must be 'int' or 'mx', got {fmt!r}")
    return _FMT[fmt]


def _require_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected a torch.Tensor")
        if not t.is_cuda:
            raise RuntimeError("libsvdq device calls need tensors on an AMD GPU (HIP device)")


def _check_int(name: str, v) -> None:
    if isinstance(v, bool) or not isinstance(v, int):
        raise ValueError(f"{name} must be a Python int")


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _host_scale(scale: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(scale.detach().to("cpu", torch.float32).numpy())


def _device_scale(scale: torch.Tensor, device) -> torch.Tensor:
    return scale.detach().to(device=device, dtype=torch.float32).contiguous()


def _check_smoothing(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor) -> None:
    """_check_smoothing: nonempty x[B,M], weight[M,N], positive finite scale[M] (ValueError)."""
    if x.dim() != 2 or weight.dim() != 2 or scale.dim() != 1:
        raise ValueError("x and weight must be 2-D and scale 1-D")
    sh = _host_scale(scale)
    L.check(L.load().svdq_check_smoothing(x.shape[0], x.shape[1], weight.shape[0], scale.shape[0], weight.shape[1],
                                          sh.ctypes.data))


def _check_rank(weight: torch.Tensor, rank) -> None:
    """_check_rank: weight is a matrix and rank a Python int in [0, min(M, N)] (ValueError)."""
    if weight.dim() != 2:
        raise ValueError("weight must be a matrix")
    _check_int("rank", rank)
    L.check(L.load().svdq_check_rank(weight.shape[0], weight.shape[1], rank))


def _check_same(x: torch.Tensor, weight: torch.Tensor) -> None:
    if x.dtype != weight.dtype:
        raise ValueError("x and weight must share one dtype")
    if x.device != weight.device:
        raise ValueError("x and weight must be on the same device")


# ----------------------------------------------------------------------------- page functions
def smooth_inputs(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor):
    """Return (x / scale, scale[:, None] * weight) on the device, in the inputs' dtype."""
    _require_gpu(x, weight, scale)
    _check_same(x, weight)
    _check_smoothing(x, weight, scale)
    lib = L.load()
    B, M = x.shape
    N = weight.shape[1]
    s = _device_scale(scale, x.device)
    xs = torch.empty((B, M), dtype=x.dtype, device=x.device)
    ws = torch.empty((M, N), dtype=x.dtype, device=x.device)
    L.check(lib.svdq_smooth_inputs(_ptr(x), B, M, x.stride(0), x.stride(1), _ptr(weight), N, weight.stride(0),
                                   weight.stride(1), _ptr(s), _dtype_code(x), _ptr(xs), M, _ptr(ws), N, _stream(x)))
    return xs, ws


def calibrate_scale(x: torch.Tensor, weight: torch.Tensor, alpha: float) -> torch.Tensor:
    """Smoothing scale from a calibration batch on the device: float32 [M] with
    max|x[:,m]|^alpha / max|W[m,:]|^(1-alpha) (1 where a maximum is 0)."""
    _require_gpu(x, weight)
    _check_same(x, weight)
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[0]:
        raise ValueError("x [B,M] and weight [M,N] must share M")
    lib = L.load()
    xc = x if x.stride(1) == 1 else x.contiguous()
    wc = weight if weight.stride(1) == 1 else weight.contiguous()
    B, M = xc.shape
    N = wc.shape[1]
    wsb = ctypes.c_size_t()
    L.check(lib.svdq_calibrate_workspace_bytes(B, M, ctypes.byref(wsb)))
    work = torch.empty(wsb.value, dtype=torch.uint8, device=x.device)
    out = torch.empty(M, dtype=torch.float32, device=x.device)
    L.check(lib.svdq_calibrate_scale(_ptr(xc), B, M, xc.stride(0), _ptr(wc), N, wc.stride(0), _dtype_code(x),
                                     float(alpha), _ptr(out), _ptr(work), wsb.value, _stream(x)))
    return out


def split_weight(weight: torch.Tensor, rank: int):
    """Return (left [M,r], right [r,N], residual [M,N]) of the library's truncated SVD.

    The factorisation runs on the host (one-time preparation); results come back on the
    weight's device and in its dtype.
    """
    _check_rank(weight, rank)
    lib = L.load()
    M, N = weight.shape
    code = _dtype_code(weight)
    host = weight.detach().to("cpu").contiguous()
    left = torch.empty((M, rank), dtype=weight.dtype)
    right = torch.empty((rank, N), dtype=weight.dtype)
    res = torch.empty((M, N), dtype=weight.dtype)
    L.check(lib.svdq_split_weight(_ptr(host), M, N, N, code, rank, _ptr(left) if rank else None,
                                  _ptr(right) if rank else None, _ptr(res)))
    dev = weight.device
    return left.to(dev), right.to(dev), res.to(dev)


def fake_quantize(x: torch.Tensor, bits: int = 4) -> torch.Tensor:
    """Per-tensor symmetric INT quantise-dequantise of x (same shape, dtype and device)."""
    _require_gpu(x)
    _check_int("bits", bits)
    lib = L.load()
    shape = x.shape
    z = x if x.dim() == 2 else x.reshape(1, -1) if x.dim() <= 1 else x.reshape(-1, x.shape[-1])
    if z.numel() == 0:
        raise ValueError("empty input")
    rows, cols = z.shape
    out = torch.empty((rows, cols), dtype=x.dtype, device=x.device)
    wsb = lib.svdq_fake_quantize_workspace(rows, cols)
    work = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    L.check(lib.svdq_fake_quantize(_ptr(z), rows, cols, z.stride(0), z.stride(1), _dtype_code(x), bits, _ptr(out), cols,
                                   None, _ptr(work), wsb, _stream(x)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------- prepared operator
@dataclass
class Prepared:
    """Device copy of the prepared weights of one layer (see include/svdq.h) and its shape."""

    blob: torch.Tensor
    M: int
    N: int
    rank: int
    fmt: str
    bits: int
    dtype: torch.dtype
    offsets: tuple
    left: torch.Tensor | None = None  # exact factors and residual the blob was built from (host)
    right: torch.Tensor | None = None
    residual: torch.Tensor | None = None

    def section(self, sec: int) -> torch.Tensor:
        return self.blob[self.offsets[sec]:self.offsets[sec + 1]]


def prepared_layout(M: int, N: int, rank: int, fmt: str = "int", bits: int = 4, dtype=torch.bfloat16) -> tuple:
    off = (ctypes.c_int64 * L.NSEC)()
    L.check(L.load().svdq_prepared_layout(M, N, rank, _fmt_code(fmt), bits, _DT[dtype], off))
    return tuple(int(v) for v in off)


def prepare(weight: torch.Tensor, scale: torch.Tensor, rank: int, bits: int = 4, fmt: str = "int",
            device=None, keep_factors: bool = False, layout: str = "mn", svd_on_gpu: bool = False,
            x_global_scale: float | None = None) -> Prepared:
    """One-time preparation: fold scale into W, split, quantise and pack the residual (host),
    then copy the blob to ``device`` (default: the weight's device, which must be a GPU).

    ``layout="mn"`` takes W as [M, N] (input by output channels); ``layout="nm"`` takes a
    Linear-layout weight [N, M] (output by input channels, i.e. W transposed) without a copy
    into the other orientation; both give the same blob. ``svd_on_gpu`` runs the truncated
    SVD's large products on ``device`` (layout "mn" only). ``x_global_scale`` (MXFP4, layout
    "mn", host SVD) selects two-level scaling: the activations are quantised as
    RN(X^ * x_global_scale), the residual with its own global scale, and alpha applies once
    in the GEMM epilogue (svdq_prepare_two_level)."""
    if layout not in ("mn", "nm"):
        raise ValueError('layout must be "mn" ([M, N]) or "nm" (Linear layout [N, M])')
    if weight.dim() != 2 or scale.dim() != 1:
        raise ValueError("weight must be 2-D and scale 1-D")
    M, N = weight.shape if layout == "mn" else (weight.shape[1], weight.shape[0])
    if scale.shape[0] != M:
        raise ValueError("scale must have one entry per input channel")
    _check_rank(weight, rank)
    _check_int("bits", bits)
    lib = L.load()
    code = _dtype_code(weight)
    offs = prepared_layout(M, N, rank, fmt, bits, weight.dtype)  # raises for float64
    host_w = weight.detach().to("cpu").contiguous()
    host_s = torch.from_numpy(_host_scale(scale))
    blob = torch.empty(offs[L.SEC_END], dtype=torch.uint8)
    left = right = res = None
    if keep_factors:
        left = torch.empty((M, rank), dtype=weight.dtype)
        right = torch.empty((rank, N), dtype=weight.dtype)
        res = torch.empty((M, N), dtype=weight.dtype)
    dev = weight.device if device is None else torch.device(device)
    outs = (_ptr(left) if keep_factors and rank else None, _ptr(right) if keep_factors and rank else None, _ptr(res))
    if x_global_scale is not None:
        if fmt != "mx" or layout != "mn" or svd_on_gpu:
            raise ValueError("x_global_scale (two-level scaling) needs fmt 'mx', layout 'mn' and the host SVD")
        L.check(lib.svdq_prepare_two_level(_ptr(host_w), M, N, N, _ptr(host_s), rank, float(x_global_scale), code,
                                           _ptr(blob), *outs))
    elif svd_on_gpu:
        if layout != "mn" or dev.type != "cuda":
            raise ValueError("svd_on_gpu needs layout 'mn' and a GPU device")
        need = ctypes.c_size_t()
        L.check(lib.svdq_prepare_gpu_workspace_bytes(M, N, rank, ctypes.byref(need)))
        work = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)
        L.check(lib.svdq_prepare_gpu(_ptr(host_w), M, N, N, _ptr(host_s), rank, _fmt_code(fmt), bits, code,
                                     _ptr(blob), *outs, _ptr(work), need.value, ctypes.c_void_p(stream.cuda_stream)))
        del work
    else:
        fn, ld = (lib.svdq_prepare, N) if layout == "mn" else (lib.svdq_prepare_linear, M)
        a, b = (M, N) if layout == "mn" else (N, M)
        L.check(fn(_ptr(host_w), a, b, ld, _ptr(host_s), rank, _fmt_code(fmt), bits, code, _ptr(blob), *outs))
    # a host blob is only for inspection; linear() needs it on the GPU
    return Prepared(blob.to(dev), M, N, rank, fmt, bits, weight.dtype, offs, left, right, res)


def workspace_bytes(B: int, prep: Prepared) -> int:
    out = ctypes.c_size_t()
    L.check(L.load().svdq_workspace_bytes(B, prep.M, prep.N, prep.rank, _fmt_code(prep.fmt), prep.bits,
                                          _DT[prep.dtype], ctypes.byref(out)))
    return int(out.value)


def linear(x: torch.Tensor, prep: Prepared, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, bias: torch.Tensor | None = None) -> torch.Tensor:
    """The per-call operator Y = (X^ L1) L2 + Q(X^) Q(R) (+ bias[N]) on prepared weights
    (with two-level MXFP4 weights: Y = alpha (Q(X^ g_x) Q(R g_R) + (X^ L1) L2 / alpha) (+ bias))."""
    _require_gpu(x, prep.blob)
    if prep.blob.device != x.device:
        raise ValueError("x and the prepared weights must be on the same device")
    if x.dim() != 2 or x.shape[1] != prep.M:
        raise ValueError(f"x must be [B, {prep.M}]")
    if x.dtype != prep.dtype:
        raise ValueError("x must have the prepared weights' dtype")
    if x.stride(1) != 1:
        x = x.contiguous()
    B = x.shape[0]
    if out is None:
        out = torch.empty((B, prep.N), dtype=x.dtype, device=x.device)
    wsb = workspace_bytes(B, prep)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    if bias is not None:
        if bias.dim() != 1 or bias.shape[0] != prep.N or bias.dtype != x.dtype or bias.device != x.device:
            raise ValueError(f"bias must be a [{prep.N}] tensor with x's dtype and device")
        bias = bias.contiguous()
    L.check(L.load().svdq_linear_bias(_ptr(x), B, prep.M, x.stride(0), _ptr(prep.blob), prep.N, prep.rank,
                                      _fmt_code(prep.fmt), prep.bits, _DT[prep.dtype],
                                      _ptr(bias) if bias is not None else None, _ptr(out), out.stride(0),
                                      _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def svdquant_linear(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor, rank: int, bits: int = 4,
                    fmt: str = "int") -> torch.Tensor:
    """Smooth, split the smoothed weight, and return (X^ L1) L2 + Q(X^) Q(R) as one [B, N] tensor."""
    _require_gpu(x, weight, scale)
    _check_same(x, weight)
    _check_smoothing(x, weight, scale)
    return linear(x, prepare(weight, scale, rank, bits, fmt))


def quantize_activations(x: torch.Tensor, scale: torch.Tensor, fmt: str = "int", bits: int = 4):
    """Step (a) alone: codes [B, padded bytes] (uint8), MX scales [B, Kp/32] (uint8) and s_x."""
    _require_gpu(x, scale)
    _check_int("bits", bits)
    lib = L.load()
    if x.stride(1) != 1:
        x = x.contiguous()
    B, M = x.shape
    code = _dtype_code(x)
    Kp = -(-M // 256) * 256
    nib = fmt == "mx" or bits <= 4
    codes = torch.empty((B, Kp // 2 if nib else Kp), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, Kp // 32), dtype=torch.uint8, device=x.device) if fmt == "mx" else None
    sx = torch.empty(1, dtype=torch.float32, device=x.device)
    wsb = ctypes.c_size_t()
    L.check(lib.svdq_workspace_bytes(B, M, 1, 0, _fmt_code(fmt), bits, code, ctypes.byref(wsb)))
    work = torch.empty(wsb.value, dtype=torch.uint8, device=x.device)
    s = _device_scale(scale, x.device)
    L.check(lib.svdq_quantize_activations(_ptr(x), B, M, x.stride(0), _ptr(s), _fmt_code(fmt), bits, code,
                                          _ptr(codes), codes.stride(0), _ptr(scales),
                                          scales.stride(0) if scales is not None else 0, _ptr(sx), _ptr(work),
                                          wsb.value, _stream(x)))
    return codes, scales, sx
