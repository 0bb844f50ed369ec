"""Numpy oracle for the SVDQuant linear operator — test infrastructure only.

Sources (cited by page title and section):
  [P1] "SVDQuant Smoothing, Low-rank and Residual Quantization" (paperleet exercise),
       sections "Functions / Return requirements" and "Formula and conventions".
  [P4] "SVDQuant 参数配置流程指南" (msModelSlim SVDQuant usage guide), step 2
       (recommended YAML: MXFP4, per_block, symmetric, minmax for act and weight).
  [P5] "Contraction-Gauge Preconditioning for Quantized Matrix Multiplication",
       abstract: the product identity AB = (AT)(T^-1 B).
  [P2] "flashinfer.gemm.svdquant_linear" (API page): the activation global scale, the
       per-tensor residual dequantisation scale alpha and the up-projection factor
       prepared divided by alpha (its l1_scaled parameter).

Precision conventions (readings where the pages are silent; each one is listed
in the design notes):
  * elementwise steps run in IEEE binary32 with subnormals, no contraction
    (numpy float32 ops), or binary64 for float64 inputs;
  * bf16 is a storage type: values are upcast exactly to float32, the step runs
    in float32, the result is rounded once (RNE) to bf16;
  * reference products and sums run in float64.

Every function here is a plain transcription of a definition; nothing is
blocked, fused or reordered. Tensors are numpy arrays; bf16 tensors are float32
arrays holding bf16-representable values.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

DTYPES = ("f32", "bf16", "f64")
MX_BLOCK = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# --------------------------------------------------------------------------- dtype rounding
def round_to_format(v, mant_bits: int, emin: int) -> np.ndarray:
    """Round float64 values to a binary format with ``mant_bits`` fraction bits and
    minimum normal exponent ``emin`` (round half to even, gradual underflow).

    The spacing of representable numbers around v is 2^(max(floor(log2|v|), emin) - mant_bits);
    v / spacing is an exact power-of-two rescaling, so rint() performs the one rounding.
    Overflow is not handled (inputs are finite and far from the format's maximum).
    """
    v = np.asarray(v, dtype=np.float64)
    _, E = np.frexp(v)  # v = f * 2^E with 0.5 <= |f| < 1, so floor(log2|v|) = E - 1
    e = np.maximum(E - 1, emin)
    q = np.ldexp(np.ones_like(v), e - mant_bits)
    return np.rint(v / q) * q


def to_dtype(v, dtype: str) -> np.ndarray:
    """D(.): round to the storage dtype ("f32" or "bf16" -> float32 array, "f64" -> float64)."""
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return round_to_format(v, 7, -126).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _work(dtype: str):
    """Arithmetic type of elementwise steps: float64 for f64 tensors, float32 otherwise."""
    return np.float64 if dtype == "f64" else np.float32


# --------------------------------------------------------------------------- validation
def check_smoothing(x, weight, scale) -> None:
    """[P1] _check_smoothing: nonempty x[B,M], weight[M,N], positive finite scale[M]."""
    x, weight, scale = np.asarray(x), np.asarray(weight), np.asarray(scale)
    if x.ndim != 2 or weight.ndim != 2 or scale.ndim != 1:
        raise ValueError("x and weight must be 2-D and scale 1-D")
    if x.size == 0 or weight.size == 0 or scale.size == 0:
        raise ValueError("empty input")
    if not (x.shape[1] == weight.shape[0] == scale.shape[0]):
        raise ValueError("input-channel sizes of x, weight and scale differ")
    s = scale.astype(np.float64)
    if not np.all(np.isfinite(s)) or not np.all(s > 0):
        raise ValueError("scale must be positive and finite")


def check_rank(weight, rank) -> None:
    """[P1] _check_rank: weight is a matrix and rank a Python int in [0, min(M, N)]."""
    weight = np.asarray(weight)
    if weight.ndim != 2:
        raise ValueError("weight must be a matrix")
    if isinstance(rank, bool) or not isinstance(rank, int):
        raise ValueError("rank must be a Python int")
    if rank < 0 or rank > min(weight.shape):
        raise ValueError("rank out of range")


def check_bits(bits) -> None:
    """[P1] "Formula and conventions" item 3: 2 <= bits <= 8."""
    if isinstance(bits, bool) or not isinstance(bits, int) or not 2 <= bits <= 8:
        raise ValueError("bits must be an int in [2, 8]")


# --------------------------------------------------------------------------- smoothing
def smooth_activations(x, scale, dtype: str) -> np.ndarray:
    """Activation half of [P1] smooth_inputs: xs = D(x / scale[None, :])."""
    w = _work(dtype)
    return to_dtype(np.asarray(x, w) / np.asarray(scale, w)[None, :], dtype)


def smooth_weight(weight, scale, dtype: str) -> np.ndarray:
    """Weight half of [P1] smooth_inputs: ws = D(scale[:, None] * weight)."""
    w = _work(dtype)
    return to_dtype(np.asarray(scale, w)[:, None] * np.asarray(weight, w), dtype)


def smooth_inputs(x, weight, scale, dtype: str):
    """[P1] smooth_inputs / "Formula and conventions" item 1: (x/scale, scale[:,None]*weight).

    Moving the per-channel factor from x into W leaves the product unchanged
    ([P5]'s identity with T = diag(1/scale)).
    """
    check_smoothing(x, weight, scale)
    return smooth_activations(x, scale, dtype), smooth_weight(weight, scale, dtype)


# --------------------------------------------------------------------------- low-rank split
def residual_of(weight, left, right, dtype: str) -> np.ndarray:
    """R = D(weight - left @ right), the product taken in float64 from the stored factors."""
    w64 = np.asarray(weight, np.float64)
    prod = np.asarray(left, np.float64) @ np.asarray(right, np.float64)
    return to_dtype(w64 - prod, dtype)


def split_weight(weight, rank: int, dtype: str):
    """[P1] split_weight / "Formula and conventions" item 2.

    Truncated SVD in float64: left = D(U_r diag(sigma_r)), right = D(V_r^T),
    residual = D(weight - left @ right). rank 0 gives [M,0] and [0,N] factors
    and the weight itself as residual.
    """
    check_rank(weight, rank)
    w64 = np.asarray(weight, np.float64)
    M, N = w64.shape
    if rank == 0:
        left = np.zeros((M, 0), np.float64)
        right = np.zeros((0, N), np.float64)
    else:
        U, s, Vt = np.linalg.svd(w64, full_matrices=False)
        left = U[:, :rank] * s[:rank]
        right = Vt[:rank]
    left = to_dtype(left, dtype)
    right = to_dtype(right, dtype)
    return left, right, residual_of(weight, left, right, dtype)


# --------------------------------------------------------------------------- per-tensor INT
def quantize_int(z, bits: int, dtype: str = "f32"):
    """[P1] fake_quantize rule: one symmetric scale for the whole tensor.

    qmax = 2^(bits-1) - 1, s = max|z| / qmax, codes = clamp(round_half_even(z / s), -qmax, qmax).
    Divisions are IEEE in the working precision. An all-zero tensor gives s = 0
    and zero codes. Returns (codes int32, s).
    """
    check_bits(bits)
    w = _work(dtype)
    qmax = 2 ** (bits - 1) - 1
    z = np.asarray(z, w)
    a = np.max(np.abs(z)) if z.size else w(0)
    if a == 0:
        return np.zeros(z.shape, np.int32), w(0)
    s = w(a) / w(qmax)
    codes = np.clip(np.rint(z / s), -qmax, qmax).astype(np.int32)
    return codes, w(s)


def fake_quantize(z, bits: int, dtype: str) -> np.ndarray:
    """[P1] fake_quantize: dequantised values D(s * codes), same shape as z."""
    codes, s = quantize_int(z, bits, dtype)
    w = _work(dtype)
    return to_dtype(w(s) * codes.astype(w), dtype)


# --------------------------------------------------------------------------- per-block MXFP4
def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent of an MXFP4 block from its max magnitude (minmax, [P4] step 2).

    e is the smallest integer with amax <= 6 * 2^e (6 = largest E2M1 magnitude), so the
    block maximum never saturates; e is clamped to the E8M0 range [-127, 127] and an
    all-zero block takes -127.  With amax = f * 2^E (0.5 <= f < 1): 6 * 2^(E-4) < amax < 6 * 2^(E-2),
    so the answer is E-3 when amax <= 6 * 2^(E-3) and E-2 otherwise.
    """
    a = np.asarray(amax, np.float64)
    _, E = np.frexp(a)
    e = np.where(a <= 6.0 * np.ldexp(1.0, E - 3), E - 3, E - 2)
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def e2m1_code(v) -> np.ndarray:
    """4-bit E2M1 code of v: magnitude rounded to the nearest of {0,.5,1,1.5,2,3,4,6}
    (codes 0..7), a tie going to the even code; bit 3 = sign bit of v (so -0 -> 8).
    Magnitudes above 6 take code 7."""
    v = np.asarray(v, np.float64)
    d = np.abs(np.abs(v)[..., None] - E2M1_GRID)  # distance to each grid point
    is_min = d == d.min(axis=-1, keepdims=True)
    even_min = is_min & (np.arange(8) % 2 == 0)
    idx = np.where(even_min.any(axis=-1), np.argmax(even_min, axis=-1), np.argmax(is_min, axis=-1))
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def quantize_mx(z, block: int = MX_BLOCK):
    """MXFP4 quantisation of z[rows, K] along K in blocks of ``block`` (the last one may be short).

    Per block: e from the block max (mx_block_exponent), v = z * 2^-e (exact), code = e2m1_code(v).
    Returns (codes uint8 [rows, K] in 0..15, scale bytes uint8 [rows, ceil(K/block)] = e + 127).
    """
    z = np.asarray(z, np.float64)
    rows, K = z.shape
    nb = -(-K // block)
    codes = np.zeros((rows, K), np.uint8)
    sbytes = np.zeros((rows, nb), np.uint8)
    for j in range(nb):
        blk = z[:, j * block:(j + 1) * block]
        e = mx_block_exponent(np.max(np.abs(blk), axis=1))
        v = blk * np.ldexp(1.0, -e)[:, None]
        codes[:, j * block:(j + 1) * block] = e2m1_code(v)
        sbytes[:, j] = (e + 127).astype(np.uint8)
    return codes, sbytes


def dequant_mx(codes, sbytes, block: int = MX_BLOCK) -> np.ndarray:
    """Exact float64 values of MXFP4 codes: grid[code & 7] * (-1)^bit3 * 2^(byte - 127)."""
    codes = np.asarray(codes)
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    e = np.repeat(np.asarray(sbytes, np.int64) - 127, block, axis=1)[:, : codes.shape[1]]
    return val * np.ldexp(1.0, e)


# --------------------------------------------------------------------------- packed layouts
def pack_nibbles(codes4) -> np.ndarray:
    """Pack 4-bit codes [rows, K] two per byte, even k in the low nibble: [rows, ceil(K/2)]."""
    c = np.asarray(codes4).astype(np.uint8) & 0xF
    rows, K = c.shape
    if K % 2:
        c = np.concatenate([c, np.zeros((rows, 1), np.uint8)], axis=1)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def pack_int_codes(codes, bits: int) -> np.ndarray:
    """Canonical INT code layout: 4-bit two's-complement nibbles for bits <= 4, else int8 bytes."""
    codes = np.asarray(codes, np.int64)
    if bits <= 4:
        return pack_nibbles(codes & 0xF)
    return codes.astype(np.int8).view(np.uint8)


# --------------------------------------------------------------------------- the operator
def forward_ref(x, scale, left, right, residual, fmt: str, bits: int, dtype: str, bias=None,
                x_global_scale=None) -> np.ndarray:
    """[P1] "Formula and conventions" item 3, Y = (X^ L1) L2 + Q(X^) Q(R), in float64, plus an
    optional per-output-channel bias [N] (the GPU library page's optional bias parameter).

    X^ = D(x/scale). The low-rank branch uses the unquantised X^ and the stored
    factors; only R is quantised on the weight side. fmt "int": per-tensor INT
    (s_x * s_R * integer product, exact); fmt "mx": MXFP4 along K for X^ rows and
    R columns ([P4] per_block), the product of exactly dequantised values.

    ``x_global_scale`` (fmt "mx" only) selects two-level scaling, [P2]'s chain: see
    forward_two_level.
    """
    if x_global_scale is not None:
        if fmt != "mx":
            raise ValueError("two-level scaling is an MXFP4 scheme")
        return forward_two_level(x, scale, left, right, residual, dtype, x_global_scale, bias)
    xs = smooth_activations(x, scale, dtype)
    low = (np.asarray(xs, np.float64) @ np.asarray(left, np.float64)) @ np.asarray(right, np.float64)
    if fmt == "int":
        cx, sx = quantize_int(xs, bits, dtype)
        cr, sr = quantize_int(residual, bits, dtype)
        res = float(sx) * float(sr) * (cx.astype(np.float64) @ cr.astype(np.float64))
    elif fmt == "mx":
        if bits != 4:
            raise ValueError("MXFP4 uses 4-bit codes")
        cx, bx = quantize_mx(xs)
        cr, br = quantize_mx(np.asarray(residual).T)
        res = dequant_mx(cx, bx) @ dequant_mx(cr, br).T
    else:
        raise ValueError(f"unknown format {fmt!r}")
    y = low + res
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


# --------------------------------------------------------------------------- two-level MXFP4 scaling
def two_level_residual_scale(residual) -> np.float32:
    """Residual global scale g_R (a reading: [P2] names a per-tensor residual dequantisation
    scale but not how it is chosen). With max|R| / 6 in [2^(ex-1), 2^ex), g_R is
    6 * 2^ex / max|R| rounded once to binary32, so g_R lies in (1, 2] and the largest
    |R * g_R| sits at 6 * 2^ex: the top E2M1 value at its block's scale. An all-zero R
    takes g_R = 1.

    ex comes from exact rational comparisons; float(Fraction) rounds the exact quotient to
    binary64 and the second rounding to binary32 cannot differ from a direct one, since a
    quotient of two 24-bit significands rounded to 53 bits and then to 24 is correctly
    rounded (Figueroa's double-rounding condition 53 >= 2 * 24 + 2).
    """
    r = np.asarray(residual, np.float64)
    a = Fraction(float(np.max(np.abs(r)))) if r.size else Fraction(0)
    if a == 0:
        return np.float32(1.0)
    q = a / 6
    ex = 0
    while Fraction(2) ** ex <= q:
        ex += 1
    while Fraction(2) ** (ex - 1) > q:
        ex -= 1
    return np.float32(float(6 * Fraction(2) ** ex / a))


def two_level_alpha(x_global_scale, g_resid) -> np.float32:
    """[P2] alpha, the per-tensor dequantisation scale of the quantised product: the
    reciprocal of g_x * g_R, taken in binary64 (the product of two binary32 numbers is exact
    there) and rounded once to binary32 (a reading: the page leaves the rounding open)."""
    return np.float32(1.0 / (float(np.float32(x_global_scale)) * float(np.float32(g_resid))))


def forward_two_level(x, scale, left, right, residual, dtype: str, x_global_scale, bias=None) -> np.ndarray:
    """[P2] svdquant_linear's three steps with MXFP4 in place of NVFP4, in float64:

      1. X^ = D(x/scale), z_x = RN_f32(X^ * g_x), MXFP4 codes of z_x along K;
      2. down = X^ L1 (the unquantised low-rank input);
      3. Y = alpha * (Q(z_x) Q(z_R) + down * D(L2 / alpha)) [+ bias],

    where z_R = RN_f32(R * g_R) is quantised per column of R along K, g_R and alpha are as in
    two_level_residual_scale and two_level_alpha, and D(L2 / alpha) is the up-projection
    factor divided by alpha and rounded to the storage dtype, as [P2] prepares l1_scaled.
    Both products are sums of exactly dequantised values taken in float64.
    """
    if dtype == "f64":
        raise ValueError("two-level scaling quantises binary32 products; use f32 or bf16")
    gx = np.float32(x_global_scale)
    gr = two_level_residual_scale(residual)
    alpha = two_level_alpha(gx, gr)
    xs = smooth_activations(x, scale, dtype)
    zx = np.asarray(xs, np.float32) * gx
    zr = np.asarray(residual, np.float32) * gr
    cx, bx = quantize_mx(zx)
    cr, br = quantize_mx(zr.T)
    acc = dequant_mx(cx, bx) @ dequant_mx(cr, br).T
    down = np.asarray(xs, np.float64) @ np.asarray(left, np.float64)
    up = np.asarray(to_dtype(np.asarray(right, np.float64) / float(alpha), dtype), np.float64)
    y = float(alpha) * (acc + down @ up)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def svdquant_linear(x, weight, scale, rank: int, bits: int = 4):
    """[P1] svdquant_linear on float32/float64 inputs: smooth, split the smoothed weight,
    Y = (X^ L1) L2 + fake_quantize(X^) @ fake_quantize(R), returned in the input dtype."""
    x = np.asarray(x)
    dtype = "f64" if x.dtype == np.float64 else "f32"
    check_smoothing(x, weight, scale)
    check_rank(weight, rank)
    check_bits(bits)
    xs, ws = smooth_inputs(x, weight, scale, dtype)
    left, right, res = split_weight(ws, rank, dtype)
    qx = np.asarray(fake_quantize(xs, bits, dtype), np.float64)
    qr = np.asarray(fake_quantize(res, bits, dtype), np.float64)
    y = (np.asarray(xs, np.float64) @ np.asarray(left, np.float64)) @ np.asarray(right, np.float64) + qx @ qr
    return to_dtype(y, dtype)


# --------------------------------------------------------------------------- scale calibration
def calibrate_scale(x, weight, alpha: float) -> np.ndarray:
    """Per-input-channel smoothing scale from a calibration batch, the step before the path:
    s[m] = max_b |x[b,m]|^alpha / max_n |W[m,n]|^(1 - alpha), evaluated in float64 and
    rounded once to float32, with s[m] = 1 where either maximum is 0 (so the scale stays a
    valid positive divisor). [P4] step 2 names the migration strength iter_smooth.alpha
    (0.25 in its diffusion example); the closed form is the reading of the design notes (R16),
    the same one the synthetic workloads use for their input scales.

    x: [B, M] calibration activations, weight: [M, N]; alpha in [0, 1]."""
    x = np.asarray(x)
    weight = np.asarray(weight)
    if x.ndim != 2 or weight.ndim != 2 or x.shape[1] != weight.shape[0] or x.size == 0 or weight.size == 0:
        raise ValueError("x [B,M] and weight [M,N] must be nonempty with matching M")
    if not (0.0 <= alpha <= 1.0):
        raise ValueError("alpha must be in [0, 1]")
    ax = np.max(np.abs(x.astype(np.float64)), axis=0)
    aw = np.max(np.abs(weight.astype(np.float64)), axis=1)
    s = np.ones(x.shape[1], np.float64)
    ok = (ax > 0) & (aw > 0)
    s[ok] = np.power(ax[ok], alpha) / np.power(aw[ok], 1.0 - alpha)
    return s.astype(np.float32)


def rel_fro(y, ref) -> float:
    """Relative Frobenius error ||y - ref||_F / ||ref||_F (float64)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))
