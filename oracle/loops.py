"""Second, loop-based oracle for tiny inputs — test infrastructure only.

Pure Python (lists of floats, ``struct`` for binary32 rounding), written
independently of ``oracle.svdquant`` so the two can check each other. It
follows the same page definitions:
  "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and
  conventions" items 1 and 3 (smoothing, per-tensor INT fake quantisation,
  the two-branch output), and the MXFP4 per-block minmax quantiser of the
  msModelSlim SVDQuant guide, step 2.

The MX helpers here are brute force on purpose: the shared exponent is found by
scanning every E8M0 value and the E2M1 code by trying all 16 codes.

Binary32 arithmetic: a float64 quotient or product of two binary32 values,
rounded once to binary32, equals the correctly rounded binary32 result (float64
has more than 2*24+2 significand bits), so f32(a / b) below is IEEE division.
"""
from __future__ import annotations

import math
import struct

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(v: float) -> float:
    """Round a Python float to the nearest binary32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16(v: float) -> float:
    """Round to bfloat16 through the binary32 bit pattern (input already binary32)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    upper, lower = u >> 16, u & 0xFFFF
    if lower > 0x8000 or (lower == 0x8000 and (upper & 1)):
        upper += 1
    return struct.unpack("<f", struct.pack("<I", (upper & 0xFFFF) << 16))[0]


def store(v: float, dtype: str) -> float:
    return f32(v) if dtype == "f32" else bf16(f32(v))


def rint_even(v: float) -> int:
    """Round half to even, written out."""
    fl = int(v // 1)
    frac = v - fl
    if frac > 0.5:
        return fl + 1
    if frac < 0.5:
        return fl
    return fl if fl % 2 == 0 else fl + 1


def smooth(x, scale, dtype):
    return [[store(f32(x[b][m]) / f32(scale[m]), dtype) for m in range(len(scale))] for b in range(len(x))]


def int_quantize(z, bits):
    """Per-tensor symmetric codes and scale of a list-of-lists z (binary32 arithmetic)."""
    qmax = 2 ** (bits - 1) - 1
    a = 0.0
    for row in z:
        for v in row:
            a = max(a, abs(v))
    if a == 0.0:
        return [[0] * len(row) for row in z], 0.0
    s = f32(a / qmax)
    codes = [[max(-qmax, min(qmax, rint_even(f32(v / s)))) for v in row] for row in z]
    return codes, s


def mx_exponent_bruteforce(amax: float) -> int:
    """Smallest e in [-127, 127] with amax <= 6 * 2^e; -127 when none is smaller."""
    for e in range(-127, 128):
        if amax <= 6.0 * 2.0 ** e:
            return e
    return 127


def e2m1_bruteforce(v: float, sign_negative: bool) -> int:
    """Code (0..15) whose value is nearest to v; among equally near codes the even one.
    The sign bit follows the sign of the input (including -0.0)."""
    best, best_d = None, None
    for code in range(16):
        mag = E2M1[code & 7]
        val = -mag if code & 8 else mag
        if (code & 8) != (8 if sign_negative else 0):
            continue  # the sign bit is fixed by the input's sign
        d = abs(val - v)
        if best_d is None or d < best_d or (d == best_d and (code & 7) % 2 == 0 and (best & 7) % 2 == 1):
            best, best_d = code, d
    return best


def mx_quantize_row(row, block=32):
    """MXFP4 codes and scale bytes of one row, blocks along the row."""
    codes, sbytes = [], []
    for j in range(0, len(row), block):
        blk = row[j:j + block]
        e = mx_exponent_bruteforce(max(abs(v) for v in blk))
        sbytes.append(e + 127)
        for v in blk:
            neg = struct.unpack("<I", struct.pack("<f", v))[0] >> 31 == 1
            codes.append(e2m1_bruteforce(v * 2.0 ** (-e), neg))
    return codes, sbytes


def mx_value(code: int, sbyte: int) -> float:
    mag = E2M1[code & 7] * 2.0 ** (sbyte - 127)
    return -mag if code & 8 else mag


def forward(x, scale, left, right, residual, fmt, bits, dtype):
    """Y = (X^ L1) L2 + Q(X^) Q(R) with loops; returns (Y, activation codes, weight codes)."""
    B, M, N = len(x), len(scale), len(residual[0])
    r = len(right)
    xs = smooth(x, scale, dtype)
    down = [[sum(xs[b][m] * left[m][j] for m in range(M)) for j in range(r)] for b in range(B)]
    low = [[sum(down[b][j] * right[j][n] for j in range(r)) for n in range(N)] for b in range(B)]
    if fmt == "int":
        cx, sx = int_quantize(xs, bits)
        cr, sr = int_quantize(residual, bits)
        res = [[sx * sr * sum(cx[b][m] * cr[m][n] for m in range(M)) for n in range(N)] for b in range(B)]
        act, wgt = (cx, sx), (cr, sr)
    else:
        act_rows = [mx_quantize_row(xs[b]) for b in range(B)]
        wgt_cols = [mx_quantize_row([residual[m][n] for m in range(M)]) for n in range(N)]
        res = [[sum(mx_value(act_rows[b][0][m], act_rows[b][1][m // 32]) *
                    mx_value(wgt_cols[n][0][m], wgt_cols[n][1][m // 32]) for m in range(M))
                for n in range(N)] for b in range(B)]
        act, wgt = act_rows, wgt_cols
    y = [[low[b][n] + res[b][n] for n in range(N)] for b in range(B)]
    return y, act, wgt


def calibrate_scale(x, weight, alpha):
    """Brute force of the calibrated smoothing scale: column maxima of |x| and row maxima of
    |W| by plain loops, then max|x|^alpha / max|W|^(1-alpha) with math.pow, rounded to f32;
    1 where a maximum is 0."""
    B, M = len(x), len(x[0])
    N = len(weight[0])
    out = []
    for m in range(M):
        ax = 0.0
        for b in range(B):
            ax = max(ax, abs(float(x[b][m])))
        aw = 0.0
        for n in range(N):
            aw = max(aw, abs(float(weight[m][n])))
        out.append(1.0 if ax == 0.0 or aw == 0.0 else f32(math.pow(ax, alpha) / math.pow(aw, 1.0 - alpha)))
    return out
