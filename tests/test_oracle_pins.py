"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value worked
by hand from a page's rule (tests/golden), a closed form (Eckart-Young), an
invariant (product identity, scaling and sign symmetry), a library routine
(numpy/torch casts, eigvalsh) or brute force (tests against oracle.loops).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import loops
from oracle import svdquant as O
from workloads import WORKLOADS, make_inputs


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- dtype rounding
def test_bf16_rounding_matches_torch_cast():
    rng = _rng(1)
    v = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32)
    # exact ties: a bf16 value plus half of its spacing
    base = torch.from_numpy(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    half = np.abs(base) * np.float32(2.0**-8)
    ties = np.concatenate([base + half, base - half, np.array([0.0, -0.0, 1e-40, -1e-40], np.float32)])
    for arr in (v, ties.astype(np.float32)):
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float32).numpy()
        got = O.to_dtype(arr, "bf16")
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_round_to_format_f32_matches_numpy_cast():
    rng = _rng(2)
    v = rng.standard_normal(50000) * 10.0 ** rng.integers(-45, 38, 50000)
    v = np.concatenate([v, [0.0, -0.0, 2.0**-149, 3 * 2.0**-150, 1 + 2.0**-24, 1 + 3 * 2.0**-24]])
    assert np.array_equal(O.round_to_format(v, 23, -126).astype(np.float32).view(np.uint32),
                          v.astype(np.float32).view(np.uint32))


# ----------------------------------------------------------------------------- smoothing
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_smoothing_preserves_product(dtype):
    x, w, s = make_inputs(1)
    if dtype == "f64":
        x, w, s = x.astype(np.float64), w.astype(np.float64), s.astype(np.float64)
    xs, ws = O.smooth_inputs(x, w, s, dtype)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    got = xs.astype(np.float64) @ ws.astype(np.float64)
    assert O.rel_fro(got, ref) <= (1e-6 if dtype == "f32" else 1e-14)
    # the activation side is divided, not multiplied: outlier columns shrink
    big = np.argmax(np.abs(x).max(0))
    assert np.abs(xs[:, big]).max() < np.abs(x[:, big]).max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_smoothing_power_of_two_scales_exact(dtype):
    rng = _rng(3)
    x = O.to_dtype(rng.standard_normal((8, 40)), dtype)
    w = O.to_dtype(rng.standard_normal((40, 24)), dtype)
    s = np.ldexp(1.0, rng.integers(-6, 7, 40)).astype(np.float32)
    xs, ws = O.smooth_inputs(x, w, s, dtype)
    assert np.array_equal(xs * s[None, :], x)
    assert np.array_equal(ws / s[:, None], w)
    assert np.array_equal(xs.astype(np.float64) @ ws.astype(np.float64), x.astype(np.float64) @ w.astype(np.float64))


def test_smoothing_leaves_inputs_unchanged_and_keeps_dtype():
    x, w, s = make_inputs(1)
    xc, wc, sc = x.copy(), w.copy(), s.copy()
    xs, ws = O.smooth_inputs(x, w, s, "f32")
    assert xs.dtype == np.float32 and ws.dtype == np.float32
    assert xs.shape == x.shape and ws.shape == w.shape
    assert np.array_equal(x, xc) and np.array_equal(w, wc) and np.array_equal(s, sc)


@pytest.mark.parametrize("case", [
    lambda x, w, s: (x[0], w, s),                       # x not 2-D
    lambda x, w, s: (x, w[:, 0], s),                    # weight not 2-D
    lambda x, w, s: (x, w, s[None]),                    # scale not 1-D
    lambda x, w, s: (x[:, :0], w[:0], s[:0]),           # empty
    lambda x, w, s: (x[:, 1:], w, s),                   # M mismatch
    lambda x, w, s: (x, w, np.where(np.arange(s.size) == 3, 0.0, s)),
    lambda x, w, s: (x, w, np.where(np.arange(s.size) == 3, -1.0, s)),
    lambda x, w, s: (x, w, np.where(np.arange(s.size) == 3, np.inf, s)),
    lambda x, w, s: (x, w, np.where(np.arange(s.size) == 3, np.nan, s)),
])
def test_check_smoothing_rejects(case):
    x, w, s = make_inputs(1)
    with pytest.raises(ValueError):
        O.check_smoothing(*case(x, w, s))


@pytest.mark.parametrize("rank", [-1, 49, True, 2.0, np.int64(3)])
def test_check_rank_rejects(rank):
    _, w, _ = make_inputs(1)
    with pytest.raises(ValueError):
        O.check_rank(w, rank)
    with pytest.raises(ValueError):
        O.check_rank(w[0], 1)


@pytest.mark.parametrize("bits", [1, 9, True, 4.0])
def test_check_bits_rejects(bits):
    with pytest.raises(ValueError):
        O.quantize_int(np.ones(3, np.float32), bits)


# ----------------------------------------------------------------------------- split
def _tail(ws, r):
    sig2 = np.sort(np.linalg.eigvalsh(ws.astype(np.float64).T @ ws.astype(np.float64)))[::-1]
    return float(np.sqrt(np.clip(sig2[r:], 0, None).sum()))


def test_split_rank0_empty_factors_and_full_residual():
    _, w, _ = make_inputs(1)
    left, right, res = O.split_weight(w, 0, "f32")
    assert left.shape == (64, 0) and right.shape == (0, 48)
    assert np.array_equal(res.view(np.uint32), w.view(np.uint32))


@pytest.mark.parametrize("dtype,tol", [("f32", 1e-5), ("bf16", 1e-2), ("f64", 1e-12)])
def test_split_full_rank_residual_vanishes(dtype, tol):
    x, w, s = make_inputs(1)
    ws = O.smooth_weight(w, s, dtype)
    left, right, res = O.split_weight(ws, min(ws.shape), dtype)
    assert np.linalg.norm(res.astype(np.float64)) / np.linalg.norm(ws.astype(np.float64)) <= tol


def test_full_rank_recovers_product():
    x, w, s = make_inputs(1)
    y = O.svdquant_linear(x, w, s, 48, 4)
    assert y.dtype == np.float32 and y.shape == (16, 48)
    assert O.rel_fro(y, x.astype(np.float64) @ w.astype(np.float64)) <= 1e-4
    y64 = O.svdquant_linear(x.astype(np.float64), w.astype(np.float64), s.astype(np.float64), 48, 4)
    assert y64.dtype == np.float64
    assert O.rel_fro(y64, x.astype(np.float64) @ w.astype(np.float64)) <= 1e-10


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("rank", [1, 4, 8, 20])
def test_split_eckart_young(dtype, rank):
    x, w, s = make_inputs(1)
    ws = O.smooth_weight(w, s, dtype)
    left, right, res = O.split_weight(ws, rank, dtype)
    tail = _tail(ws, rank)
    err = abs(np.linalg.norm(res.astype(np.float64)) - tail)
    if dtype == "f64":
        assert err <= 1e-9 * tail
    else:  # factors and R stored in binary32
        assert err <= 1e-5 * np.linalg.norm(ws.astype(np.float64))


def test_split_factor_structure():
    x, w, s = make_inputs(1)
    ws = O.smooth_weight(w, s, "f64")
    left, right, res = O.split_weight(ws, 8, "f64")
    assert np.allclose(right @ right.T, np.eye(8), atol=1e-12)
    g = left.T @ left
    assert np.allclose(g - np.diag(np.diag(g)), 0, atol=1e-10 * np.abs(g).max())
    norms = np.sqrt(np.diag(g))
    assert np.all(np.diff(norms) <= 1e-12)  # singular values descending
    assert np.allclose(norms**2, np.sort(np.linalg.eigvalsh(ws.T @ ws))[::-1][:8], rtol=1e-10)


# ----------------------------------------------------------------------------- per-tensor INT
def test_int_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "int_worked.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        z = np.array(c["z"], np.float32)
        codes, s = O.quantize_int(z, c["bits"])
        assert float(s) == c["s"]
        assert codes.tolist() == c["codes"]
        assert O.fake_quantize(z, c["bits"], "f32").tolist() == c["fake"]


def test_int_zero_input():
    z = np.zeros((3, 5), np.float32)
    codes, s = O.quantize_int(z, 4)
    assert s == 0 and not codes.any()
    assert not O.fake_quantize(z, 4, "f32").any()


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_int_invariants(bits):
    rng = _rng(bits)
    qmax = 2 ** (bits - 1) - 1
    z = (rng.standard_normal((9, 31)) * 3).astype(np.float32)
    c, s = O.quantize_int(z, bits)
    # the max-magnitude element maps to +-qmax
    i = np.unravel_index(np.argmax(np.abs(z)), z.shape)
    assert abs(c[i]) == qmax and np.abs(c).max() == qmax
    # power-of-two rescaling: same codes, scale times 2^k
    for k in (-5, 3):
        c2, s2 = O.quantize_int(z * np.float32(2.0**k), bits)
        assert np.array_equal(c2, c) and s2 == s * np.float32(2.0**k)
    # sign symmetry
    c3, s3 = O.quantize_int(-z, bits)
    assert np.array_equal(c3, -c) and s3 == s
    # permutation equivariance
    p = rng.permutation(z.size)
    c4, _ = O.quantize_int(z.reshape(-1)[p], bits)
    assert np.array_equal(c4, c.reshape(-1)[p])
    # dequantisation error bound: |z - s*c| <= s/2
    assert np.all(np.abs(z.astype(np.float64) - float(s) * c) <= float(s) / 2 * (1 + 1e-6))


def test_int_packing_layout():
    codes = np.array([[1, -1, 7, -7, 0]], np.int64)
    assert O.pack_int_codes(codes, 4).tolist() == [[0xF1, 0x97, 0x00]]
    assert O.pack_int_codes(codes, 8).tolist() == [[1, 255, 7, 249, 0]]


# ----------------------------------------------------------------------------- MXFP4
def test_mx_worked_blocks(golden_dir):
    with open(os.path.join(golden_dir, "mx_worked.json")) as f:
        g = json.load(f)
    for b in g["blocks"]:
        z = np.array([b["z"]], np.float32)
        codes, sb = O.quantize_mx(z)
        assert sb.tolist() == [[b["scale_byte"]]]
        assert codes.tolist() == [b["codes"]]


def _sweep_values():
    """Dense sweep of binary32 patterns with |v| <= 8, every tie point, subnormals, signed zeros."""
    pats = np.arange(0, 0x41000001, 2749, dtype=np.uint64).astype(np.uint32)
    v = pats.view(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    extra = np.concatenate([ties, np.nextafter(ties, 0), np.nextafter(ties, 10),
                            np.array([0.0, 1e-40, 1e-45, 6.0, 8.0, 5.9999995], np.float32)])
    v = np.concatenate([v, extra])
    return np.concatenate([v, -v])


def test_e2m1_code_bruteforce():
    v = _sweep_values()
    got = O.e2m1_code(v)
    want = np.array([loops.e2m1_bruteforce(float(a), bool(np.signbit(a))) for a in v], np.uint8)
    assert np.array_equal(got, want)


def test_mx_exponent_bruteforce():
    rng = _rng(5)
    a = np.concatenate([
        np.abs(_sweep_values()).astype(np.float64),
        np.ldexp(rng.random(3000) + 0.5, rng.integers(-150, 128, 3000)),
        6.0 * np.ldexp(1.0, np.arange(-130, 127)),          # exact powers: a == 6*2^e boundary
        np.nextafter(6.0 * np.ldexp(1.0, np.arange(-120, 120)), np.inf),
        [0.0, 2.0**-149, 2.0**-126, 3.3e38],
    ])
    with np.errstate(over="ignore"):
        a = a.astype(np.float32).astype(np.float64)  # block maxima are finite binary32 values
    a = a[np.isfinite(a)]
    got = O.mx_block_exponent(a)
    want = np.array([loops.mx_exponent_bruteforce(float(t)) for t in a])
    assert np.array_equal(got, want)


def test_mx_scaling_and_zero():
    rng = _rng(6)
    z = rng.standard_normal((5, 70)).astype(np.float32)  # ragged: 3 blocks, the last of 6
    c, sb = O.quantize_mx(z)
    assert sb.shape == (5, 3) and c.shape == (5, 70)
    for k in (-9, 4):
        c2, sb2 = O.quantize_mx(z * np.float32(2.0**k))
        assert np.array_equal(c2, c) and np.array_equal(sb2.astype(int), sb.astype(int) + k)
    c3, sb3 = O.quantize_mx(-z)
    assert np.array_equal(c3, c ^ 8) and np.array_equal(sb3, sb)
    cz, sz = O.quantize_mx(np.zeros((2, 40), np.float32))
    assert not cz.any() and not sz.any()
    # dequantised magnitude never exceeds the block max, error within half a grid step (<= 2^(e-1)... 1 unit at 4..6)
    dq = O.dequant_mx(c, sb)
    e = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)[:, :70]
    assert np.all(np.abs(dq - z) <= np.ldexp(1.0, e) + 0)


def test_mx_quantises_along_k_per_column():
    """R with a different exponent per column n, every 32-block along M holding +-6*2^(e_n):
    quantising R^T along M is exact; along N it would lose the small columns."""
    M, N = 64, 8
    rng = _rng(7)
    mags = O.E2M1_GRID[rng.integers(0, 8, (M, N))] * np.where(rng.random((M, N)) < 0.5, -1, 1)
    mags[0::32, :] = 6.0
    R = (mags * np.ldexp(1.0, np.arange(N) - 4)[None, :]).astype(np.float32)
    c, sb = O.quantize_mx(R.T)
    assert np.array_equal(O.dequant_mx(c, sb), R.T.astype(np.float64))
    assert np.array_equal(sb.astype(int) - 127, np.repeat((np.arange(N) - 4)[:, None], 2, axis=1))
    # the exact case through the whole forward: rank 0, unit scale, x rows also exact
    x = (O.E2M1_GRID[rng.integers(0, 8, (3, M))] * np.ldexp(1.0, np.arange(3) - 1)[:, None]).astype(np.float32)
    x[:, 0::32] = 6.0 * np.ldexp(1.0, np.arange(3) - 1)[:, None]
    y = O.forward_ref(x, np.ones(M, np.float32), np.zeros((M, 0)), np.zeros((0, N)), R, "mx", 4, "f32")
    assert np.array_equal(y, x.astype(np.float64) @ R.astype(np.float64))


def test_mx_packing_layout():
    codes = np.array([[1, 2, 15, 8, 3]], np.uint8)
    assert O.pack_nibbles(codes).tolist() == [[0x21, 0x8F, 0x03]]


# ----------------------------------------------------------------------------- whole operator
def test_forward_int_exact_special_case():
    """rank 0, unit scale, integer activations and residual with max |.| = 7: s_x = s_R = 1,
    so Q is the identity and Y equals the integer product exactly."""
    rng = _rng(8)
    x = rng.integers(-7, 8, (16, 64)).astype(np.float32)
    R = rng.integers(-7, 8, (64, 48)).astype(np.float32)
    x[0, 0], R[0, 0] = 7, -7
    y = O.forward_ref(x, np.ones(64, np.float32), np.zeros((64, 0)), np.zeros((0, 48)), R, "int", 4, "f32")
    assert np.array_equal(y, x.astype(np.float64) @ R.astype(np.float64))


def test_forward_toy_workload_against_loops():
    x, w, s = make_inputs(1)
    ws = O.smooth_weight(w, s, "f32")
    left, right, res = O.split_weight(ws, 8, "f32")
    y = O.forward_ref(x, s, left, right, res, "int", 4, "f32")
    yl, (cx, sx), (cr, sr) = loops.forward(x.tolist(), s.tolist(), left.tolist(), right.tolist(), res.tolist(), "int", 4, "f32")
    xs = O.smooth_activations(x, s, "f32")
    ocx, osx = O.quantize_int(xs, 4)
    ocr, osr = O.quantize_int(res, 4)
    assert np.array_equal(ocx, np.array(cx)) and np.array_equal(ocr, np.array(cr))
    assert float(osx) == sx and float(osr) == sr
    assert O.rel_fro(y, np.array(yl)) <= 1e-12


def test_forward_mx_bf16_against_loops():
    rng = _rng(9)
    B, M, N, r = 4, 80, 12, 3  # ragged K: blocks of 32, 32, 16
    x = O.to_dtype(rng.standard_t(3, (B, M)), "bf16")
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)), "bf16")
    s = np.abs(rng.standard_normal(M)).astype(np.float32) + np.float32(0.1)
    ws = O.smooth_weight(w, s, "bf16")
    left, right, res = O.split_weight(ws, r, "bf16")
    y = O.forward_ref(x, s, left, right, res, "mx", 4, "bf16")
    yl, act, wgt = loops.forward(x.tolist(), s.tolist(), left.tolist(), right.tolist(), res.tolist(), "mx", 4, "bf16")
    xs = O.smooth_activations(x, s, "bf16")
    cx, bx = O.quantize_mx(xs)
    cr, br = O.quantize_mx(res.T)
    assert cx.tolist() == [a[0] for a in act] and bx.tolist() == [a[1] for a in act]
    assert cr.tolist() == [c[0] for c in wgt] and br.tolist() == [c[1] for c in wgt]
    assert O.rel_fro(y, np.array(yl)) <= 1e-12


def test_two_branch_beats_naive_and_improves_with_rank():
    """Toy experiment of the exercise page (qualitative): with outlier channels, the two-branch
    output error falls with rank and is below naive W4A4 and smoothing-only quantisation."""
    x, w, s = make_inputs(1)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    naive = O.fake_quantize(x, 4, "f32").astype(np.float64) @ O.fake_quantize(w, 4, "f32").astype(np.float64)
    xs, ws = O.smooth_inputs(x, w, s, "f32")
    smooth_only = O.fake_quantize(xs, 4, "f32").astype(np.float64) @ O.fake_quantize(ws, 4, "f32").astype(np.float64)
    errs = [O.rel_fro(O.svdquant_linear(x, w, s, r, 4), ref) for r in range(0, 7)]
    assert errs[6] < errs[0] and errs[4] < O.rel_fro(smooth_only, ref) < O.rel_fro(naive, ref)


# ----------------------------------------------------------------------------- workloads
@pytest.mark.parametrize("cid", [1, 2])
def test_workload_inputs(cid):
    wl = WORKLOADS[cid]
    x, w, s = make_inputs(cid, B=min(wl.B, 64))
    assert x.dtype == w.dtype == s.dtype == np.float32
    assert w.shape == (wl.M, wl.N) and s.shape == (wl.M,)
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    if wl.dtype == "bf16":
        assert not (x.view(np.uint32) & 0xFFFF).any() and not (w.view(np.uint32) & 0xFFFF).any()
    x2, w2, s2 = make_inputs(cid, B=min(wl.B, 64))
    assert np.array_equal(x, x2) and np.array_equal(w, w2) and np.array_equal(s, s2)


@pytest.mark.parametrize("fmt", ["int", "mx"])
def test_forward_full_rank_recovers_product(fmt):
    """Full rank leaves a numerically zero residual, so Y is the unquantised low-rank branch
    and recovers x @ W (the residual's quantisation error is relative to a ~1e-7 residual)."""
    x, w, s = make_inputs(1)
    ws = O.smooth_weight(w, s, "f32")
    left, right, res = O.split_weight(ws, 48, "f32")
    y = O.forward_ref(x, s, left, right, res, fmt, 4, "f32")
    assert O.rel_fro(y, x.astype(np.float64) @ w.astype(np.float64)) <= 1e-5


# ----------------------------------------------------------------------------- scale calibration
def test_calibrate_scale_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "calib_worked.json")))
    x, w = np.array(g["x"], np.float32), np.array(g["w"], np.float32)
    for c in g["cases"]:
        got = O.calibrate_scale(x, w, c["alpha"])
        assert got.dtype == np.float32 and np.array_equal(got, np.array(c["scale"], np.float32)), c


def test_calibrate_scale_against_loops_and_invariants():
    rng = np.random.default_rng(21)
    x = (rng.standard_t(3, (9, 12)) * 10.0 ** rng.integers(-3, 3, (9, 12))).astype(np.float32)
    w = (rng.standard_normal((12, 7)) * 10.0 ** rng.integers(-2, 2, (12, 7))).astype(np.float32)
    x[:, 3] = 0.0
    w[5] = 0.0
    for alpha in (0.0, 0.25, 0.5, 0.9, 1.0):
        got = O.calibrate_scale(x, w, alpha)
        assert np.array_equal(got, np.array(loops.calibrate_scale(x.tolist(), w.tolist(), alpha), np.float32))
        assert got[3] == 1.0 and got[5] == 1.0 and np.all(got > 0)
    # alpha = 1: the column maximum itself; scaling x by 4 doubles the scale at alpha = 0.5
    # and leaves it at alpha = 0
    ax = np.max(np.abs(x), axis=0)
    ok = (ax > 0) & (np.max(np.abs(w), axis=1) > 0)
    assert np.array_equal(O.calibrate_scale(x, w, 1.0)[ok], ax[ok])
    assert np.array_equal(O.calibrate_scale(4 * x, w, 0.5), np.where(ok, 2, 1) * O.calibrate_scale(x, w, 0.5))
    assert np.array_equal(O.calibrate_scale(4 * x, w, 0.0), O.calibrate_scale(x, w, 0.0))
    # a smoothing with the calibrated scale balances the channel maxima: max|x/s| and
    # max|s W| agree up to rounding where alpha = 0.5
    s = O.calibrate_scale(x, w, 0.5).astype(np.float64)
    mx = np.max(np.abs(x / s), axis=0)
    mw = np.max(np.abs(s[:, None] * w), axis=1)
    assert np.allclose(mx[ok], mw[ok], rtol=1e-6)


@pytest.mark.parametrize("alpha", [-0.1, 1.5])
def test_calibrate_scale_rejects(alpha):
    with pytest.raises(ValueError):
        O.calibrate_scale(np.ones((2, 3), np.float32), np.ones((3, 2), np.float32), alpha)
    with pytest.raises(ValueError):
        O.calibrate_scale(np.ones((2, 3), np.float32), np.ones((4, 2), np.float32), 0.5)


def test_forward_bias_is_added_per_output_channel():
    """Zero activations give codes 0 and a zero low-rank branch, so Y is the bias itself; a
    bias shifts every row of a nonzero forward by the same vector."""
    x, w, s = make_inputs(1)
    left, right, res = O.split_weight(O.smooth_weight(w, s, "f32"), 8, "f32")
    bias = np.arange(w.shape[1], dtype=np.float32) - 20.0
    y0 = O.forward_ref(np.zeros_like(x), s, left, right, res, "int", 4, "f32", bias=bias)
    assert np.array_equal(y0, np.broadcast_to(bias.astype(np.float64), y0.shape))
    y = O.forward_ref(x, s, left, right, res, "mx", 4, "f32")
    yb = O.forward_ref(x, s, left, right, res, "mx", 4, "f32", bias=bias)
    assert np.allclose(yb - y, bias[None, :], rtol=0, atol=1e-12 * np.abs(y).max())


# ----------------------------------------------------------------------------- two-level MXFP4 scaling
def test_two_level_residual_scale_worked(golden_dir):
    from fractions import Fraction
    with open(os.path.join(golden_dir, "two_level_worked.json")) as f:
        g = json.load(f)
    for case in g["residual_scale"]:
        r = np.zeros((3, 2), np.float32)
        r[1, 0] = -case["amax"]
        r[2, 1] = case["amax"] / 2
        assert O.two_level_residual_scale(r) == np.float32(float(Fraction(case["g"]))), case


def test_two_level_residual_scale_places_the_max_at_the_top_code():
    """g_R lies in (1, 2] and maps max|R| to 6 * 2^ex up to one rounding of the binary32
    product, so the block holding the max takes exponent ex (or ex + 1 when that product
    rounds just above 6 * 2^ex)."""
    rng = _rng(41)
    for t in range(300):
        r = (rng.standard_normal((8, 5)) * 2.0 ** rng.integers(-60, 60)).astype(np.float32)
        g = O.two_level_residual_scale(r)
        assert 1.0 < g <= 2.0
        top = np.max(np.abs(r * g))  # binary32 products
        e = int(O.mx_block_exponent(top))
        assert abs(float(top) / (6.0 * 2.0 ** e) - 1.0) <= 2.0 ** -22 or abs(float(top) / (6.0 * 2.0 ** (e - 1)) - 1.0) <= 2.0 ** -22


def test_two_level_forward_worked(golden_dir):
    with open(os.path.join(golden_dir, "two_level_worked.json")) as f:
        g = json.load(f)["forward"]
    x = np.zeros((1, 32), np.float32)
    x[0, : len(g["x"])] = g["x"]
    res = np.zeros((32, 1), np.float32)
    res[: len(g["residual"]), 0] = g["residual"]
    left = np.zeros((32, 1), np.float32)
    left[1, 0] = g["left_row1"]
    right = np.full((1, 1), g["right"], np.float32)
    s = np.ones(32, np.float32)
    y = O.forward_ref(x, s, left, right, res, "mx", 4, "f32")
    assert y[0, 0] == g["y_plain"]
    y2 = O.forward_ref(x, s, left, right, res, "mx", 4, "f32", x_global_scale=g["x_global_scale"])
    assert abs(y2[0, 0] / g["y_two_level"] - 1.0) <= g["rel_tol_two_level"]
    assert y2[0, 0] != y[0, 0]


@pytest.mark.parametrize("dtype,j", [("f32", 3), ("bf16", -5), ("f32", 0)])
def test_two_level_with_power_of_two_scales_is_plain_mx(dtype, j):
    """When g_x = 2^j and max|R| = 3 * 2^k (so g_R = 2), every scale is a power of two: the
    codes are those of plain MXFP4, the block exponents move by j and 1, alpha = 2^-(j+1)
    and L2 / alpha is exact, so the two-level forward equals the plain one bit for bit."""
    rng = _rng(7 + j)
    x = O.to_dtype(rng.standard_t(3, (24, 100)), dtype)
    w = O.to_dtype(0.1 * rng.standard_normal((100, 40)), dtype)
    s = np.ones(100, np.float32)
    left, right, res = O.split_weight(O.smooth_weight(w, s, dtype), 6, dtype)
    res = np.array(res, np.float32)
    k = int(np.ceil(np.log2(np.max(np.abs(res)) / 3.0))) + 1
    res[3, 7] = 3.0 * 2.0 ** k
    assert O.two_level_residual_scale(res) == 2.0
    y = O.forward_ref(x, s, left, right, res, "mx", 4, dtype)
    y2 = O.forward_ref(x, s, left, right, res, "mx", 4, dtype, x_global_scale=2.0 ** j)
    assert np.array_equal(y, y2)


def test_two_level_differs_from_plain_and_rejects_int():
    """A non-power-of-two g_x changes the activation codes (the scaled values land on other
    E2M1 points), and two-level scaling is an MXFP4-only scheme."""
    x, w, s = make_inputs(1)
    left, right, res = O.split_weight(O.smooth_weight(w, s, "f32"), 8, "f32")
    y = O.forward_ref(x, s, left, right, res, "mx", 4, "f32")
    y2 = O.forward_ref(x, s, left, right, res, "mx", 4, "f32", x_global_scale=1.37)
    assert not np.array_equal(y, y2)
    exact = x.astype(np.float64) @ w.astype(np.float64)
    assert O.rel_fro(y2, exact) < 0.2 and O.rel_fro(y, exact) < 0.2
    with pytest.raises(ValueError):
        O.forward_ref(x, s, left, right, res, "int", 4, "f32", x_global_scale=1.0)
