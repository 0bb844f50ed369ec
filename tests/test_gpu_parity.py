"""GPU parity of libsvdq against the CPU oracle (runs through the C ABI on an MI355X).

Integer and byte outputs (activation codes, E8M0 scales, s_x, smoothing results,
fake-quantised values) must match the oracle bit for bit. The operator output Y must be
within a relative Frobenius error of 2e-3 (float32 inputs) or 1e-2 (bfloat16 inputs) of
the oracle's float64 forward on the library's own exported factors and residual; exact
special cases (rank 0, unit scale, values the quantiser reproduces exactly) must match
x @ W bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import rank_bit_residual_amd as R
from rank_bit_residual_amd import _lib
from oracle import svdquant as O
from workloads import WORKLOADS, make_inputs

from cases import double_boundary_case

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": 2e-3, "bf16": 1e-2}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _g(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(TD[dtype]).to(dev())


def _np(t):
    return t.detach().to("cpu", torch.float32).numpy()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ----------------------------------------------------------------------------- elementwise calls
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_smooth_inputs_bit_exact(dtype):
    rng = np.random.default_rng(10)
    x = O.to_dtype(rng.standard_t(3, (37, 300)) * 10.0 ** rng.integers(-3, 4, (37, 300)), dtype)
    w = O.to_dtype(rng.standard_normal((300, 70)), dtype)
    s = np.abs(rng.standard_normal(300)).astype(np.float32) * np.float32(3) + np.float32(1e-3)
    x[0, :5] = [0.0, -0.0, 1e-38, -3e-39, 65504.0]
    xs, ws = R.smooth_inputs(_g(x, dtype), _g(w, dtype), torch.from_numpy(s).to(dev()))
    oxs, ows = O.smooth_inputs(x, w, s, dtype)
    assert np.array_equal(_bits(_np(xs)), _bits(oxs)) and np.array_equal(_bits(_np(ws)), _bits(ows))
    # strided (transposed) inputs
    xt = _g(x.T.copy(), dtype).t()
    xs2, _ = R.smooth_inputs(xt, _g(w, dtype), torch.from_numpy(s).to(dev()))
    assert torch.equal(xs2, xs)


def test_smooth_bf16_every_value():
    """Every finite bf16 x (both signs) against 64 scales: workload-like values, powers of
    two, values whose reciprocal is inexact, and scales outside [2^-90, 2^90]."""
    rng = np.random.default_rng(15)
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    xv = np.concatenate([h, h | 0x8000]).astype(np.uint32) << 16
    x = xv.view(np.float32)[:, None] * np.ones((1, 64), np.float32)
    s = np.concatenate([
        np.abs(rng.standard_normal(40)) * 3 + 0.01,
        [1.0, 2.0, 0.5, 3.0, 0.1, 7.0, 1e-3, 1e3, 2.0**-90, 2.0**90, 2.0**-91, 2.0**91, 2.0**-120, 2.0**120],
        np.ldexp(rng.random(10) + 0.5, rng.integers(-89, 90, 10)),
    ]).astype(np.float32)
    w = np.ones((64, 3), np.float32)
    xs, _ = R.smooth_inputs(_g(x, "bf16"), _g(w, "bf16"), torch.from_numpy(s).to(dev()))
    want = O.smooth_activations(x, s, "bf16")
    got = _np(xs)
    bad = np.argwhere(_bits(got) != _bits(want))
    assert bad.size == 0, f"{len(bad)} mismatches, first x={x[tuple(bad[0])]!r} s={s[bad[0][1]]!r}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_fake_quantize_bit_exact(dtype, bits):
    rng = np.random.default_rng(bits)
    z = O.to_dtype(rng.standard_normal((129, 77)) * 3, dtype)
    got = R.fake_quantize(_g(z, dtype), bits)
    assert got.dtype == TD[dtype] and got.shape == (129, 77)
    assert np.array_equal(_bits(_np(got)), _bits(O.fake_quantize(z, bits, dtype)))


def test_fake_quantize_zero_and_worked_ties():
    z = torch.zeros(5, 9, device=dev())
    assert not R.fake_quantize(z, 4).any()
    t = torch.tensor([[7, 3.5, 2.5, -0.5, -1.5, 0]], device=dev())
    assert R.fake_quantize(t, 4).tolist() == [[7, 4, 2, 0, -2, 0]]
    t = torch.tensor([[105, 37.5]], device=dev())
    assert R.fake_quantize(t, 4).tolist() == [[105, 30]]


# ----------------------------------------------------------------------------- step (a): codes
def _act_codes_ref(x, s, fmt, bits, dtype):
    xs = O.smooth_activations(x, s, dtype)
    if fmt == "mx":
        c, sb = O.quantize_mx(xs)
        return O.pack_nibbles(c), sb, None
    c, sx = O.quantize_int(xs, bits, dtype)
    return O.pack_int_codes(c, bits), None, sx


def _check_codes(x, s, fmt, bits, dtype):
    codes, scales, sx = R.quantize_activations(_g(x, dtype), torch.from_numpy(s).to(dev()), fmt, bits)
    torch.cuda.synchronize()
    wc, ws, wsx = _act_codes_ref(x, s, fmt, bits, dtype)
    codes = codes.cpu().numpy()
    assert np.array_equal(codes[:, : wc.shape[1]], wc)
    assert not codes[:, wc.shape[1]:].any()
    if fmt == "mx":
        sc = scales.cpu().numpy()
        assert np.array_equal(sc[:, : ws.shape[1]], ws)
    else:
        assert sx.cpu().numpy()[0] == np.float32(wsx)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_activation_codes_bit_exact_workloads(cid):
    wl = WORKLOADS[cid]
    x, w, s = make_inputs(cid)
    _check_codes(x, s, wl.fmt, wl.bits, wl.dtype)


def _workspace_codes(ws, B, M, mx):
    """The activation codes at the start of svdq_linear's workspace as [B, Kp/2] bytes:
    row-major for INT, and for MXFP4 (both MXFP4 GEMMs; operand arrays past 2 GiB, which take
    the generic kernel, are not used here) 1 KB tiles of 16 rows x 128 codes, tile
    (b / 16, k / 128) at ((b / 16) * Kp / 128 + k / 128) KB."""
    row = ((M + 255) // 256 * 256) // 2
    if mx:
        rows16 = -(-B // 16) * 16
        t = ws[: rows16 * row].cpu().numpy().reshape(rows16 // 16, row // 64, 16, 64)
        return t.transpose(0, 2, 1, 3).reshape(rows16, row)[:B]
    return ws[: B * row].cpu().numpy().reshape(B, row)


@pytest.mark.parametrize("cid,B,rank", [(2, None, None), (5, None, None), (2, 48, 64), (5, 40, 96), (3, 300, None)])
def test_linear_workspace_codes_bit_exact(cid, B, rank):
    """The codes svdq_linear itself writes (white-box: its workspace begins with the
    activation codes, [B, Kp/2] nibbles, row-major for INT or, for MXFP4, in 1 KB tiles of 16
    rows x 128 codes) equal the oracle's. At the INT and decode shapes the
    activation kernel splits the rank over several blocks and shares the coding between
    them, a path svdq_quantize_activations (one rank chunk) does not take."""
    wl = WORKLOADS[cid]
    x, w, s = make_inputs(cid, B=B)
    rank = wl.rank if rank is None else rank
    p = R.prepare(_g(w, wl.dtype), torch.from_numpy(s), rank, wl.bits, wl.fmt)
    ws = torch.full((R.workspace_bytes(x.shape[0], p),), 0xA5, dtype=torch.uint8, device=dev())
    R.linear(_g(x, wl.dtype), p, workspace=ws)
    torch.cuda.synchronize()
    want, _, _ = _act_codes_ref(x, s, wl.fmt, wl.bits, wl.dtype)
    got = _workspace_codes(ws, x.shape[0], x.shape[1], wl.fmt == "mx")
    assert np.array_equal(got[:, : want.shape[1]], want)
    assert not got[:, want.shape[1]:].any()


def test_int_linear_graph_replay_matches_eager():
    """The INT path (max pre-pass, activation kernel, INT4 GEMM) captured in a HIP graph:
    every replay must equal the eager result."""
    rng = np.random.default_rng(17)
    B, M, N = 64, 2048, 512
    x = O.to_dtype(rng.standard_normal((B, M)), "bf16")
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)), "bf16")
    from workloads import smoothing_scale
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(smoothing_scale(x, w, 0.5)), 32, 4, "int")
    xg = _g(x, "bf16")
    want = R.linear(xg, p)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(dev())
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        out = R.linear(xg, p)  # warm-up on the capture stream (allocates the workspace)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            out = R.linear(xg, p)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want)


def test_int_small_batch_many_calls_same_results():
    """The INT path (maximum pre-pass, activation kernel, GEMM) keeps no state between calls:
    1100 back-to-back calls on one workspace alternate two batches of different ranges (so
    s_x changes every call); each must reproduce its batch's first result bit for bit, and
    the first results match the oracle."""
    rng = np.random.default_rng(23)
    B, M, N = 64, 2048, 384
    xs = [O.to_dtype(rng.standard_normal((B, M)) * (1 + 3 * k), "bf16") for k in range(2)]
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)), "bf16")
    from workloads import smoothing_scale
    s = smoothing_scale(xs[0], w, 0.5)
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(s), 32, 4, "int", keep_factors=True)
    ws = torch.empty(R.workspace_bytes(B, p), dtype=torch.uint8, device=dev())
    want = [R.linear(_g(x, "bf16"), p, workspace=ws).clone() for x in xs]
    for x, y in zip(xs, want):
        ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "int", 4, "bf16")
        assert O.rel_fro(_np(y), ref) <= TOL["bf16"]
    xg = [_g(x, "bf16") for x in xs]
    outs = torch.empty((100, B, N), dtype=torch.bfloat16, device=dev())
    for rnd in range(11):
        outs.fill_(float("nan"))
        for k in range(100):
            R.linear(xg[k % 2], p, out=outs[k], workspace=ws)
        torch.cuda.synchronize()
        for k in range(100):
            assert torch.equal(outs[k], want[k % 2]), f"call {100 * rnd + k} differs"


@pytest.mark.parametrize("B,M,N", [(4200, 1536, 256), (300, 4096, 200)])
def test_int_linear_batch_routes(B, M, N):
    """B = 4200: 263 row blocks, no K split, two K steps per wave of the activation kernel;
    B = 300: K split into four chunks whose partials the INT4 GEMM sums."""
    assert _int_case(B, M, N, 32, "bf16", B) <= TOL["bf16"]


def test_activation_codes_double_rounding_boundaries():
    x, s = double_boundary_case()
    _check_codes(x, s, "mx", 4, "bf16")
    _check_codes(x, s, "int", 8, "bf16")


@pytest.mark.parametrize("fmt,bits,dtype", [("mx", 4, "bf16"), ("mx", 4, "f32"), ("int", 4, "bf16"), ("int", 3, "f32"),
                                             ("int", 8, "bf16"), ("int", 6, "f32")])
def test_activation_codes_edge_values(fmt, bits, dtype):
    """Ragged K (M = 300: a short last block), ties, signed zeros, subnormals, huge values."""
    rng = np.random.default_rng(11)
    B, M = 19, 300
    x = rng.standard_normal((B, M)) * 10.0 ** rng.integers(-2, 3, (B, M))
    grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.0])
    x[1] = grid[rng.integers(0, len(grid), M)]
    x[2] = 0.0
    x[3, :40] = -0.0
    x[4] = rng.standard_normal(M) * 1e-39
    x[5] = rng.standard_normal(M) * 1e30
    x = O.to_dtype(x, dtype)
    s = np.ones(M, np.float32)
    s[100:] = np.abs(rng.standard_normal(M - 100)).astype(np.float32) + np.float32(0.01)
    _check_codes(x, s, fmt, bits, dtype)


# ----------------------------------------------------------------------------- exact special cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_int_exact_special_case(dtype):
    """rank 0, unit scale, integer x and W with max |.| = 7: s_x = s_R = 1 and Y = x @ W exactly."""
    rng = np.random.default_rng(12)
    B, M, N = 40, 320, 300
    x = rng.integers(-7, 8, (B, M)).astype(np.float32)
    w = rng.integers(-7, 8, (M, N)).astype(np.float32)
    x[0, 0] = w[0, 0] = 7
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, 4, "int")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x.astype(np.float64) @ w.astype(np.float64), dtype)
    assert np.array_equal(_bits(_np(y)), _bits(want))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_exact_special_case(dtype):
    """rank 0, unit scale, E2M1-grid values whose every 32-block (rows of x, columns of W)
    has max 4 or 6: the shared exponent is 0, Q is the identity and Y = x @ W exactly."""
    rng = np.random.default_rng(13)
    B, M, N = 40, 320, 300
    grid = O.E2M1_GRID
    x = grid[rng.integers(0, 8, (B, M))] * np.where(rng.random((B, M)) < 0.5, -1, 1)
    w = grid[rng.integers(0, 8, (M, N))] * np.where(rng.random((M, N)) < 0.5, -1, 1)
    x[:, 0::32] = np.where(rng.random((B, M // 32)) < 0.5, 6.0, -4.0)
    w[0::32, :] = np.where(rng.random((M // 32, N)) < 0.5, -6.0, 4.0)
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, 4, "mx")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x @ w, dtype)
    assert np.array_equal(_bits(_np(y)), _bits(want))


# ----------------------------------------------------------------------------- exact cases per GEMM kernel
def _gemm_route(B, M, N, fmt, bits, dtype):
    """The residual GEMM kernel (and MXFP4 tile) svdq_linear launches for a shape: the launch
    rules of the library, restated so that each exact case below names the kernel it aims at."""
    if fmt == "mx" and B <= 64:
        return "decode"
    def pick(prefix, us_per_elem):
        # fewest rounds of 256 compute units x per-round time 10 us + us_per_elem per tile
        # element; 192-wide tiles only when N % 192 == 0; the first of equal estimates wins
        best = None
        for bm, bn in ((128, 192), (128, 256), (256, 192), (256, 256)):
            if bn == 192 and N % 192:
                continue
            rounds = -(-(-(-B // bm) * -(-N // bn)) // 256)
            t = rounds * (10.0 + us_per_elem * bm * bn)
            if best is None or t < best[0]:
                best = (t, f"{prefix}{bm}x{bn}")
        return best[1]
    if fmt == "mx":
        return pick("mx", 0.3e-3)
    # INT takes the large tiles once the 64 x 64 kernel needs four rounds
    if -(-B // 64) * -(-N // 64) >= 4 * 256:
        return pick("int", 0.6e-3)
    return "int4" if bits <= 4 else "int8"


def _e2m1_exact_operands(rng, B, M, N):
    """x [B, M] and W [M, N] on the E2M1 grid with every 32-block (rows of x, columns of W)
    holding a 4 or a 6 as its largest magnitude: the shared exponents are 0 and quantisation
    is the identity, so with rank 0 and unit scale Y = x @ W, a sum of multiples of 1/4 below
    2^24 / 4 in magnitude, exact in float32 and rounded once to bf16."""
    grid = O.E2M1_GRID
    x = grid[rng.integers(0, 8, (B, M))] * np.where(rng.random((B, M)) < 0.5, -1, 1)
    w = grid[rng.integers(0, 8, (M, N))] * np.where(rng.random((M, N)) < 0.5, -1, 1)
    x[:, 0::32] = np.where(rng.random((B, -(-M // 32))) < 0.5, 6.0, -4.0)
    w[0::32, :] = np.where(rng.random((-(-M // 32), N)) < 0.5, -6.0, 4.0)
    return x, w


@pytest.mark.parametrize("B,M,N,bits,dtype", [
    (256, 4096, 4096, 4, "bf16"),   # the INT4 workload's shape: 64 x 64 tiles, 16 K stages
    (130, 1792, 200, 3, "f32"),     # 7 stages (one odd steady iteration), ragged B and N, float32 io
    (70, 1536, 328, 2, "bf16"),     # exactly the 6 stages kept in flight, ragged N tile
    (130, 768, 200, 8, "bf16"),     # int8 codes: exactly 6 stages of 128 codes, ragged B and N
    (64, 2048, 328, 6, "f32"),      # int8 codes, 16 stages, float32 io
    (300, 896, 136, 5, "bf16"),     # int8 codes, 7 stages (one odd steady iteration)
    (40, 320, 300, 4, "bf16"),      # 2 stages: fewer than the 6 kept in flight, all issued at once
    (70, 200, 96, 3, "f32"),        # 1 stage (K = 200 padded to 256), float32 io
    (130, 1280, 200, 4, "bf16"),    # 5 stages, the longest short run
    (33, 384, 72, 8, "f32"),        # int8 codes: 4 stages of 128 codes
])
def test_int4_kernel_exact_special_case(B, M, N, bits, dtype):
    """Rank 0, unit scale, integer x and W with max |.| = qmax through the INT kernel (K from
    one stage of 256 nibble codes or 128 int8 codes up, both sides of the six it keeps in
    flight): s_x = s_R = 1 and Y = x @ W bit for bit. |Y| <= qmax^2 K < 2^24, so the float32
    result is exact and the bf16 one is its single rounding."""
    q = 2 ** (bits - 1) - 1
    assert q * q * M < 2 ** 24
    assert _gemm_route(B, M, N, "int", bits, dtype) == ("int4" if bits <= 4 else "int8")
    rng = np.random.default_rng(B + M + bits)
    x = rng.integers(-q, q + 1, (B, M)).astype(np.float32)
    w = rng.integers(-q, q + 1, (M, N)).astype(np.float32)
    x[0, 0] = w[0, 0] = q
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, bits, "int")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x.astype(np.float64) @ w.astype(np.float64), dtype)
    got = _np(y)
    bad = np.argwhere(_bits(got) != _bits(want))
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("B,M,N,bits,route,dtype", [
    (1024, 768, 4096, 8, "int128x256", "bf16"),  # int8 codes: 64 per stage, one MFMA per chunk
    (4096, 512, 3072, 6, "int256x192", "f32"),
    (1100, 256, 4000, 5, "int128x256", "bf16"),  # ragged B and N, four stages of 64 codes
])
def test_int8_codes_large_tile_exact_special_case(B, M, N, bits, route, dtype):
    """Rank 0, unit scale, integer x and W with max |.| = qmax through the large-tile INT kernel
    with int8 codes (5-8 bits): Y = x @ W bit for bit (|Y| <= qmax^2 K < 2^24)."""
    q = 2 ** (bits - 1) - 1
    assert q * q * M < 2 ** 24
    assert _gemm_route(B, M, N, "int", bits, dtype) == route
    rng = np.random.default_rng(B + N + bits)
    x = rng.integers(-q, q + 1, (B, M)).astype(np.float32)
    w = rng.integers(-q, q + 1, (M, N)).astype(np.float32)
    x[0, 0] = w[0, 0] = q
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, bits, "int")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x.astype(np.float64) @ w.astype(np.float64), dtype)
    bad = np.argwhere(_bits(_np(y)) != _bits(want))
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("B,M,N,route,dtype", [
    (1024, 256, 4096, "int128x256", "bf16"),   # four rounds of 64 x 64 tiles: the large tiles take over
    (1100, 320, 4000, "int128x256", "bf16"),   # ragged B and N, four K stages
    (2048, 256, 3072, "int128x192", "bf16"),
    (4096, 256, 3072, "int256x192", "f32"),    # float32 io (its f32 tile leaves in row chunks)
    (4096, 256, 4096, "int256x256", "bf16"),
])
def test_int_large_tile_exact_special_case(B, M, N, route, dtype):
    """INT4 exact case (rank 0, unit scale, integer x and W with max |.| = 7) through each tile
    of the large-tile INT kernel: nibbles unpacked to int8 times 16 on the int8 MFMAs, exact
    int32 sums, Y = x @ W bit for bit."""
    assert _gemm_route(B, M, N, "int", 4, dtype) == route
    rng = np.random.default_rng(B + N)
    x = rng.integers(-7, 8, (B, M)).astype(np.float32)
    w = rng.integers(-7, 8, (M, N)).astype(np.float32)
    x[0, 0] = w[0, 0] = 7
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, 4, "int")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x.astype(np.float64) @ w.astype(np.float64), dtype)
    bad = np.argwhere(_bits(_np(y)) != _bits(want))
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("B,M,N,rank,dtype", [
    (1024, 2048, 4096, 32, "bf16"),
    (4096, 1024, 4096, 64, "bf16"),
    (2048, 768, 3072, 96, "f32"),
])
def test_int_large_tile_shapes(B, M, N, rank, dtype):
    """The large-tile INT kernel with a low-rank branch (up-projection after the K loop, on the
    dequantised accumulators) against the oracle."""
    assert _gemm_route(B, M, N, "int", 4, dtype) not in ("int4", "int8")
    rng = np.random.default_rng(B + M + rank)
    x = O.to_dtype(rng.standard_normal((B, M)), dtype)
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.5)
    p = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, 4, "int", keep_factors=True)
    y = R.linear(_g(x, dtype), p)
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "int", 4, dtype)
    assert O.rel_fro(_np(y), ref) <= TOL[dtype]


@pytest.mark.parametrize("B,M,N,route", [
    (4096, 256, 3072, "mx256x192"),  # the attention-projection tile: 256 tiles, one round
    (520, 512, 576, "mx128x192"),    # 15 tiles of 128 x 192, ragged B
    (200, 512, 392, "mx128x256"),    # two 128-row tiles, the second with 72 live rows, ragged N
    (100, 512, 576, "mx128x192"),    # B <= 128: 128-row tiles, N a multiple of 192
    (128, 768, 512, "mx128x256"),    # one full 128-row tile
    (65, 256, 300, "mx128x256"),     # one live row past the decode range, ragged N
    (4096, 256, 8192, "mx256x256"),  # 512 tiles of 256 x 256: the MLP up-projection's tile choice
    (16, 1024, 392, "decode"),       # decode kernel, one 16-row tile, eight waves
    (17, 1280, 200, "decode"),       # decode kernel, two row tiles (the second with one live row)
    (40, 768, 96, "decode"),         # decode kernel, four row tiles and four waves
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_kernel_exact_special_case(B, M, N, route, dtype):
    """Plain (not two-level) MXFP4 exact case through each MXFP4 kernel and tile choice, with
    bf16 io (one rounding of the exact product) and f32 io (the exact product itself; the f32
    tile leaves the kernel in row chunks)."""
    assert _gemm_route(B, M, N, "mx", 4, dtype) == route
    x, w = _e2m1_exact_operands(np.random.default_rng(B + N), B, M, N)
    p = R.prepare(_g(w, dtype), torch.ones(M), 0, 4, "mx")
    y = R.linear(_g(x, dtype), p)
    want = O.to_dtype(x @ w, dtype)
    got = _np(y)
    bad = np.argwhere(_bits(got) != _bits(want))
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}"


# ----------------------------------------------------------------------------- the hardware E2M1 conversion
def _sweep_blocks(dtype, values_for):
    """Activation rows for a sweep of the E2M1 coding: for every shared exponent e from -127 to
    126, blocks of 32 whose element 0 is the block maximum (6 * 2^e, or the dtype's largest
    finite value where 6 * 2^e is beyond it; sign alternating) and whose other 31 elements are
    the values under test (values_for(e), all at most that maximum in magnitude). Rows hold 256
    blocks (K = 8192); the last row is padded with zero blocks."""
    fmax = {"bf16": float(np.uint32(0x7F7F0000).view(np.float32)), "f32": float(np.finfo(np.float32).max)}[dtype]
    blocks = []
    for e in range(-127, 127):
        cap = min(6.0 * 2.0 ** e, fmax)
        v = values_for(e, cap)
        assert np.all(np.abs(v.astype(np.float64)) <= cap)
        nb = -(-len(v) // 31)
        body = np.zeros(nb * 31, np.float32)
        body[: len(v)] = v
        blk = np.empty((nb, 32), np.float32)
        blk[:, 1:] = body.reshape(nb, 31)
        blk[:, 0] = np.where(np.arange(nb) % 2 == 0, cap, -cap)
        blocks.append(blk)
    allb = np.concatenate(blocks)
    rows = -(-len(allb) // 256)
    out = np.zeros((rows * 256, 32), np.float32)
    out[: len(allb)] = allb
    return out.reshape(rows, 256 * 32)


def _check_codes_chunked(x, dtype):
    s = np.ones(x.shape[1], np.float32)
    codes, scales, _ = R.quantize_activations(_g(x, dtype), torch.from_numpy(s).to(dev()), "mx", 4)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    for r0 in range(0, x.shape[0], 64):
        c, sb = O.quantize_mx(x[r0:r0 + 64].astype(np.float64))
        wc = O.pack_nibbles(c)
        gc = codes[r0:r0 + 64, : wc.shape[1]]
        bad = np.argwhere(gc != wc)
        assert bad.size == 0, f"codes differ at row {r0 + bad[0][0]}, byte {bad[0][1]}"
        assert np.array_equal(scales[r0:r0 + 64, : sb.shape[1]], sb), f"E8M0 bytes differ in rows {r0}.."


def test_e2m1_conversion_every_bf16_value():
    """Every finite bf16 value of either sign, against every shared exponent e in [-127, 126]
    whose block maximum 6 * 2^e it does not exceed (subnormal values, subnormal 2^-127 block
    scales, every tie and every E2M1 boundary included): codes and E8M0 bytes bit-equal to the
    oracle's quantize_mx."""
    mags = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)

    def values_for(e, cap):
        v = mags[mags.astype(np.float64) <= cap]
        return np.concatenate([v, -v])

    _check_codes_chunked(_sweep_blocks("bf16", values_for), "bf16")


def test_e2m1_conversion_dense_f32():
    """float32 activations: for every shared exponent, 1024 significands per binade over the
    whole coded range [2^-4, 6] * 2^e, every E2M1 rounding midpoint and its neighbours within 2
    ulps, and values far below the smallest code, both signs; the values are RN_f32(m * 2^e), so
    at the bottom of the range they are float32 subnormals."""
    rng = np.random.default_rng(5)
    sig = np.concatenate([np.ldexp(1.0 + np.arange(1024) / 1024.0, k) for k in range(-4, 3)])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 8),
                           np.nextafter(np.nextafter(mids, 0), 0), np.nextafter(np.nextafter(mids, 8), 8)])
    ms = np.concatenate([sig[sig <= 6.0], near.astype(np.float64), [4.0, 6.0, 0.0, 1e-3, 3e-9],
                         rng.random(64) * 6.0])

    def values_for(e, cap):
        v = (ms * 2.0 ** e).astype(np.float32)
        v = v[np.abs(v.astype(np.float64)) <= cap]
        return np.concatenate([v, -v])

    _check_codes_chunked(_sweep_blocks("f32", values_for), "f32")


# ----------------------------------------------------------------------------- the operator
def _parity(cid, B=None, rank=None, rows=None):
    wl = WORKLOADS[cid]
    rank = wl.rank if rank is None else rank
    x, w, s = make_inputs(cid, B=B)
    p = R.prepare(_g(w, wl.dtype), torch.from_numpy(s), rank, wl.bits, wl.fmt, keep_factors=True)
    xg = _g(x, wl.dtype)
    y = R.linear(xg, p)
    y2 = R.linear(xg, p)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "repeated calls differ"
    assert torch.equal(xg, _g(x, wl.dtype)), "input modified"
    l, r, res = _np(p.left), _np(p.right), _np(p.residual)
    if rows is not None:  # MXFP4 rows are independent: check a sample against the oracle
        sel = np.random.default_rng(0).choice(x.shape[0], rows, replace=False)
        ref = O.forward_ref(x[sel], s, l, r, res, wl.fmt, wl.bits, wl.dtype)
        got = _np(y)[sel]
    else:
        ref = O.forward_ref(x, s, l, r, res, wl.fmt, wl.bits, wl.dtype)
        got = _np(y)
    err = O.rel_fro(got, ref)
    print(f"workload {cid} B={x.shape[0]} rank={rank}: rel Frobenius error {err:.3e}")
    assert err <= TOL[wl.dtype]
    return err


@pytest.mark.parametrize("cid", [1, 2, 5])
def test_operator_parity_full_size(cid):
    _parity(cid)


@pytest.mark.parametrize("cid", [3, 4])
def test_operator_parity_full_size_every_row(cid):
    """The two large MXFP4 workloads (4096 rows) against the oracle on every output."""
    _parity(cid)


@pytest.mark.parametrize("cid,B", [(3, 77), (4, 130), (2, 33)])
def test_operator_parity_ragged_batch(cid, B):
    _parity(cid, B=B)


@pytest.mark.parametrize("rank", [0, 1, 40, 48])
def test_operator_parity_toy_ranks(rank):
    _parity(1, rank=rank)


def test_full_rank_recovers_product():
    x, w, s = make_inputs(1)
    y = R.svdquant_linear(_g(x, "f32"), _g(w, "f32"), torch.from_numpy(s).to(dev()), 48, 4)
    assert O.rel_fro(_np(y), x.astype(np.float64) @ w.astype(np.float64)) <= 1e-4


def test_strided_activations_match_contiguous():
    x, w, s = make_inputs(3, B=64)
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(s), 32, 4, "mx")
    big = torch.zeros(64, 3072 + 64, dtype=torch.bfloat16, device=dev())
    big[:, 16:16 + 3072] = _g(x, "bf16")
    assert torch.equal(R.linear(big[:, 16:16 + 3072], p), R.linear(_g(x, "bf16"), p))


@pytest.mark.parametrize("fmt", ["mx", "int"])
def test_activation_row_stride_past_quad_offsets(fmt):
    """Full activation steps load x by quads with 32-bit element offsets spanning 17 row
    strides; a row stride above INT32_MAX / 17 elements takes the per-lane loads instead. Two
    rows 130 M elements apart (a 260 MB view) give the same output as their contiguous copy."""
    x, w, s = make_inputs(3, B=2)
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(s), 32, 4, fmt)
    ldx, M = 130_000_000, x.shape[1]
    assert ldx > (2**31 - 1) // 17 and ldx % 8 == 0
    big = torch.zeros(ldx + M, dtype=torch.bfloat16, device=dev())
    view = big.as_strided((2, M), (ldx, 1))
    view.copy_(_g(x, "bf16"))
    got = R.linear(view, p)
    want = R.linear(_g(x, "bf16"), p)
    torch.cuda.synchronize()
    del big, view
    assert torch.equal(got, want)


# ----------------------------------------------------------------------------- large-batch MXFP4 kernel
def _mx_case(B, M, N, rank, seed):
    rng = np.random.default_rng(seed)
    x = O.to_dtype(rng.standard_t(3, (B, M)), "bf16")
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)), "bf16")
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.25)
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(s), rank, 4, "mx", keep_factors=True)
    y = R.linear(_g(x, "bf16"), p)
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "mx", 4, "bf16")
    return O.rel_fro(_np(y), ref)


@pytest.mark.parametrize("B,M,N,rank", [
    (300, 512, 576, 32),    # ragged batch, N a multiple of 192 with a partial last padded block
    (513, 320, 200, 7),     # N not a multiple of 192 (256-wide tiles), short K (2 stages < ring depth)
    (256, 256, 1000, 64),   # one K stage pair, N tail
    (1024, 1024, 384, 0),   # rank 0: no up-projection
])
def test_mx_large_batch_shapes(B, M, N, rank):
    assert _mx_case(B, M, N, rank, B + N) <= TOL["bf16"]


@pytest.mark.parametrize("B,M,N,rank", [
    (4096, 1024, 4352, 32),   # 272 tiles of 256 x 256: more tiles than compute units
    (4100, 768, 4032, 64),    # 357 ragged 256 x 192 tiles (17 x 21), two 32-wide up-projection rounds
    (2048, 512, 12288, 96),   # 512 tiles of 256 x 192, three up-projection rounds
])
def test_mx_large_batch_several_tiles_per_block(B, M, N, rank):
    """More output tiles than compute units (a compute unit runs several tiles in turn), with
    ragged tiles and ranks above 32, against the oracle."""
    assert _mx_case(B, M, N, rank, B + N) <= TOL["bf16"]


def test_mx_exact_special_case_ragged_tiles_per_block():
    """Rank 0, E2M1-grid operands (exact product) over 357 ragged tiles, more than compute units."""
    B, M, N = 4100, 256, 4032
    assert _gemm_route(B, M, N, "mx", 4, "bf16") == "mx256x192"
    x, w = _e2m1_exact_operands(np.random.default_rng(77), B, M, N)
    p = R.prepare(_g(w, "bf16"), torch.ones(M), 0, 4, "mx")
    y = R.linear(_g(x, "bf16"), p)
    bad = np.argwhere(_bits(_np(y)) != _bits(O.to_dtype(x @ w, "bf16")))
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}"


def test_mx_exact_special_case_large_batch():
    rng = np.random.default_rng(14)
    B, M, N = 520, 320, 392
    grid = O.E2M1_GRID
    x = grid[rng.integers(0, 8, (B, M))] * np.where(rng.random((B, M)) < 0.5, -1, 1)
    w = grid[rng.integers(0, 8, (M, N))] * np.where(rng.random((M, N)) < 0.5, -1, 1)
    x[:, 0::32] = np.where(rng.random((B, M // 32)) < 0.5, 6.0, -4.0)
    w[0::32, :] = np.where(rng.random((M // 32, N)) < 0.5, -6.0, 4.0)
    p = R.prepare(_g(w, "bf16"), torch.ones(M), 0, 4, "mx")
    y = R.linear(_g(x, "bf16"), p)
    assert np.array_equal(_bits(_np(y)), _bits(O.to_dtype(x @ w, "bf16")))


# ----------------------------------------------------------------------------- INT4 kernel (K >= 1536)
def _int_case(B, M, N, rank, dtype, seed):
    rng = np.random.default_rng(seed)
    x = O.to_dtype(rng.standard_normal((B, M)) * np.where(rng.random(M) < 0.01, 30.0, 1.0), dtype)
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.5)
    p = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, 4, "int", keep_factors=True)
    y = R.linear(_g(x, dtype), p)
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "int", 4, dtype)
    return O.rel_fro(_np(y), ref)


@pytest.mark.parametrize("B,M,N,rank,dtype", [
    (70, 1536, 200, 32, "bf16"),   # K stages = stages in flight: no steady-state iteration
    (64, 1792, 130, 0, "bf16"),    # 7 stages: one steady iteration (odd), rank 0
    (130, 2048, 200, 96, "f32"),   # 8 stages, f32 io, up-projection beyond the prefetched steps
    (256, 2560, 4104, 32, "bf16"), # ragged N across the last 64-column tile
])
def test_int4_gemm_shapes(B, M, N, rank, dtype):
    assert _int_case(B, M, N, rank, dtype, B + M) <= TOL[dtype]


# ----------------------------------------------------------------------------- decode-batch MXFP4 kernel
@pytest.mark.parametrize("B,M,N,rank", [
    (16, 8192, 1024, 128),  # decode kernel: split-K partials of down, two up-projection rounds
    (40, 3072, 200, 160),   # decode kernel, four row tiles and waves, three up-projection rounds
    (100, 1024, 576, 64),   # 128-row tiles, N a multiple of 192
    (300, 768, 1000, 32),   # 256 x 256 tiles, ragged B and N
    (520, 1536, 768, 96),   # 256 x 192 tiles, three 32-wide up-projection steps
])
def test_mx_f32_io_shapes(B, M, N, rank):
    """MXFP4 with float32 io through the MXFP4 kernels: the up-projection takes f32 down and
    L2 split into bf16 high and low parts (three bf16 products, relative error near 2^-16).
    Measured against the oracle: 3e-7 to 5e-6. The bound is 1e-4, far inside the float32
    tolerance; rounding down and L2 to plain bf16 (relative error near 2^-9 on the low-rank
    term) would exceed it."""
    rng = np.random.default_rng(B + N + rank)
    x = O.to_dtype(rng.standard_t(3, (B, M)), "f32")
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)), "f32")
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.25)
    p = R.prepare(_g(w, "f32"), torch.from_numpy(s), rank, 4, "mx", keep_factors=True)
    y = R.linear(_g(x, "f32"), p)
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "mx", 4, "f32")
    assert O.rel_fro(_np(y), ref) <= 1e-4


@pytest.mark.parametrize("B,M,N,rank", [
    (1, 9216, 1000, 32),    # single row; each of the 8 waves gets 9 K stages (one batch of 8 + a tail)
    (17, 2048, 520, 16),    # two 16-row tiles, the second with one live row
    (33, 4352, 300, 128),   # four row tiles (4 waves); uneven K quarters (8 and 9 stages)
    (64, 1024, 4104, 0),    # full 64 rows, rank 0, N tail inside the last 32-column block
    (5, 1024, 640, 48),     # K in one chunk: the finished down-projection, no split-K partials
    (12, 16384, 256, 200),  # 16 split-K partials (more than are prefetched); a second up-projection round
    (40, 3072, 200, 160),   # four row tiles, three up-projection rounds of 64 rank columns
])
def test_mx_decode_batch_shapes(B, M, N, rank):
    assert _mx_case(B, M, N, rank, B + N) <= TOL["bf16"]


# ----------------------------------------------------------------------------- scale calibration
def _ulp32(a):
    a = np.abs(np.asarray(a, np.float32))
    return np.spacing(a)


@pytest.mark.parametrize("cid,alpha", [(1, 0.5), (2, 0.5), (3, 0.25), (5, 0.25), (4, 0.9)])
def test_calibrate_scale_matches_oracle(cid, alpha):
    """Exact maxima; the power and quotient in binary64 on both sides, so the float32 scales
    agree bit for bit unless the two binary64 results straddle a float32 rounding boundary
    (then by one ulp)."""
    wl = WORKLOADS[cid]
    x, w, _ = make_inputs(cid)
    got = _np(R.calibrate_scale(_g(x, wl.dtype), _g(w, wl.dtype), alpha))
    want = O.calibrate_scale(x, w, alpha)
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(diff <= _ulp32(want)), "more than one float32 ulp apart"
    assert np.mean(got == want) >= 0.999


def test_calibrate_scale_edges():
    """Zero columns and rows give 1; strided x; ragged M (not a multiple of 64) and N."""
    rng = np.random.default_rng(22)
    B, M, N = 37, 131, 45
    x = O.to_dtype(rng.standard_t(3, (B, M)) * 10.0 ** rng.integers(-2, 3, (B, M)), "bf16")
    w = O.to_dtype(rng.standard_normal((M, N)), "bf16")
    x[:, 7] = 0.0
    w[100] = 0.0
    for alpha in (0.0, 0.5, 1.0):
        xt = _g(x.T.copy(), "bf16").t()  # column-major x: the binding copies it
        got = _np(R.calibrate_scale(xt, _g(w, "bf16"), alpha))
        want = O.calibrate_scale(x, w, alpha)
        assert got[7] == 1.0 and got[100] == 1.0
        assert np.all(np.abs(got.astype(np.float64) - want) <= _ulp32(want))
    big = torch.zeros(B, M + 9, dtype=torch.float32, device=dev())
    big[:, 3:3 + M] = _g(x, "f32")
    got = _np(R.calibrate_scale(big[:, 3:3 + M], _g(w, "f32"), 0.5))  # row stride M + 9, unaligned rows
    assert np.all(np.abs(got.astype(np.float64) - O.calibrate_scale(x, w, 0.5)) <= _ulp32(O.calibrate_scale(x, w, 0.5)))


# ----------------------------------------------------------------------------- toy experiment
def test_toy_experiment_through_library():
    """The exercise page's toy experiment run through the library: the same ordering as the
    page describes (two-branch below smoothing-only below naive W4A4, falling with rank), the
    oracle's numbers for naive and smoothing-only (bit-exact quantisation), the two-branch
    errors within 2% of the oracle's (different but equivalent truncated-SVD bases), and the
    singular values from the library's split equal to numpy's."""
    dev()
    import bench

    r = bench.toy_experiment()
    lib, orc = r["library"], r["oracle"]
    assert lib["naive_w4a4"] == pytest.approx(orc["naive_w4a4"], rel=1e-12)
    assert lib["smoothing_only"] == pytest.approx(orc["smoothing_only"], rel=1e-12)
    assert np.allclose(lib["two_branch"], orc["two_branch"], rtol=0.02)
    tb = lib["two_branch"]
    assert tb[6] < tb[0] and tb[4] < lib["smoothing_only"] < lib["naive_w4a4"]
    for name in ("W", "smoothed_W"):
        a = np.array(r["singular_values_library"][name])
        b = np.array(r["singular_values_oracle"][name])
        assert np.allclose(a[:8], b[:8], rtol=1e-5, atol=1e-6 * b[0])


# ----------------------------------------------------------------------------- operand arrays past 2 GiB
@pytest.mark.parametrize("fmt", ["int", "mx"])
def test_activation_codes_past_2gib_take_the_generic_kernel(fmt):
    """262144 x 16384 bf16 activations (8 GiB) give a 2 GiB activation-code array, past the
    32-bit buffer offsets of the INT and MXFP4 kernels, so the residual GEMM runs on the
    generic kernel (64-bit addressing). Unit smoothing and |x| <= 4 except one planted 8 in
    a sampled row, so the INT per-tensor maximum of the sample is the tensor's; sampled rows
    at the start, middle and end are compared with the oracle."""
    B, M, N, rank = 262144, 16384, 64, 16
    torch.manual_seed(5)
    xg = torch.randn((B, M), dtype=torch.bfloat16, device=dev()).clamp_(-4, 4)
    rows = np.array([0, 1, 77, B // 2, B // 2 + 1, B - 2, B - 1])
    xg[B // 2, 1234] = 8.0
    rng = np.random.default_rng(6)
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 2)) @ rng.standard_normal((2, N)), "bf16")
    s = np.ones(M, np.float32)
    p = R.prepare(_g(w, "bf16"), torch.from_numpy(s), rank, 4, fmt, keep_factors=True)
    y = R.linear(xg, p)
    torch.cuda.synchronize()
    got = _np(y[torch.from_numpy(rows).to(dev())])
    xs = _np(xg[torch.from_numpy(rows).to(dev())])
    del xg, y
    torch.cuda.empty_cache()
    ref = O.forward_ref(xs, s, _np(p.left), _np(p.right), _np(p.residual), fmt, 4, "bf16")
    assert O.rel_fro(got, ref) <= TOL["bf16"]


# ----------------------------------------------------------------------------- output bias
@pytest.mark.parametrize("B,M,N,fmt,dtype", [
    (40, 2048, 300, "int", "bf16"),   # INT4 kernel
    (512, 512, 576, "mx", "bf16"),    # large-batch MXFP4 kernel (256 x 192 tiles)
    (16, 1024, 200, "mx", "bf16"),    # decode MXFP4 kernel
    (48, 320, 130, "int", "f32"),     # INT kernel, short K (two stages)
])
def test_linear_bias_matches_oracle(B, M, N, fmt, dtype):
    rng = np.random.default_rng(B + N)
    x = O.to_dtype(rng.standard_t(3, (B, M)), dtype)
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 2)) @ rng.standard_normal((2, N)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.5)
    bias = O.to_dtype(rng.standard_normal(N), dtype)
    p = R.prepare(_g(w, dtype), torch.from_numpy(s), 32, 4, fmt, keep_factors=True)
    xg = _g(x, dtype)
    y = R.linear(xg, p, bias=_g(bias, dtype))
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), fmt, 4, dtype, bias=bias)
    assert O.rel_fro(_np(y), ref) <= TOL[dtype]
    # without the bias the result is the plain operator
    y0 = R.linear(xg, p)
    ref0 = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), fmt, 4, dtype)
    assert O.rel_fro(_np(y0), ref0) <= TOL[dtype]


def test_linear_bias_exact_special_case():
    """Rank 0, unit scale, integer x and W with max 7 (exact INT4 product) plus an integer
    bias: Y = x @ W + bias bit for bit."""
    rng = np.random.default_rng(23)
    B, M, N = 40, 320, 300
    x = rng.integers(-7, 8, (B, M)).astype(np.float32)
    w = rng.integers(-7, 8, (M, N)).astype(np.float32)
    x[0, 0] = w[0, 0] = 7
    bias = rng.integers(-50, 50, N).astype(np.float32)
    p = R.prepare(_g(w, "f32"), torch.ones(M), 0, 4, "int")
    y = R.linear(_g(x, "f32"), p, bias=_g(bias, "f32"))
    want = x.astype(np.float64) @ w.astype(np.float64) + bias
    assert np.array_equal(_bits(_np(y)), _bits(want.astype(np.float32)))


# ----------------------------------------------------------------------------- truncated SVD on the GPU
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prepare_with_gpu_svd(dtype):
    """The randomized route on the GPU (float64): the split meets the Eckart-Young bound like
    the host route's, its factors have the split's structure (L2 rows orthonormal, L1 columns
    orthogonal, sigma descending), and the prepared operator matches the oracle. The two routes
    orthonormalise their panels differently, so their rank-r factors may differ where the
    singular values inside the noise bulk are close (several results are correct)."""
    rng = np.random.default_rng(24)
    M, N, rank = 1024, 768, 32
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + (rng.standard_normal((M, 6)) * 0.3) @ rng.standard_normal((6, N)), dtype)
    x = O.to_dtype(rng.standard_t(3, (64, M)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.5)
    pg = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, 4, "int", keep_factors=True, svd_on_gpu=True)
    ph = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, 4, "int", keep_factors=True)
    ws = O.smooth_weight(w, s, dtype).astype(np.float64)
    sig2 = np.sort(np.linalg.eigvalsh(ws.T @ ws))[::-1]
    tail = np.sqrt(np.clip(sig2[rank:], 0, None).sum())
    ulp = {"f32": 2.0**-24, "bf16": 2.0**-8}[dtype]
    for p_ in (pg, ph):
        res = _np(p_.residual).astype(np.float64)
        assert abs(np.linalg.norm(res) - tail) <= 1e-3 * tail + 4 * ulp * np.linalg.norm(ws)
    l1, l2 = _np(pg.left).astype(np.float64), _np(pg.right).astype(np.float64)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.abs(l2 @ l2.T - np.eye(rank)).max() <= tol
    g = l1.T @ l1
    sig = np.sqrt(np.diag(g))
    assert np.abs(g - np.diag(np.diag(g))).max() <= tol * sig[0] ** 2
    assert np.all(sig[:-1] >= sig[1:] * (1 - tol))
    y = R.linear(_g(x, dtype), pg)
    ref = O.forward_ref(x, s, _np(pg.left), _np(pg.right), _np(pg.residual), "int", 4, dtype)
    assert O.rel_fro(_np(y), ref) <= TOL[dtype]


def test_prepare_gpu_svd_eckart_young_at_decode_shape():
    """The GPU split at 8192 x 8192, rank 128 (the decode workload's weight, where the rank
    cuts into the noise bulk): ||R||_F within 1e-3 of the exact tail sqrt(sum_{i>r} sigma_i^2),
    taken from the float64 Gram matrix's eigenvalues on the host (no SVD)."""
    import scipy.linalg

    wl = WORKLOADS[5]
    _, w, s = make_inputs(5, B=64)
    p = R.prepare(_g(w, wl.dtype), torch.from_numpy(s), wl.rank, wl.bits, wl.fmt, keep_factors=True, svd_on_gpu=True)
    ws = O.smooth_weight(w, s, wl.dtype).astype(np.float64)
    gram = ws.T @ ws
    n = gram.shape[0]
    top = scipy.linalg.eigh(gram, eigvals_only=True, subset_by_index=[n - wl.rank, n - 1])
    tail = np.sqrt(np.sum(ws * ws) - top.sum())
    res = np.linalg.norm(_np(p.residual).astype(np.float64))
    print(f"decode-shape GPU split: ||R|| {res:.6f}, tail {tail:.6f}, rel {(res - tail) / tail:.2e}")
    assert abs(res - tail) <= 1e-3 * tail


# ----------------------------------------------------------------------------- two-level MXFP4 scaling
def _two_level_case(B, M, N, rank, dtype, gx, seed, bias=False):
    rng = np.random.default_rng(seed)
    x = O.to_dtype(rng.standard_t(3, (B, M)), dtype)
    w = O.to_dtype(0.02 * rng.standard_normal((M, N)) + 0.05 * rng.standard_normal((M, 3)) @ rng.standard_normal((3, N)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.25)
    b = O.to_dtype(rng.standard_normal(N), dtype) if bias else None
    p = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, 4, "mx", keep_factors=True, x_global_scale=gx)
    y = R.linear(_g(x, dtype), p, bias=None if b is None else _g(b, dtype))
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), "mx", 4, dtype, bias=b, x_global_scale=gx)
    return O.rel_fro(_np(y), ref)


@pytest.mark.parametrize("B,M,N,rank,dtype,gx,bias", [
    (512, 512, 576, 32, "bf16", 1.37, False),   # large-batch kernel
    (300, 1024, 392, 0, "bf16", 0.011, True),   # large-batch kernel, rank 0, bias
    (16, 1024, 200, 48, "bf16", 5.5, True),     # decode kernel, bias
    (33, 4352, 300, 128, "bf16", 0.7, False),   # decode kernel, split-K partials
    (100, 640, 300, 32, "bf16", 1.37, False),   # general kernel (64 < B < 256)
    (40, 320, 130, 16, "f32", 3.1, True),       # general kernel, float32 io
])
def test_two_level_parity(B, M, N, rank, dtype, gx, bias):
    err = _two_level_case(B, M, N, rank, dtype, gx, B + N, bias)
    print(f"two-level B={B} M={M} N={N} rank={rank} {dtype}: rel Frobenius error {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("cid,rows", [(3, 256), (5, None)])
def test_two_level_parity_workloads(cid, rows):
    wl = WORKLOADS[cid]
    x, w, s = make_inputs(cid)
    xs = O.smooth_activations(x, s, wl.dtype)
    gx = float(np.float32(448.0 / np.max(np.abs(xs))))  # a calibrated, non-power-of-two g_x
    p = R.prepare(_g(w, wl.dtype), torch.from_numpy(s), wl.rank, 4, "mx", keep_factors=True, x_global_scale=gx)
    y = _np(R.linear(_g(x, wl.dtype), p))
    sel = np.arange(x.shape[0]) if rows is None else np.random.default_rng(1).choice(x.shape[0], rows, replace=False)
    ref = O.forward_ref(x[sel], s, _np(p.left), _np(p.right), _np(p.residual), "mx", 4, wl.dtype, x_global_scale=gx)
    err = O.rel_fro(y[sel], ref)
    print(f"two-level workload {cid}: rel Frobenius error {err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("cid,B,gx", [(5, None, 0.37), (3, 512, 1.37), (3, 100, 9.0)])
def test_two_level_workspace_codes_bit_exact(cid, B, gx):
    """svdq_linear's activation codes under two-level scaling are the MXFP4 codes of the
    binary32 products RN(X^ * g_x) (white-box: the workspace begins with them, in 16-row
    tiles)."""
    wl = WORKLOADS[cid]
    x, w, s = make_inputs(cid, B=B)
    p = R.prepare(_g(w, wl.dtype), torch.from_numpy(s), wl.rank, 4, "mx", x_global_scale=gx)
    ws = torch.full((R.workspace_bytes(x.shape[0], p),), 0xA5, dtype=torch.uint8, device=dev())
    R.linear(_g(x, wl.dtype), p, workspace=ws)
    torch.cuda.synchronize()
    z = O.smooth_activations(x, s, wl.dtype).astype(np.float32) * np.float32(gx)
    c, _ = O.quantize_mx(z)
    want = O.pack_nibbles(c)
    got = _workspace_codes(ws, x.shape[0], x.shape[1], True)
    assert np.array_equal(got[:, : want.shape[1]], want)
    assert not got[:, want.shape[1]:].any()


@pytest.mark.parametrize("B", [520, 16, 100])
def test_two_level_exact_special_case(B):
    """Rank 0, unit scale, x and W on the E2M1 grid with a 6 in every block: g_R = 2 and
    g_x = 1/4 keep every value exact and alpha = 2, so Y = x @ W bit for bit through each
    MXFP4 kernel."""
    rng = np.random.default_rng(31 + B)
    M, N = 320, 392
    grid = O.E2M1_GRID
    x = grid[rng.integers(0, 8, (B, M))] * np.where(rng.random((B, M)) < 0.5, -1, 1)
    w = grid[rng.integers(0, 8, (M, N))] * np.where(rng.random((M, N)) < 0.5, -1, 1)
    x[:, 0::32] = np.where(rng.random((B, M // 32)) < 0.5, 6.0, -4.0)
    w[0::32, :] = np.where(rng.random((M // 32, N)) < 0.5, -6.0, 4.0)
    p = R.prepare(_g(w, "bf16"), torch.ones(M), 0, 4, "mx", x_global_scale=0.25)
    glob = p.section(_lib.SEC_GLOBAL)[:16].cpu().numpy().view(np.float32)
    assert glob.tolist() == [0.25, 2.0, 2.0, 0.0]
    y = R.linear(_g(x, "bf16"), p)
    assert np.array_equal(_bits(_np(y)), _bits(O.to_dtype(x @ w, "bf16")))


# ----------------------------------------------------------------------------- seeded shape sweep
def _sweep_cases(n=24, seed=2026):
    """Ragged shapes drawn from a fixed seed: B in [1, 600] (every kernel route), M in [1, 2600]
    (short and multi-stage K, partial 32-blocks), N in [1, 700], rank in [0, min(M, N, 80)],
    both formats, INT widths 2-8, both dtypes, and a bias on every third case."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        fmt = "mx" if c % 2 else "int"
        dtype = "f32" if c % 5 == 0 else "bf16"
        bits = 4 if fmt == "mx" else int(rng.integers(2, 9))
        B = int(rng.choice([1, 3, 16, 17, 40, 64, 65, 130, 255, 256, 300, 600]))
        M = int(rng.integers(1, 2601))
        N = int(rng.integers(1, 701))
        rank = int(rng.integers(0, min(M, N, 80) + 1))
        out.append((c, B, M, N, rank, fmt, bits, dtype, c % 3 == 0))
    return out


def _sweep_cases_large(n=8, seed=2027):
    """Larger ragged shapes from a fixed seed, for the large-batch routes: B in [700, 4200], N in
    [1000, 4200] (so INT takes the large tiles whenever 64 x 64 tiles would need four rounds,
    and MXFP4 meets every tile shape), M in [64, 800], rank in [0, 64], INT widths 2-8, both
    dtypes, a bias on every third case."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        fmt = "mx" if c % 2 else "int"
        dtype = "f32" if c % 3 == 1 else "bf16"
        bits = 4 if fmt == "mx" else int(rng.integers(2, 9))
        B = int(rng.integers(700, 4201))
        M = int(rng.integers(64, 801))
        N = int(rng.integers(1000, 4201))
        rank = int(rng.integers(0, 65))
        out.append((100 + c, B, M, N, rank, fmt, bits, dtype, c % 3 == 0))
    return out


@pytest.mark.parametrize("c,B,M,N,rank,fmt,bits,dtype,bias", _sweep_cases() + _sweep_cases_large())
def test_parity_shape_sweep(c, B, M, N, rank, fmt, bits, dtype, bias):
    rng = np.random.default_rng(1000 + c)
    x = O.to_dtype(rng.standard_t(3, (B, M)), dtype)
    w = O.to_dtype(0.05 * rng.standard_normal((M, N)) + 0.1 * rng.standard_normal((M, 2)) @ rng.standard_normal((2, N)), dtype)
    from workloads import smoothing_scale
    s = smoothing_scale(x, w, 0.5)
    b = O.to_dtype(rng.standard_normal(N), dtype) if bias else None
    print(f"case {c}: B={B} M={M} N={N} rank={rank} {fmt}{bits} {dtype} bias={bias}", flush=True)
    p = R.prepare(_g(w, dtype), torch.from_numpy(s), rank, bits, fmt, keep_factors=True)
    xg = _g(x, dtype)
    bg = None if b is None else _g(b, dtype)
    y = R.linear(xg, p, bias=bg)
    y2 = R.linear(xg, p, bias=bg)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    ref = O.forward_ref(x, s, _np(p.left), _np(p.right), _np(p.residual), fmt, bits, dtype, bias=b)
    err = O.rel_fro(_np(y), ref)
    print(f"case {c}: rel Frobenius error {err:.3e}", flush=True)
    assert err <= TOL[dtype]


# ----------------------------------------------------------------------------- measured ceilings
def test_ceiling_probes_run_and_count_their_work():
    """svdq_ceiling: the FP4 and INT8 MFMA loops and the read stream run through the C ABI and
    report the work of one launch (flops: CUs x 2 blocks x 4 waves x iterations x 8 MFMAs x
    the instruction's flops; bytes: the buffer rounded down to 16)."""
    lib = _lib.load()
    d = dev()
    cus = torch.cuda.get_device_properties(d).multi_processor_count
    scratch = torch.empty(1 << 22, dtype=torch.uint8, device=d)
    stream = ctypes.c_void_p(torch.cuda.current_stream(d).cuda_stream)
    work = ctypes.c_double()
    for kind, per in ((0, 2 * 32 * 32 * 64), (1, 2 * 32 * 32 * 32)):
        assert lib.svdq_ceiling(kind, 3, None, 0, ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), stream,
                                ctypes.byref(work)) == 0, lib.svdq_last_error()
        assert work.value == cus * 2 * 4 * 3 * 8 * per
    buf = torch.arange(1 << 20, dtype=torch.int32, device=d)
    assert lib.svdq_ceiling(2, 64, ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4 + 7,
                            ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), stream, ctypes.byref(work)) == 0
    assert work.value == buf.numel() * 4
    # a scratch buffer too small for the launch is refused
    assert lib.svdq_ceiling(2, 1 << 14, ctypes.c_void_p(buf.data_ptr()), 1024, ctypes.c_void_p(scratch.data_ptr()),
                            1024, stream, ctypes.byref(work)) == _lib.SVDQ_EINVAL
    torch.cuda.synchronize()
