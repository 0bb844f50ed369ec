"""Host preparation of libsvdq (C++) against the oracle, on the CPU.

svdq_prepare folds the smoothing scale into W, splits it with the library's truncated
SVD and quantises the residual; the oracle checks each stage on the library's exported
factors: the fold and the residual codes/scales bit-exactly, the split by Eckart-Young.
"""
import zlib

import numpy as np
import pytest
import torch

import rank_bit_residual_amd as R
from rank_bit_residual_amd import _lib
from oracle import svdquant as O
from workloads import make_inputs, to_bf16_values

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(TD[dtype])


def _np(t):
    return t.to(torch.float32).numpy()


def _case(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "toy":
        x, w, s = make_inputs(1)
        return w, s, "f32"
    M, N, dtype = {"bf16_small": (320, 200, "bf16"), "bf16_ragged": (100, 70, "bf16"), "f32_mid": (600, 640, "f32")}[name]
    w = 0.02 * rng.standard_normal((M, N)) + (rng.standard_normal((M, 4)) * 0.3) @ rng.standard_normal((4, N))
    x = rng.standard_t(3, (32, M))
    x[:, :3] *= 40
    w = w.astype(np.float32)
    x = x.astype(np.float32)
    if dtype == "bf16":
        w, x = to_bf16_values(w), to_bf16_values(x)
    from workloads import smoothing_scale
    return w, smoothing_scale(x, w, 0.25), dtype


def _prep(w, s, dtype, rank, fmt, bits):
    return R.prepare(_t(w, dtype), torch.from_numpy(s), rank, bits, fmt, device="cpu", keep_factors=True)


def _sections(p):
    M, N = p.M, p.N
    Kp, Np, rp = -(-M // 256) * 256, -(-N // 256) * 256, -(-p.rank // 32) * 32
    nib = p.fmt == "mx" or p.bits <= 4
    rb = Kp // 2 if nib else Kp
    codes = p.section(_lib.SEC_RCODES)[: Np * rb].numpy()
    if p.fmt == "mx":
        # 1 KB tiles: [Np/16][Kp/128][16 columns][64 bytes]
        codes = codes.reshape(Np // 16, Kp // 128, 16, 64).transpose(0, 2, 1, 3)
    codes = codes.reshape(Np, rb)
    dt = np.float32 if p.dtype == torch.float32 else np.uint16
    E = 16 // np.dtype(dt).itemsize
    # L1^T tiles: [rp/16][Kp/128][32/E K-slices][4 blocks][16 rows][E]
    tiles = p.section(_lib.SEC_L1T).numpy().view(dt)[: rp * Kp].reshape(rp // 16, Kp // 128, 32 // E, 4, 16, E)
    l1t = tiles.transpose(0, 4, 1, 3, 2, 5).reshape(rp, Kp)
    l2t = p.section(_lib.SEC_L2T).numpy().view(dt)[: Np * rp].reshape(Np, rp)
    return codes, l1t, l2t, Kp, Np, rp, nib


@pytest.mark.parametrize("name", ["toy", "bf16_small", "bf16_ragged"])
def test_fold_is_bit_exact(name):
    w, s, dtype = _case(name)
    p = _prep(w, s, dtype, 0, "int", 4)
    want = O.smooth_weight(w, s, dtype)
    assert np.array_equal(_np(p.residual).view(np.uint32), want.view(np.uint32))
    assert p.left.shape == (w.shape[0], 0) and p.right.shape == (0, w.shape[1])


@pytest.mark.parametrize("name,rank,fmt,bits", [
    ("toy", 8, "int", 4), ("toy", 0, "int", 4), ("toy", 48, "int", 4), ("toy", 8, "int", 8), ("toy", 5, "int", 2),
    ("bf16_small", 32, "mx", 4), ("bf16_small", 32, "int", 4), ("bf16_ragged", 7, "mx", 4), ("bf16_ragged", 40, "int", 6),
    ("f32_mid", 16, "mx", 4),
])
def test_residual_codes_bit_exact(name, rank, fmt, bits):
    w, s, dtype = _case(name)
    p = _prep(w, s, dtype, rank, fmt, bits)
    M, N = w.shape
    res = _np(p.residual)
    codes, l1t, l2t, Kp, Np, rp, nib = _sections(p)
    if fmt == "int":
        c, sr = O.quantize_int(res, bits, dtype)
        want = O.pack_int_codes(c.T, bits)
        got_s = p.section(_lib.SEC_RSCALES)[:4].numpy().view(np.float32)[0]
        assert got_s == np.float32(sr)
    else:
        c, sb = O.quantize_mx(res.T)
        want = O.pack_nibbles(c)
        nb = -(-M // 32)
        tiled = p.section(_lib.SEC_RSCALES)[: Np * (Kp // 32)].numpy()
        # stage-tiled layout: [Np/64][Kp/128][64 rows][4 blocks]
        scales = tiled.reshape(Np // 64, Kp // 128, 64, 4).transpose(0, 2, 1, 3).reshape(Np, Kp // 32)
        assert np.array_equal(scales[:N, :nb], sb)
        assert not scales[N:].any() and not scales[:, nb:].any()
    assert np.array_equal(codes[:N, : want.shape[1]], want)
    assert not codes[N:].any() and not codes[:, want.shape[1]:].any()
    # transposed, zero-padded factors
    if dtype == "f32":
        l1, l2 = p.left.numpy(), p.right.numpy()
        assert np.array_equal(l1t[:rank, :M], l1.T) and np.array_equal(l2t[:N, :rank], l2.T)
    else:
        l1 = p.left.view(torch.int16).numpy().view(np.uint16)
        l2 = p.right.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(l1t[:rank, :M], l1.T) and np.array_equal(l2t[:N, :rank], l2.T)
    assert not l1t[rank:].any() and not l1t[:, M:].any() and not l2t[N:].any() and not l2t[:, rank:].any()


@pytest.mark.parametrize("name,rank", [("toy", 1), ("toy", 8), ("toy", 30), ("bf16_small", 32), ("f32_mid", 16)])
def test_split_eckart_young(name, rank):
    w, s, dtype = _case(name)
    p = _prep(w, s, dtype, rank, "int", 4)
    ws = O.smooth_weight(w, s, dtype).astype(np.float64)
    sig2 = np.sort(np.linalg.eigvalsh(ws.T @ ws))[::-1]
    tail = np.sqrt(np.clip(sig2[rank:], 0, None).sum())
    res = _np(p.residual).astype(np.float64)
    # the residual is exactly D(ws - left @ right) from the exported factors
    want_res = O.residual_of(ws.astype(np.float32), _np(p.left), _np(p.right), dtype)
    assert np.array_equal(_np(p.residual), want_res)
    # Eckart-Young: ||R|| equals the singular-value tail, up to the split's own accuracy
    # (exact for the Jacobi route, 1e-3 relative for the randomized route) plus the rounding
    # of the stored factors to the dtype, which is relative to ||ws||
    err = abs(np.linalg.norm(res) - tail)
    algo = 1e-9 if min(w.shape) <= 512 else 1e-3
    ulp = {"f32": 2.0**-24, "bf16": 2.0**-8}[dtype]
    assert err <= algo * tail + 4 * ulp * np.linalg.norm(ws), (err, tail)


def test_split_full_rank_and_factor_structure():
    w, s, dtype = _case("toy")
    ws = O.smooth_weight(w, s, dtype)
    left, right, res = R.split_weight(torch.from_numpy(ws), 48)
    assert np.linalg.norm(res.numpy()) / np.linalg.norm(ws) <= 1e-5
    l, r = left.numpy().astype(np.float64), right.numpy().astype(np.float64)
    assert np.allclose(r @ r.T, np.eye(48), atol=1e-5)
    g = l.T @ l
    assert np.allclose(g - np.diag(np.diag(g)), 0, atol=1e-5 * np.abs(g).max())
    assert np.all(np.diff(np.sqrt(np.diag(g))) <= 1e-5 * np.sqrt(g.max()))


def test_split_weight_matches_prepare_and_is_deterministic():
    w, s, dtype = _case("bf16_small")
    ws = O.smooth_weight(w, s, dtype)
    a = R.split_weight(_t(ws, dtype), 32)
    b = R.split_weight(_t(ws, dtype), 32)
    p = _prep(w, s, dtype, 32, "mx", 4)
    for u, v, q in zip(a, b, (p.left, p.right, p.residual)):
        assert torch.equal(u, v) and torch.equal(u, q)
        assert u.dtype == torch.bfloat16


def test_split_rank0():
    w, s, dtype = _case("toy")
    left, right, res = R.split_weight(torch.from_numpy(w), 0)
    assert left.shape == (64, 0) and right.shape == (0, 48)
    assert torch.equal(res, torch.from_numpy(w))


def test_inputs_unchanged():
    w, s, dtype = _case("bf16_small")
    wt, st = _t(w, dtype), torch.from_numpy(s.copy())
    w0, s0 = wt.clone(), st.clone()
    R.prepare(wt, st, 8, 4, "mx", device="cpu")
    R.split_weight(wt, 8)
    assert torch.equal(wt, w0) and torch.equal(st, s0)


@pytest.mark.parametrize("rank", [-1, 49, True, 3.0])
def test_rank_errors(rank):
    w, s, _ = _case("toy")
    with pytest.raises(ValueError):
        R.split_weight(torch.from_numpy(w), rank)
    with pytest.raises(ValueError):
        R.prepare(torch.from_numpy(w), torch.from_numpy(s), rank, device="cpu")


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan")])
def test_scale_errors(bad):
    w, s, _ = _case("toy")
    s = s.copy()
    s[5] = bad
    with pytest.raises(ValueError):
        R.prepare(torch.from_numpy(w), torch.from_numpy(s), 4, device="cpu")


def test_format_and_dtype_errors():
    w, s, _ = _case("toy")
    wt, st = torch.from_numpy(w), torch.from_numpy(s)
    for fmt, bits in (("int", 1), ("int", 9), ("mx", 3), ("fp8", 4)):
        with pytest.raises(ValueError):
            R.prepare(wt, st, 4, bits, fmt, device="cpu")
    with pytest.raises(TypeError):
        R.prepare(wt.double(), st, 4, device="cpu")
    with pytest.raises(ValueError):
        R.prepare(wt, st[:10], 4, device="cpu")
    with pytest.raises(ValueError):
        R.prepare(wt[0], st, 4, device="cpu")


def test_device_calls_need_a_gpu():
    w, s, _ = _case("toy")
    x = torch.zeros(2, 64)
    with pytest.raises(RuntimeError):
        R.smooth_inputs(x, torch.from_numpy(w), torch.from_numpy(s))
    with pytest.raises(RuntimeError):
        R.fake_quantize(x)
    p = _prep(w, s, "f32", 4, "int", 4)
    with pytest.raises(RuntimeError):
        R.linear(x, p)


@pytest.mark.parametrize("name,rank,fmt,bits", [("bf16_small", 32, "mx", 4), ("toy", 8, "int", 4),
                                                ("f32_mid", 16, "mx", 4), ("bf16_ragged", 7, "int", 6)])
def test_linear_layout_prepare_gives_the_same_blob(name, rank, fmt, bits):
    """A weight handed over in the Linear layout [N, M] (W transposed) prepares to the same
    bytes, and the same factors, as W itself."""
    w, s, dtype = _case(name)
    a = R.prepare(_t(w, dtype), torch.from_numpy(s), rank, bits, fmt, device="cpu", keep_factors=True)
    b = R.prepare(_t(w.T.copy(), dtype), torch.from_numpy(s), rank, bits, fmt, device="cpu", keep_factors=True,
                  layout="nm")
    assert torch.equal(a.blob, b.blob)
    assert torch.equal(a.residual, b.residual) and (rank == 0 or torch.equal(a.left, b.left))
    with pytest.raises(ValueError):
        R.prepare(_t(w.T.copy(), dtype), torch.from_numpy(s), rank, bits, fmt, device="cpu", layout="km")


# ----------------------------------------------------------------------------- two-level MXFP4 scaling
def _glob(p):
    return p.section(_lib.SEC_GLOBAL)[:16].numpy().view(np.float32)


@pytest.mark.parametrize("name,rank,fmt,bits", [("toy", 8, "int", 4), ("bf16_small", 32, "mx", 4)])
def test_plain_preparation_has_unit_global_scales(name, rank, fmt, bits):
    w, s, dtype = _case(name)
    assert _glob(_prep(w, s, dtype, rank, fmt, bits)).tolist() == [1.0, 1.0, 1.0, 0.0]


@pytest.mark.parametrize("name,rank,gx", [("bf16_small", 32, 0.37), ("bf16_ragged", 7, 3.0), ("f32_mid", 16, 1.0),
                                          ("toy", 0, 2.0 ** -20)])
def test_two_level_blob_matches_oracle(name, rank, gx):
    """Global scales, residual codes and block scales of RN(R * g_R), and the up-projection
    factor divided by alpha, bit for bit against the oracle; L1 and the unscaled factors are
    those of the plain preparation."""
    w, s, dtype = _case(name)
    M, N = w.shape
    p = R.prepare(_t(w, dtype), torch.from_numpy(s), rank, 4, "mx", device="cpu", keep_factors=True,
                  x_global_scale=gx)
    plain = _prep(w, s, dtype, rank, "mx", 4)
    res = _np(p.residual)
    assert torch.equal(p.residual, plain.residual)
    gr = O.two_level_residual_scale(res)
    alpha = O.two_level_alpha(gx, gr)
    assert _glob(p).tolist() == [np.float32(gx), gr, alpha, 0.0]
    codes, l1t, l2t, Kp, Np, rp, _ = _sections(p)
    c, sb = O.quantize_mx((res * gr).T)
    want = O.pack_nibbles(c)
    assert np.array_equal(codes[:N, : want.shape[1]], want)
    assert not codes[N:].any() and not codes[:, want.shape[1]:].any()
    nb = -(-M // 32)
    tiled = p.section(_lib.SEC_RSCALES)[: Np * (Kp // 32)].numpy()
    scales = tiled.reshape(Np // 64, Kp // 128, 64, 4).transpose(0, 2, 1, 3).reshape(Np, Kp // 32)
    assert np.array_equal(scales[:N, :nb], sb)
    pc, pl1t, pl2t = _sections(plain)[:3]
    assert np.array_equal(l1t, pl1t)
    if rank:
        up = O.to_dtype(_np(p.right).astype(np.float64) / float(alpha), dtype)
        if dtype == "bf16":
            up = (up.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(l2t[:N, :rank], up.T)
        assert torch.equal(p.right, plain.right) and torch.equal(p.left, plain.left)
    assert not l2t[N:].any() and not l2t[:, rank:].any()


@pytest.mark.parametrize("gx", [0.0, -1.0, float("inf"), float("nan"), 2.0 ** 65, 2.0 ** -65])
def test_two_level_rejects_global_scales_out_of_range(gx):
    w, s, dtype = _case("toy")
    with pytest.raises(ValueError):
        R.prepare(_t(w, dtype), torch.from_numpy(s), 8, 4, "mx", device="cpu", x_global_scale=gx)


def test_two_level_needs_mx_and_the_host_split():
    w, s, dtype = _case("toy")
    with pytest.raises(ValueError):
        R.prepare(_t(w, dtype), torch.from_numpy(s), 8, 4, "int", device="cpu", x_global_scale=1.0)
    with pytest.raises(ValueError):
        R.prepare(_t(w.T.copy(), dtype), torch.from_numpy(s), 8, 4, "mx", device="cpu", layout="nm",
                  x_global_scale=1.0)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_split_eckart_young_at_workload_shapes(cid):
    """The library's truncated SVD at the shapes it serves (4096 x 4096 rank 32, 3072 x 3072
    rank 32, 3072 x 12288 rank 32, 8192 x 8192 rank 128: all on the randomized subspace
    route): ||R||_F of svdq_prepare's residual within 1e-3 of the exact tail
    sqrt(sum_{i>r} sigma_i^2) of the smoothed weight. The tail comes from an independent route:
    ||ws||_F^2 minus the r largest eigenvalues of the float64 Gram matrix (LAPACK's symmetric
    eigensolver), no SVD. At 8192 x 8192 the rank (128) cuts into the noise bulk, where
    consecutive singular values are closest."""
    import scipy.linalg

    from workloads import WORKLOADS

    wl = WORKLOADS[cid]
    _, w, s = make_inputs(cid, B=64)
    p = R.prepare(torch.from_numpy(w).to(TD[wl.dtype]), torch.from_numpy(s), wl.rank, wl.bits, wl.fmt, device="cpu",
                  keep_factors=True)
    ws = O.smooth_weight(w, s, wl.dtype).astype(np.float64)
    gram = ws @ ws.T if ws.shape[0] <= ws.shape[1] else ws.T @ ws
    n = gram.shape[0]
    top = scipy.linalg.eigh(gram, eigvals_only=True, subset_by_index=[n - wl.rank, n - 1])
    tail = np.sqrt(np.sum(ws * ws) - top.sum())
    res = np.linalg.norm(_np(p.residual).astype(np.float64))
    assert abs(res - tail) <= 1e-3 * tail, (res, tail)
