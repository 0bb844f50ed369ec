"""Seeded synthetic workloads for the SVDQuant linear operator.

Five workloads mirror the settings the source pages describe: the page-1 toy
(one outlier-heavy activation matrix, a weight with a low-rank spike, INT4
per-tensor fake quantisation), an INT4 W4A4 layer, the MXFP4 W4A4 diffusion
transformer projections of the quantisation-tool guide (page 4: alpha 0.25,
rank 32, MXFP4 per-block minmax), and a decode-shaped MXFP4 layer.

Recipe (numpy ``default_rng(seed)``, all draws in float64 in this order):
  1. x ~ N(0,1) or Student-t(nu=3) of shape [B, M];
  2. outlier channels: ``rng.choice(M, k, replace=False)``; those columns of x
     are multiplied by the outlier factor;
  3. W noise ~ sigma_w * N(0,1) of shape [M, N];
  4. the spike: toy workload U [M,4], V [N,4] ~ N(0, 0.1^2), spike = U V^T;
     otherwise U, V = Q factors of QR of Gaussian [M,k], [N,k] and
     spike = U diag(s) V^T with s_i = 4 * (1/4)^((i-1)/(k-1)), i = 1..k;
  5. cast to float32, then round to bfloat16 (RNE, via torch) for bf16 workloads;
  6. smoothing scale s_m = max_b|x[b,m]|^alpha / max_n|W[m,n]|^(1-alpha)
     from the cast tensors, in float64, cast to float32 (1 where a max is 0).
     alpha = 0.5 is the square-root form sqrt(max|x| / max|W|).

Sizes, formats and seeds are listed in ``WORKLOADS``; the seed of workload c is
c - 1. No public dataset, checkpoint or calibration set is used: real diffusion
activations are stood in for by the heavy-tailed draws above.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    M: int
    N: int
    rank: int
    dtype: str  # "f32" or "bf16"
    fmt: str  # "int" (per-tensor symmetric INT) or "mx" (MXFP4, 32-element E8M0 blocks)
    bits: int
    alpha: float
    x_dist: str  # "normal" or "t3"
    n_outliers: int
    outlier_factor: float
    w_sigma: float
    spike: str  # "toy4" or "geom"
    spike_rank: int
    seed: int

    @property
    def flops(self) -> int:
        """Residual GEMM work 2*B*M*N, the throughput numerator."""
        return 2 * self.B * self.M * self.N


WORKLOADS = {
    1: Workload("toy_int4_f32", 16, 64, 48, 8, "f32", "int", 4, 0.5, "normal", 2, 20.0, 0.02, "toy4", 4, 0),
    2: Workload("int4_w4a4_bf16", 256, 4096, 4096, 32, "bf16", "int", 4, 0.5, "normal", 41, 30.0, 0.02, "geom", 16, 1),
    3: Workload("mxfp4_dit_attn_proj", 4096, 3072, 3072, 32, "bf16", "mx", 4, 0.25, "t3", 15, 50.0, 0.02, "geom", 32, 2),
    4: Workload("mxfp4_dit_mlp_up", 4096, 3072, 12288, 32, "bf16", "mx", 4, 0.25, "t3", 15, 50.0, 0.02, "geom", 32, 3),
    5: Workload("mxfp4_decode", 16, 8192, 8192, 128, "bf16", "mx", 4, 0.25, "normal", 82, 30.0, 0.015, "geom", 64, 4),
}


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE, torch's cast) and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def smoothing_scale(x: np.ndarray, w: np.ndarray, alpha: float) -> np.ndarray:
    """Per-input-channel scale max|x[:,m]|^alpha / max|W[m,:]|^(1-alpha), float32, positive."""
    ax = np.max(np.abs(x.astype(np.float64)), axis=0)
    aw = np.max(np.abs(w.astype(np.float64)), axis=1)
    ok = (ax > 0) & (aw > 0)
    s = np.ones_like(ax)
    s[ok] = ax[ok] ** alpha / aw[ok] ** (1.0 - alpha)
    return s.astype(np.float32)


def _spike(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    M, N, k = wl.M, wl.N, wl.spike_rank
    if wl.spike == "toy4":
        U = rng.normal(0.0, 0.1, size=(M, k))
        V = rng.normal(0.0, 0.1, size=(N, k))
        return U @ V.T
    U, _ = np.linalg.qr(rng.standard_normal((M, k)))
    V, _ = np.linalg.qr(rng.standard_normal((N, k)))
    s = 4.0 * (0.25 ** (np.arange(k) / max(k - 1, 1)))
    return (U * s) @ V.T


def make_inputs(wl: Workload | int, B: int | None = None, seed: int | None = None):
    """Return (x, W, scale) as float32 arrays (bf16-representable values for bf16 workloads).

    ``B`` overrides the batch (rows of x) for reduced-size parity cases; ``seed``
    overrides the workload's seed.
    """
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if wl.x_dist == "t3":
        x = rng.standard_t(3.0, size=(B, wl.M))
    else:
        x = rng.standard_normal((B, wl.M))
    cols = rng.choice(wl.M, wl.n_outliers, replace=False)
    x[:, cols] *= wl.outlier_factor
    w = wl.w_sigma * rng.standard_normal((wl.M, wl.N)) + _spike(rng, wl)
    x = x.astype(np.float32)
    w = w.astype(np.float32)
    if wl.dtype == "bf16":
        x = to_bf16_values(x)
        w = to_bf16_values(w)
    scale = smoothing_scale(x, w, wl.alpha)
    return x, w, scale
