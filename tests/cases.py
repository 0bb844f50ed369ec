"""Constructed inputs shared by the GPU parity tests and the CPU checks of their sensitivity."""
import numpy as np

from oracle import svdquant as O

E2M1_TIES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def double_boundary_case(B=48, nblocks=16, seed=16):
    """bf16 x and float32 scale with x / scale within a few f32 ulps of a bf16 rounding
    midpoint next to an E2M1 tie (0.25, 0.75, ..., 5), in blocks whose shared exponent is
    0 (column 0 of every 32-block holds X^ = 6). Rounding X^ to the wrong neighbour moves it
    off (or onto) the tie, which changes the FP4 code."""
    rng = np.random.default_rng(seed)
    M = 32 * nblocks
    k = rng.integers(0, len(E2M1_TIES), M)
    tie = E2M1_TIES[k]
    half_ulp = np.ldexp(1.0, np.floor(np.log2(tie)).astype(int) - 8)  # half a bf16 ulp at the tie
    t = tie + np.where(rng.random(M) < 0.5, -1.0, 1.0) * half_ulp      # a bf16 rounding midpoint
    x0 = O.to_dtype(rng.uniform(0.5, 4.0, M), "bf16").astype(np.float64)
    s = (x0 / t).astype(np.float32)  # x0 / s = t (1 + O(2^-24))
    s[0::32] = 1.0
    rowscale = np.ldexp(1.0, rng.integers(-3, 4, B))  # powers of two keep every ratio's position
    sign = np.where(rng.random((B, M)) < 0.5, -1.0, 1.0)
    x = sign * x0[None, :] * rowscale[:, None]
    x[:, 0::32] = 6.0 * rowscale[:, None]
    return O.to_dtype(x, "bf16"), s
