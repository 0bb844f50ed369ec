"""CPU checks that the constructed GPU parity inputs can catch the mistakes they target.

Each planted mistake is applied to the oracle's own arithmetic (never to the library); the
constructed case must change many outputs under it, so a device path that made the same
mistake could not pass the bit-exact GPU comparison on that case.
"""
import numpy as np

from cases import double_boundary_case
from oracle import svdquant as O


def _codes(xs):
    return O.quantize_mx(xs)[0]


def test_double_boundary_case_catches_rounding_mistakes():
    x, s = double_boundary_case()
    good = _codes(O.smooth_activations(x, s, "bf16"))
    # one rounding straight from the exact quotient to bf16 (skipping RN_f32)
    single = _codes(O.to_dtype(x.astype(np.float64) / s.astype(np.float64), "bf16"))
    # the uncorrected product with the rounded reciprocal
    y = (np.float32(1) / s).astype(np.float32)
    prod = _codes(O.to_dtype((x.astype(np.float32) * y[None, :]).astype(np.float32), "bf16"))
    # truncation instead of round-to-nearest-even when narrowing to bf16
    q = (x.astype(np.float32) / s[None, :]).astype(np.float32)
    trunc = _codes((q.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32))
    for bad in (single, prod, trunc):
        assert (bad != good).sum() > 0.01 * good.size
