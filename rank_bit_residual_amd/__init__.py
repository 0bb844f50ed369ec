"""SVDQuant linear operator for AMD Instinct MI355X (gfx950).

Y = (X^ L1) L2 + Q(X^) Q(R): smoothed activations X^ = x / scale, a rank-r truncated
SVD L1 L2 of the smoothed weight, and the 4-bit (per-tensor INT or MXFP4) residual R.
The per-call path is hand-written HIP in libsvdq.so; this package is its ctypes binding.
"""
from .api import (Prepared, calibrate_scale, fake_quantize, linear, prepare, prepared_layout, quantize_activations,
                  smooth_inputs, split_weight, svdquant_linear, workspace_bytes)

__all__ = ["Prepared", "calibrate_scale", "fake_quantize", "linear", "prepare", "prepared_layout", "quantize_activations",
           "smooth_inputs", "split_weight", "svdquant_linear", "workspace_bytes"]
