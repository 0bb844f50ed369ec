"""Seeded synthetic inputs for the SVDQuant linear operator.

This package is shared by the tests, the benchmark and the oracle's checks. It
draws x, W and the smoothing scale for each workload and holds none of the
operator's own arithmetic (no smoothing, factorisation or quantisation).
"""
from .synth import WORKLOADS, Workload, make_inputs, smoothing_scale, to_bf16_values

__all__ = ["WORKLOADS", "Workload", "make_inputs", "smoothing_scale", "to_bf16_values"]
