"""CPU oracle for the SVDQuant linear operator — TEST INFRASTRUCTURE ONLY.

A plain, slow, readable numpy implementation of what the operator computes,
written from the source pages' definitions. It shares no code with the GPU
library (no kernels, headers, tables or helpers) and never imports it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``rank_bit_residual_amd``)
must never call it.

Modules:
  svdquant  -- vectorised numpy oracle (smoothing, truncated SVD split, per-tensor
               INT and per-block MXFP4 quantisers, packed layouts, reference forward)
  loops     -- a second, pure-Python loop implementation for tiny inputs, used
               to cross-check the numpy oracle
"""
