"""Float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this package. The library and its Python binding never do; they share no code
with it (no kernels, helpers, tables or pre/post-processing). Inputs come from the separate
seeded generator module, which holds none of the attention arithmetic.

Modules:
  attention  the definition (stable row-max softmax) forward and the analytic backward, fp64
  tiled      a float64 model of the tiled forward with the online (m, l, u) merge, used only to
             pin the algorithm the pages describe (never the device's ground truth)
  blocksparse exact attention restricted to allowed 128 x 128 (query, key) blocks
  dropout    attention with dropout on P and its Philox4x32-10 keep mask
  splitkv    split-KV partials (O_s, LSE_s) over key ranges and their merge by the page-3 rule
  traffic    the analytic naive-versus-tiled HBM traffic model
  metrics    max-abs / per-slice max-rel / rel-L2 and the tolerances

Every function is pinned by tests that do not retype it: the pages' worked examples
(tests/golden), closed forms, invariances, library cross-checks (scipy) and finite-difference
gradients.
"""
from . import attention, blocksparse, dropout, metrics, splitkv, tiled, traffic  # noqa: F401
