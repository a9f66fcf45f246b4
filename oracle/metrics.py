"""Error metrics and tolerances used to compare a device result with the float64 oracle.

Test infrastructure only.

* max-abs: max |x - r| over the whole tensor.
* max-rel: per (b, h) slice, max |x - r| / max(max |r|, floor), then the max over slices. An
  element-wise relative error is meaningless where r is near 0, and attention outputs cluster
  near 0. ``floor`` (0 unless given) only matters for a slice whose largest exact magnitude is
  below it: the gradient tests pass 1e-3 of the largest exact gradient magnitude, so that a slice
  whose exact gradient is zero (dQ and dK when every row sees a single key) is measured against
  that instead of against its own rounding noise; every other slice keeps its own denominator.
* rel-L2: ||x - r|| / ||r|| over the tensor (reported, not gated).

Tolerances: float32 path O max-abs 1e-5; fp16/bf16 O max-abs 1e-2 and max-rel 2e-2 against the
oracle run on the same rounded inputs; LSE max-abs 1e-3; dQ/dK/dV max-rel 5e-2.
"""
from __future__ import annotations

import numpy as np

TOL = {
    "f32": {"o_abs": 1e-5, "o_rel": None, "lse_abs": 1e-3, "grad_rel": 5e-2},
    "f16": {"o_abs": 1e-2, "o_rel": 2e-2, "lse_abs": 1e-3, "grad_rel": 5e-2},
    "bf16": {"o_abs": 1e-2, "o_rel": 2e-2, "lse_abs": 1e-3, "grad_rel": 5e-2},
}


def max_abs(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - r)))


def max_rel(x, r, slice_ndim: int = 2, floor: float = 0.0):
    """Per-slice relative error; slices are the trailing ``slice_ndim`` axes.

    The denominator of a slice is max(max |r|, floor): the floor binds only for slices whose
    exact values are all smaller than it in magnitude (with floor = 0, never).
    """
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    if x.size == 0:
        return 0.0
    lead = x.shape[: x.ndim - slice_ndim]
    xs = x.reshape((-1,) + x.shape[x.ndim - slice_ndim:])
    rs = r.reshape((-1,) + r.shape[r.ndim - slice_ndim:])
    worst = 0.0
    for a, b in zip(xs, rs):
        den = max(float(np.max(np.abs(b))), floor)
        num = float(np.max(np.abs(a - b)))
        if den == 0.0:
            rel = 0.0 if num == 0.0 else np.inf
        else:
            rel = num / den
        worst = max(worst, rel)
    del lead
    return worst


def rel_l2(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    den = float(np.linalg.norm(r))
    num = float(np.linalg.norm(x - r))
    return 0.0 if den == 0.0 and num == 0.0 else (num / den if den else np.inf)


def report(x, r):
    return {"max_abs": max_abs(x, r), "max_rel": max_rel(x, r), "rel_l2": rel_l2(x, r)}
