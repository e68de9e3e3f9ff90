"""Shared helpers for the tests: oracle-side layers and error metrics."""
from __future__ import annotations

import sys

import numpy as np

import moe_inputs as mi
import oracle


def say(*a):
    """Print and flush, so a GPU failure can be traced to its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err_inf(y, ref) -> float:
    """Global infinity-norm relative error: max|y - ref| / max|ref|."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def oracle_layer(wl: mi.Workload, layer: int, experts) -> oracle.Layer:
    """The oracle's view of a generated layer, holding only ``experts``
    (regenerated on the host with the same counter-based generator)."""
    W, b = mi.router(wl, layer)
    ex = {int(e): mi.expert_canon(wl, layer, int(e)).numpy() for e in set(int(v) for v in experts)}
    sh = mi.expert_canon(wl, layer, -1).numpy() if wl.Is else None
    grid = mi.codebook_grid(wl.seed) if wl.codebook else None
    return oracle.Layer(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, W, b, ex, sh, grid=grid)


# layer-output tolerance: global infinity-norm relative error max|y - ref| / max|ref|
TOL_LAYER = 2e-3

# Regression envelope of the decode path with fp16 hi + lo activations (not
# the tolerance of the method, which is TOL_LAYER): its products are exact and
# its roundings are fp32 accumulation and the ~22-bit activation split, so
# observed errors are 2e-7 (median) to 5e-6 (largest); a single wrongly
# decoded weight or a dropped block would exceed this long before TOL_LAYER.
TOL_DECODE_PATH = 1e-5


def row_rel_err(y, ref) -> float:
    """Largest per-row relative error max_t ||y_t - ref_t|| / ||ref_t|| (2-norms)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))
