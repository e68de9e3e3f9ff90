"""Build packed layers of a workload on the GPU.

The canonical bytes come from this package's counter-based generator, run on
the device; the product library then packs them (``moe_pack_experts``).  Used
by the GPU tests, the benchmark and the smoke check; the CPU oracle never
imports this module.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Workload, codebook_grid, expert_canon, layer_experts_canon, router


def packed_layer(wl: Workload, layer: int, device="cuda", canon_hook=None):
    """Generate one layer's weights on ``device`` and pack them.

    ``canon_hook(canon, shared)`` may edit the canonical tensors in place
    before packing (used by invariance tests).
    """
    import bit_quantized_experts_amd as bqe

    canon = layer_experts_canon(wl, layer, device)
    shared = expert_canon(wl, layer, -1, device) if wl.Is else None
    if canon_hook is not None:
        canon_hook(canon, shared)
    W, b = router(wl, layer)
    Wd = torch.from_numpy(W).to(device)
    bd = torch.from_numpy(b).to(device) if b is not None else None
    desc = bqe.make_desc(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, codebook=wl.codebook)
    grid = torch.from_numpy(codebook_grid(wl.seed)).to(device) if wl.codebook else None
    L = bqe.PackedLayer(desc, canon, shared, Wd, bd, device, grid=grid)
    del canon, shared, Wd, bd, grid
    return L


def activations_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
