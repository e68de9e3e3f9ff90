"""The allocation-free layer entry point (moe_layer_forward_noalloc, the
library's static device scratch instead of a caller's workspace) gives the
same results as moe_layer_forward on the same inputs, bit for bit, on
consecutive calls whose second call is smaller (the scratch keeps the first
call's contents), and rejects a call whose workspace exceeds the scratch."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_inputs.device import activations_device, packed_layer
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def bqe():
    import bit_quantized_experts_amd as m
    m.lib()
    return m


def _run(bqe, L, x_np, noalloc):
    T = x_np.shape[0]
    d, E, k = L.desc.d_model, L.desc.n_experts, L.desc.top_k
    x = activations_device(x_np)
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device=DEV)
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    r = bqe.RouteIO(None, None, logits.data_ptr(), idx.data_ptr(), w.data_ptr())
    if noalloc:
        bqe.moe_layer_forward_noalloc(L.handle, x, y, r)
    else:
        bqe.moe_layer_forward(L.handle, x, y, bqe.new_workspace(L.layer_workspace_bytes(T)), r)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (y, logits, idx, w)]


@pytest.mark.parametrize("which", ["full", "tiny"])
def test_noalloc_equals_workspace_entry(bqe, which):
    if which == "full":
        wl = mi.small(mi.WORKLOADS["layer_t1"], layers=1)
        sizes = (8, 3)            # decode kernels, the second call smaller
    else:
        wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1)
        sizes = (8, 5, 40, 12)    # decode, then grouped-GEMM chunks
    L = packed_layer(wl, 0)
    for T in sizes:
        say(f"[noalloc] {which}: T={T}")
        assert L.layer_workspace_bytes(T) <= bqe.NOALLOC_SCRATCH_BYTES
        x = mi.activations(wl, T=T, stream=700 + T)
        ref = _run(bqe, L, x, noalloc=False)
        got = _run(bqe, L, x, noalloc=True)
        for name, a, b in zip(("y", "logits", "idx", "w"), ref, got):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (which, T, name)


def test_noalloc_rejects_oversized_call(bqe):
    wl = mi.small(mi.WORKLOADS["layer_t1"], layers=1)
    L = packed_layer(wl, 0)
    T = 4096  # a long prefill chunk: its workspace is far above the scratch
    assert L.layer_workspace_bytes(T) > bqe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, wl.d), dtype=torch.float32, device=DEV)
    y = torch.zeros((T, wl.d), dtype=torch.float32, device=DEV)
    with pytest.raises(bqe.MoeError) as e:
        bqe.moe_layer_forward_noalloc(L.handle, x, y)
    assert e.value.code == bqe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not torch.any(y != 0)  # nothing was launched
