"""HIP-graph capture of the forward calls: every replay equals the eager
result bit for bit, with eager calls on other inputs (through the same
workspace, whose control words the route kernel resets) between the replays.
The benchmark times graph replays, so this is the check that a replay
computes what the eager path computes."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_inputs.device import packed_layer, activations_device
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def bqe():
    import bit_quantized_experts_amd as m
    m.lib()
    return m


def _replays_match(run, outs, other, n_replay=3):
    """run(): the call, writing into `outs`; other(): an eager call on other
    inputs through the same workspace."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(n_replay):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            a, b = o.cpu().numpy(), r.cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {i}"
    say(f"    {n_replay} replays equal the eager result")


@pytest.mark.parametrize("mode", ["decode", "decode_T12", "f16act", "prefill_T200"])
def test_stack_graph_replays(bqe, mode):
    wl = mi.small(mi.WORKLOADS["stack_t8_2bit"], layers=2) if mode != "prefill_T200" else \
        mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1, layers=3)
    T = {"decode": 8, "decode_T12": 12, "f16act": 16, "prefill_T200": 200}[mode]
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    handles = [L.handle for L in layers]
    nL, d, k = wl.layers, wl.d, wl.k
    x = activations_device(mi.activations(wl, T=T, stream=70))
    x2 = activations_device(mi.activations(wl, T=T, stream=71))
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    y2 = torch.empty((T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    fwd = bqe.moe_stack_forward_f16act if mode == "f16act" else bqe.moe_stack_forward
    say(f"[graph] stack {mode}: layers={nL} T={T}")
    _replays_match(lambda: fwd(handles, x, y, ws, 1e-6, None, il, wr), [y, il, wr],
                   lambda: fwd(handles, x2, y2, ws, 1e-6))


@pytest.mark.parametrize("T", [1, 8, 12, 40])
def test_layer_graph_replays(bqe, T):
    wl = mi.small(mi.WORKLOADS["layer_t1"], layers=1)
    L = packed_layer(wl, 0)
    d, E, k = wl.d, wl.E, wl.k
    x = activations_device(mi.activations(wl, T=T, stream=80))
    x2 = activations_device(mi.activations(wl, T=T, stream=81))
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    y2 = torch.empty((T, d), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(L.workspace_bytes(T))
    r = bqe.RouteIO(None, None, logits.data_ptr(), idx.data_ptr(), w.data_ptr())
    outs = [y, idx, w, logits]
    say(f"[graph] layer T={T}")
    _replays_match(lambda: bqe.moe_layer_forward(L.handle, x, y, ws, r), outs,
                   lambda: bqe.moe_layer_forward(L.handle, x2, y2, ws))
