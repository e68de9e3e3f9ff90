"""GPU parity of the decode path at 9..16 tokens (one pass with 16 token rows
at full precision: every weight fragment multiplied by the tokens' fp16 hi
parts and then their lo parts) against the CPU oracle.

Bars as for the 8-token decode path: routing bit-exact given the GPU's
logits, logits within 1e-5 of the fp64 router, layer outputs within the
decode path's envelope (1e-5 infinity-norm relative error, per row too) with
the oracle fed the GPU's routing; stacks per layer.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_inputs.device import packed_layer, activations_device
from tests.helpers import TOL_DECODE_PATH, TOL_LAYER, oracle_layer, rel_err_inf, row_rel_err, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def bqe():
    import bit_quantized_experts_amd as m
    m.lib()
    return m


def _forward(bqe, L, x_np):
    T = x_np.shape[0]
    d, E, k = L.desc.d_model, L.desc.n_experts, L.desc.top_k
    x = activations_device(x_np)
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(L.workspace_bytes(T))
    r = bqe.RouteIO(None, None, logits.data_ptr(), idx.data_ptr(), w.data_ptr())
    bqe.moe_layer_forward(L.handle, x, y, ws, r)
    torch.cuda.synchronize()
    return y.cpu().numpy(), logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _check_layer(wl, layer, L, x_np, bqe, tag, tol=TOL_DECODE_PATH):
    say(f"[mid-T] {tag}: T={x_np.shape[0]} d={wl.d} E={wl.E} k={wl.k} bits={wl.bits} Is={wl.Is}")
    y, logits, idx, w = _forward(bqe, L, x_np)
    oi, ow = oracle.topk(logits, wl.k)
    assert np.array_equal(idx, oi), tag
    assert np.array_equal(w.view(np.uint32), ow.view(np.uint32)), tag
    W, b = mi.router(wl, layer)
    assert rel_err_inf(logits, oracle.router_logits(x_np, W, b)) < 1e-5, tag
    OL = oracle_layer(wl, layer, idx.reshape(-1))
    oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
    err, rerr = rel_err_inf(y, oy), row_rel_err(y, oy)
    say(f"    rel err {err:.3e} (largest per-row {rerr:.3e})")
    assert err <= tol and rerr <= tol, (tag, err, rerr)
    assert np.all(np.isfinite(y))
    return y


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("Is", [0, 64, 96])
def test_midt_layer_tiny_all_T(bqe, bits, Is):
    wl = mi.small(mi.WORKLOADS["tiny"], bits=bits, Is=Is, zipf_s=1.1 if Is else None)
    L = packed_layer(wl, 0)
    for T in range(9, 17):
        x = mi.activations(wl, T=T, stream=400 + T)
        _check_layer(wl, 0, L, x, bqe, f"tiny bits={bits} Is={Is}")


@pytest.mark.parametrize("bits", [2, 3])
def test_midt_layer_full_size(bqe, bits):
    # d = 2560: the gate/up kernel stages the 16-token fragments in two LDS
    # windows
    base = mi.WORKLOADS["layer_t1"] if bits == 2 else mi.WORKLOADS["stack_3bit"]
    wl = mi.small(base, layers=1)
    L = packed_layer(wl, 0)
    for T in (9, 16):
        x = mi.activations(wl, T=T, stream=500 + T)
        _check_layer(wl, 0, L, x, bqe, f"full bits={bits}")


def test_midt_layer_odd_shapes(bqe):
    # E not a multiple of 16, k = E, a shared expert wider than the routed
    # ones, and inputs of one to six LDS windows (d = 256 .. 8192)
    for kw in (dict(E=20, k=3, I=96, Is=32), dict(E=1, k=1, I=32, Is=0), dict(E=5, k=5, I=160, Is=288),
               dict(d=512, E=40, k=4, I=64, Is=64), dict(d=1536, E=24, k=2, I=32, Is=0),
               dict(d=4096, E=32, k=4, I=64, Is=96, bits=3), dict(d=8192, E=24, k=3, I=96, Is=32)):
        wl = mi.small(mi.WORKLOADS["tiny"], zipf_s=None, **kw)
        L = packed_layer(wl, 0)
        for T in (9, 13, 16):
            x = mi.activations(wl, T=T, stream=80 + T)
            _check_layer(wl, 0, L, x, bqe, f"odd {kw}")


@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_midt_layer_extreme_scales(bqe, shape):
    """Inputs far from unit scale and block scales near the packer's limit:
    the power-of-two scaling per (slice, token) and per (down item, token)
    keeps every row's precision relative to its own norm."""
    base = mi.WORKLOADS["tiny"] if shape == "tiny" else mi.small(mi.WORKLOADS["layer_t1"], E=24, layers=1)
    for scale_lo, scale_hi in ((0.01, 0.05), (6.0, 7.9)):
        wl = mi.small(base, Is=64 if shape == "tiny" else base.Is, zipf_s=1.1, scale_lo=scale_lo, scale_hi=scale_hi)
        L = packed_layer(wl, 0)
        for T, p in ((9, 20), (16, -20), (12, -60)):
            x = (mi.activations(wl, T=T, stream=190 + T) * np.float32(2.0 ** p)).astype(np.float32)
            # rows of very different norms in one call
            x[::3] *= np.float32(2.0 ** 12)
            _check_layer(wl, 0, L, x, bqe, f"{shape} scales U({scale_lo},{scale_hi}) x*2^{p}")


@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_midt_codebook(bqe, shape):
    kw = dict(bits=3, codebook=True, scale_lo=0.002, scale_hi=0.008)
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1, **kw) if shape == "tiny" else \
        mi.small(mi.WORKLOADS["layer_t1"], layers=1, **kw)
    L = packed_layer(wl, 0)
    for T in ((10, 16) if shape == "tiny" else (16,)):
        x = mi.activations(wl, T=T, stream=610 + T)
        _check_layer(wl, 0, L, x, bqe, f"codebook {shape}")


@pytest.mark.parametrize("T", [12, 16])
def test_midt_same_as_grouped_gemms(bqe, T, monkeypatch):
    """MOE_MID_T=0 sends the same call through the grouped GEMMs, whose
    router sums the logits in another order (gate weights may differ in the
    last bit): each path within its own bar of the oracle under its own
    routing, and the two outputs within the looser bar of each other."""
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1)
    L = packed_layer(wl, 0)
    x_np = mi.activations(wl, T=T, stream=700 + T)
    errs, ys = [], []
    for mid, tol in (("1", TOL_DECODE_PATH), ("0", TOL_LAYER)):
        monkeypatch.setenv("MOE_MID_T", mid)
        y, logits, idx, w = _forward(bqe, L, x_np)
        oi, ow = oracle.topk(logits, wl.k)
        assert np.array_equal(idx, oi) and np.array_equal(w.view(np.uint32), ow.view(np.uint32)), mid
        OL = oracle_layer(wl, 0, idx.reshape(-1))
        oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
        errs.append(rel_err_inf(y, oy))
        assert errs[-1] <= tol, (mid, errs[-1])
        ys.append(y)
    say(f"[mid-T] T={T}: 16-row decode pass {errs[0]:.3e}, grouped GEMMs {errs[1]:.3e}")
    assert rel_err_inf(ys[0], ys[1]) <= TOL_LAYER


def test_midt_forced_routing_invalid_and_repeated(bqe):
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64)
    L = packed_layer(wl, 0)
    T = 14
    x_np = mi.activations(wl, T=T, stream=71)
    g = np.random.default_rng(19)
    idx = np.stack([g.permutation(wl.E)[:wl.k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, wl.k)).astype(np.float32)
    idx[2, 1] = wl.E + 5   # out of range: skipped
    idx[9, 0] = -1         # out of range: skipped
    idx[13, 1] = idx[13, 0]  # repeated: the first occurrence only
    x = activations_device(x_np)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=DEV)
    fi = torch.from_numpy(idx).to(DEV)
    fw = torch.from_numpy(w).to(DEV)
    oi = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    ow = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(L.workspace_bytes(T))
    say(f"[mid-T] forced routing T={T}")
    bqe.moe_layer_forward(L.handle, x, y, ws, bqe.RouteIO(fi.data_ptr(), fw.data_ptr(), None, oi.data_ptr(),
                                                          ow.data_ptr()))
    torch.cuda.synchronize()
    assert np.array_equal(oi.cpu().numpy(), idx) and np.array_equal(ow.cpu().numpy(), w)
    OL = oracle_layer(wl, 0, idx[(idx >= 0) & (idx < wl.E)])
    oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
    assert rel_err_inf(y.cpu().numpy(), oy) <= TOL_DECODE_PATH


@pytest.mark.parametrize("which,T", [("tiny", 12), ("full", 16), ("full_3bit", 9)])
def test_midt_stack_teacher_forced(bqe, which, T):
    """Every layer of a stack of 9..16 tokens (one pass per layer) against
    the oracle under the stack's own routing."""
    if which == "tiny":
        wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1, layers=4)
    elif which == "full":
        wl = mi.small(mi.WORKLOADS["stack_t8_2bit"], layers=3)
    else:
        wl = mi.small(mi.WORKLOADS["stack_3bit"], layers=2)
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    x_np = mi.activations(wl, T=T, stream=55)
    nL, d, k = wl.layers, wl.d, wl.k
    x = activations_device(x_np)
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    yl = torch.empty((nL, T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wlr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    say(f"[mid-T stack] {which} layers={nL} T={T}")
    bqe.moe_stack_forward([L.handle for L in layers], x, y, ws, 1e-6, yl, il, wlr)
    torch.cuda.synchronize()
    yl, il, wlr = yl.cpu().numpy(), il.cpu().numpy(), wlr.cpu().numpy()
    assert np.array_equal(y.cpu().numpy(), yl[-1])
    h = x_np
    for l in range(nL):
        if l > 0:
            h = oracle.rmsnorm(yl[l - 1], 1e-6)
        OL = oracle_layer(wl, l, il[l].reshape(-1))
        oy, _, _, _ = oracle.layer_forward(OL, h, force_idx=il[l], force_w=wlr[l])
        err, rerr = rel_err_inf(yl[l], oy), row_rel_err(yl[l], oy)
        say(f"    layer {l}: rel err {err:.3e} (largest per-row {rerr:.3e})")
        assert err <= TOL_DECODE_PATH and rerr <= TOL_DECODE_PATH, (l, err, rerr)
