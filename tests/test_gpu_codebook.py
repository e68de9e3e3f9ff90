"""GPU parity of codebook blocks (15 bytes per 32 weights: fp16 scale, eight
9-bit indices into a 512 x 4 grid of magnitudes, 32 sign bits) against the CPU
oracle, with the synthetic grid of the input generator.

Bars as for b-bit blocks: codes and dequantised weights bit-exact through the
scalar export and through the expert kernels' own decoders (the decode
fragment decoder, and the grouped GEMMs' fp16 dequantization, one rounding of
scale times code); routing bit-exact given the logits; layer outputs within
the decode path's envelope (and the 2e-3 bar) on the decode kernels, within
2e-3 on the grouped GEMMs, with the oracle fed the GPU's routing.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_inputs.device import packed_layer, activations_device
from tests.helpers import TOL_DECODE_PATH, TOL_LAYER, oracle_layer, rel_err_inf, row_rel_err, say
from tests.test_gpu_decode import _check_layer, _forward

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def bqe():
    import bit_quantized_experts_amd as m
    m.lib()
    return m


def _cb(base, **kw):
    kw.setdefault("bits", 3)
    return mi.small(mi.WORKLOADS[base], codebook=True, scale_lo=0.002, scale_hi=0.008, **kw)


def test_cb_generator_cpu_equals_gpu():
    for first, count in ((0, 1000), (98765, 4097)):
        a = mi.canon_blocks(0, 3, mi.STREAM_ROUTED, first, count, 3, 0.002, 0.008, device="cpu", codebook=True)
        b = mi.canon_blocks(0, 3, mi.STREAM_ROUTED, first, count, 3, 0.002, 0.008, device=DEV, codebook=True).cpu()
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_cb_unpack_bitexact(bqe, shape):
    """The scalar export and the decode kernels' fragment decoder (index
    bytes, index high bits, LDS grid lookup, sign bits) against the oracle."""
    if shape == "tiny":
        wl = _cb("tiny", Is=96)
        experts = list(range(wl.E)) + [-1]
    else:
        wl = _cb("layer_t1", E=12)
        experts = [0, 6, 11, -1]
    grid = mi.codebook_grid(wl.seed)
    say(f"[cb unpack] {shape}")
    L = packed_layer(wl, 0)
    for e in experts:
        canon = mi.expert_canon(wl, 0, e).numpy()
        I = wl.Is if e < 0 else wl.I
        parts = oracle.split_expert(canon, wl.d, I, 3, grid)
        for mat, (rows, cols) in enumerate(((I, wl.d), (I, wl.d), (wl.d, I))):
            oc, _ = oracle.cb_unpack_matrix(parts[mat], rows, cols, grid)
            ow = oracle.cb_dequant_matrix(parts[mat], rows, cols, grid)
            codes = torch.full((rows, cols), 99, dtype=torch.int8, device=DEV)
            w32 = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
            w16 = torch.full((rows, cols), -1, dtype=torch.int16, device=DEV)
            bqe.moe_debug_unpack(L.handle, e, mat, codes, w32, w16)
            torch.cuda.synchronize()
            assert np.array_equal(codes.cpu().numpy(), oc), (e, mat, "scalar codes")
            assert np.array_equal(w32.cpu().numpy().astype(np.float64), ow), (e, mat, "scalar weights")
            assert np.array_equal(w16.cpu().numpy().view(np.uint16), oracle.double_to_half_array(ow)), (e, mat)
            codes.fill_(99)
            w32.fill_(float("nan"))
            bqe.moe_debug_unpack_path(L.handle, e, mat, 0, codes, w32, None)
            torch.cuda.synchronize()
            assert np.array_equal(codes.cpu().numpy(), oc), (e, mat, "decode-path codes")
            assert np.array_equal(w32.cpu().numpy().astype(np.float64), ow), (e, mat, "decode-path weights")
            o16 = oracle.double_to_half_array(ow)
            for path in (1, 2):  # the grouped GEMMs' dequantization from half and whole chunks
                w16.fill_(-1)
                bqe.moe_debug_unpack_path(L.handle, e, mat, path, None, None, w16)
                torch.cuda.synchronize()
                assert np.array_equal(w16.cpu().numpy().view(np.uint16), o16), (e, mat, path)


def test_cb_pack_checks(bqe):
    wl = _cb("tiny")
    canon = mi.layer_experts_canon(wl, 0, DEV)
    W, _ = mi.router(wl, 0)
    Wd = torch.from_numpy(W).to(DEV)
    desc = bqe.make_desc(wl.d, wl.E, wl.I, 0, wl.k, 3, codebook=True)
    buf = torch.empty(bqe.moe_packed_bytes(desc), dtype=torch.uint8, device=DEV)
    with pytest.raises(bqe.MoeError) as ei:  # codebook blocks need the grid
        bqe.moe_pack_experts(desc, canon, None, Wd, None, buf)
    assert ei.value.code == bqe.MOE_ERR_ARG
    grid = torch.from_numpy(mi.codebook_grid()).to(DEV)
    bad = grid.clone()
    bad[300, 2] = 128
    with pytest.raises(bqe.MoeError) as ei:
        bqe.moe_pack_experts_cb(desc, canon, None, bad, Wd, None, buf)
    assert ei.value.code == bqe.MOE_ERR_DATA
    with pytest.raises(bqe.MoeError) as ei:  # the 3-bit class only
        bqe.moe_packed_bytes(bqe.make_desc(wl.d, wl.E, wl.I, 0, wl.k, 2, codebook=True))
    assert ei.value.code == bqe.MOE_ERR_UNSUPPORTED
    big = canon.clone()
    big[15 * 7: 15 * 7 + 2] = torch.tensor([0x00, 0x5C], dtype=torch.uint8)  # block 7's scale = 256.0
    with pytest.raises(bqe.MoeError) as ei:  # scale * code must stay below 2^15 in fp16
        bqe.moe_pack_experts_cb(desc, big, None, grid, Wd, None, buf)
    assert ei.value.code == bqe.MOE_ERR_DATA
    h = bqe.moe_pack_experts_cb(desc, canon, None, grid, Wd, None, buf)
    got = bqe.moe_layer_get_desc(h)
    assert (got.bits, got.codebook, got.block) == (3, 1, 32)
    bqe.moe_layer_release(h)


@pytest.mark.parametrize("Is", [0, 64])
def test_cb_layer_tiny_all_T(bqe, Is):
    wl = _cb("tiny", Is=Is, zipf_s=1.1)
    L = packed_layer(wl, 0)
    for T in range(1, 9):
        x = mi.activations(wl, T=T, stream=T)
        _check_layer(wl, 0, L, x, bqe, f"cb tiny Is={Is} T={T}")


@pytest.mark.parametrize("T", [1, 8])
def test_cb_layer_full_size(bqe, T):
    wl = _cb("layer_t1")
    L = packed_layer(wl, 0)
    x = mi.activations(wl, T=T, stream=21)
    _check_layer(wl, 0, L, x, bqe, f"cb full T={T}")


def test_cb_f16act_full_size(bqe):
    wl = _cb("layer_t1")
    L = packed_layer(wl, 0)
    T = 16
    x_np = mi.activations(wl, T=T, stream=22)
    d, k = wl.d, wl.k
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(L.workspace_bytes(T))
    r = bqe.RouteIO(None, None, None, idx.data_ptr(), w.data_ptr())
    say(f"[cb f16act] T={T}")
    bqe.moe_layer_forward_f16act(L.handle, activations_device(x_np), y, ws, r)
    torch.cuda.synchronize()
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    OL = oracle_layer(wl, 0, idx.reshape(-1))
    oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
    err = rel_err_inf(y.cpu().numpy(), oy)
    say(f"    rel err {err:.3e}")
    assert err <= TOL_LAYER


@pytest.mark.parametrize("T", [8, 1])
def test_cb_stack_teacher_forced(bqe, T):
    """Three stacked full-size codebook layers, each against the oracle under
    the stack's routing (the input of a layer is the RMSNorm of the last)."""
    wl = _cb("stack_cb3", layers=3)
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    x_np = mi.activations(wl, T=T, stream=23)
    nL, d, k = wl.layers, wl.d, wl.k
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    yl = torch.empty((nL, T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    say(f"[cb stack] layers={nL} T={T}")
    bqe.moe_stack_forward([L.handle for L in layers], activations_device(x_np), y, ws, 1e-6, yl, il, wr)
    torch.cuda.synchronize()
    yl, il, wr = yl.cpu().numpy(), il.cpu().numpy(), wr.cpu().numpy()
    assert np.array_equal(y.cpu().numpy(), yl[-1])
    h = x_np
    for l in range(nL):
        if l > 0:
            h = oracle.rmsnorm(yl[l - 1], 1e-6)
        OL = oracle_layer(wl, l, il[l].reshape(-1))
        oy, _, _, _ = oracle.layer_forward(OL, h, force_idx=il[l], force_w=wr[l])
        err, rerr = rel_err_inf(yl[l], oy), row_rel_err(yl[l], oy)
        say(f"    layer {l}: rel err {err:.3e} (largest per-row {rerr:.3e})")
        assert err <= TOL_DECODE_PATH and rerr <= TOL_DECODE_PATH, (l, err, rerr)


@pytest.mark.parametrize("shape,T", [("tiny", 9), ("tiny", 37), ("tiny", 200), ("full", 300)])
def test_cb_prefill_layer(bqe, shape, T, monkeypatch):
    """Chunks of more than 8 tokens through the grouped GEMMs (codebook
    weights dequantized in registers from the LDS grid), teacher-forced
    (MOE_MID_T=0: T = 9 too)."""
    monkeypatch.setenv("MOE_MID_T", "0")
    wl = _cb("tiny", Is=64, zipf_s=1.1) if shape == "tiny" else _cb("layer_t1")
    L = packed_layer(wl, 0)
    x_np = mi.activations(wl, T=T, stream=24)
    say(f"[cb prefill] {shape} T={T}")
    y, logits, idx, w = _forward(bqe, L, x_np)
    oi, ow = oracle.topk(logits, wl.k)
    assert np.array_equal(idx, oi) and np.array_equal(w.view(np.uint32), ow.view(np.uint32))
    rows = np.arange(T) if shape == "tiny" else np.unique(np.linspace(0, T - 1, 24).astype(int))
    OL = oracle_layer(wl, 0, idx[rows].reshape(-1))
    oy, _, _, _ = oracle.layer_forward(OL, x_np[rows], force_idx=idx[rows], force_w=w[rows])
    err = rel_err_inf(y[rows], oy)
    say(f"    rel err {err:.3e} on {len(rows)} rows")
    assert err <= TOL_LAYER


def test_cb_prefill_stack(bqe):
    """Three stacked tiny codebook layers over 50 tokens (the chunked-prefill
    stack), each against the oracle under the stack's routing."""
    wl = _cb("tiny", Is=64, zipf_s=1.1, layers=3)
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    T, nL, d, k = 50, wl.layers, wl.d, wl.k
    x_np = mi.activations(wl, T=T, stream=25)
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    yl = torch.empty((nL, T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    say(f"[cb prefill stack] layers={nL} T={T}")
    bqe.moe_stack_forward([L.handle for L in layers], activations_device(x_np), y, ws, 1e-6, yl, il, wr)
    torch.cuda.synchronize()
    yl, il, wr = yl.cpu().numpy(), il.cpu().numpy(), wr.cpu().numpy()
    h = x_np
    for l in range(nL):
        if l > 0:
            h = oracle.rmsnorm(yl[l - 1], 1e-6)
        OL = oracle_layer(wl, l, il[l].reshape(-1))
        oy, _, _, _ = oracle.layer_forward(OL, h, force_idx=il[l], force_w=wr[l])
        err = rel_err_inf(yl[l], oy)
        say(f"    layer {l}: rel err {err:.3e}")
        assert err <= TOL_LAYER, (l, err)
