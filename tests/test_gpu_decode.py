"""GPU parity of the decode path (T <= 8) against the CPU oracle.

Bars: unpacked codes and dequantised weights bit-exact; top-k indices and
gate weights bit-exact given the same logits; layer outputs within a global
infinity-norm relative error of 2e-3 with the oracle fed the GPU's own
routing (teacher forcing), per layer for stacks.
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


def _forward(bqe, L, x_np, route=True):
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


def _check_layer(wl, layer, L, x_np, bqe, tag):
    say(f"[decode] {tag}: T={x_np.shape[0]} d={wl.d} E={wl.E} k={wl.k} bits={wl.bits} Is={wl.Is}")
    y, logits, idx, w = _forward(bqe, L, x_np)
    # routing: bit-exact against the oracle's selection on the GPU's logits
    oi, ow = oracle.topk(logits, wl.k)
    assert np.array_equal(idx, oi), tag
    assert np.array_equal(w.view(np.uint32), ow.view(np.uint32)), tag
    # logits close to the oracle's fp64 router
    W, b = mi.router(wl, layer)
    ol = oracle.router_logits(x_np, W, b)
    assert rel_err_inf(logits, ol) < 1e-5, tag
    # layer output, teacher-forced with the GPU routing
    OL = oracle_layer(wl, layer, idx.reshape(-1))
    oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
    err = rel_err_inf(y, oy)
    rerr = row_rel_err(y, oy)
    say(f"    rel err {err:.3e} (largest per-row {rerr:.3e})")
    assert err <= TOL_LAYER, (tag, err)
    assert err <= TOL_DECODE_PATH and rerr <= TOL_DECODE_PATH, (tag, err, rerr)
    assert np.all(np.isfinite(y))
    return y, idx, w, err


def test_generator_cpu_equals_gpu():
    for bits in (2, 3):
        for first, count in ((0, 1000), (123457, 4097)):
            a = mi.canon_blocks(0, 5, mi.STREAM_ROUTED, first, count, bits, 0.01, 0.05, device="cpu")
            b = mi.canon_blocks(0, 5, mi.STREAM_ROUTED, first, count, bits, 0.01, 0.05, device=DEV).cpu()
            assert torch.equal(a, b)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_debug_unpack_bitexact(bqe, bits, shape):
    if shape == "tiny":
        wl = mi.small(mi.WORKLOADS["tiny"], bits=bits, Is=96)
        experts = list(range(wl.E)) + [-1]
    else:
        wl = mi.small(mi.WORKLOADS["layer_t1"], bits=bits, E=12)
        experts = [0, 5, 11, -1]
    say(f"[unpack] {shape} bits={bits}")
    L = packed_layer(wl, 0)
    for e in experts:
        canon = mi.expert_canon(wl, 0, e).numpy()
        I = wl.Is if e < 0 else wl.I
        parts = oracle.split_expert(canon, wl.d, I, bits)
        for mat, (rows, cols) in enumerate(((I, wl.d), (I, wl.d), (wl.d, I))):
            codes = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
            w32 = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
            w16 = torch.empty((rows, cols), dtype=torch.int16, device=DEV)
            bqe.moe_debug_unpack(L.handle, e, mat, codes, w32, w16)
            torch.cuda.synchronize()
            oc, _ = oracle.unpack_matrix(parts[mat], rows, cols, bits)
            ow = oracle.dequant_matrix(parts[mat], rows, cols, bits)
            assert np.array_equal(codes.cpu().numpy(), oc), (e, mat)
            assert np.array_equal(w32.cpu().numpy().astype(np.float64), ow), (e, mat)
            o16 = oracle.double_to_half_array(ow)
            assert np.array_equal(w16.cpu().numpy().view(np.uint16), o16), (e, mat)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_debug_unpack_path_bitexact(bqe, bits, shape):
    """The weights as the expert kernels' own decoders see them: the decode
    kernels' fragment decode (codes and fp32 scale x code) and the grouped
    GEMMs' fp16 register dequantization from half and whole chunks, bit for
    bit against the oracle's unpack and dequant."""
    if shape == "tiny":
        wl = mi.small(mi.WORKLOADS["tiny"], bits=bits, Is=96)
        experts = list(range(wl.E)) + [-1]
    else:
        base = mi.WORKLOADS["layer_t1"] if bits == 2 else mi.WORKLOADS["stack_3bit"]
        wl = mi.small(base, E=12, layers=1)
        experts = [0, 7, 11, -1]
    say(f"[unpack path] {shape} bits={bits}")
    L = packed_layer(wl, 0)
    for e in experts:
        canon = mi.expert_canon(wl, 0, e).numpy()
        I = wl.Is if e < 0 else wl.I
        parts = oracle.split_expert(canon, wl.d, I, bits)
        for mat, (rows, cols) in enumerate(((I, wl.d), (I, wl.d), (wl.d, I))):
            oc, _ = oracle.unpack_matrix(parts[mat], rows, cols, bits)
            ow = oracle.dequant_matrix(parts[mat], rows, cols, bits)
            o16 = oracle.double_to_half_array(ow)
            codes = torch.full((rows, cols), 99, dtype=torch.int8, device=DEV)
            w32 = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
            bqe.moe_debug_unpack_path(L.handle, e, mat, 0, codes, w32, None)
            torch.cuda.synchronize()
            assert np.array_equal(codes.cpu().numpy(), oc), (e, mat, "decode codes")
            assert np.array_equal(w32.cpu().numpy().astype(np.float64), ow), (e, mat, "decode weights")
            for path in (1, 2):
                w16 = torch.full((rows, cols), -1, dtype=torch.int16, device=DEV)
                bqe.moe_debug_unpack_path(L.handle, e, mat, path, None, None, w16)
                torch.cuda.synchronize()
                assert np.array_equal(w16.cpu().numpy().view(np.uint16), o16), (e, mat, path)


@pytest.mark.parametrize("E,k,T", [(16, 2, 5), (512, 10, 64), (512, 16, 33), (4096, 8, 9), (3, 3, 7), (1, 1, 4),
                                   (1000, 12, 6), (2048, 16, 3), (65, 16, 5)])
def test_route_topk_bitexact(bqe, E, k, T):
    say(f"[topk] E={E} k={k} T={T}")
    g = np.random.default_rng(E * 31 + k)
    cases = [g.standard_normal((T, E)).astype(np.float32) * 2,
             g.integers(0, 3, (T, E)).astype(np.float32),
             np.where(g.random((T, E)) < 0.5, -0.0, 0.0).astype(np.float32)]
    if E == 512:
        cases.append(mi.direct_logits(mi.WORKLOADS["layer_t1"], T))
    # experts e with e % 64 < 16 (one wavefront lane in four holds them) all
    # rank above the rest: more than 64 logits reach the k-th largest of the
    # per-lane maxima when E is large, which takes the selection's second path
    cases.append((((np.arange(E) % 64) < 16).astype(np.float32)[None, :]
                  + g.random((T, E)).astype(np.float32) * 1e-3).astype(np.float32))
    for l in cases:
        lt = torch.from_numpy(l).to(DEV)
        idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        bqe.moe_route_topk(lt, k, idx, w)
        torch.cuda.synchronize()
        oi, ow = oracle.topk(l, k)
        assert np.array_equal(idx.cpu().numpy(), oi)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("Is", [0, 64, 96])
def test_layer_tiny_all_T(bqe, bits, Is):
    wl = mi.small(mi.WORKLOADS["tiny"], bits=bits, Is=Is, zipf_s=1.1 if Is else None)
    L = packed_layer(wl, 0)
    for T in range(1, 9):
        x = mi.activations(wl, T=T, stream=T)
        _check_layer(wl, 0, L, x, bqe, f"tiny bits={bits} Is={Is} T={T}")


@pytest.mark.parametrize("bits", [2, 3])
def test_layer_full_size(bqe, bits):
    base = mi.WORKLOADS["layer_t1"] if bits == 2 else mi.WORKLOADS["stack_3bit"]
    wl = mi.small(base, layers=1)
    L = packed_layer(wl, 0)
    for T in (1, 3, 8):
        x = mi.activations(wl, T=T, stream=100 + T)
        _check_layer(wl, 0, L, x, bqe, f"full bits={bits} T={T}")


@pytest.mark.parametrize("shape", ["tiny", "full"])
def test_layer_extreme_scales(bqe, shape):
    """Inputs far from unit scale (x times 2^20 and 2^-20) and block scales
    near the largest the packer accepts: every row keeps the decode path's
    precision relative to its own norm (the activations and the intermediate
    h are scaled by powers of two before they are split into fp16 parts)."""
    base = mi.WORKLOADS["tiny"] if shape == "tiny" else mi.small(mi.WORKLOADS["layer_t1"], E=24, layers=1)
    for scale_lo, scale_hi in ((0.01, 0.05), (6.0, 7.9)):
        wl = mi.small(base, Is=64 if shape == "tiny" else base.Is, zipf_s=1.1, scale_lo=scale_lo, scale_hi=scale_hi)
        L = packed_layer(wl, 0)
        for T, p in ((3, 20), (8, -20), (1, -60)):
            x = (mi.activations(wl, T=T, stream=90 + T) * np.float32(2.0 ** p)).astype(np.float32)
            _check_layer(wl, 0, L, x, bqe, f"{shape} scales U({scale_lo},{scale_hi}) x*2^{p} T={T}")


def test_layer_odd_shapes(bqe):
    # E not a multiple of 16, intermediate sizes not multiples of 64, k = E,
    # a shared expert wider than the routed ones, and inputs wider than one
    # LDS window of the gate/up kernel (d = 4096 and 8192: two and three
    # windows)
    for kw in (dict(E=20, k=3, I=96, Is=32), dict(E=1, k=1, I=32, Is=0), dict(E=5, k=5, I=160, Is=288),
               dict(d=512, E=40, k=4, I=64, Is=64), dict(d=4096, E=32, k=4, I=64, Is=96, bits=3),
               dict(d=8192, E=24, k=3, I=96, Is=32)):
        wl = mi.small(mi.WORKLOADS["tiny"], zipf_s=None, **kw)
        L = packed_layer(wl, 0)
        for T in (1, 5, 8):
            x = mi.activations(wl, T=T, stream=60 + T)
            _check_layer(wl, 0, L, x, bqe, f"odd {kw} T={T}")


@pytest.mark.parametrize("T,mid", [(6, "1"), (12, "1"), (12, "0")])
def test_forced_routing_and_invalid_entries(bqe, T, mid, monkeypatch):
    # T = 6: the 8-row decode pass; T = 12: the 16-row decode pass, or with
    # MOE_MID_T=0 the grouped-GEMM kernels
    monkeypatch.setenv("MOE_MID_T", mid)
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64)
    L = packed_layer(wl, 0)
    x_np = mi.activations(wl, T=T, stream=7)
    g = np.random.default_rng(9)
    idx = np.stack([g.permutation(wl.E)[:wl.k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, wl.k)).astype(np.float32)
    idx[2, 1] = wl.E + 5   # out of range: skipped
    idx[4, 0] = -1         # out of range: skipped
    idx[5, 1] = idx[5, 0]  # repeated: the first occurrence only
    if T > 8:
        idx[10, 0] = idx[10, 1]
    x = activations_device(x_np)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=DEV)
    fi = torch.from_numpy(idx).to(DEV)
    fw = torch.from_numpy(w).to(DEV)
    oi = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    ow = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(L.workspace_bytes(T))
    r = bqe.RouteIO(fi.data_ptr(), fw.data_ptr(), None, oi.data_ptr(), ow.data_ptr())
    bqe.moe_layer_forward(L.handle, x, y, ws, r)
    torch.cuda.synchronize()
    assert np.array_equal(oi.cpu().numpy(), idx) and np.array_equal(ow.cpu().numpy(), w)
    # the oracle applies the same rule to the raw rows (out-of-range ids
    # skipped, a repeated id counted once at its first rank)
    OL = oracle_layer(wl, 0, idx[(idx >= 0) & (idx < wl.E)])
    oy, _, _, _ = oracle.layer_forward(OL, x_np, force_idx=idx, force_w=w)
    assert rel_err_inf(y.cpu().numpy(), oy) <= TOL_LAYER


def test_workspace_reuse_control_words(bqe):
    """The route kernel counts finished workgroups in the workspace's control
    words; every call must leave them at zero, so one workspace serves calls
    of any shape in turn with results identical to a fresh workspace's."""
    wa = mi.small(mi.WORKLOADS["tiny"], Is=64)
    wb = mi.small(mi.WORKLOADS["layer_t1"], layers=1)
    La, Lb = packed_layer(wa, 0), packed_layer(wb, 0)
    nbytes = max(La.workspace_bytes(8), Lb.workspace_bytes(8))
    shared = bqe.new_workspace(nbytes)
    g = np.random.default_rng(31)

    def run(L, wl, T, ws, forced):
        x = activations_device(mi.activations(wl, T=T, stream=100 + T))
        y = torch.empty((T, wl.d), dtype=torch.float32, device=DEV)
        idx = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
        if forced:
            fi = torch.from_numpy(np.stack([g.permutation(wl.E)[:wl.k] for _ in range(T)]).astype(np.int32)).to(DEV)
            fw = torch.from_numpy(g.random((T, wl.k)).astype(np.float32)).to(DEV)
            r = bqe.RouteIO(fi.data_ptr(), fw.data_ptr(), None, idx.data_ptr(), w.data_ptr())
        else:
            r = bqe.RouteIO(None, None, None, idx.data_ptr(), w.data_ptr())
        bqe.moe_layer_forward(L.handle, x, y, ws, r)
        torch.cuda.synchronize()
        return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()

    for L, wl, T, forced in [(La, wa, 3, False), (Lb, wb, 8, False), (La, wa, 5, True), (Lb, wb, 1, False),
                             (La, wa, 8, False), (Lb, wb, 2, True), (Lb, wb, 7, False)]:
        say(f"[decode] workspace reuse: E={wl.E} d={wl.d} T={T} forced={forced}")
        state = g.bit_generator.state
        y1, i1, w1 = run(L, wl, T, shared, forced)
        assert int(shared[:256].count_nonzero()) == 0, "control words left set"
        g.bit_generator.state = state
        y2, i2, w2 = run(L, wl, T, bqe.new_workspace(nbytes), forced)
        assert np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_determinism_and_T8_vs_T1(bqe):
    wl = mi.small(mi.WORKLOADS["layer_t1"], layers=1)
    L = packed_layer(wl, 0)
    x = mi.activations(wl, T=8, stream=55)
    y1, _, i1, w1 = _forward(bqe, L, x)
    y2, _, i2, w2 = _forward(bqe, L, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(i1, i2) and np.array_equal(w1, w2)
    # verify pass == token-by-token decode (routing bit-exact, outputs within fp32 rounding)
    for t in range(8):
        yt, _, it, wt = _forward(bqe, L, x[t:t + 1])
        assert np.array_equal(it[0], i1[t]) and np.array_equal(wt[0], w1[t])
        assert rel_err_inf(yt[0], y1[t]) < 1e-5


def test_unused_experts_do_not_change_output(bqe):
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1)
    x = mi.activations(wl, T=3, stream=77)
    L = packed_layer(wl, 0)
    y, _, idx, w = _forward(bqe, L, x)
    used = set(idx.reshape(-1).tolist())
    eb = wl.expert_bytes()

    def scramble(canon, shared):
        g = torch.Generator(device="cpu").manual_seed(3)
        for e in range(wl.E):
            if e not in used:
                noise = torch.randint(0, 256, (eb,), generator=g, dtype=torch.uint8)
                blk = noise.view(-1, wl.block_bytes())
                blk[:, 1] &= 0x3F  # keep scales finite and small
                canon[e * eb:(e + 1) * eb] = noise.to(canon.device)

    L2 = packed_layer(wl, 0, canon_hook=scramble)
    y2, _, idx2, w2 = _forward(bqe, L2, x)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("path", ["phases", "persist"])
@pytest.mark.parametrize("which", ["tiny", "full", "full_3bit_T8", "full_3bit_T1"])
def test_stack_teacher_forced(bqe, which, path, monkeypatch):
    """Every layer of a stack against the oracle under the stack's own
    routing, on both decode paths: the per-phase kernels, and the persistent
    pass (one launch for the stack, which must leave its abort word clear)."""
    monkeypatch.setenv("MOE_PERSIST", "1" if path == "persist" else "0")
    if which == "tiny":
        wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1, layers=5)
        T = 7
    elif which == "full":
        wl = mi.small(mi.WORKLOADS["stack_t8_2bit"], layers=3)
        T = 8
    else:
        # the first layers of the 3-bit stack, at both of its decode sizes
        wl = mi.small(mi.WORKLOADS["stack_3bit"], layers=3)
        T = 8 if which.endswith("T8") else 1
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    x_np = mi.activations(wl, T=T, stream=5)
    nL, d, k = wl.layers, wl.d, wl.k
    x = activations_device(x_np)
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    yl = torch.empty((nL, T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wlr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    say(f"[stack] {which} layers={nL} T={T} path={path}")
    bqe.moe_stack_forward([L.handle for L in layers], x, y, ws, 1e-6, yl, il, wlr)
    torch.cuda.synchronize()
    assert bqe.moe_workspace_status(ws) == 0
    yl, il, wlr = yl.cpu().numpy(), il.cpu().numpy(), wlr.cpu().numpy()
    assert np.array_equal(y.cpu().numpy(), yl[-1])
    h = x_np
    for l in range(nL):
        if l > 0:
            h = oracle.rmsnorm(yl[l - 1], 1e-6)
        OL = oracle_layer(wl, l, il[l].reshape(-1))
        oy, ologits, _, _ = oracle.layer_forward(OL, h, force_idx=il[l], force_w=wlr[l])
        err = rel_err_inf(yl[l], oy)
        rerr = row_rel_err(yl[l], oy)
        say(f"    layer {l}: rel err {err:.3e} (largest per-row {rerr:.3e})")
        assert err <= TOL_LAYER, (l, err)
        assert err <= TOL_DECODE_PATH and rerr <= TOL_DECODE_PATH, (l, err, rerr)


def test_stack_mixed_layer_shapes(bqe):
    """Consecutive stacked layers with different expert counts and expert
    sizes (same d and k): each layer's workspace layout differs, and every
    layer must still read its input from the previous layer's output."""
    wls = [mi.small(mi.WORKLOADS["tiny"], E=16, k=4, I=64, Is=0, zipf_s=None, layers=4),
           mi.small(mi.WORKLOADS["tiny"], E=512, k=4, I=96, Is=64, zipf_s=1.1, layers=4),
           mi.small(mi.WORKLOADS["tiny"], E=40, k=4, I=32, Is=160, zipf_s=None, layers=4),
           mi.small(mi.WORKLOADS["tiny"], E=16, k=4, I=64, Is=0, zipf_s=None, layers=4)]
    layers = [packed_layer(wl, l) for l, wl in enumerate(wls)]
    T, d, k, nL = 8, wls[0].d, 4, len(wls)
    x_np = mi.activations(wls[0], T=T, stream=44)
    x = activations_device(x_np)
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    yl = torch.empty((nL, T, d), dtype=torch.float32, device=DEV)
    il = torch.empty((nL, T, k), dtype=torch.int32, device=DEV)
    wlr = torch.empty((nL, T, k), dtype=torch.float32, device=DEV)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))
    say(f"[stack] mixed shapes: E={[w.E for w in wls]} I={[w.I for w in wls]} Is={[w.Is for w in wls]} T={T}")
    bqe.moe_stack_forward([L.handle for L in layers], x, y, ws, 1e-6, yl, il, wlr)
    torch.cuda.synchronize()
    yl, il, wlr = yl.cpu().numpy(), il.cpu().numpy(), wlr.cpu().numpy()
    assert np.array_equal(y.cpu().numpy(), yl[-1])
    h = x_np
    for l, wl in enumerate(wls):
        if l > 0:
            h = oracle.rmsnorm(yl[l - 1], 1e-6)
        OL = oracle_layer(wl, l, il[l].reshape(-1))
        oy, _, _, _ = oracle.layer_forward(OL, h, force_idx=il[l], force_w=wlr[l])
        err = rel_err_inf(yl[l], oy)
        say(f"    layer {l}: rel err {err:.3e}")
        assert err <= TOL_DECODE_PATH, (l, err)


def test_stack_chunks_of_eight(bqe, monkeypatch):
    """With MOE_MID_T=0, 9..16 tokens run the decode kernels 8 tokens at a
    time: a 12-token stack call equals calls on rows 0..7 and 8..11, bit for
    bit, in the output, the per-layer outputs and the per-layer routing."""
    monkeypatch.setenv("MOE_MID_T", "0")
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64, zipf_s=1.1, layers=3)
    layers = [packed_layer(wl, l) for l in range(wl.layers)]
    nL, d, k, T = wl.layers, wl.d, wl.k, 12
    x_np = mi.activations(wl, T=T, stream=15)
    ws = bqe.new_workspace(max(L.workspace_bytes(T) for L in layers))

    def run(xs):
        n = xs.shape[0]
        y = torch.empty((n, d), dtype=torch.float32, device=DEV)
        yl = torch.empty((nL, n, d), dtype=torch.float32, device=DEV)
        il = torch.empty((nL, n, k), dtype=torch.int32, device=DEV)
        wr = torch.empty((nL, n, k), dtype=torch.float32, device=DEV)
        bqe.moe_stack_forward([L.handle for L in layers], activations_device(xs), y, ws, 1e-6, yl, il, wr)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (y, yl, il, wr)]

    say(f"[stack] chunks of eight: T={T}")
    full = run(x_np)
    a, b = run(x_np[:8]), run(x_np[8:])
    for name, f, pa, pb in zip(("y", "y_layers", "idx_layers", "w_layers"), full, a, b):
        joined = np.concatenate([pa, pb], axis=0 if name == "y" else 1)
        assert np.array_equal(f.view(np.uint32), joined.view(np.uint32)), name
