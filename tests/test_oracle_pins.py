"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test ties one oracle function to an independent route: numpy's own
binary16 conversion, numpy ``unpackbits`` for the bitstream order, exact
rationals, brute-force sorting, a dense fp64 numpy evaluation of every
expert, closed forms and invariants, and the hand-worked blocks in
``tests/golden/blocks.json``.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent decoders used only by the pins
# ---------------------------------------------------------------------------
def np_decode(canon, rows, cols, bits):
    """Dequantised fp64 weights via numpy's fp16 view and unpackbits (bit order 'little')."""
    bb = 2 + 4 * bits
    blk = np.asarray(canon, dtype=np.uint8).reshape(rows, cols // 32, bb)
    scale = np.ascontiguousarray(blk[..., :2]).view(np.float16)[..., 0].astype(np.float64)
    bitarr = np.unpackbits(blk[..., 2:], axis=-1, bitorder="little").astype(np.int64)
    q = (bitarr.reshape(rows, cols // 32, 32, bits) * (1 << np.arange(bits))).sum(-1)
    c = q - (1 << (bits - 1))
    return (scale[..., None] * c).reshape(rows, cols), c.reshape(rows, cols)


def np_expert(canon, d, I, bits):
    bb = 2 + 4 * bits
    g = I * (d // 32) * bb
    dn = d * (I // 32) * bb
    c = np.asarray(canon, dtype=np.uint8)
    Wg = np_decode(c[:g], I, d, bits)[0]
    Wu = np_decode(c[g:2 * g], I, d, bits)[0]
    Wd = np_decode(c[2 * g:2 * g + dn], d, I, bits)[0]
    return Wg, Wu, Wd


def np_ffn(Wg, Wu, Wd, x):
    g = Wg @ x
    u = Wu @ x
    h = g / (1.0 + np.exp(-g)) * u
    return Wd @ h


# ---------------------------------------------------------------------------
# fp16
# ---------------------------------------------------------------------------
def test_half_to_double_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_double_to_half_matches_numpy(orc):
    g = np.random.default_rng(1)
    vals = np.concatenate([
        g.standard_normal(4000) * 10.0 ** g.integers(-9, 6, 4000),
        # exact ties between neighbouring fp16 values, normal and subnormal
        (np.arange(0, 2048, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -10,
        [65504.0, 65519.99, 65520.0, 1e6, -65520.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 0.0, -0.0],
    ])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.double_to_half(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# unpack
# ---------------------------------------------------------------------------
def test_golden_blocks(orc):
    with open(os.path.join(GOLDEN, "blocks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        blk = bytes.fromhex(case["bytes"].replace(" ", ""))
        codes, scale = orc.unpack_block(blk, case["bits"])
        assert scale == case["scale"], case["note"]
        assert codes.tolist() == case["codes"], case["note"]


def test_unpack_2bit_all_bytes(orc):
    # every byte value at every code position: 256 blocks x 8 positions
    blocks = np.zeros((256 * 8, 10), dtype=np.uint8)
    blocks[:, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), dtype=np.uint8)
    for pos in range(8):
        blocks[pos * 256:(pos + 1) * 256, 2 + pos] = np.arange(256)
    rows = blocks.shape[0]
    codes, scales = orc.unpack_matrix(blocks.reshape(-1), rows, 32, 2)
    _, ref = np_decode(blocks.reshape(-1), rows, 32, 2)
    assert np.array_equal(codes, ref)
    assert np.all(scales == 1.0)
    assert set(np.unique(codes).tolist()) == {-2, -1, 0, 1}


@pytest.mark.slow
def test_unpack_3bit_all_24bit_groups(orc):
    # all 2^24 three-byte groups (eight 3-bit codes each), four groups per block
    n = 1 << 24
    v = np.arange(n, dtype=np.uint32)
    grp = np.stack([v & 0xFF, (v >> 8) & 0xFF, v >> 16], axis=1).astype(np.uint8).reshape(-1, 12)
    nblk = grp.shape[0]
    chunk = 1 << 19
    for c0 in range(0, nblk, chunk):
        g = grp[c0:c0 + chunk]
        blocks = np.zeros((g.shape[0], 14), dtype=np.uint8)
        blocks[:, 0:2] = np.frombuffer(np.float16(-0.5).tobytes(), dtype=np.uint8)
        blocks[:, 2:] = g
        codes, scales = orc.unpack_matrix(blocks.reshape(-1), g.shape[0], 32, 3)
        _, ref = np_decode(blocks.reshape(-1), g.shape[0], 32, 3)
        assert np.array_equal(codes, ref)
        assert np.all(scales == -0.5)


def test_unpack_generated_matrices(orc):
    for bits in (2, 3):
        wl = mi.small(mi.WORKLOADS["tiny"], bits=bits)
        ex = mi.expert_canon(wl, 0, 7).numpy()
        gate, up, down = orc.split_expert(ex, wl.d, wl.I, bits)
        for canon, rows, cols in ((gate, wl.I, wl.d), (up, wl.I, wl.d), (down, wl.d, wl.I)):
            codes, _ = orc.unpack_matrix(canon, rows, cols, bits)
            w = orc.dequant_matrix(canon, rows, cols, bits)
            wref, cref = np_decode(canon, rows, cols, bits)
            assert np.array_equal(codes, cref)
            assert np.array_equal(w, wref)
            lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
            assert codes.min() == lo and codes.max() == hi


def test_dequant_all_scales_exact(orc):
    # every finite positive fp16 scale times every 3-bit code; the product of
    # an 11-bit significand and |c| <= 4 is exact in fp64 and in fp32
    s = np.arange(1, 0x7C00, dtype=np.uint16)
    blocks = np.zeros((s.size, 14), dtype=np.uint8)
    blocks[:, 0] = s & 0xFF
    blocks[:, 1] = s >> 8
    blocks[:, 2:] = np.frombuffer(bytes.fromhex("88c6fa" * 4), dtype=np.uint8)
    w = orc.dequant_matrix(blocks.reshape(-1), s.size, 32, 3)
    sf = s.view(np.float16).astype(np.float64)
    codes = np.tile(np.arange(-4, 4), 4)
    exact = [Fraction(float(a)) * int(c) for a, c in zip(sf[::997], codes[:1].repeat(1))]
    assert np.array_equal(w, sf[:, None] * codes[None, :])
    assert all(Fraction(float(v)) == e for v, e in zip(w[::997, 0], exact))
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


# ---------------------------------------------------------------------------
# exp64
# ---------------------------------------------------------------------------
def test_exp64_constants_are_nearest(orc):
    coeff = orc.exp64_coefficients()
    for i, c in enumerate(coeff):
        assert c == float(Fraction(1, math.factorial(i))), i
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    hi, lo, inv = orc.exp64_ln2_parts()
    assert hi == float(ln2)
    assert lo == float(ln2 - Decimal(hi))
    assert inv == float(1 / ln2)


def test_exp64_vs_libm(orc):
    g = np.random.default_rng(2)
    z = np.concatenate([-g.random(3000) * 745.0, -g.random(2000) * 30.0, -g.random(1000) * 1e-3,
                        [0.0, -0.0, -1e-300, -708.0, -744.0, -1.0, -math.log(2.0) * 10]])
    got = orc.exp64(z)
    ref = np.exp(z)
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got - ref) <= ulp * 1.0 + 0.0)
    assert orc.exp64(np.array([0.0]))[0] == 1.0
    assert orc.exp64(np.array([-2000.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# router, top-k, gate weights
# ---------------------------------------------------------------------------
def test_router_vs_numpy_and_one_hot(orc):
    wl = mi.WORKLOADS["tiny"]
    W, _ = mi.router(wl, 0)
    bias = np.linspace(-1, 1, wl.E).astype(np.float32)
    x = mi.activations(wl, T=9)
    got = orc.router_logits(x, W, bias)
    ref = (x.astype(np.float64) @ W.astype(np.float64).T + bias.astype(np.float64)).astype(np.float32)
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(ref)).astype(np.float64))
    assert np.mean(got == ref) > 0.99
    # one-hot activation picks out a column of W plus the bias exactly
    xo = np.zeros((wl.d, wl.d), dtype=np.float32)
    np.fill_diagonal(xo, 1.0)
    lo = orc.router_logits(xo[:40], W, bias)
    exact = (W[:, :40].T.astype(np.float64) + bias.astype(np.float64)).astype(np.float32)
    assert np.array_equal(lo, exact)


def _brute_topk(l, k):
    order = sorted(range(len(l)), key=lambda e: (-float(l[e]), e))
    return order[:k]


def test_topk_brute_force_and_ties(orc):
    g = np.random.default_rng(3)
    cases = [g.standard_normal((50, 64)).astype(np.float32),
             g.integers(0, 3, (200, 40)).astype(np.float32),       # heavy ties
             np.where(g.random((50, 33)) < 0.5, -0.0, 0.0).astype(np.float32),
             mi.direct_logits(mi.WORKLOADS["layer_t1"], T=64)]
    for l in cases:
        for k in (1, 2, 7, min(10, l.shape[1])):
            idx, w = orc.topk(l, k)
            for t in range(l.shape[0]):
                assert idx[t].tolist() == _brute_topk(l[t], k)
            assert np.all(w > 0)
            assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)


def test_gate_weight_closed_forms(orc):
    g = np.random.default_rng(4)
    l = g.standard_normal((400, 20)).astype(np.float32) * 3
    idx, w = orc.topk(l, 2)
    l0 = l[np.arange(400), idx[:, 0]].astype(np.float64)
    l1 = l[np.arange(400), idx[:, 1]].astype(np.float64)
    w0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.all(np.abs(w[:, 0] - w0) <= np.spacing(w0.astype(np.float32)))
    # all-equal logits: every weight is fp32(1/k)
    for k in (1, 3, 7, 10):
        le = np.full((3, 16), 0.25, dtype=np.float32)
        _, we = orc.topk(le, k)
        assert np.all(we == np.float32(1.0 / k))


def test_topk_rejects_nonfinite(orc):
    l = np.zeros((2, 8), dtype=np.float32)
    l[1, 3] = np.nan
    with pytest.raises(RuntimeError):
        orc.topk(l, 2)


# ---------------------------------------------------------------------------
# expert FFN and layer
# ---------------------------------------------------------------------------
def test_expert_ffn_vs_dense_numpy(orc):
    for bits in (2, 3):
        wl = mi.small(mi.WORKLOADS["tiny"], bits=bits)
        ex = mi.expert_canon(wl, 0, 2).numpy()
        x = mi.activations(wl, T=1)[0].astype(np.float64)
        got = orc.expert_ffn(ex, wl.d, wl.I, bits, x)
        ref = np_ffn(*np_expert(ex, wl.d, wl.I, bits), x)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def _tiny_layer(orc, wl, layer=0, shared=False):
    W, bias = mi.router(wl, layer)
    allx = mi.layer_experts_canon(wl, layer).numpy()
    eb = wl.expert_bytes()
    experts = {e: allx[e * eb:(e + 1) * eb] for e in range(wl.E)}
    sh = mi.expert_canon(wl, layer, -1).numpy() if wl.Is else None
    return orc.Layer(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, W, bias, experts, sh)


def test_layer_vs_dense_masked_all_experts(orc):
    for wl in (mi.WORKLOADS["tiny"],
               mi.small(mi.WORKLOADS["tiny"], bits=3, Is=96, k=3, zipf_s=1.1, T=6)):
        L = _tiny_layer(orc, wl)
        x = mi.activations(wl)
        y, logits, idx, w = orc.layer_forward(L, x)
        # dense: every expert evaluated, gate g_e = w if selected else 0
        xd = x.astype(np.float64)
        eb = wl.expert_bytes()
        dense = [np_expert(L.experts[e], wl.d, wl.I, wl.bits) for e in range(wl.E)]
        ref = np.zeros((x.shape[0], wl.d))
        for t in range(x.shape[0]):
            gate = np.zeros(wl.E)
            gate[idx[t]] = w[t]
            for e in range(wl.E):
                ref[t] += gate[e] * np_ffn(*dense[e], xd[t])
            if wl.Is:
                ref[t] += np_ffn(*np_expert(L.shared, wl.d, wl.Is, wl.bits), xd[t])
        assert np.max(np.abs(y - ref)) <= 4 * np.spacing(np.float32(np.max(np.abs(ref))))
        # routing equals brute force on the oracle's own logits
        for t in range(x.shape[0]):
            assert idx[t].tolist() == _brute_topk(logits[t], wl.k)
        assert eb > 0


def test_single_expert_is_textbook_swiglu(orc):
    wl = mi.small(mi.WORKLOADS["tiny"], E=1, k=1)
    L = _tiny_layer(orc, wl)
    x = mi.activations(wl)
    y, _, idx, w = orc.layer_forward(L, x)
    assert np.all(idx == 0) and np.all(w == 1.0)
    Wg, Wu, Wd = np_expert(L.experts[0], wl.d, wl.I, wl.bits)
    for t in range(x.shape[0]):
        ref = np_ffn(Wg, Wu, Wd, x[t].astype(np.float64))
        assert np.max(np.abs(y[t] - ref)) <= 2 * np.spacing(np.float32(np.max(np.abs(ref))))


def test_unused_experts_do_not_change_output(orc):
    wl = mi.WORKLOADS["tiny"]
    L = _tiny_layer(orc, wl)
    x = mi.activations(wl)
    y, _, idx, _ = orc.layer_forward(L, x)
    used = set(idx.reshape(-1).tolist())
    g = np.random.default_rng(5)
    for e in range(wl.E):
        if e not in used:
            L.experts[e] = g.integers(0, 256, L.experts[e].size).astype(np.uint8)
    y2, _, idx2, _ = orc.layer_forward(L, x)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(y, y2)
    # and they may be absent altogether
    for e in range(wl.E):
        if e not in used:
            del L.experts[e]
    y3, _, _, _ = orc.layer_forward(L, x)
    assert np.array_equal(y, y3)


def test_row_independence_and_forcing(orc):
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64)
    L = _tiny_layer(orc, wl)
    x = mi.activations(wl, T=5)
    y, _, idx, w = orc.layer_forward(L, x)
    for t in range(5):
        yt, _, it, wt = orc.layer_forward(L, x[t:t + 1])
        assert np.array_equal(yt[0], y[t]) and np.array_equal(it[0], idx[t]) and np.array_equal(wt[0], w[t])
    yf, _, _, _ = orc.layer_forward(L, x, force_idx=idx, force_w=w)
    assert np.array_equal(yf, y)


def test_zero_scale_expert_and_shared_linearity(orc):
    wl = mi.small(mi.WORKLOADS["tiny"], Is=64)
    L = _tiny_layer(orc, wl)
    x = mi.activations(wl)
    y, _, idx, w = orc.layer_forward(L, x)
    # zero every scale of the rank-0 expert of token 0: its term vanishes
    e0 = int(idx[0, 0])
    z = L.experts[e0].copy().reshape(-1, 2 + 4 * wl.bits)
    z[:, :2] = 0
    L.experts[e0] = z.reshape(-1)
    yz, _, _, _ = orc.layer_forward(L, x, force_idx=idx, force_w=w)
    ffn0 = orc.expert_ffn(_tiny_layer(orc, wl).experts[e0], wl.d, wl.I, wl.bits, x[0].astype(np.float64))
    assert np.max(np.abs((y[0] - yz[0]) - w[0, 0] * ffn0)) <= 1e-5 * np.max(np.abs(y[0]))
    # removing the shared expert subtracts exactly its FFN
    L2 = _tiny_layer(orc, wl)
    Lns = orc.Layer(wl.d, wl.E, wl.I, 0, wl.k, wl.bits, L2.router_w, L2.router_bias, L2.experts, None)
    yn, _, _, _ = orc.layer_forward(Lns, x, force_idx=idx, force_w=w)
    for t in range(x.shape[0]):
        fs = orc.expert_ffn(L2.shared, wl.d, wl.Is, wl.bits, x[t].astype(np.float64))
        assert np.max(np.abs((y[t].astype(np.float64) - yn[t]) - fs)) <= 1e-5 * np.max(np.abs(y[t]))


def test_rmsnorm_closed_forms(orc):
    d = 64
    for c in (1.0, -3.5, 1e-4):
        x = np.full((2, d), c, dtype=np.float32)
        y = orc.rmsnorm(x, 1e-6)
        assert np.all(y == np.float32(c / math.sqrt(c * c + 1e-6)))
    x = mi.activations(mi.WORKLOADS["tiny"], T=3)
    y = orc.rmsnorm(x, 1e-6)
    xd = x.astype(np.float64)
    ref = xd / np.sqrt((xd * xd).mean(1, keepdims=True) + 1e-6)
    assert np.max(np.abs(y - ref)) <= np.spacing(np.float32(np.abs(ref).max()))


def test_generator_is_deterministic_and_device_agnostic_shape():
    wl = mi.WORKLOADS["tiny"]
    a = mi.layer_experts_canon(wl, 3)
    b = mi.layer_experts_canon(wl, 3)
    assert a.dtype == b.dtype and bool((a == b).all())
    c = mi.layer_experts_canon(wl, 4)
    assert not bool((a == c).all())
    eb = wl.expert_bytes()
    assert bool((mi.expert_canon(wl, 3, 5) == a[5 * eb:6 * eb]).all())


def _group_brute(idx, E):
    """Brute force: list every used (t, r), sort by (expert, token)."""
    T, k = idx.shape
    pairs = []
    for t in range(T):
        seen = set()
        for r in range(k):
            e = int(idx[t, r])
            if 0 <= e < E and e not in seen:
                pairs.append((e, t, t * k + r))
            seen.add(e)
    pairs.sort()
    counts = np.bincount([p[0] for p in pairs], minlength=E).astype(np.int32)
    perm = np.full(T * k, -1, np.int32)
    perm[:len(pairs)] = [p[2] for p in pairs]
    return counts, perm


def test_group_tokens_brute_force(orc):
    rng = np.random.default_rng(11)
    for T, E, k in ((1, 4, 2), (37, 16, 2), (300, 512, 10), (64, 3, 3)):
        # distinct experts per token, Zipf-like skew
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm = orc.group_tokens(idx, E)
        bc, bp = _group_brute(idx, E)
        assert np.array_equal(counts, bc)
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(bc)]).astype(np.int32))
        assert np.array_equal(perm, bp)
        assert offsets[E] == T * k


def test_group_tokens_invalid_and_repeated_entries(orc):
    # ids outside [0, E) and repeats within a token are left out
    idx = np.array([[2, 2, 5], [-1, 0, 7], [1, 3, 1], [0, 9, 0]], np.int32)
    E = 8
    counts, offsets, perm = orc.group_tokens(idx, E)
    bc, bp = _group_brute(idx, E)
    assert np.array_equal(counts, bc) and np.array_equal(perm, bp)
    # hand count: expert 0 <- (1,1),(3,0); 1 <- (2,0); 2 <- (0,0); 3 <- (2,1); 5 <- (0,2); 7 <- (1,2)
    assert counts.tolist() == [2, 1, 1, 1, 0, 1, 0, 1]
    assert perm.tolist() == [4, 9, 6, 0, 7, 2, 5, -1, -1, -1, -1, -1]
    assert offsets[E] == 7


def test_group_tokens_closed_form(orc):
    # token t routes to experts (t + r) mod E: expert e gets the tokens with
    # (e - t) mod E < k, in token order
    T, E, k = 50, 7, 3
    idx = np.array([[(t + r) % E for r in range(k)] for t in range(T)], np.int32)
    counts, offsets, perm = orc.group_tokens(idx, E)
    for e in range(E):
        toks = [t for t in range(T) if (e - t) % E < k]
        assert counts[e] == len(toks)
        got = perm[offsets[e]:offsets[e + 1]]
        assert got.tolist() == [t * k + (e - t) % E for t in toks]


# ---------------------------------------------------------------------------
# codebook blocks (reading R7) and the forced-routing rule (reading R8)
# ---------------------------------------------------------------------------
def np_cb_decode(canon, rows, cols, grid):
    """Independent numpy decoder of codebook blocks: fields by slicing, sign
    bits by unpackbits, magnitudes by fancy indexing into the grid."""
    blk = np.asarray(canon, dtype=np.uint8).reshape(rows, cols // 32, 15)
    scale = np.ascontiguousarray(blk[..., :2]).view(np.float16)[..., 0].astype(np.float64)
    hi = np.unpackbits(blk[..., 10:11], axis=-1, bitorder="little").astype(np.int64)  # [.., 8]
    index = blk[..., 2:10].astype(np.int64) + 256 * hi                                    # [.., 8]
    mag = np.asarray(grid, dtype=np.int64)[index]                                        # [.., 8, 4]
    sign = np.unpackbits(blk[..., 11:15], axis=-1, bitorder="little").astype(np.int64)  # [.., 32]
    c = mag.reshape(rows, cols // 32, 32) * (1 - 2 * sign)
    return (scale[..., None] * c).reshape(rows, cols), c.reshape(rows, cols)


def np_cb_expert(canon, d, I, grid):
    g = I * (d // 32) * 15
    dn = d * (I // 32) * 15
    c = np.asarray(canon, dtype=np.uint8)
    return (np_cb_decode(c[:g], I, d, grid)[0], np_cb_decode(c[g:2 * g], I, d, grid)[0],
            np_cb_decode(c[2 * g:2 * g + dn], d, I, grid)[0])


def test_cb_golden_blocks(orc):
    with open(os.path.join(GOLDEN, "cb_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        grid = np.zeros((512, 4), np.uint8)
        for i, v in case["grid"].items():
            grid[int(i)] = v
        blk = bytes.fromhex(case["bytes"].replace(" ", ""))
        assert len(blk) == 15 == orc.block_bytes(3, grid)
        codes, scale = orc.cb_unpack_block(blk, grid)
        assert scale == case["scale"], case["note"]
        assert codes.tolist() == case["codes"], case["note"]


def test_cb_every_index_and_sign_byte(orc):
    """Each of the 512 indices at each of the 8 positions, and each sign byte
    value at each of the 4 sign bytes, against a direct table walk of the
    field values the block was built from."""
    g = np.random.default_rng(11)
    grid = g.integers(0, 128, (512, 4)).astype(np.uint8)
    for pos in range(8):
        for index in range(512):
            blk = bytearray(15)
            blk[0:2] = b"\x00\x3c"
            blk[2 + pos] = index & 0xFF
            blk[10] = (index >> 8) << pos
            codes, _ = orc.cb_unpack_block(bytes(blk), grid)
            expect = np.tile(grid[0], 8).astype(np.int64)      # other positions: index 0
            expect[4 * pos:4 * pos + 4] = grid[index]
            assert codes.tolist() == expect.tolist(), (pos, index)
    for sb in range(4):
        for v in range(256):
            blk = bytearray(15)
            blk[0:2] = b"\x00\x3c"
            blk[11 + sb] = v
            codes, _ = orc.cb_unpack_block(bytes(blk), grid)
            expect = np.tile(grid[0], 8).astype(np.int64)
            for bit in range(8):
                if (v >> bit) & 1:
                    expect[8 * sb + bit] *= -1
            assert codes.tolist() == expect.tolist(), (sb, v)


def test_cb_generated_matrices_vs_numpy(orc):
    wl = mi.small(mi.WORKLOADS["tiny"], bits=3, codebook=True, scale_lo=0.002, scale_hi=0.008)
    grid = mi.codebook_grid()
    ex = mi.expert_canon(wl, 0, 3).numpy()
    n = wl.I * (wl.d // 32) * 15
    w, c = np_cb_decode(ex[:n], wl.I, wl.d, grid)
    codes, scales = orc.cb_unpack_matrix(ex[:n], wl.I, wl.d, grid)
    assert np.array_equal(codes.astype(np.int64), c)
    assert np.array_equal(orc.cb_dequant_matrix(ex[:n], wl.I, wl.d, grid), w)
    assert np.array_equal(np.repeat(scales, 32, axis=1) * codes, w)


def test_cb_reduces_to_plain_2bit(orc):
    """With grid entry i (i < 256) = the base-4 digits of i, a 2-bit block
    rewritten as a codebook block (index = sum |c| 4^m, sign = c < 0) must
    dequantise to the same weights as the plain 2-bit decoder."""
    grid = np.zeros((512, 4), np.uint8)
    for i in range(256):
        grid[i] = [(i >> (2 * m)) & 3 for m in range(4)]
    wl = mi.small(mi.WORKLOADS["tiny"], bits=2)
    canon = mi.expert_canon(wl, 0, 1).numpy()[: 64 * 8 * 10]          # 64 rows x 256 inputs
    codes, scales = orc.unpack_matrix(canon, 64, 256, 2)
    cb = np.zeros((64, 8, 15), np.uint8)
    blk = canon.reshape(64, 8, 10)
    cb[..., 0:2] = blk[..., 0:2]
    c = codes.reshape(64, 8, 8, 4).astype(np.int64)
    index = (np.abs(c) * (4 ** np.arange(4))).sum(-1)                  # [64, 8, 8] < 256
    cb[..., 2:10] = index.astype(np.uint8)
    sign = (codes.reshape(64, 8, 32) < 0).astype(np.uint8)
    cb[..., 11:15] = np.packbits(sign, axis=-1, bitorder="little")
    w_cb = orc.cb_dequant_matrix(cb.reshape(-1), 64, 256, grid)
    assert np.array_equal(w_cb, orc.dequant_matrix(canon, 64, 256, 2))


def test_cb_dequant_exact_all_scales(orc):
    """Every positive finite fp16 scale times magnitudes up to 127 with both
    signs: the fp64 product is exact and also exact in fp32."""
    grid = np.zeros((512, 4), np.uint8)
    grid[0] = [127, 1, 77, 0]
    grid[1] = [3, 101, 126, 15]
    scales = np.arange(1, 0x7C00, dtype=np.uint16)
    rows = scales.size
    canon = np.zeros((rows, 15), np.uint8)
    canon[:, 0] = scales & 0xFF
    canon[:, 1] = scales >> 8
    canon[:, 2:10] = [0, 1, 0, 1, 0, 1, 0, 1]
    canon[:, 11:15] = [0x5A, 0xC3, 0x0F, 0xF0]
    w = orc.cb_dequant_matrix(canon.reshape(-1), rows, 32, grid)
    s = scales.view(np.float16).astype(np.float64)
    _, c = np_cb_decode(canon.reshape(-1), rows, 32, grid)
    from fractions import Fraction as F
    for r in range(0, rows, 97):
        for j in range(32):
            assert F(w[r, j]) == F(s[r]) * int(c[r, j])
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


def test_cb_expert_ffn_and_layer_vs_dense(orc):
    grid = mi.codebook_grid()
    wl = mi.small(mi.WORKLOADS["tiny"], bits=3, codebook=True, Is=64, k=3, zipf_s=1.1, T=5,
                  scale_lo=0.002, scale_hi=0.008)
    ex = mi.expert_canon(wl, 0, 2).numpy()
    x = mi.activations(wl, T=1)[0].astype(np.float64)
    got = orc.expert_ffn(ex, wl.d, wl.I, 3, x, grid=grid)
    ref = np_ffn(*np_cb_expert(ex, wl.d, wl.I, grid), x)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))

    W, bias = mi.router(wl, 0)
    allx = mi.layer_experts_canon(wl, 0).numpy()
    eb = wl.expert_bytes()
    assert eb == 3 * wl.I * (wl.d // 32) * 15
    experts = {e: allx[e * eb:(e + 1) * eb] for e in range(wl.E)}
    sh = mi.expert_canon(wl, 0, -1).numpy()
    L = orc.Layer(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits, W, bias, experts, sh, grid=grid)
    xs = mi.activations(wl)
    y, _, idx, w = orc.layer_forward(L, xs)
    dense = [np_cb_expert(experts[e], wl.d, wl.I, grid) for e in range(wl.E)]
    dsh = np_cb_expert(sh, wl.d, wl.Is, grid)
    for t in range(xs.shape[0]):
        gate = np.zeros(wl.E)
        gate[idx[t]] = w[t]
        xt = xs[t].astype(np.float64)
        r = sum(gate[e] * np_ffn(*dense[e], xt) for e in range(wl.E)) + np_ffn(*dsh, xt)
        assert np.max(np.abs(y[t] - r)) <= 4 * np.spacing(np.float32(np.max(np.abs(r))))


def test_forced_routing_invalid_and_repeated_ids(orc):
    """Reading R8: an id outside [0, E) contributes nothing and a repeated id
    counts once, at its first rank: the output equals the closed form
    w_first * FFN_e(x) (+ the other valid experts)."""
    wl = mi.small(mi.WORKLOADS["tiny"], k=3)
    L = _tiny_layer(orc, wl)
    x = mi.activations(wl, T=2)
    fi = np.array([[5, 5, 99], [-1, 7, 7]], np.int32)
    fw = np.array([[0.75, 0.25, 0.5], [0.5, 0.375, 0.125]], np.float32)
    y, _, _, _ = orc.layer_forward(L, x, force_idx=fi, force_w=fw)
    r0 = 0.75 * orc.expert_ffn(L.experts[5], wl.d, wl.I, wl.bits, x[0].astype(np.float64))
    r1 = 0.375 * orc.expert_ffn(L.experts[7], wl.d, wl.I, wl.bits, x[1].astype(np.float64))
    assert np.array_equal(y[0], r0.astype(np.float32))
    assert np.array_equal(y[1], r1.astype(np.float32))
