"""Seeded synthetic inputs for the low-bit MoE layer.

This module is the only code that both the HIP path's tests/benchmark and the
CPU oracle draw on.  It holds none of the layer's arithmetic: it produces raw
bytes and plain float arrays, nothing else.

Expert weights come in the canonical block format {fp16 scale, 32 b-bit
codes}.  Codes are uniform over their range, so every bit pattern of a
block's code bytes is equally likely; the generator therefore writes uniform
random bytes for the codes and never packs individual values.  Scales are
uniform in [lo, hi) rounded to fp16.

Weight bytes come from a counter-based hash (the "lowbias32" integer mixer,
applied twice with two stream keys), evaluated with int64 torch arithmetic
that never overflows, so the same call gives the same bytes on the CPU and on
the GPU.  That lets the GPU build a 48-layer stack (tens of GB) in place
while the oracle regenerates on the host only the experts a check touches.

Float inputs that need a normal distribution (activations, router weights)
come from numpy's PCG64 on the host; they are small.

Workloads (one table; the sizes follow the model the pages describe: 48
layers of 512 small experts, about ten routed per token, plus a shared
expert [cnyes profile of Strata, section "Strata 到底是什麼？"]):
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

M32 = 0xFFFFFFFF


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    E: int
    I: int
    Is: int          # shared-expert intermediate size, 0 = none
    k: int
    bits: int
    T: int
    layers: int
    scale_lo: float
    scale_hi: float
    router_sigma: float = 0.02
    zipf_s: float | None = 1.1   # None = no router bias
    seed: int = 0
    extra_T: tuple = field(default_factory=tuple)
    codebook: bool = False       # codebook blocks (15 bytes per 32 weights) instead of b-bit codes

    def block_bytes(self) -> int:
        return CB_BLOCK_BYTES if self.codebook else 2 + 4 * self.bits

    def expert_blocks(self, I: int | None = None) -> int:
        I = self.I if I is None else I
        return 3 * I * (self.d // 32)

    def expert_bytes(self, I: int | None = None) -> int:
        return self.expert_blocks(I) * self.block_bytes()


WORKLOADS = {
    # small case the oracle finishes in seconds
    "tiny": Workload("tiny", d=256, E=16, I=64, Is=0, k=2, bits=2, T=4, layers=1,
                     scale_lo=0.01, scale_hi=0.05, zipf_s=None),
    # one full-size layer, single-token decode
    "layer_t1": Workload("layer_t1", d=2560, E=512, I=640, Is=640, k=10, bits=2, T=1,
                         layers=1, scale_lo=0.01, scale_hi=0.05),
    # 48-layer stack, 8 tokens per pass (1 real + 7 drafts), 2-bit
    "stack_t8_2bit": Workload("stack_t8_2bit", d=2560, E=512, I=640, Is=640, k=10, bits=2,
                              T=8, layers=48, scale_lo=0.01, scale_hi=0.05),
    # 48-layer stack, 3-bit, decode at T=1 and T=8
    "stack_3bit": Workload("stack_3bit", d=2560, E=512, I=640, Is=640, k=10, bits=3,
                           T=8, layers=48, scale_lo=0.005, scale_hi=0.03, extra_T=(1,)),
    # chunked prefill through one layer
    "prefill": Workload("prefill", d=2560, E=512, I=640, Is=640, k=10, bits=2, T=8192,
                        layers=1, scale_lo=0.01, scale_hi=0.05),
    # chunked prefill through the 48-layer 2-bit stack (the same layers as stack_t8_2bit)
    "stack_prefill": Workload("stack_prefill", d=2560, E=512, I=640, Is=640, k=10, bits=2, T=8192,
                              layers=48, scale_lo=0.01, scale_hi=0.05),
}

# codebook-block variants (a synthetic grid stands in for the real tables)
WORKLOADS["layer_t1_cb3"] = replace(WORKLOADS["layer_t1"], name="layer_t1_cb3", bits=3, codebook=True,
                                    scale_lo=0.002, scale_hi=0.008)
WORKLOADS["stack_cb3"] = replace(WORKLOADS["stack_t8_2bit"], name="stack_cb3", bits=3, codebook=True,
                                 scale_lo=0.002, scale_hi=0.008)

# codebook blocks: fp16 scale + 13 payload bytes (index bytes, index high
# bits, sign bits); grid of 512 entries of 4 magnitudes
CB_BLOCK_BYTES = 15
CB_ENTRIES = 512

# stream ids inside one (seed, layer)
STREAM_ROUTED = 1
STREAM_SHARED = 2


# ---------------------------------------------------------------------------
# counter-based hash (lowbias32 mixer), int64 torch arithmetic, no overflow
# ---------------------------------------------------------------------------
def _mul32_t(x: torch.Tensor, c: int) -> torch.Tensor:
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + ((x * hi) & 0xFFFF) * 65536) & M32


def _mix32_t(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32_t(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32_t(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def stream_keys(seed: int, layer: int, stream: int) -> tuple[int, int]:
    k0 = _mix32(_mix32(seed ^ 0x243F6A88) ^ _mix32(layer + 0x13198A2E) ^ _mix32(stream * 0x03707344 + 1))
    k1 = _mix32(k0 ^ 0xA4093822 ^ _mix32(seed + 0x299F31D0))
    return k0, k1


def hash_words(k0: int, k1: int, ctr: torch.Tensor) -> torch.Tensor:
    """32-bit words (as int64 in [0, 2^32)) for 32-bit counters."""
    return _mix32_t(_mix32_t((ctr + k0) & M32) ^ k1)


def canon_blocks(seed: int, layer: int, stream: int, first: int, count: int, bits: int,
                 scale_lo: float, scale_hi: float, device="cpu", chunk: int = 1 << 22,
                 codebook: bool = False) -> torch.Tensor:
    """Canonical blocks [first, first+count) of one stream, as uint8 [count, bytes].

    b-bit blocks (2 + 4*bits bytes): block n uses counters 4n .. 4n+bits; word
    4n gives the scale (u = word / 2^32, s = fp16(fp32(lo + (hi-lo) u))),
    words 4n+1.. give the 4*bits code bytes, little endian.

    Codebook blocks (15 bytes): block n uses counters 8n .. 8n+4; word 8n gives
    the scale as above, words 8n+1..8n+4 give the 13 payload bytes (the first
    13 of their 16 little-endian bytes), so grid indices and signs are uniform.
    """
    assert bits in (2, 3)
    per = 8 if codebook else 4
    assert per * (first + count) < (1 << 32), "counter space of one stream exceeded"
    k0, k1 = stream_keys(seed, layer, stream)
    bb = CB_BLOCK_BYTES if codebook else 2 + 4 * bits
    n_words = 4 if codebook else bits
    out = torch.empty((count, bb), dtype=torch.uint8, device=device)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        base = torch.arange(first + c0, first + c0 + n, dtype=torch.int64, device=device) * per
        w0 = hash_words(k0, k1, base)
        u = w0.to(torch.float64) * (2.0 ** -32)
        s = (u * (scale_hi - scale_lo) + scale_lo).to(torch.float32).to(torch.float16)
        sb = s.view(torch.int16).to(torch.int64) & 0xFFFF
        cols = [sb & 0xFF, sb >> 8]
        for j in range(n_words):
            wj = hash_words(k0, k1, base + (1 + j))
            cols += [wj & 0xFF, (wj >> 8) & 0xFF, (wj >> 16) & 0xFF, wj >> 24]
        out[c0:c0 + n] = torch.stack(cols[:bb], dim=1).to(torch.uint8)
        del base, w0, u, s, sb, cols
    return out


def codebook_grid(seed: int = 0) -> np.ndarray:
    """Synthetic codebook [512, 4] uint8: 512 distinct 4-vectors of odd
    magnitudes 1..15 (a seeded choice among the 8^4 = 4096 such vectors)."""
    g = _rng(seed, 404)
    pick = g.permutation(8 ** 4)[:CB_ENTRIES]
    digits = np.stack([(pick >> (3 * c)) & 7 for c in range(4)], axis=1)
    return (2 * digits + 1).astype(np.uint8)


def expert_canon(wl: Workload, layer: int, expert: int, device="cpu") -> torch.Tensor:
    """Canonical bytes of one expert (expert = -1: the shared expert), flat uint8."""
    if expert < 0:
        nb = wl.expert_blocks(wl.Is)
        blk = canon_blocks(wl.seed, layer, STREAM_SHARED, 0, nb, wl.bits, wl.scale_lo, wl.scale_hi, device,
                           codebook=wl.codebook)
    else:
        nb = wl.expert_blocks()
        blk = canon_blocks(wl.seed, layer, STREAM_ROUTED, expert * nb, nb, wl.bits,
                           wl.scale_lo, wl.scale_hi, device, codebook=wl.codebook)
    return blk.reshape(-1)


def layer_experts_canon(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    """Canonical bytes of all routed experts of one layer, [E * expert_bytes] uint8."""
    nb = wl.expert_blocks()
    blk = canon_blocks(wl.seed, layer, STREAM_ROUTED, 0, wl.E * nb, wl.bits,
                       wl.scale_lo, wl.scale_hi, device, codebook=wl.codebook)
    return blk.reshape(-1)


# ---------------------------------------------------------------------------
# float inputs (host, numpy PCG64)
# ---------------------------------------------------------------------------
def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def router(wl: Workload, layer: int):
    """(W_r [E, d] fp32 ~ N(0, sigma^2), bias [E] fp32 or None).

    Zipf-skewed bias: b_e = -s * ln(pi(e) + 1) for a seeded random permutation
    pi of the experts, i.e. the log of the Zipf(s) weights (the normalising
    constant is a common shift and does not change the routing).
    """
    g = _rng(wl.seed, 101, layer)
    W = (g.standard_normal((wl.E, wl.d)) * wl.router_sigma).astype(np.float32)
    if wl.zipf_s is None:
        return W, None
    perm = g.permutation(wl.E)
    bias = (-wl.zipf_s * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    return W, bias


def activations(wl: Workload, T: int | None = None, stream: int = 0) -> np.ndarray:
    """x [T, d] fp32 ~ N(0, 1)."""
    T = wl.T if T is None else T
    g = _rng(wl.seed, 202, stream)
    return g.standard_normal((T, wl.d)).astype(np.float32)


def direct_logits(wl: Workload, T: int, stream: int = 0) -> np.ndarray:
    """Router logits drawn directly: N(0,1) plus the workload's Zipf bias (fp32)."""
    g = _rng(wl.seed, 303, stream)
    l = g.standard_normal((T, wl.E))
    _, bias = router(wl, 0)
    if bias is not None:
        l = l + bias.astype(np.float64)[None, :]
    return l.astype(np.float32)


def small(wl: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (for reduced test sizes)."""
    return replace(wl, **kw)
