"""The C ABI library loads and exports every declared symbol; host-side
argument checks reject bad input before anything touches the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bqe():
    import bit_quantized_experts_amd as m
    if not os.path.exists(m.LIB_PATH):
        from bit_quantized_experts_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_and_binding_agree(bqe):
    decl = declared_functions()
    assert len(decl) >= 14
    assert sorted(decl) == sorted(bqe.EXPORTED)


def test_library_exports_every_symbol(bqe):
    out = subprocess.run(["nm", "-D", "--defined-only", bqe.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(bqe.lib(), name)


def test_packed_bytes_matches_format(bqe):
    for name in ("tiny", "layer_t1", "stack_3bit", "prefill"):
        wl = mi.WORKLOADS[name]
        desc = bqe.make_desc(wl.d, wl.E, wl.I, wl.Is, wl.k, wl.bits)
        n = bqe.moe_packed_bytes(desc)
        # the packed weights are exactly the canonical bytes (no expansion),
        # plus the router (fp32, and an fp16 hi/lo copy with row exponents for
        # the prefill router), bias, a status word and 256-byte alignment
        weights = wl.E * wl.expert_bytes() + (wl.expert_bytes(wl.Is) if wl.Is else 0)
        E16 = (wl.E + 15) // 16 * 16
        router = wl.E * wl.d * 4 + wl.E * 4 + E16 * wl.d * 4 + E16 * 4
        assert weights + router <= n <= weights + router + 256 * (4 * wl.E + 8), name


@pytest.mark.parametrize("field,value,code", [
    ("block", 16, 2), ("bits", 4, 2), ("d_model", 2560 + 32, 2), ("n_experts", 0, 2),
    ("n_experts", 5000, 2), ("d_ff", 48, 2), ("d_ff_shared", 40, 2), ("top_k", 0, 1), ("top_k", 17, 1),
])
def test_packed_bytes_rejects(bqe, field, value, code):
    desc = bqe.make_desc(2560, 512, 640, 640, 10, 2)
    setattr(desc, field, value)
    with pytest.raises(bqe.MoeError) as ei:
        bqe.moe_packed_bytes(desc)
    assert ei.value.code == code
    assert bqe.moe_last_error()


def test_host_checks_without_gpu(bqe):
    L = bqe.lib()
    assert L.moe_route_topk(None, -1, 8, 2, None, None, None) == bqe.MOE_ERR_ARG
    assert L.moe_route_topk(None, 4, 8, 9, None, None, None) == bqe.MOE_ERR_ARG
    assert L.moe_route_topk(None, 4, 5000, 2, None, None, None) == bqe.MOE_ERR_ARG
    assert L.moe_route_topk(None, 0, 8, 2, None, None, None) == bqe.MOE_OK  # T = 0: nothing to do
    assert L.moe_rmsnorm(None, 2, 6, ctypes.c_float(1e-6), None, None) == bqe.MOE_ERR_ARG
    assert L.moe_workspace_init(None, 1024, None) == bqe.MOE_ERR_ARG
    assert L.moe_layer_forward(None, None, 1, None, None, None, 0, None) == bqe.MOE_ERR_ARG
    assert L.moe_stack_forward(None, 0, None, 1, ctypes.c_float(1e-6), None, None, None, None, None, 0, None) == bqe.MOE_ERR_ARG
    # fp16-activation entry points: at most 16 tokens, then the usual checks
    assert L.moe_layer_forward_f16act(None, None, 17, None, None, None, 0, None) == bqe.MOE_ERR_UNSUPPORTED
    assert L.moe_layer_forward_f16act(None, None, 1, None, None, None, 0, None) == bqe.MOE_ERR_ARG
    assert L.moe_stack_forward_f16act(None, 1, None, 17, ctypes.c_float(1e-6), None, None, None, None, None, 0,
                                      None) == bqe.MOE_ERR_UNSUPPORTED
    assert L.moe_stack_forward_f16act(None, 0, None, 1, ctypes.c_float(1e-6), None, None, None, None, None, 0,
                                      None) == bqe.MOE_ERR_ARG
    assert L.moe_timing_start(9, 1) == bqe.MOE_ERR_ARG
    assert L.moe_group_workspace_bytes(-1, 8, 2, ctypes.byref(ctypes.c_size_t())) == bqe.MOE_ERR_ARG
    assert L.moe_group_tokens(None, 4, 8, 2, None, None, None, None, 0, None) == bqe.MOE_ERR_ARG
    assert L.moe_timing_stop(None, None) == bqe.MOE_ERR_ARG
    assert L.moe_debug_unpack(None, 0, 0, None, None, None, None) == bqe.MOE_ERR_ARG
    n = ctypes.c_size_t()
    assert L.moe_workspace_bytes(None, 1, ctypes.byref(n)) == bqe.MOE_ERR_ARG
