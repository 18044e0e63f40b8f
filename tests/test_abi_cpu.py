"""The C-ABI library builds, loads and exports every symbol include/moe.h declares; its
host-only entry points (capacity, workspace size, argument checks) work without a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.moe_oracle as O
from capacity_routing_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from capacity_routing_expert_amd import build
        build.build()
    return B.lib()


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert declared == sorted(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_capacity_matches_oracle(lib):
    assert B.capacity(8, 1, 4, 1.25) == 2
    rng = np.random.Generator(np.random.PCG64(3))
    for _ in range(2000):
        T = int(rng.integers(0, 200000)); k = int(rng.integers(1, 9)); E = int(rng.integers(1, 257))
        C = float(rng.choice([0.1, 0.7, 1.0, 1.1, 1.25, 1.5, 2.0, 3.3, 4.0, 0.3333333333333333]))
        assert B.capacity(T, k, E, C) == O.capacity(T, k, E, C), (T, k, E, C)
    assert B.capacity(10, 1, 7, 0.7) == 0
    assert B.capacity(-1, 1, 1, 1.0) == -1
    assert B.capacity(1, 0, 1, 1.0) == -1
    assert B.capacity(1, 1, 1, float("nan")) == -1
    assert B.capacity(1, 1, 1, -0.5) == -1


def test_workspace_and_max_rows(lib):
    s = B.make_shape(4096, 2048, 8192, 8, 2, 1280, B.MOE_BF16)
    assert B.max_kept_rows(s) == min(4096 * 2, 8 * 1280)
    ws = B.workspace_bytes(s)
    # at least H and Y for the largest possible number of kept rows
    assert ws >= 8192 * 8192 * 2 + 8192 * 2048 * 2
    assert ws % 256 == 0
    bad = B.make_shape(16, 64, 64, 4, 5, 4, B.MOE_BF16)  # k > E
    assert B.workspace_bytes(bad) == 0 and B.max_kept_rows(bad) == -1


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 0, 1), ("top_k", 9, 1), ("n_experts", 0, 1), ("n_experts", 300, 1),
    ("capacity", -1, 1), ("T", -5, 1), ("d_model", 12, 2), ("dtype", 7, 2),
    # 32-bit limits: T * top_k assignments, bytes of x, tile offsets into d_ff rows
    ("T", 1 << 30, 2), ("T", 1 << 24, 2), ("d_ff", 1 << 22, 2),
])
def test_shape_errors_before_any_launch(lib, field, value, status):
    s = B.make_shape(16, 64, 64, 8, 2, 4, B.MOE_BF16)
    setattr(s, field, value)
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = lib.moe_route(ctypes.byref(s), p, p, None, p, p, None, p, 1 << 30, None)
    assert rc == status, (rc, B.last_error())
    assert B.last_error()


def test_pointer_errors_before_any_launch(lib):
    s = B.make_shape(16, 64, 64, 8, 2, 4, B.MOE_BF16)
    p = ctypes.c_void_p(4096)
    assert lib.moe_route(ctypes.byref(s), None, p, None, p, p, None, p, 1 << 30, None) == 1
    assert "x is NULL" in B.last_error()
    assert lib.moe_route(ctypes.byref(s), ctypes.c_void_p(4098), p, None, p, p, None, p, 1 << 30, None) == 2
    assert "aligned" in B.last_error()
    assert lib.moe_route(ctypes.byref(s), p, p, None, p, p, None, p, 16, None) == 3
    assert "workspace" in B.last_error()
    assert lib.moe_combine(ctypes.byref(s), p, p, p, p, p, None) == 1  # out aliases x
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"


def test_weight_layout_checks_on_the_host(lib):
    """The packed weight layout is checked before anything runs: unknown layout values, fp32,
    and experts too large for 32-bit offsets are refused; the packed size rounds columns up to
    whole 32-column blocks."""
    ok = B.make_shape(64, 2048, 8192, 8, 2, 32, B.MOE_BF16, B.MOE_WEIGHTS_PACKED)
    assert B.workspace_bytes(ok) > 0
    assert B.packed_weights_bytes(ok, 8192, 2048) == 8 * 8192 * 2048 * 2
    assert B.packed_weights_bytes(ok, 136, 72) == 8 * 3 * 136 * 32 * 2  # 72 -> 3 blocks of 32
    assert B.workspace_bytes(B.make_shape(64, 2048, 8192, 8, 2, 32, B.MOE_BF16, 2)) == 0
    assert "weight_layout" in B.last_error()
    assert B.workspace_bytes(B.make_shape(8, 8, 8, 4, 1, 2, B.MOE_F32, B.MOE_WEIGHTS_PACKED)) == 0
    assert "bf16" in B.last_error()
    assert B.workspace_bytes(B.make_shape(8, 32768, 32768, 4, 1, 0, B.MOE_BF16,
                                          B.MOE_WEIGHTS_PACKED)) == 0
    assert "4 GiB" in B.last_error()
    # packing refuses fp32 and ragged columns before launching anything
    f32 = B.make_shape(8, 8, 8, 2, 1, 0, B.MOE_F32)
    assert lib.moe_pack_weights(ctypes.byref(f32), ctypes.c_void_p(16), 8, 8, ctypes.c_void_p(4096),
                                None) == 2
    bf = B.make_shape(8, 8, 8, 2, 1, 0, B.MOE_BF16)
    assert lib.moe_pack_weights(ctypes.byref(bf), ctypes.c_void_p(16), 8, 12, ctypes.c_void_p(4096),
                                None) == 2


def test_gemm_timing_arm_checks_on_the_host(lib):
    """moe_set_gemm_timing only stores the handles: a half-NULL pair or four NULLs are refused,
    one GEMM's pair may be NULL, NULL disarms (no GPU call is made, so stand-in handles are
    enough here)."""
    half = (ctypes.c_void_p * 4)(1, 2, 0, 4)
    assert lib.moe_set_gemm_timing(half) == 1
    assert "events[2] and events[3]" in B.last_error()
    none = (ctypes.c_void_p * 4)(0, 0, 0, 0)
    assert lib.moe_set_gemm_timing(none) == 1
    assert lib.moe_set_gemm_timing(None) == 0
    for ok in ((1, 2, 3, 4), (1, 2, 0, 0), (0, 0, 3, 4)):
        assert lib.moe_set_gemm_timing((ctypes.c_void_p * 4)(*ok)) == 0
    assert lib.moe_set_gemm_timing(None) == 0  # disarmed before any layer call


def test_stage_timing_arm_checks_on_the_host(lib):
    """moe_set_stage_timing (router and combine kernels) only stores the handles, with the same
    rules as the GEMM timing: a half-NULL pair or four NULLs are refused, one kernel's pair may
    be NULL, NULL disarms."""
    half = (ctypes.c_void_p * 4)(0, 2, 3, 4)
    assert lib.moe_set_stage_timing(half) == 1
    assert "events[0] and events[1]" in B.last_error()
    assert lib.moe_set_stage_timing((ctypes.c_void_p * 4)(0, 0, 0, 0)) == 1
    for ok in ((1, 2, 3, 4), (1, 2, 0, 0), (0, 0, 3, 4)):
        assert lib.moe_set_stage_timing((ctypes.c_void_p * 4)(*ok)) == 0
    assert lib.moe_set_stage_timing(None) == 0  # disarmed before any layer call


def test_dispatch_gather_argument_checks(lib):
    """moe_dispatch takes x and x_routed together or not at all, and refuses overlapping ones,
    before anything is launched."""
    s = B.make_shape(16, 64, 64, 8, 2, 4, B.MOE_BF16)
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    args = [ctypes.byref(s), p, p, p, p, p, p, p]
    assert lib.moe_dispatch(*args, p, None, ws, 1 << 30, None) == 1
    assert "x_routed" in B.last_error()
    assert lib.moe_dispatch(*args, None, p, ws, 1 << 30, None) == 1
    # x [16, 64] bf16 = 2 KiB at 4096, x_routed [max_rows = 16 * 2 ... 32 rows] overlapping it
    assert lib.moe_dispatch(*args, ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 1024), ws,
                            1 << 30, None) == 1
    assert "overlaps" in B.last_error()


def _cpu(n, dtype):
    import torch
    return torch.zeros(n, dtype=dtype)


ROUTE_ARGS = ["x", "w_router", "b_router", "topk_ids", "topk_gates", "logits"]


@pytest.mark.parametrize("which", ROUTE_ARGS)
def test_binding_refuses_undersized_route_tensors(lib, which):
    """The binding checks every tensor's size against the shape before its pointer reaches the
    library.  Only the tensor under test is passed (a CPU tensor: its size is checked before
    its device), every other argument is None."""
    import torch
    T, d, E, k = 16, 64, 8, 2
    s = B.make_shape(T, d, 64, E, k, 4, B.MOE_BF16)
    need = {"x": (T * d, torch.bfloat16), "w_router": (E * d, torch.bfloat16),
            "b_router": (E, torch.float32), "topk_ids": (T * k, torch.int32),
            "topk_gates": (T * k, torch.float32), "logits": (T * E, torch.float32)}
    n, dt = need[which]
    for size, msg in ((n - 1, f"{which} holds {n - 1} elements, the shape needs {n}"),
                      (n, "must be on the GPU")):
        args = {a: None for a in ROUTE_ARGS}
        args[which] = _cpu(size, dt)
        with pytest.raises(ValueError, match=msg):
            B.moe_route(s, *[args[a] for a in ROUTE_ARGS], _cpu(256, torch.uint8))


LAYER_ARGS = ["x", "w_router", "b_router", "w1", "b1", "w2", "b2", "out"]


@pytest.mark.parametrize("which", ["x", "w1", "b1", "w2", "b2", "out", "topk_ids",
                                   "expert_counts", "slot_of"])
def test_binding_refuses_undersized_layer_tensors(lib, which):
    import torch
    T, d, f, E, k = 16, 64, 96, 8, 2
    s = B.make_shape(T, d, f, E, k, 4, B.MOE_BF16)
    bf = torch.bfloat16
    need = {"x": (T * d, bf), "w1": (E * f * d, bf), "b1": (E * f, bf), "w2": (E * d * f, bf),
            "b2": (E * d, bf), "out": (T * d, bf), "topk_ids": (T * k, torch.int32),
            "expert_counts": (E, torch.int32), "slot_of": (T * k, torch.int32)}
    n, dt = need[which]
    pos = {a: None for a in LAYER_ARGS}
    kw = {"topk_ids": None, "expert_counts": None, "slot_of": None}
    (pos if which in pos else kw)[which] = _cpu(n - 1, dt)
    with pytest.raises(ValueError, match=f"{which} holds {n - 1} elements"):
        B.moe_layer_forward(s, *[pos[a] for a in LAYER_ARGS], ws=_cpu(256, torch.uint8), **kw)


def test_binding_packed_weight_sizes(lib):
    """Packed weights need ceil(cols / 32) * 32 columns: a row-major-sized W2 is refused."""
    import torch
    T, d, f, E, k = 16, 72, 104, 4, 2  # W2's 104 columns pack into 4 blocks of 32
    s = B.make_shape(T, d, f, E, k, 4, B.MOE_BF16, B.MOE_WEIGHTS_PACKED)
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="w2 holds"):
        B.moe_expert_ffn(s, None, _cpu(0, torch.int32), None, None, None, _cpu(E * d * f, bf),
                         None, _cpu(0, bf), _cpu(256, torch.uint8))
    with pytest.raises(ValueError, match="must be on the GPU"):
        B.moe_expert_ffn(s, None, _cpu(0, torch.int32), None, None, None,
                         _cpu(E * 4 * d * 32, bf), None, _cpu(0, bf), _cpu(256, torch.uint8))
