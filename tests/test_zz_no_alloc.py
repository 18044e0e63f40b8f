"""moe_layer_forward_noalloc (the workspace is the library's fixed device scratch) against
moe_layer_forward with a caller workspace: the same kernels, so every output is bitwise equal,
on consecutive calls that reuse the scratch, the second with a smaller input."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import parity as P
from capacity_routing_expert_amd import binding as B
from capacity_routing_expert_amd import layer as L
from capacity_routing_expert_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    B.lib()  # loud failure if the library is missing
    yield
    torch.cuda.synchronize()


def _noalloc(dev, k, cap):
    shape = L.shape_of(dev, k, cap)
    T, E = shape.T, shape.n_experts
    res = {
        "out": torch.empty_like(dev["x"]),
        "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
        "gates": torch.empty((T, k), dtype=torch.float32, device=DEV),
        "slot_of": torch.empty((T, k), dtype=torch.int32, device=DEV),
        "drop_mask": torch.empty((T, k), dtype=torch.uint8, device=DEV),
        "counts": torch.empty((E,), dtype=torch.int32, device=DEV),
    }
    B.moe_layer_forward_noalloc(shape, dev["x"], dev["w_router"], dev["b_router"], dev["w1"],
                                dev["b1"], dev["w2"], dev["b2"], res["out"], topk_ids=res["ids"],
                                topk_gates=res["gates"], slot_of=res["slot_of"],
                                drop_mask=res["drop_mask"], expert_counts=res["counts"])
    return res


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _cases():
    """A bf16 layer of 2500 tokens (5000 assignments: the two-launch dispatch), the decode layer
    (T 64, d_model 2048, d_ff 8192, 8 experts, top-2, capacity 64), then smaller inputs: 40 of
    its tokens with capacity 8 (drops), a small bf16 layer, the fp32 worked example."""
    mid = W.make_shape_inputs(2500, 256, 512, 8, "bf16", seed=23, router_bias_std=1.0)
    dec = W.make_inputs("decode")
    wl = dec["workload"]
    cap = O.capacity(wl.T, wl.top_k, wl.n_experts, wl.capacity_factor)
    part = dict(dec)
    part["x"] = dec["x"][:40].copy()
    small = W.make_shape_inputs(300, 128, 256, 8, "bf16", seed=17, router_bias_std=1.0)
    we = W.make_inputs("worked_example")
    return [("bf16 T2500", mid, 2, O.capacity(2500, 2, 8, 1.0)), ("decode T64", dec, 2, cap),
            ("decode T40 cap 8", part, 2, 8),
            ("bf16 T300", small, 2, O.capacity(300, 2, 8, 1.0)), ("worked example", we, 1, 2)]


def test_noalloc_matches_layer_forward_on_consecutive_calls():
    """Each case through both entry points, one after another on the same scratch (every later
    case is smaller than the first); all outputs bitwise equal, and the float outputs within
    the dtype's tolerance of the oracle."""
    for name, inp, k, cap in _cases():
        say(f"[noalloc] {name}")
        dev = L.upload(inp, DEV)
        want = L.layer_forward(dev, k, cap)
        got = _noalloc(dev, k, cap)
        torch.cuda.synchronize()
        for key in ("out", "ids", "gates", "slot_of", "drop_mask", "counts"):
            assert _same(got[key], want[key]), (name, key)
        dt = inp["dtype"]
        f64 = lambda a: W.to_float64(a, dt)
        ref = O.forward(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"], f64(inp["w1"]),
                        f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]), k,
                        cap * inp["w1"].shape[0] / (inp["x"].shape[0] * k))
        assert ref["cap"] == cap
        ids, gates = P.to_np(got["ids"]), P.to_np(got["gates"])
        P.compare_route(ids, gates, ref, x=f64(inp["x"]), w=f64(inp["w_router"]),
                        b=inp["b_router"])
        dref = O.dispatch(ids, gates, inp["w1"].shape[0], cap)
        assert np.array_equal(P.to_np(got["slot_of"]), dref["slot_of"])
        assert P.max_abs_rel(P.to_np(got["out"]), ref["out"]) <= P.TOL[dt]


def test_noalloc_repeated_and_after_a_larger_call():
    """The scratch keeps the last call's contents: a small call right after a large one, and
    the same call twice, give the workspace path's bits."""
    big, small = _cases()[1], _cases()[3]
    for name, inp, k, cap in (big, small, small, big):
        dev = L.upload(inp, DEV)
        a = _noalloc(dev, k, cap)
        b = L.layer_forward(dev, k, cap)
        torch.cuda.synchronize()
        assert _same(a["out"], b["out"]) and _same(a["slot_of"], b["slot_of"]), name


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the fixed scratch (the mid layer needs about 160 MiB) is
    refused on the host with MOE_ERR_WORKSPACE; nothing is launched."""
    shape = B.make_shape(4096, 2048, 8192, 8, 2, 1280, B.MOE_BF16)
    assert B.workspace_bytes(shape) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, 2048), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x)
    wr = torch.zeros((8, 2048), dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros((8, 8192, 2048), dtype=torch.bfloat16, device=DEV)
    b1 = torch.zeros((8, 8192), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((8, 2048, 8192), dtype=torch.bfloat16, device=DEV)
    b2 = torch.zeros((8, 2048), dtype=torch.bfloat16, device=DEV)
    out.fill_(1.0)
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward_noalloc(shape, x, wr, None, w1, b1, w2, b2, out)
    assert ei.value.status == 3 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 1.0).all())  # untouched
    del w1, w2
    torch.cuda.empty_cache()
