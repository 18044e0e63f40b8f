"""Kernel timing of the expert GEMMs (moe_set_gemm_timing) and of the router and the combine
(moe_set_stage_timing): the timed call returns the untimed call's bits, and the events bracket
the kernels in order."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
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
    B.moe_set_gemm_timing(None)
    B.moe_set_stage_timing(None)
    torch.cuda.synchronize()


def new_events(n=4):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for ev in evs:
        ev.record()  # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    return evs


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check_events(evs, empty=False):
    up = evs[0].elapsed_time(evs[1])
    gap = evs[1].elapsed_time(evs[2])
    down = evs[2].elapsed_time(evs[3])
    say(f"    up {up * 1e3:.1f} us, gap {gap * 1e3:.1f} us, down {down * 1e3:.1f} us")
    assert gap >= 0.0
    if empty:
        assert up >= 0.0 and down >= 0.0
    else:
        assert up > 0.0 and down > 0.0


@pytest.mark.parametrize("T,d,f,E,k,C,dt", [
    (1000, 136, 264, 8, 2, 1.0, "bf16"),   # large tiles
    (65, 264, 328, 8, 2, 1.25, "bf16"),    # decode-sized tiles
    (65, 12, 20, 8, 2, 0.75, "f32"),       # fp32 FMA path
])
def test_timed_layer_same_bits(T, d, f, E, k, C, dt):
    say(f"[timing] layer T={T} d={d} f={f} E={E} k={k} {dt}")
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=T + E, router_bias_std=1.0)
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, C)
    a = L.layer_forward(dev, k, cap)
    evs = new_events()
    B.moe_set_gemm_timing(evs)
    b = L.layer_forward(dev, k, cap)
    torch.cuda.synchronize()
    assert torch.equal(bits(a["out"]), bits(b["out"]))
    check_events(evs)
    # the arm was consumed: the next call records nothing into these events
    t_before = evs[0].elapsed_time(evs[3])
    L.layer_forward(dev, k, cap)
    torch.cuda.synchronize()
    assert evs[0].elapsed_time(evs[3]) == t_before


def test_timed_dropless_and_expert_ffn():
    T, d, f, E, k = 700, 128, 264, 8, 2
    say(f"[timing] dropless and staged T={T}")
    inp = W.make_shape_inputs(T, d, f, E, "bf16", seed=11, router_bias_std=1.0)
    dev = L.upload(inp, DEV)
    a = L.layer_forward_dropless(dev, k)
    evs = new_events()
    B.moe_set_gemm_timing(evs)
    b = L.layer_forward_dropless(dev, k)
    torch.cuda.synchronize()
    assert torch.equal(bits(a["out"]), bits(b["out"]))
    check_events(evs)
    cap = O.capacity(T, k, E, 1.0)
    shape = L.shape_of(dev, k, cap)
    r = L.layer_forward(dev, k, cap)
    st = L.dispatch(shape, r["ids"], r["gates"])
    n = int(st["offsets"][-1].item())
    y0 = L.expert_ffn(shape, dev, st["row_token"], st["offsets"])
    evs = new_events()
    B.moe_set_gemm_timing(evs)
    y1 = L.expert_ffn(shape, dev, st["row_token"], st["offsets"])
    torch.cuda.synchronize()
    assert torch.equal(bits(y0[:n]), bits(y1[:n]))
    check_events(evs)


def test_one_gemm_timed():
    """Only the down-projection's pair armed: its events bracket a kernel, the others stay
    as they were."""
    T, d, f, E, k = 1000, 136, 264, 8, 2
    inp = W.make_shape_inputs(T, d, f, E, "bf16", seed=5, router_bias_std=1.0)
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, 1.0)
    a = L.layer_forward(dev, k, cap)
    evs = new_events()
    t01 = evs[0].elapsed_time(evs[1])
    B.moe_set_gemm_timing([None, None, evs[2], evs[3]])
    b = L.layer_forward(dev, k, cap)
    torch.cuda.synchronize()
    assert torch.equal(bits(a["out"]), bits(b["out"]))
    assert evs[2].elapsed_time(evs[3]) > 0.0
    assert evs[0].elapsed_time(evs[1]) == t01


def test_timed_layer_without_kept_rows():
    """Capacity 0: no expert GEMM is launched; the events are recorded back to back."""
    T, d, f, E, k = 64, 64, 128, 4, 1
    inp = W.make_shape_inputs(T, d, f, E, "bf16", seed=3)
    dev = L.upload(inp, DEV)
    evs = new_events()
    B.moe_set_gemm_timing(evs)
    res = L.layer_forward(dev, k, 0)
    torch.cuda.synchronize()
    assert torch.equal(bits(res["out"]), bits(dev["x"]))  # every token dropped: out is x
    check_events(evs, empty=True)


@pytest.mark.parametrize("T,d,f,E,k,C,dt", [
    (1000, 136, 264, 8, 2, 1.0, "bf16"),   # router for at most 8 experts (d slices)
    (3000, 64, 96, 40, 4, 1.0, "bf16"),    # 16 x 16 router tiles, mid-size dispatch
    (65, 12, 20, 8, 2, 0.75, "f32"),       # fp32 inputs
])
def test_stage_timed_layer_same_bits(T, d, f, E, k, C, dt):
    """Router and combine kernels timed together with both GEMMs: same bits as an untimed call,
    and the eight events in launch order (router, up-projection, down-projection, combine)."""
    say(f"[stage timing] layer T={T} d={d} f={f} E={E} k={k} {dt}")
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=T * 3 + E, router_bias_std=1.0)
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, C)
    a = L.layer_forward(dev, k, cap)
    gev, sev = new_events(), new_events()
    B.moe_set_gemm_timing(gev)
    B.moe_set_stage_timing(sev)
    b = L.layer_forward(dev, k, cap)
    torch.cuda.synchronize()
    assert torch.equal(bits(a["out"]), bits(b["out"]))
    assert torch.equal(a["ids"], b["ids"]) and torch.equal(a["slot_of"], b["slot_of"])
    route = sev[0].elapsed_time(sev[1])
    combine = sev[2].elapsed_time(sev[3])
    say(f"    route {route * 1e3:.1f} us, combine {combine * 1e3:.1f} us")
    assert route > 0.0 and combine > 0.0
    assert sev[1].elapsed_time(gev[0]) >= 0.0  # the router ends before the up-projection starts
    assert gev[3].elapsed_time(sev[2]) >= 0.0  # the down-projection ends before the combine
    # the arm was consumed
    t_before = sev[0].elapsed_time(sev[3])
    L.layer_forward(dev, k, cap)
    torch.cuda.synchronize()
    assert sev[0].elapsed_time(sev[3]) == t_before


def test_stage_timing_of_an_empty_batch():
    """T = 0 launches nothing: the router and combine events are recorded back to back."""
    inp = W.make_shape_inputs(4, 64, 64, 4, "bf16", seed=3)
    dev = L.upload(inp, DEV)
    dev["x"] = dev["x"][:0]
    sev = new_events()
    B.moe_set_stage_timing(sev)
    res = L.layer_forward(dev, 2, 0)
    torch.cuda.synchronize()
    assert res["out"].shape == (0, 64)
    assert sev[0].elapsed_time(sev[1]) >= 0.0 and sev[2].elapsed_time(sev[3]) >= 0.0
