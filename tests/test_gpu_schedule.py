"""Parity of the batch consolidation path (Token Scheduler, pooled per-batch layer) against the
CPU oracle, on the GPU, through the C interface."""
from __future__ import annotations

import json
import os
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
GOLDEN_SCHED = os.path.join(os.path.dirname(__file__), "golden", "batch_consolidation.json")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    B.lib()  # loud failure if the library is missing
    yield
    torch.cuda.synchronize()


def test_schedule_diagram_pool():
    """The diagram's pool (8 tokens, top-1 over 4 experts, two batches of 4 with every expert
    once per batch): the GPU's order equals the oracle's and each new batch activates 2
    experts, each original batch 4."""
    with open(GOLDEN_SCHED) as fh:
        g = json.load(fh)["facts"]
    ids = np.array(g["batch1_experts"]["value"] + [2, 0, 3, 1], dtype=np.int32)[:, None]
    ref = O.schedule_batches(ids, 4)
    res = L.schedule_batches(torch.from_numpy(ids).to(DEV), 4, 4)
    assert np.array_equal(P.to_np(res["order"]), ref["order"])
    assert list(P.to_np(res["batch_experts"])) == [g["optimized_active_per_batch"]["value"]] * 2
    assert list(P.to_np(res["orig_batch_experts"])) == [g["original_active_per_batch"]["value"]] * 2


@pytest.mark.parametrize("seed", range(6))
def test_schedule_forced(seed):
    """Pools from 1 to 8192 tokens, 1 to 256 experts, top-1 to top-5, many equal expert sets
    (token index decides), and ids outside [0, E) (sorted as E, not counted)."""
    rng = np.random.Generator(np.random.PCG64(500 + seed))
    T, Bsz, E, k = [(1, 1, 1, 1), (512, 64, 8, 2), (8192, 128, 64, 6), (4096, 256, 256, 5),
                    (3000, 100, 4, 3), (960, 32, 16, 1)][seed]
    say(f"[schedule] seed={seed} T={T} B={Bsz} E={E} k={k}")
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    bad = np.zeros((T, k), bool)
    if seed == 4:
        bad = rng.random((T, k)) < 0.05
        ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    res = L.schedule_batches(torch.from_numpy(ids).to(DEV), Bsz, E)
    ref = O.schedule_batches(np.where(bad, E, ids), Bsz)  # an invalid id sorts as E
    assert np.array_equal(P.to_np(res["order"]), ref["order"])
    # active experts: distinct valid ids per batch
    valid = np.where(bad, -1, ids)
    want = [len({int(e) for e in valid[b].ravel() if e >= 0}) for b in ref["batches"]]
    want0 = [len({int(e) for e in valid[b].ravel() if e >= 0}) for b in ref["orig_batches"]]
    assert list(P.to_np(res["batch_experts"])) == want
    assert list(P.to_np(res["orig_batch_experts"])) == want0


POOLS = [
    # T_pool, batch, d, f, E, k, C, dtype
    (8, 4, 4, 8, 4, 1, 1.0, "f32"),
    (60, 12, 12, 20, 4, 2, 2.0, "f32"),
    (60, 12, 12, 20, 4, 2, 0.5, "f32"),
    (256, 64, 72, 136, 8, 2, 4.0, "bf16"),
    (256, 64, 72, 136, 8, 2, 1.0, "bf16"),
    (900, 100, 64, 200, 16, 3, 1.25, "bf16"),
]


@pytest.mark.parametrize("T,Bsz,d,f,E,k,C,dt", POOLS)
def test_batches_small(T, Bsz, d, f, E, k, C, dt):
    """The pooled layer, original grouping and consolidated, against the oracle's per-batch
    layer: routing exact, order and active experts exact, every output row within
    tolerance (capacities below and at the batch size)."""
    say(f"[batches] T={T} B={Bsz} E={E} k={k} C={C} {dt}")
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=T + 7 * E, router_bias_std=1.0)
    f64 = lambda a: W.to_float64(a, dt)
    dev = L.upload(inp, DEV)
    cap = O.capacity(Bsz, k, E, C)
    for cons in (False, True):
        res = L.layer_forward_batches(dev, k, cap, Bsz, cons)
        ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
        ref = O.forward_batches(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"],
                                f64(inp["w1"]), f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]),
                                k, C, Bsz, cons)
        P.compare_route(ids, gates, ref, x=f64(inp["x"]), w=f64(inp["w_router"]),
                        b=inp["b_router"])
        sched = O.schedule_batches(ids, Bsz)
        batches = sched["batches"] if cons else sched["orig_batches"]
        if cons:
            assert np.array_equal(P.to_np(res["order"]), sched["order"])
        assert np.array_equal(P.to_np(res["batch_experts"]),
                              sched["active"] if cons else sched["orig_active"])
        # the oracle's per-batch layer on the GPU's routing
        out = np.zeros((T, d))
        for b in batches:
            out[b] = O.forward_with_routing(f64(inp["x"])[b], ids[b], gates[b], cap, E,
                                            f64(inp["w1"]), f64(inp["b1"]), f64(inp["w2"]),
                                            f64(inp["b2"]))["out"]
        err = P.max_abs_rel(P.to_np(res["out"]), out)
        say(f"    consolidate={cons}: out max-abs-rel {err:.3e}, active {list(P.to_np(res['batch_experts']))}")
        assert err <= P.TOL[dt]


def test_decode_pool_consolidation():
    """Eight decode batches (capacity 64 = batch size: nothing drops): the consolidated run
    activates fewer experts per batch and returns the original grouping's output bit for bit
    (each token's rows see the same products in the same order); every token against the
    oracle."""
    inp = W.make_inputs("decode_pool")
    wl = inp["workload"]
    dt = inp["dtype"]
    cap = O.capacity(wl.batch_size, wl.top_k, wl.n_experts, wl.capacity_factor)
    assert cap == wl.batch_size
    dev = L.upload(inp, DEV)
    a = L.layer_forward_batches(dev, wl.top_k, cap, wl.batch_size, False)
    b = L.layer_forward_batches(dev, wl.top_k, cap, wl.batch_size, True)
    torch.cuda.synchronize()
    ea, eb = P.to_np(a["batch_experts"]), P.to_np(b["batch_experts"])
    say(f"[decode_pool] active experts per batch: original {list(ea)}, consolidated {list(eb)}")
    assert eb.sum() < ea.sum()
    assert torch.equal(a["ids"], b["ids"])
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    ids, gates = P.to_np(b["ids"]), P.to_np(b["gates"])
    x64, wr64 = W.to_float64(inp["x"], dt), W.to_float64(inp["w_router"], dt)
    r = O.route(x64, wr64, None, wl.top_k)
    P.compare_route(ids, gates, r, x=x64, w=wr64)
    assert np.array_equal(P.to_np(b["order"]), O.schedule_batches(ids, wl.batch_size)["order"])
    # every token of the pool against the oracle (nothing drops: capacity = batch size)
    w1, b1, w2, b2 = (inp[n] for n in ("w1", "b1", "w2", "b2"))
    want = x64.copy()
    for e in range(wl.n_experts):
        sel = np.nonzero(ids == e)
        if len(sel[0]) == 0:
            continue
        y = O.expert_ffn(x64[sel[0]], W.to_float64(w1[e], dt), W.to_float64(b1[e], dt),
                         W.to_float64(w2[e], dt), W.to_float64(b2[e], dt))
        np.add.at(want, sel[0], gates[sel][:, None].astype(np.float64) * y)
    got = P.to_np(b["out"])
    err = P.max_abs_rel(got, want)
    say(f"    out max-abs-rel {err:.3e} (element-wise {P.elementwise_rel(got, want):.3e}) over "
        f"all {wl.T} tokens")
    assert err <= P.TOL[dt]
    del dev, a, b
    torch.cuda.empty_cache()


def test_schedule_limits():
    """More than 8192 pool tokens cannot be consolidated (one workgroup sorts the pool); the
    original grouping has no such limit; an empty pool is a no-op."""
    inp = W.make_shape_inputs(8200, 8, 8, 4, "f32", seed=2)
    dev = L.upload(inp, DEV)
    with pytest.raises(B.MoeError) as ei:
        L.layer_forward_batches(dev, 2, 41, 41, True)  # 200 batches of 41 tokens
    assert ei.value.status == 2
    res = L.layer_forward_batches(dev, 2, 41, 41, False)
    assert res["out"].shape == (8200, 8)
    dev["x"] = dev["x"][:0]
    res = L.layer_forward_batches(dev, 2, 4, 4, True)
    assert res["out"].shape == (0, 8)
