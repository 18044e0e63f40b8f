"""Parity of the dropless pair-order flow (pair dispatch, pair-order expert GEMMs, moe_sum)
against the CPU oracle, on the GPU, through the C interface."""
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


class F64:
    """Per-expert float64 view of a stored weight array, converted on access."""

    def __init__(self, arr, dt):
        self.arr, self.dt = arr, dt

    def __getitem__(self, e):
        return W.to_float64(self.arr[e], self.dt)


def compare_pairs(gpu: dict, ref: dict, E: int):
    """Exact equality of the pair grouping (counts, offsets, sorted pairs, row tokens)."""
    assert np.array_equal(P.to_np(gpu["counts"]), ref["counts"][:E]), "expert counts"
    assert np.array_equal(P.to_np(gpu["offsets"]), ref["offsets"][:E + 1]), "expert offsets"
    assert np.array_equal(P.to_np(gpu["sorted_pairs"]), ref["sorted_pairs"]), "sorted pairs"
    assert np.array_equal(P.to_np(gpu["row_token"]), ref["row_token"]), "row tokens"


def _expert(inp, gated):
    dt = inp["dtype"]
    if gated:
        w13, w2 = F64(inp["w1"], dt), F64(inp["w2"], dt)
        return lambda e, rows: O.expert_ffn_gated(rows, w13[e], w2[e])
    w1, b1, w2, b2 = (F64(inp[n], dt) for n in ("w1", "b1", "w2", "b2"))
    return lambda e, rows: O.expert_ffn(rows, w1[e], b1[e], w2[e], b2[e])


# --------------------------------------------------------------------------- small shapes
DROPLESS_SMALL = [
    # T, d, f, E, k, gated   (skinny tiles up to 64 E pairs, large tiles above; ragged d_ff
    # and K tails; one block of pairs up to 2048, several above)
    (1, 64, 64, 1, 1, False),
    (7, 72, 136, 2, 2, False),
    (65, 264, 328, 8, 2, False),
    (1000, 136, 72, 8, 3, False),
    (1500, 64, 520, 64, 6, False),
    (517, 256, 264, 5, 1, False),
    (7, 72, 136, 2, 2, True),
    (65, 264, 328, 8, 2, True),
    (300, 128, 200, 16, 4, True),
    (1000, 136, 72, 8, 3, True),
    (700, 64, 96, 256, 8, False),  # 256 experts: multi-pass router, many small expert groups
    (4000, 64, 96, 128, 4, True),
]


@pytest.mark.parametrize("T,d,f,E,k,gated", DROPLESS_SMALL)
def test_dropless_small_shapes(T, d, f, E, k, gated):
    """The whole dropless layer against the oracle's flow: routing and pair grouping exact,
    every pair row and every output row within tolerance; the staged calls give the layer's
    bits."""
    say(f"[dropless small] T={T} d={d} f={f} E={E} k={k} gated={gated}")
    inp = W.make_shape_inputs(T, d, f, E, "bf16", seed=T * 17 + E, router_bias_std=2.0,
                              gated=gated)
    f64 = lambda a: W.to_float64(a, "bf16")
    dev = L.upload(inp, DEV)
    res = L.layer_forward_dropless(dev, k, gated=gated)
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    r = O.route(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"], k)
    P.compare_route(ids, gates, r, x=f64(inp["x"]), w=f64(inp["w_router"]), b=inp["b_router"])
    full = O.forward_dropless_with_routing(f64(inp["x"]), ids, gates, E, _expert(inp, gated))
    assert np.array_equal(P.to_np(res["counts"]), full["counts"])
    rows_err = P.max_abs_rel(P.to_np(res["pair_rows"]), full["pair_rows"])
    out_err = P.max_abs_rel(P.to_np(res["out"]), full["out"])
    say(f"    pair rows max-abs-rel {rows_err:.3e}, out {out_err:.3e}")
    assert rows_err <= P.TOL["bf16"] and out_err <= P.TOL["bf16"]

    shape = L.shape_of(dev, k, 0)
    disp = L.dispatch_pairs(shape, res["ids"])
    compare_pairs(disp, full, E)
    rows = L.expert_ffn_pairs(shape, dev, disp, res["gates"], gated=gated)
    assert torch.equal(rows.view(torch.int16), res["pair_rows"].view(torch.int16))
    out = L.moe_sum(shape, dev["x"], res["ids"], rows)
    assert torch.equal(out.view(torch.int16), res["out"].view(torch.int16))


# --------------------------------------------------------------------------- pair dispatch
@pytest.mark.parametrize("seed", range(6))
def test_dispatch_pairs_forced(seed):
    """moe_dispatch_pairs on caller-made routings: one block and many, one hot expert over
    many blocks, 256 experts, and ids outside [0, E) (placed after offsets[E], uncounted)."""
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    T = [5, 3000, 20000, 70000, 1, 1024][seed]
    E = [3, 8, 64, 4, 1, 256][seed]
    k = min(E, [2, 2, 6, 2, 1, 2][seed])
    say(f"[dispatch pairs] seed={seed} T={T} E={E} k={k}")
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if seed == 3:
        ids[:, 0] = 0
    bad = np.zeros((T, k), bool)
    if seed in (1, 5):
        bad = rng.random((T, k)) < 0.03
        ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    shape = B.make_shape(T, 8, 8, E, k, 0, B.MOE_BF16)
    res = L.dispatch_pairs(shape, torch.from_numpy(ids).to(DEV))
    # the oracle knows no invalid ids: an extra last expert E takes them, which leaves the
    # valid experts' groups unchanged and lists the invalid pairs, ascending, after them
    ref = O.dispatch_pairs(np.where(bad, E, ids).astype(np.int32), E + 1)
    compare_pairs(res, ref, E)


# --------------------------------------------------------------------------- moe_sum
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_moe_sum_variants(dt):
    """moe_sum with and without the residual and the ids, against the oracle's moe_sum over
    the present rows; a token with no present row is a bit copy of x (zeros without x)."""
    rng = np.random.Generator(np.random.PCG64(11))
    for T, d, k, E in ((1, 8, 1, 1), (37, 264, 3, 5), (500, 2048, 2, 8), (64, 72, 6, 64)):
        say(f"[moe_sum] dt={dt} T={T} d={d} k={k}")
        inp = W.make_shape_inputs(T * k, d, 8, 1, dt, seed=T + d)  # pair rows from x's draw
        rows_h = inp["x"]
        x_h = W.make_shape_inputs(T, d, 8, 1, dt, seed=T + d + 1)["x"]
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        absent = rng.random((T, k)) < 0.2
        absent[0, :] = True  # token 0: nothing to add
        ids[absent] = -1
        rows = L.to_device(rows_h, dt, DEV)
        x = L.to_device(x_h, dt, DEV)
        ids_d = torch.from_numpy(ids).to(DEV)
        shape = B.make_shape(T, d, 8, E, k, 0, B.MOE_BF16 if dt == "bf16" else B.MOE_F32)
        r64 = W.to_float64(rows_h, dt)
        x64 = W.to_float64(x_h, dt)
        present = r64 * (~absent).reshape(-1, 1)
        for with_x in (True, False):
            for with_ids in (True, False):
                out = L.moe_sum(shape, x if with_x else None, ids_d if with_ids else None, rows)
                want = O.moe_sum(present if with_ids else r64, k, x64 if with_x else None)
                assert P.max_abs_rel(P.to_np(out), want) <= P.TOL[dt]
                if with_ids:
                    ref0 = P.bits(x[0]) if with_x else np.zeros_like(P.bits(x[0]))
                    assert np.array_equal(P.bits(out[0]), ref0)


# --------------------------------------------------------------------------- full sizes
@pytest.mark.parametrize("key", ["mid", "decode", "fine", "gated"])
def test_dropless_config_end_to_end(key):
    """The workloads run dropless at full size: routing and pair grouping exact, then every
    pair row and every token's output against the oracle's flow (no capacity: every pair
    kept)."""
    inp = W.make_inputs(key)
    wl = inp["workload"]
    dt = inp["dtype"]
    gated = wl.expert == "gated"
    say(f"[dropless {key}] {wl.name}")
    dev = L.upload(inp, DEV)
    res = L.layer_forward_dropless(dev, wl.top_k, gated=gated)
    torch.cuda.synchronize()
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    x64, wr64 = W.to_float64(inp["x"], dt), W.to_float64(inp["w_router"], dt)
    r = O.route(x64, wr64, inp["b_router"], wl.top_k)
    info = P.compare_route(ids, gates, r, x=x64, w=wr64, b=inp["b_router"])
    ref = O.dispatch_pairs(ids, wl.n_experts)
    shape = L.shape_of(dev, wl.top_k, 0)
    compare_pairs(L.dispatch_pairs(shape, res["ids"]), ref, wl.n_experts)
    assert np.array_equal(P.to_np(res["counts"]), ref["counts"])
    say(f"    route certified {info['certified']}; pair grouping exact; largest expert "
        f"{int(ref['counts'].max())} of {wl.T * wl.top_k} pairs")
    full = O.forward_dropless_with_routing(x64, ids, gates, wl.n_experts, _expert(inp, gated))
    got_rows, got_out = P.to_np(res["pair_rows"]), P.to_np(res["out"])
    rows_err = P.max_abs_rel(got_rows, full["pair_rows"])
    out_err = P.max_abs_rel(got_out, full["out"])
    say(f"    pair rows max-abs-rel {rows_err:.3e} (element-wise "
        f"{P.elementwise_rel(got_rows, full['pair_rows']):.3e}), out {out_err:.3e} (element-wise "
        f"{P.elementwise_rel(got_out, full['out']):.3e}) over all {wl.T} tokens")
    assert rows_err <= P.TOL[dt] and out_err <= P.TOL[dt]
    del dev, res
    torch.cuda.empty_cache()


def test_dropless_matches_capacity_layer_without_drops():
    """The decode workload's capacity (64 = T) drops nothing, so the capacity layer and the
    dropless flow compute the same layer: same routing and counts, outputs within the bf16
    tolerance of each other (they round at different points: Y rows vs weighted pair rows)."""
    inp = W.make_inputs("decode")
    wl = inp["workload"]
    cap = O.capacity(wl.T, wl.top_k, wl.n_experts, wl.capacity_factor)
    dev = L.upload(inp, DEV)
    a = L.layer_forward(dev, wl.top_k, cap)
    b = L.layer_forward_dropless(dev, wl.top_k)
    assert int(a["drop_mask"].sum()) == 0
    assert torch.equal(a["ids"], b["ids"]) and torch.equal(a["counts"], b["counts"])
    assert P.max_abs_rel(P.to_np(b["out"]), P.to_np(a["out"])) <= P.TOL["bf16"]


def test_dropless_refusals():
    """fp32 is refused by the dropless layer (bf16 only); an empty batch is a no-op; a short
    workspace is refused."""
    inp = W.make_shape_inputs(8, 8, 8, 4, "f32", seed=1)
    dev = L.upload(inp, DEV)
    with pytest.raises(B.MoeError) as ei:
        L.layer_forward_dropless(dev, 2)
    assert ei.value.status == 2
    inp = W.make_shape_inputs(64, 64, 64, 4, "bf16", seed=3)
    dev = L.upload(inp, DEV)
    shape = L.shape_of(dev, 2, 0)
    ws = torch.empty(B.workspace_bytes_dropless(shape) - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.MoeError) as ei:
        L.layer_forward_dropless(dev, 2, ws=ws)
    assert ei.value.status == 3
    dev["x"] = dev["x"][:0]
    res = L.layer_forward_dropless(dev, 2)
    assert res["out"].shape == (0, 64)
