"""Parity of the HIP path (through the C interface) against the CPU oracle, on the GPU."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import parity as P
import pins
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


_CACHE: dict = {}


def case(key):
    if key not in _CACHE:
        say(f"[case] generating {key}")
        inp = W.make_inputs(key)
        wl = inp["workload"]
        dt = inp["dtype"]
        ref = O.route(W.to_float64(inp["x"], dt), W.to_float64(inp["w_router"], dt),
                      inp["b_router"], wl.top_k)
        cap = O.capacity(wl.T, wl.top_k, wl.n_experts, wl.capacity_factor)
        _CACHE.clear()  # keep one large case in memory at a time
        _CACHE[key] = (inp, ref, cap)
    return _CACHE[key]


def route_inputs(inp):
    """The router inputs in float64 (x, W_r, b_r), for the rounding bound of compare_route."""
    dt = inp["dtype"]
    return dict(x=W.to_float64(inp["x"], dt), w=W.to_float64(inp["w_router"], dt),
                b=inp["b_router"])


def check_all_outputs(inp, res, y_rows, ids, gates, dref, tag):
    """Every kept slot's expert output and every token's layer output against the oracle
    (max-abs-rel within the dtype's tolerance; the element-wise diagnostic reported), and the
    tokens with every choice dropped bit for bit equal to x."""
    dt = inp["dtype"]
    x64 = W.to_float64(inp["x"], dt)
    n = dref["n_kept"]
    Y = O.expert_ffn_slots(x64, dref["row_token"], dref["offsets"], F64(inp["w1"], dt),
                           F64(inp["b1"], dt), F64(inp["w2"], dt), F64(inp["b2"], dt))
    out_ref, all_dropped = O.combine(x64, gates, dref["slot_of"], Y)
    y_got = P.to_np(y_rows[:n])
    out_got = P.to_np(res["out"])
    y_err, y_el = P.max_abs_rel(y_got, Y), P.elementwise_rel(y_got, Y)
    o_err, o_el = P.max_abs_rel(out_got, out_ref), P.elementwise_rel(out_got, out_ref)
    say(f"    {tag}: Y max-abs-rel {y_err:.3e} (element-wise {y_el:.3e}) over {n} rows; "
        f"out max-abs-rel {o_err:.3e} (element-wise {o_el:.3e}) over {len(out_ref)} tokens")
    assert y_err <= P.TOL[dt], y_err
    assert o_err <= P.TOL[dt], o_err
    dropped = np.nonzero(all_dropped)[0]
    if len(dropped):
        idx = torch.as_tensor(dropped, device=res["out"].device)
        xb = L.to_device(inp["x"], dt, res["out"].device)
        assert np.array_equal(P.bits(res["out"][idx]), P.bits(xb[idx])), "dropped rows differ from x"
    return len(dropped)


# --------------------------------------------------------------------------- worked example
def test_worked_example_forced_dispatch():
    g = pins.golden()
    ids = torch.tensor(g["assignment"]["ids"], dtype=torch.int32, device=DEV)[:, None].contiguous()
    gates = torch.tensor(pins.FORCED_GATES, dtype=torch.float32, device=DEV)[:, None].contiguous()
    shape = B.make_shape(8, 4, 8, 4, 1, g["capacity"]["value"], B.MOE_F32)
    res = L.dispatch(shape, ids, gates)
    dref = O.dispatch(ids.cpu().numpy(), gates.cpu().numpy(), 4, g["capacity"]["value"])
    P.compare_dispatch(res, dref)
    drop = P.to_np(res["drop_mask"])[:, 0]
    assert list(np.nonzero(drop)[0]) == [g["dropped_token"]["value"]]
    off = P.to_np(res["offsets"]); rt = P.to_np(res["row_token"])
    kept = [sorted(rt[off[e]:off[e + 1]].tolist()) for e in range(4)]
    assert kept == [sorted(b) for b in g["kept_batches"]["value"]]


def _forced_routing_inputs():
    """d = E = 4; router = 4 * permutation so expert e reads feature pi(e); x rows are chosen
    so routing reproduces the worked example's assignment, token 0 is the page's x_0, and
    token 4 is the least confident of expert 0's three tokens."""
    g = pins.golden()
    pi = [2, 0, 1, 3]
    w_router = np.zeros((4, 4), np.float32)
    for e, j in enumerate(pi):
        w_router[e, j] = 4.0
    x = np.array([g["x0"]["value"],
                  [1.2, 0.1, 0.3, -0.2],
                  [0.1, 0.0, 1.0, -0.5],
                  [0.2, 1.5, -0.4, 0.1],
                  [0.3, 0.2, 0.45, -0.0],
                  [0.9, -0.2, 0.1, 0.4],
                  [0.1, 0.2, -0.3, 1.1],
                  [-0.5, 0.3, 0.2, 0.7]], np.float32)
    inp = W.make_inputs("worked_example")
    inp["x"], inp["w_router"], inp["b_router"] = x, w_router, None
    return inp


def test_worked_example_forced_end_to_end():
    g = pins.golden()
    inp = _forced_routing_inputs()
    f64 = lambda a: W.to_float64(a, "f32")
    ref = O.forward(f64(inp["x"]), f64(inp["w_router"]), None, f64(inp["w1"]), f64(inp["b1"]),
                    f64(inp["w2"]), f64(inp["b2"]), 1, 1.25)
    assert list(ref["ids"][:, 0]) == g["assignment"]["ids"]
    assert list(np.nonzero(ref["drop_mask"][:, 0])[0]) == [g["dropped_token"]["value"]]
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, 1, ref["cap"])
    assert list(P.to_np(res["ids"])[:, 0]) == g["assignment"]["ids"]
    P.compare_route(P.to_np(res["ids"]), P.to_np(res["gates"]), ref, x=f64(inp["x"]),
                    w=f64(inp["w_router"]))
    P.compare_dispatch(res, ref)
    err = P.max_abs_rel(P.to_np(res["out"]), ref["out"])
    assert err <= P.TOL["f32"], err
    t4 = g["dropped_token"]["value"]
    assert np.array_equal(P.bits(res["out"][t4]), P.bits(dev["x"][t4]))
    assert np.signbit(P.to_np(res["out"])[t4, 3])


def test_worked_example_config_end_to_end():
    inp, ref, cap = case("worked_example")
    wl = inp["workload"]
    f64 = lambda a: W.to_float64(a, "f32")
    full = O.forward(f64(inp["x"]), f64(inp["w_router"]), None, f64(inp["w1"]), f64(inp["b1"]),
                     f64(inp["w2"]), f64(inp["b2"]), wl.top_k, wl.capacity_factor)
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, wl.top_k, cap)
    P.compare_route(P.to_np(res["ids"]), P.to_np(res["gates"]), full, x=f64(inp["x"]),
                    w=f64(inp["w_router"]))
    P.compare_dispatch(res, full)
    assert P.max_abs_rel(P.to_np(res["out"]), full["out"]) <= P.TOL["f32"]
    dropped = np.nonzero(full["all_dropped"])[0]
    for t in dropped:
        assert np.array_equal(P.bits(res["out"][int(t)]), P.bits(dev["x"][int(t)]))


# --------------------------------------------------------------------------- full-size configs
@pytest.mark.parametrize("key", ["mid", "decode", "fine", "collapse"])
def test_config_end_to_end(key):
    """The workload at full size: routing and dispatch bit-exact against the oracle, then every
    kept slot's expert output and every token's output against the oracle's float64 layer;
    the staged calls return the layer's bits."""
    inp, ref, cap = case(key)
    wl = inp["workload"]
    say(f"[{key}] {wl.name} cap={cap}")
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, wl.top_k, cap)
    torch.cuda.synchronize()
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    info = P.compare_route(ids, gates, ref, **route_inputs(inp))
    say(f"    route: {info['certified']} tokens differ (each certified by the rounding bound), "
        f"max gate difference {info['max_gate_ulp']} fp32 ulp")
    dref = O.dispatch(ids, gates, wl.n_experts, cap)
    P.compare_dispatch(res, dref)
    say(f"    dispatch exact; kept {dref['n_kept']} of {wl.T * wl.top_k}")

    # staged calls: same kernels, bitwise-identical results; their Y rows go to the oracle
    shape = L.shape_of(dev, wl.top_k, cap)
    st = L.dispatch(shape, res["ids"], res["gates"])
    P.compare_dispatch(st, dref)
    y = L.expert_ffn(shape, dev, st["row_token"], st["offsets"])
    out2 = L.combine(shape, dev["x"], res["gates"], st["slot_of"], y)
    assert torch.equal(out2.view(torch.int16), res["out"].view(torch.int16))
    del out2, st
    n_dropped = check_all_outputs(inp, res, y, ids, gates, dref, key)
    say(f"    {n_dropped} tokens fully dropped, bitwise equal to x")
    del dev, res, y
    torch.cuda.empty_cache()


def test_determinism_mid():
    inp, ref, cap = case("mid")
    wl = inp["workload"]
    dev = L.upload(inp, DEV)
    ws = L.workspace(L.shape_of(dev, wl.top_k, cap), DEV)
    a = L.layer_forward(dev, wl.top_k, cap, ws=ws)
    ws.fill_(0xA5)  # stale workspace content must not matter
    b = L.layer_forward(dev, wl.top_k, cap, ws=ws)
    for name in a:
        assert np.array_equal(P.bits(a[name]) if a[name].is_floating_point() else P.to_np(a[name]),
                              P.bits(b[name]) if b[name].is_floating_point() else P.to_np(b[name])), name


# --------------------------------------------------------------------------- randomized shapes
SMALL = [
    # T, d, f, E, k, C, dtype
    (1, 64, 64, 1, 1, 1.0, "bf16"),
    (7, 72, 136, 2, 2, 1.0, "bf16"),
    (63, 128, 200, 3, 2, 0.5, "bf16"),
    (65, 264, 328, 8, 2, 1.25, "bf16"),
    (1000, 136, 72, 8, 3, 1.0, "bf16"),
    (1000, 64, 520, 64, 6, 1.5, "bf16"),
    (300, 128, 256, 16, 4, 0.25, "bf16"),
    (517, 256, 264, 5, 1, 8.0, "bf16"),
    # decode-sized batches (at most 64 E kept rows) with experts past 32 and 64 rows: the
    # up-projection's 32-row token tiles come several to an expert
    (60, 72, 136, 4, 2, 2.0, "bf16"),
    (200, 64, 264, 8, 2, 4.0, "bf16"),
    # more than 32 experts: the router takes several passes of 32 over x (bf16 inputs)
    (700, 64, 96, 256, 8, 1.0, "bf16"),
    (90, 32, 64, 160, 4, 2.0, "bf16"),
    (4000, 64, 96, 128, 4, 2.0, "bf16"),  # ... with the large-batch expert tiles
    # 8192 tokens or more: 4-wave router blocks; 40 experts leave the last pass half empty
    (8192, 32, 48, 40, 3, 1.0, "bf16"),
    # at most 8 experts with many tokens: 8-wave and 4-wave router blocks, ragged counts
    (4100, 64, 96, 6, 2, 1.0, "bf16"),
    (17000, 40, 24, 8, 3, 0.9, "bf16"),
    (1, 4, 8, 4, 1, 1.25, "f32"),
    (7, 5, 9, 3, 2, 1.0, "f32"),
    (65, 12, 20, 8, 2, 0.75, "f32"),
    (333, 24, 40, 64, 8, 1.0, "f32"),
    (200, 16, 16, 200, 3, 2.0, "f32"),
    (8200, 8, 12, 24, 2, 1.0, "f32"),
    # the layer's one-launch mid-size dispatch: just past the one-workgroup limit (3 runs, the
    # last of 2 keys), a single expert with half the assignments dropped, 256 experts
    (513, 8, 8, 4, 2, 1.0, "bf16"),
    (1030, 8, 16, 1, 1, 0.5, "f32"),
    (3000, 16, 24, 256, 4, 1.0, "bf16"),
]


@pytest.mark.parametrize("T,d,f,E,k,C,dt", SMALL)
def test_random_small_shapes(T, d, f, E, k, C, dt):
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=T * 31 + E, router_bias_std=1.0)
    f64 = lambda a: W.to_float64(a, dt)
    full = O.forward(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"], f64(inp["w1"]),
                     f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]), k, C)
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, k, full["cap"])
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    P.compare_route(ids, gates, full, x=f64(inp["x"]), w=f64(inp["w_router"]), b=inp["b_router"])
    dref = O.dispatch(ids, gates, E, full["cap"])
    P.compare_dispatch(res, dref)
    Y = O.expert_ffn_slots(f64(inp["x"]), dref["row_token"], dref["offsets"], f64(inp["w1"]),
                           f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]))
    out_ref, all_dropped = O.combine(f64(inp["x"]), gates, dref["slot_of"], Y)
    assert P.max_abs_rel(P.to_np(res["out"]), out_ref) <= P.TOL[dt]
    for t in np.nonzero(all_dropped)[0]:
        assert np.array_equal(P.bits(res["out"][int(t)]), P.bits(dev["x"][int(t)]))


@pytest.mark.parametrize("T", [500, 5000])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gate_ties(dt, T):
    """Integer-valued x and router weights: many tokens share exactly the same gates, so the
    fill order's token and choice tie-breaks decide the slots."""
    d, f, E, k = 16, 24, 6, 2
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=5, x_values=(-1.0, 0.0, 1.0))
    f64 = lambda a: W.to_float64(a, dt)
    full = O.forward(f64(inp["x"]), f64(inp["w_router"]), None, f64(inp["w1"]), f64(inp["b1"]),
                     f64(inp["w2"]), f64(inp["b2"]), k, 0.75)
    n_tied = len(full["gates"].ravel()) - len(np.unique(full["gates"].ravel()))
    assert n_tied > 100
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, k, full["cap"])
    P.compare_route(P.to_np(res["ids"]), P.to_np(res["gates"]), full, x=f64(inp["x"]),
                    w=f64(inp["w_router"]))
    P.compare_dispatch(res, full)
    assert P.max_abs_rel(P.to_np(res["out"]), full["out"]) <= P.TOL[dt]


@pytest.mark.parametrize("seed", range(18))
def test_dispatch_forced_patterns(seed):
    """moe_dispatch on caller-made routings: ties, -0.0, big experts spanning several sort
    chunks, capacities from 0 to above T, and out-of-range ids (dropped, not counted).
    Seeds 0, 4, 6, 7 and 8 (at most 1024 assignments) take the one-workgroup path; seeds 1 and
    9 to 15 (1025 to 16384) the two-launch run-sort and merge path; seeds 2, 3, 5, 16 and 17
    the bucketed multi-kernel path.  Seeds 8 and 9, and 15 and 16, sit on either side of a
    switch.  Seed 10 puts all 8192 assignments into one expert, seeds 11 and 12 spread 8192
    over 256 and 64 experts with 5 % invalid ids, seed 13 has 8193 assignments over 3
    experts, seed 14 keeps every assignment (capacity above the count), seed 15 puts 16384
    into one hot expert, seed 16 has 16385 over 256 experts with invalid ids, seed 17 has
    16386 over 16 experts.  Even seeds draw their gates from six values (ties and -0.0), odd
    seeds uniformly."""
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    T = [5, 3000, 20000, 70000, 1, 9000, 400, 300, 512, 1025, 8192, 8192, 2048, 2731, 1500,
         16384, 16385, 5462][seed]
    E = [3, 8, 64, 4, 1, 256, 256, 5, 16, 7, 8, 256, 64, 3, 2, 8, 256, 16][seed]
    k = min(E, [2, 2, 6, 2, 1, 3, 2, 3, 2, 1, 1, 1, 4, 3, 2, 1, 1, 3][seed])
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32) if T < 5000 else \
        np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if seed in (3, 10, 15):
        ids[:, 0] = 0  # one hot expert with T assignments
    vals = np.array([0.5, 0.25, -0.0, 0.0, 0.125, 0.75], np.float32)
    gates = vals[rng.integers(len(vals), size=(T, k))] if seed % 2 == 0 else \
        rng.random((T, k)).astype(np.float32)
    bad = np.zeros((T, k), bool)
    if seed in (1, 5, 6, 9, 11, 12, 16):
        bad = rng.random((T, k)) < (0.01 if seed in (1, 5) else 0.05)
        ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    cap = [0, 400, 1536, 16384, 1, 120, 3, 100, 40, 100, 5000, 3, 0, 2000, 3000, 9000, 40,
           1000][seed]
    shape = B.make_shape(T, 8, 8, E, k, cap, B.MOE_BF16)
    res = L.dispatch(shape, torch.from_numpy(ids).to(DEV), torch.from_numpy(gates).to(DEV))
    # the oracle knows no invalid ids: give them an extra last expert E, which leaves the
    # valid experts' counts and slots unchanged; their own slots are then ignored
    dref = O.dispatch(np.where(bad, E, ids).astype(np.int32), gates, E + 1, cap)
    counts = dref["counts"][:E]
    assert np.array_equal(P.to_np(res["counts"]), counts)
    kept = np.minimum(counts, cap)
    assert np.array_equal(P.to_np(res["offsets"]), np.concatenate([[0], np.cumsum(kept)]))
    so = dref["slot_of"].copy()
    so[bad] = -1
    assert np.array_equal(P.to_np(res["slot_of"]), so)
    assert np.array_equal(P.to_np(res["drop_mask"]), (so < 0).astype(np.uint8))
    n = int(kept.sum())
    assert np.array_equal(P.to_np(res["row_token"])[:n], dref["row_token"][:n])


def test_capacity_zero_returns_input():
    inp = W.make_shape_inputs(100, 64, 64, 8, "bf16", seed=3)
    inp["x"][5, 3] = 0x8000  # -0.0
    dev = L.upload(inp, DEV)
    res = L.layer_forward(dev, 2, 0)
    assert torch.equal(res["out"].view(torch.int16), dev["x"].view(torch.int16))
    assert int(res["drop_mask"].sum()) == 200


def test_empty_batch_is_a_no_op():
    inp = W.make_shape_inputs(4, 64, 64, 4, "bf16", seed=3)
    dev = L.upload(inp, DEV)
    dev["x"] = dev["x"][:0]
    res = L.layer_forward(dev, 2, 0)
    assert res["out"].shape == (0, 64)


def test_short_workspace_is_refused():
    inp = W.make_shape_inputs(64, 64, 64, 4, "bf16", seed=3)
    dev = L.upload(inp, DEV)
    shape = L.shape_of(dev, 2, 32)
    ws = torch.empty(B.workspace_bytes(shape) - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.MoeError) as ei:
        L.layer_forward(dev, 2, 32, ws=ws)
    assert ei.value.status == 3


# --------------------------------------------------------------------------- padded fixed buffers
PADDED_SMALL = [
    # T, d, f, E, k, C, dtype   (E * cap buffer rows; skinny and large GEMM tiles both covered)
    (7, 72, 136, 2, 2, 1.0, "bf16"),
    (65, 264, 328, 8, 2, 1.25, "bf16"),
    (1000, 136, 72, 8, 3, 1.0, "bf16"),
    (300, 128, 256, 16, 4, 0.25, "bf16"),
    (700, 64, 96, 256, 8, 1.0, "bf16"),
    (65, 12, 20, 8, 2, 0.75, "f32"),
    (200, 16, 16, 200, 3, 2.0, "f32"),
]


@pytest.mark.parametrize("T,d,f,E,k,C,dt", PADDED_SMALL)
def test_padded_small_shapes(T, d, f, E, k, C, dt):
    """moe_layer_forward_padded against the oracle's fixed buffers: every buffer row, the
    empty ones included (FFN of a zero row), the buffer slots exactly, and the layer output."""
    inp = W.make_shape_inputs(T, d, f, E, dt, seed=T * 17 + E, router_bias_std=1.0)
    f64 = lambda a: W.to_float64(a, dt)
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, C)
    res = L.layer_forward_padded(dev, k, cap)
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    full = O.forward(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"], f64(inp["w1"]),
                     f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]), k, C)
    P.compare_route(ids, gates, full, x=f64(inp["x"]), w=f64(inp["w_router"]), b=inp["b_router"])
    pref = O.dispatch_padded(ids, gates, E, cap)
    assert np.array_equal(P.to_np(res["slot_of"]), pref["slot_of"])
    Y = O.expert_ffn_padded(f64(inp["x"]), pref["row_token"], E, cap, f64(inp["w1"]),
                            f64(inp["b1"]), f64(inp["w2"]), f64(inp["b2"]))
    if E * cap:
        assert P.max_abs_rel(P.to_np(res["y_rows"]), Y) <= P.TOL[dt]
        empty = pref["row_token"] < 0
        if empty.any():
            assert P.max_abs_rel(P.to_np(res["y_rows"])[empty], Y[empty]) <= P.TOL[dt]
    out_ref, all_dropped = O.combine(f64(inp["x"]), gates, pref["slot_of"], Y)
    assert P.max_abs_rel(P.to_np(res["out"]), out_ref) <= P.TOL[dt]
    for t in np.nonzero(all_dropped)[0]:
        assert np.array_equal(P.bits(res["out"][int(t)]), P.bits(dev["x"][int(t)]))


@pytest.mark.parametrize("key", ["mid", "decode"])
def test_padded_matches_compact(key):
    """At full size the padded layout computes E * cap rows but returns the compact layout's
    output bit for bit (each kept row accumulates the same products in the same K order);
    its slots are e * cap + rank, and sampled empty rows match the oracle's FFN of a zero row."""
    inp, ref, cap = case(key)
    wl = inp["workload"]
    dev = L.upload(inp, DEV)
    a = L.layer_forward(dev, wl.top_k, cap)
    p = L.layer_forward_padded(dev, wl.top_k, cap)
    torch.cuda.synchronize()
    assert torch.equal(a["out"].view(torch.int16), p["out"].view(torch.int16))
    ids = P.to_np(a["ids"])
    so_a, so_p = P.to_np(a["slot_of"]), P.to_np(p["slot_of"])
    offs = np.concatenate([[0], np.cumsum(np.minimum(P.to_np(a["counts"]), cap))])
    kept = so_a >= 0
    assert np.array_equal(so_p >= 0, kept)
    assert np.array_equal(so_p[kept], ids[kept] * cap + so_a[kept] - offs[ids[kept]])
    pref = O.dispatch_padded(ids, P.to_np(a["gates"]), wl.n_experts, cap)
    empty = np.nonzero(pref["row_token"] < 0)[0]
    say(f"[{key}] padded: {wl.n_experts * cap} buffer rows, {len(empty)} empty")
    if len(empty):
        rows = np.random.default_rng(5).choice(empty, size=min(64, len(empty)), replace=False)
        dt = inp["dtype"]
        Y = O.expert_ffn_padded(W.to_float64(inp["x"], dt), pref["row_token"], wl.n_experts, cap,
                                F64(inp["w1"], dt), F64(inp["b1"], dt), F64(inp["w2"], dt),
                                F64(inp["b2"], dt), rows=rows)
        got = P.to_np(p["y_rows"][torch.as_tensor(rows, device=DEV)])
        assert P.max_abs_rel(got, Y) <= P.TOL[dt]
    del dev, a, p
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- gated expert
GATED_SMALL = [
    # T, d, f, E, k, C   (bf16; skinny and large GEMM tiles, ragged d_ff and K tails)
    (7, 72, 136, 2, 2, 1.0),
    (65, 264, 328, 8, 2, 1.25),
    (1000, 136, 72, 8, 3, 1.0),
    (517, 256, 264, 5, 1, 8.0),
    (300, 128, 200, 16, 4, 0.25),
    (4000, 64, 96, 128, 4, 2.0),
]


@pytest.mark.parametrize("T,d,f,E,k,C", GATED_SMALL)
def test_gated_small_shapes(T, d, f, E, k, C):
    """moe_layer_forward_gated against the oracle's gated layer: routing, slots, every output
    row, and bit copies for tokens with every choice dropped."""
    inp = W.make_shape_inputs(T, d, f, E, "bf16", seed=T * 13 + E, router_bias_std=1.0, gated=True)
    f64 = lambda a: W.to_float64(a, "bf16")
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, C)
    res = L.layer_forward_gated(dev, k, cap)
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    full = O.forward_gated(f64(inp["x"]), f64(inp["w_router"]), inp["b_router"], f64(inp["w1"]),
                           f64(inp["w2"]), k, C)
    P.compare_route(ids, gates, full, x=f64(inp["x"]), w=f64(inp["w_router"]), b=inp["b_router"])
    dref = O.dispatch(ids, gates, E, cap)
    P.compare_dispatch(res, dref)
    Y = O.expert_ffn_slots_gated(f64(inp["x"]), dref["row_token"], dref["offsets"], f64(inp["w1"]),
                                 f64(inp["w2"]))
    out_ref, all_dropped = O.combine(f64(inp["x"]), gates, dref["slot_of"], Y)
    assert P.max_abs_rel(P.to_np(res["out"]), out_ref) <= P.TOL["bf16"]
    for t in np.nonzero(all_dropped)[0]:
        assert np.array_equal(P.bits(res["out"][int(t)]), P.bits(dev["x"][int(t)]))


def test_gated_config_end_to_end():
    """The gated workload at full size: routing and dispatch exact, every token's output
    against the oracle's gated layer."""
    inp = W.make_inputs("gated")
    wl = inp["workload"]
    cap = O.capacity(wl.T, wl.top_k, wl.n_experts, wl.capacity_factor)
    dt = inp["dtype"]
    ri = route_inputs(inp)
    ref = O.route(ri["x"], ri["w"], inp["b_router"], wl.top_k)
    dev = L.upload(inp, DEV)
    res = L.layer_forward_gated(dev, wl.top_k, cap)
    ids, gates = P.to_np(res["ids"]), P.to_np(res["gates"])
    info = P.compare_route(ids, gates, ref, **ri)
    dref = O.dispatch(ids, gates, wl.n_experts, cap)
    P.compare_dispatch(res, dref)
    Y = O.expert_ffn_slots_gated(ri["x"], dref["row_token"], dref["offsets"], F64(inp["w1"], dt),
                                 F64(inp["w2"], dt))
    want, all_dropped = O.combine(ri["x"], gates, dref["slot_of"], Y)
    got = P.to_np(res["out"])
    err, el = P.max_abs_rel(got, want), P.elementwise_rel(got, want)
    say(f"[gated] route certified {info['certified']}; out max-abs-rel {err:.3e} "
        f"(element-wise {el:.3e}) over {wl.T} tokens")
    assert err <= P.TOL[dt]
    for t in np.nonzero(all_dropped)[0]:
        assert np.array_equal(P.bits(res["out"][int(t)]), P.bits(dev["x"][int(t)]))
    del dev, res
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- graph capture
@pytest.mark.parametrize("key", ["mid", "decode"])
def test_layer_forward_in_a_captured_graph(key):
    """The layer enqueues no host synchronisation, allocation or memset, so a HIP graph can
    capture it: every replay (with eager work and synchronisations between replays) returns
    the eager call's bits."""
    inp, ref, cap = case(key)
    wl = inp["workload"]
    dev = L.upload(inp, DEV)
    shape = L.shape_of(dev, wl.top_k, cap)
    ws = L.workspace(shape, DEV)
    out = torch.empty_like(dev["x"])
    ids = torch.empty((wl.T, wl.top_k), dtype=torch.int32, device=DEV)
    eager = L.layer_forward(dev, wl.top_k, cap)
    s = torch.cuda.Stream()
    args = (shape, dev["x"], dev["w_router"], dev["b_router"], dev["w1"], dev["b1"], dev["w2"],
            dev["b2"], out)
    with torch.cuda.stream(s):
        B.moe_layer_forward(*args, topk_ids=ids, ws=ws, stream=s)  # warm on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.moe_layer_forward(*args, topk_ids=ids, ws=ws, stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        ids.fill_(-7)
        ws.fill_(0xA5)  # stale workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager["out"].view(torch.int16)), f"replay {r}"
        assert torch.equal(ids, eager["ids"]), f"replay {r} ids"
        L.layer_forward(dev, wl.top_k, cap)  # eager work between replays
        torch.cuda.synchronize()
    del g, dev, ws, out
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- staged router
ROUTE_SHAPES = [
    # T, d, E, k, dtype  (one expert tile; two tiles per pass; 4-wave blocks from 8192 tokens
    # with several passes and a half-empty last tile)
    (100, 136, 8, 2, "bf16"),
    (300, 64, 40, 6, "bf16"),
    (8192, 64, 40, 3, "bf16"),
    (8200, 24, 70, 4, "f32"),
    (65, 12, 5, 2, "f32"),
    # at most 8 experts (8-token x 8-expert matrix-core tiles): 4- and 8-wave blocks, ragged
    # token counts, fewer column quads than waves (d 72, d 8), fewer than 8 experts (padding
    # columns), a single expert, every expert chosen
    (4097, 72, 8, 2, "bf16"),
    (5000, 8, 3, 1, "bf16"),
    (16385, 136, 7, 3, "bf16"),
    (16384, 512, 1, 1, "bf16"),
    (20000, 264, 8, 8, "bf16"),
    (16400, 24, 6, 2, "f32"),
    # at most 8 experts below 16384 tokens (MFMA blocks on four slices of d): several 128-column
    # quads per wave with a partial last quad (d 2056: 17 quads over 4 waves), a d with a
    # partial last chunk in fp32, fewer experts than a group, a single token
    (1001, 2056, 8, 2, "bf16"),
    (3000, 1000, 5, 3, "bf16"),
    (777, 130, 8, 4, "f32"),
    (1, 512, 8, 2, "bf16"),
]


@pytest.mark.parametrize("T,d,E,k,dt", ROUTE_SHAPES)
def test_route_staged_with_logits(T, d, E, k, dt):
    """moe_route on its own, with the optional fp32 logits: ids and gates bit-exact (certified
    rounding differences only), every logit the fp32 rounding of the oracle's float64 logit
    (bias included), except where that float64 value lies within the summation-order bound of
    an fp32 rounding midpoint."""
    say(f"[route] T={T} d={d} E={E} k={k} {dt}")
    inp = W.make_shape_inputs(T, d, 8, E, dt, seed=T + E, router_bias_std=1.0)
    f64 = lambda a: W.to_float64(a, dt)
    x64, w64 = f64(inp["x"]), f64(inp["w_router"])
    ref = O.route(x64, w64, inp["b_router"], k)
    dev = L.upload(inp, DEV)
    res = L.route(dev, k, 0, want_logits=True)
    info = P.compare_route(P.to_np(res["ids"]), P.to_np(res["gates"]), ref, x=x64, w=w64,
                           b=inp["b_router"])
    got = P.to_np(res["logits"])
    want = ref["logits"]
    diff = got != want.astype(np.float32)
    if diff.any():
        # each differing logit: adjacent fp32 values, the oracle's value within the bound of
        # their midpoint (both sides sum the same exact products in different orders)
        n = d + 1
        gamma = n * P.U64 / (1 - n * P.U64)
        A = np.abs(x64) @ np.abs(w64).T + np.abs(inp["b_router"])[None, :]
        g, r = got[diff].astype(np.float32), want.astype(np.float32)[diff]
        assert np.all(np.abs(g.view(np.int32).astype(np.int64) - r.view(np.int32).astype(np.int64)) == 1)
        mid = (g.astype(np.float64) + r.astype(np.float64)) / 2
        assert np.all(np.abs(want[diff] - mid) <= 2 * gamma * A[diff])
    say(f"    {int(diff.sum())} logits differ (certified), {info['certified']} tokens' routing")


@pytest.mark.parametrize("T,d,E,k,C,dt", [(700, 136, 8, 2, 1.0, "bf16"),
                                          (3000, 264, 64, 6, 0.5, "bf16"),
                                          (65, 13, 4, 2, 1.0, "f32"),
                                          (1500, 20, 16, 3, 2.0, "f32")])
def test_dispatch_gathers_routed_rows(T, d, E, k, C, dt):
    """moe_dispatch with x: x_routed row s is x[row_token[s]] bit for bit for every kept slot
    (16-byte rows and 4-byte-word rows); the dispatch outputs are those of the call without x."""
    say(f"[x_routed] T={T} d={d} E={E} k={k} C={C} {dt}")
    inp = W.make_shape_inputs(T, d, 8, E, dt, seed=2 * T + E, router_bias_std=1.0)
    dev = L.upload(inp, DEV)
    cap = O.capacity(T, k, E, C)
    r = L.route(dev, k, cap)
    shape = L.shape_of(dev, k, cap)
    a = L.dispatch(shape, r["ids"], r["gates"])
    b = L.dispatch(shape, r["ids"], r["gates"], x=dev["x"])
    for name in ("counts", "offsets", "slot_of", "row_token", "drop_mask"):
        n = int(a["offsets"][-1]) if name == "row_token" else None
        assert torch.equal(a[name][:n], b[name][:n]), name
    n = int(b["offsets"][-1].item())
    want = dev["x"][b["row_token"][:n].long()]
    assert np.array_equal(P.bits(b["x_routed"][:n]), P.bits(want))
    dref = O.dispatch(P.to_np(r["ids"]), P.to_np(r["gates"]), E, cap)
    assert np.array_equal(P.to_np(b["row_token"])[:n], dref["row_token"])


# --------------------------------------------------------------------------- one GPU's share
def test_ep8_hot_shard_expert_ffn():
    """The collapse layer's hot expert as one GPU's share under expert parallelism (16384
    received rows through one expert, d_model 4096, d_ff 14336), in the launch configuration
    bench.py times (packed weights, rows in receive order): every row against the oracle."""
    wl = W.WORKLOADS["ep8_hot_shard"]
    say(f"[shard] {wl.name}")
    inp = W.make_inputs(wl)
    dt = inp["dtype"]
    dev = L.pack_weights(L.upload(inp, DEV))
    rows = wl.T
    shape = L.shape_of(dev, wl.top_k, rows)
    row_token = torch.arange(rows, dtype=torch.int32, device=DEV)
    offsets = torch.tensor([0, rows], dtype=torch.int32, device=DEV)
    y = L.expert_ffn(shape, dev, row_token, offsets)
    torch.cuda.synchronize()
    got = P.to_np(y[:rows])
    del y, dev
    torch.cuda.empty_cache()
    ref = O.expert_ffn_slots(W.to_float64(inp["x"], dt), np.arange(rows), np.array([0, rows]),
                             F64(inp["w1"], dt), F64(inp["b1"], dt), F64(inp["w2"], dt),
                             F64(inp["b2"], dt))
    err, el = P.max_abs_rel(got, ref), P.elementwise_rel(got, ref)
    say(f"    Y max-abs-rel {err:.3e} (element-wise {el:.3e}) over {rows} rows")
    assert err <= P.TOL[dt], err
