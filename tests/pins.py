"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check takes the oracle module as its argument, so the same checks run against the
real oracle (tests/test_oracle_pins.py) and against copies with planted mistakes
(tests/test_oracle_mutations.py), which must each fail at least one check.

What pins what:
  * the worked example's printed numbers (tests/golden/worked_example.json, cited to
    "Expert Networks > Worked Example: Expert Specialization"): capacity 2, expert 0's
    overflow drops token 4, the kept batches, dropped output equal to the input;
  * closed forms: softmax of (0, ln2, ln3, ln4) is (0.1, 0.2, 0.3, 0.4); one expert gives
    gate 1; equal logits give 1/E; SiLU(ln 3) = 0.75 ln 3; exact-rational capacities;
  * library routines: torch float64 linear/SiLU for the expert FFN and the dense
    special case, scipy's softmax;
  * brute force: integer-valued router logits summed exactly in Python integers; top-k by
    enumerating all k-subsets; slot ranks by an independent counting definition;
  * the rounding of the gates to fp32 before top-k: two probabilities 0.5 -/+ 2.5e-10 both
    round to 0.5, so the tie goes to the lower expert although the float64 values differ;
  * invariants: counts sum to T*k, slot map is a bijection, kept gates dominate dropped
    gates, permutation equivariance, capacity 0 returns the input;
  * the gated expert: SiLU(ln 3) = (3/4) ln 3 through a gate and an up row, a zero gate
    gives zero, torch float64 linear/SiLU for the expert and the layer;
  * the padded fixed buffers: the worked example's batches in their buffers with one empty
    slot, an empty slot's output b2 exactly when b1 = 0 (SiLU(0) = 0), the same layer output
    as the compact layout;
  * the dropless pair-order flow: a hand-sorted pair list, counting-sort invariants
    (permutation, experts non-decreasing, pairs ascending inside an expert), moe_sum against
    numpy's reshape-and-sum, each pair row and token output against torch float64 linear/SiLU
    per token, and the capacity layer's output when the capacity holds every pair;
  * the batch scheduler: the Token Routing Optimization diagram's counts
    (tests/golden/batch_consolidation.json: 4 experts per batch with 1 token each become 2
    with 2 each) for every legible reading of its second batch, brute-force set counting, the
    top-1 bound E_used + M - 1, and the layer's output unchanged by the grouping when nothing
    can drop (per-token torch recomputation), per-batch capacity when it can.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
GOLDEN_SCHED = os.path.join(os.path.dirname(__file__), "golden", "batch_consolidation.json")


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)["facts"]


# Gates for the worked example's forced assignment.  The page fixes the assignment, the
# value 0.87 for token 0 and that token 4 has the lowest confidence on expert 0; the other
# values are a choice consistent with those facts.
FORCED_GATES = [0.87, 0.62, 0.71, 0.55, 0.48, 0.66, 0.59, 0.93]


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _torch_ffn(x_rows, w1, b1, w2, b2):
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    h = F.linear(t(x_rows), t(w1), t(b1))
    return F.linear(F.silu(h), t(w2), t(b2)).numpy()


def _rand_weights(rng, E, d, f, scale=1.0):
    w1 = rng.standard_normal((E, f, d)) * scale / math.sqrt(d)
    b1 = rng.standard_normal((E, f)) * 0.1
    w2 = rng.standard_normal((E, d, f)) * scale / math.sqrt(f)
    b2 = rng.standard_normal((E, d)) * 0.1
    return w1, b1, w2, b2


# ----------------------------------------------------------------------------- capacity
def check_capacity_page(o):
    g = golden()
    L = g["layer"]
    assert o.capacity(L["T"], L["top_k"], L["n_experts"], g["capacity_factor"]["value"]) == g["capacity"]["value"]


def check_capacity_closed_forms(o):
    # floor(C*T*k/E) for the four bf16 workloads
    assert o.capacity(4096, 2, 8, 1.25) == 1280
    assert o.capacity(16384, 6, 64, 1.0) == 1536
    assert o.capacity(64, 2, 8, 4.0) == 64
    assert o.capacity(32768, 2, 8, 2.0) == 16384
    # small budgets round down to zero, no lower clamp
    assert o.capacity(4, 1, 8, 0.1) == 0
    assert o.capacity(7, 1, 8, 1.0) == 0
    assert o.capacity(8, 1, 8, 1.0) == 1
    # exact rational value of the stored double: 0.7 is stored slightly below 7/10, so
    # 0.7 * 10 / 7 is just under 1 and floors to 0 (double arithmetic would give 1)
    assert Fraction(0.7) < Fraction(7, 10)
    assert o.capacity(10, 1, 7, 0.7) == 0
    # 1.1 is stored slightly above 11/10
    assert o.capacity(10, 1, 1, 1.1) == 11
    # brute-force definition: the largest n with n * E <= C*T*k
    rng = _rng(11)
    for _ in range(200):
        T = int(rng.integers(0, 5000)); k = int(rng.integers(1, 9)); E = int(rng.integers(1, 300))
        C = float(rng.choice([0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 3.3, 0.1]))
        n = o.capacity(T, k, E, C)
        assert n >= 0
        assert Fraction(n) * E <= Fraction(C) * T * k < Fraction(n + 1) * E


# ----------------------------------------------------------------------------- routing
def check_softmax_closed_forms(o):
    L = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    p = o.softmax(L)
    assert np.max(np.abs(p - np.array([[0.1, 0.2, 0.3, 0.4]]))) < 4e-16
    assert o.softmax(np.array([[3.7]]))[0, 0] == 1.0
    p = o.softmax(np.full((1, 5), -2.25))
    assert np.all(np.abs(p - 0.2) < 1e-16)
    # shift invariance at large magnitude (no overflow)
    p = o.softmax(np.array([[1000.0, 1001.0]]))
    assert abs(p[0, 0] - 1.0 / (1.0 + math.e)) < 1e-15 and abs(p[0, 1] - math.e / (1.0 + math.e)) < 1e-15
    from scipy.special import softmax as sp_softmax
    Lr = _rng(3).standard_normal((50, 13)) * 4
    assert np.max(np.abs(o.softmax(Lr) - sp_softmax(Lr, axis=1))) < 1e-15


def check_router_logits_exact(o):
    """Integer-valued inputs: every partial sum is an exactly representable integer."""
    rng = _rng(5)
    for (T, d, E) in [(6, 4, 4), (5, 7, 3), (3, 33, 9)]:
        x = rng.integers(-50, 50, size=(T, d)).astype(np.float64)
        w = rng.integers(-50, 50, size=(E, d)).astype(np.float64)
        b = rng.integers(-9, 9, size=E).astype(np.float64)
        L = o.router_logits(x, w, b)
        for t in range(T):
            for e in range(E):
                want = sum(int(x[t, j]) * int(w[e, j]) for j in range(d)) + int(b[e])
                assert L[t, e] == want


def _topk_brute(g_row, k):
    E = len(g_row)
    beats = lambda a, b: (g_row[a] > g_row[b]) or (g_row[a] == g_row[b] and a < b)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(beats(a, b) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1
    chosen = list(winners[0])
    # order inside the chosen set: by how many chosen elements beat it (0 for the first)
    return sorted(chosen, key=lambda e: sum(bool(beats(o2, e)) for o2 in chosen))


def check_topk_bruteforce(o):
    rng = _rng(7)
    vals = np.array([0.125, 0.25, 0.25, 0.375, 0.5], dtype=np.float32)
    for E in range(1, 7):
        for k in range(1, E + 1):
            for _ in range(25):
                g = vals[rng.integers(len(vals), size=(1, E))]
                ids, gates = o.top_k(g, k)
                want = _topk_brute(g[0], k)
                assert list(ids[0]) == want, (g, k, ids, want)
                assert np.array_equal(gates[0], g[0, want])


def check_gates_unrenormalised(o):
    """Top-k gates are the softmax probabilities themselves (scipy), rounded to fp32."""
    from scipy.special import softmax as sp_softmax
    rng = _rng(9)
    x = rng.standard_normal((40, 16))
    w = rng.standard_normal((6, 16)) / 4
    r = o.route(x, w, None, 2)
    p = sp_softmax(x @ w.T, axis=1)
    for t in range(40):
        for c in range(2):
            assert abs(float(r["gates"][t, c]) - p[t, r["ids"][t, c]]) <= 6e-8 * p[t, r["ids"][t, c]] + 1e-30
        assert r["gates"][t, 0] >= r["gates"][t, 1]
        assert r["ids"][t, 0] == int(np.argmax(p[t]))
    # with 6 experts the two chosen gates cannot sum to one
    assert np.all(r["gates"].astype(np.float64).sum(axis=1) < 1.0)


def check_gates_rounded_before_topk(o):
    """Top-k ranks the fp32 gates, not the float64 probabilities.  Logits (0, 1e-9) give
    probabilities 0.5 -/+ 2.5e-10; both lie within half an fp32 ulp of 0.5 (the fp32 neighbours
    of 0.5 are 0.5 - 2^-25 and 0.5 + 2^-24), so both gates are exactly 0.5 and the tie goes to
    the lower expert, although expert 1's float64 probability is the larger."""
    x = np.array([[1.0]])
    w = np.array([[0.0], [1e-9]])
    r = o.route(x, w, None, 1)
    assert r["probs"][0, 1] > r["probs"][0, 0]
    assert int(r["ids"][0, 0]) == 0
    assert r["gates"].dtype == np.float32 and float(r["gates"][0, 0]) == 0.5
    r2 = o.route(x, w, None, 2)
    assert list(r2["ids"][0]) == [0, 1] and list(r2["gates"][0]) == [0.5, 0.5]
    # (0, ln 3): 0.25 and 0.75 exactly after the rounding, whatever the last float64 bits
    r3 = o.route(np.array([[1.0]]), np.array([[0.0], [math.log(3.0)]]), None, 2)
    assert list(r3["ids"][0]) == [1, 0] and list(r3["gates"][0]) == [0.75, 0.25]
    # the fill order compares the rounded gates too: two tokens whose float64 probabilities for
    # expert 1 differ below fp32 resolution tie, and the lower token takes the single slot
    x2 = np.array([[1.0], [1.0 + 2.0 ** -20]])
    w2 = np.array([[0.0], [2.0 ** -12]])
    r4 = o.route(x2, w2, None, 1)
    assert list(r4["ids"][:, 0]) == [1, 1] and r4["probs"][1, 1] > r4["probs"][0, 1]
    assert r4["gates"][0, 0] == r4["gates"][1, 0]
    d = o.dispatch(r4["ids"], r4["gates"], 2, 1)
    assert list(d["drop_mask"][:, 0]) == [0, 1]


# ----------------------------------------------------------------------------- dispatch
def _counting_ranks(ids, gates, E, cap):
    """Independent definition: rank = number of same-expert assignments ahead in the order
    (larger gate, or equal gate and smaller token, or same token and smaller choice)."""
    T, k = ids.shape
    rank = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for c in range(k):
            e = ids[t, c]; g = float(gates[t, c])
            r = 0
            for t2 in range(T):
                for c2 in range(k):
                    if ids[t2, c2] != e or (t2, c2) == (t, c):
                        continue
                    g2 = float(gates[t2, c2])
                    if g2 > g or (g2 == g and (t2, c2) < (t, c)):
                        r += 1
            rank[t, c] = r
    counts = np.array([(ids == e).sum() for e in range(E)])
    kept = np.minimum(counts, cap)
    off = np.concatenate([[0], np.cumsum(kept)])
    slot = np.where(rank < cap, off[ids] + rank, -1)
    return rank, slot, counts, off


def check_worked_example_dispatch(o):
    g = golden()
    ids = np.array(g["assignment"]["ids"], dtype=np.int32)[:, None]
    gates = np.array(FORCED_GATES, dtype=np.float32)[:, None]
    cap = g["capacity"]["value"]
    d = o.dispatch(ids, gates, 4, cap)
    assert d["counts"][0] == g["expert0_load"]["value"]
    assert list(np.nonzero(d["drop_mask"][:, 0])[0]) == [g["dropped_token"]["value"]]
    kept_sets = []
    for e in range(4):
        s0, s1 = int(d["offsets"][e]), int(d["offsets"][e + 1])
        kept_sets.append(sorted(int(t) for t in d["row_token"][s0:s1]))
    assert kept_sets == [sorted(b) for b in g["kept_batches"]["value"]]
    assert max(e1 - e0 for e0, e1 in zip(d["offsets"][:-1], d["offsets"][1:])) == g["slowest_expert_rows"]["value"]


def check_dispatch_exhaustive(o):
    vals = [0.25, 0.5, 0.75]
    # k = 1: every id pattern and every gate pattern for T = 4 tokens over E = 3 experts
    for T, E in [(3, 2), (4, 3)]:
        for id_pat in itertools.product(range(E), repeat=T):
            ids = np.array(id_pat, dtype=np.int32)[:, None]
            for g_pat in itertools.product(vals, repeat=T):
                gates = np.array(g_pat, dtype=np.float32)[:, None]
                for cap in (0, 1, 2, T):
                    d = o.dispatch(ids, gates, E, cap)
                    rank, slot, counts, off = _counting_ranks(ids, gates, E, cap)
                    assert np.array_equal(d["slot_of"], slot)
                    assert np.array_equal(d["counts"], counts)
                    assert np.array_equal(d["offsets"], off)
    # k = 2: random ordered pairs of distinct experts and tied gates
    rng = _rng(13)
    for _ in range(400):
        T = int(rng.integers(1, 6)); E = int(rng.integers(2, 5)); k = 2
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32)
        gates = np.array(vals, dtype=np.float32)[rng.integers(3, size=(T, k))]
        cap = int(rng.integers(0, T + 1))
        d = o.dispatch(ids, gates, E, cap)
        rank, slot, counts, off = _counting_ranks(ids, gates, E, cap)
        assert np.array_equal(d["slot_of"], slot)
        assert np.array_equal(d["drop_mask"], (slot < 0).astype(np.uint8))


def check_dispatch_invariants(o):
    rng = _rng(17)
    for trial in range(30):
        T = int(rng.integers(1, 300)); E = int(rng.integers(1, 12)); k = int(rng.integers(1, E + 1))
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32)
        gates = rng.choice(np.array([0.1, 0.2, 0.3, 0.7], dtype=np.float32), size=(T, k)) if trial % 2 \
            else rng.random((T, k)).astype(np.float32)
        cap = int(rng.integers(0, max(2, T * k // E + 3)))
        d = o.dispatch(ids, gates, E, cap)
        assert d["counts"].sum() == T * k
        assert d["n_kept"] == int(np.minimum(d["counts"], cap).sum())
        s = d["slot_of"][d["slot_of"] >= 0]
        assert np.array_equal(np.sort(s), np.arange(d["n_kept"]))
        for t in range(T):
            for c in range(k):
                if d["slot_of"][t, c] >= 0:
                    sl = d["slot_of"][t, c]
                    assert d["row_token"][sl] == t
                    assert d["offsets"][ids[t, c]] <= sl < d["offsets"][ids[t, c] + 1]
        for e in range(E):
            m = ids == e
            kept_g = gates[m & (d["slot_of"] >= 0)]
            drop_g = gates[m & (d["slot_of"] < 0)]
            if len(kept_g) and len(drop_g):
                assert kept_g.min() >= drop_g.max()
            # within an expert, slots run in the fill order (gate descending)
            sl = d["slot_of"][m & (d["slot_of"] >= 0)]
            g_by_slot = gates[m & (d["slot_of"] >= 0)][np.argsort(sl)]
            assert np.all(np.diff(g_by_slot.astype(np.float64)) <= 0)


def check_permutation_equivariance(o):
    rng = _rng(19)
    T, d, f, E, k = 40, 8, 12, 5, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    cap = o.capacity(T, k, E, 1.0)
    a = o.forward(x, w, None, w1, b1, w2, b2, k, 1.0)
    perm = rng.permutation(T)
    b = o.forward(x[perm], w, None, w1, b1, w2, b2, k, 1.0)
    assert a["cap"] == cap == b["cap"]
    assert np.array_equal(a["drop_mask"][perm], b["drop_mask"])
    assert np.max(np.abs(a["out"][perm] - b["out"])) < 1e-12


# ----------------------------------------------------------------------------- FFN + combine
def check_silu_closed_forms(o):
    import torch
    import torch.nn.functional as F
    h = np.array([-800.0, -30.0, -1.5, -0.0, 0.0, 0.3, 2.0, 40.0, 800.0])
    s = o.silu(h)
    assert np.all(np.isfinite(s))
    assert np.max(np.abs(s - F.silu(torch.as_tensor(h)).numpy())) < 1e-15
    assert abs(o.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    assert o.silu(np.array([800.0]))[0] == 800.0


def check_expert_ffn_vs_torch(o):
    rng = _rng(23)
    E, d, f = 3, 6, 10
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    xr = rng.standard_normal((7, d))
    for e in range(E):
        got = o.expert_ffn(xr, w1[e], b1[e], w2[e], b2[e])
        assert np.max(np.abs(got - _torch_ffn(xr, w1[e], b1[e], w2[e], b2[e]))) < 1e-13


def check_worked_example_outputs(o):
    """Forced routing of the worked example: out_0 = x_0 + 0.87 y_0, out_4 = x_4 bit for bit."""
    g = golden()
    L = g["layer"]
    rng = _rng(29)
    T, d, f, E = L["T"], L["d_model"], L["d_ff"], L["n_experts"]
    x = rng.standard_normal((T, d))
    x[0] = g["x0"]["value"]
    x[4, 1] = -0.0  # a negative zero must survive the residual path
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    ids = np.array(g["assignment"]["ids"], dtype=np.int32)[:, None]
    gates = np.array(FORCED_GATES, dtype=np.float32)[:, None]
    assert gates[0, 0] == np.float32(g["gate0"]["value"])
    res = o.forward_with_routing(x, ids, gates, g["capacity"]["value"], E, w1, b1, w2, b2)
    dropped = g["dropped_token"]["value"]
    assert res["all_dropped"][dropped]
    assert np.array_equal(res["out"][dropped], x[dropped])
    assert np.signbit(res["out"][dropped, 1])
    for t in range(T):
        if t == dropped:
            continue
        e = ids[t, 0]
        y = _torch_ffn(x[t:t + 1], w1[e], b1[e], w2[e], b2[e])[0]
        want = x[t] + float(gates[t, 0]) * y
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13


def check_dense_special_case(o):
    """One expert, top-1, room for every token: gate is exactly 1 and the layer is a dense
    residual FFN, out = x + FFN(x)."""
    rng = _rng(31)
    T, d, f = 9, 5, 7
    x = rng.standard_normal((T, d)); w = rng.standard_normal((1, d))
    w1, b1, w2, b2 = _rand_weights(rng, 1, d, f)
    res = o.forward(x, w, None, w1, b1, w2, b2, 1, 1.0)
    assert np.all(res["gates"] == 1.0)
    want = x + _torch_ffn(x, w1[0], b1[0], w2[0], b2[0])
    assert np.max(np.abs(res["out"] - want)) < 1e-13


def check_dropless_per_token(o):
    """Capacity >= T: nothing drops and each token gets the gate-weighted sum of its k
    experts (a per-token loop with torch's linear layers, independent of dispatch)."""
    rng = _rng(37)
    T, d, f, E, k = 12, 6, 9, 4, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    b = rng.standard_normal(E)
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    res = o.forward(x, w, b, w1, b1, w2, b2, k, float(E))
    assert res["cap"] >= T
    assert not res["drop_mask"].any()
    for t in range(T):
        want = x[t].copy()
        for c in range(k):
            e = res["ids"][t, c]
            want = want + float(res["gates"][t, c]) * _torch_ffn(x[t:t + 1], w1[e], b1[e], w2[e], b2[e])[0]
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13


def check_all_experts(o):
    """k = E: every token uses every expert; with room for all, the gates sum to ~1 and
    out = x + sum_e p_e FFN_e(x)."""
    rng = _rng(41)
    T, d, f, E = 6, 4, 5, 3
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    res = o.forward(x, w, None, w1, b1, w2, b2, E, 1.0)
    assert res["cap"] == T
    assert np.all(np.sort(res["ids"], axis=1) == np.arange(E))
    assert np.all(np.abs(res["gates"].astype(np.float64).sum(axis=1) - 1.0) < 1e-6)
    for t in range(T):
        want = x[t] + sum(float(res["gates"][t, c]) * _torch_ffn(x[t:t + 1], *(a[res["ids"][t, c]] for a in (w1, b1, w2, b2)))[0]
                          for c in range(E))
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13


def check_capacity_zero(o):
    rng = _rng(43)
    T, d, f, E = 10, 4, 6, 8
    x = rng.standard_normal((T, d)); x[3, 2] = -0.0
    w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    res = o.forward(x, w, None, w1, b1, w2, b2, 1, 0.5)  # floor(0.5*10/8) = 0
    assert res["cap"] == 0 and res["n_kept"] == 0
    assert res["all_dropped"].all()
    assert np.array_equal(res["out"], x) and np.signbit(res["out"][3, 2])


# ----------------------------------------------------------------------------- padded buffers
def check_padded_worked_example(o):
    """"Why there is a buffer": with the worked example's forced assignment and capacity 2,
    the four fixed buffers hold the page's kept batches, in fill order (gate descending), and
    expert 2's buffer has one empty slot; token 4 has no slot."""
    g = golden()
    ids = np.array(g["assignment"]["ids"], dtype=np.int32)[:, None]
    gates = np.array(FORCED_GATES, dtype=np.float32)[:, None]
    cap = g["capacity"]["value"]
    d = o.dispatch_padded(ids, gates, 4, cap)
    rows = [int(t) for t in d["row_token"]]
    # buffer e holds the page's kept batch e, ordered by the forced gates (descending)
    want = []
    for batch in g["kept_batches"]["value"]:
        b = sorted(batch, key=lambda t: -FORCED_GATES[t])
        want += b + [-1] * (cap - len(b))
    assert rows == want
    assert int(d["slot_of"][g["dropped_token"]["value"], 0]) == -1
    assert sum(r < 0 for r in rows) == 4 * cap - (8 - 1)


def check_padded_empty_rows(o):
    """An empty slot's input is the zero row: with b1 = 0, SiLU(0) = 0 makes its expert output
    exactly b2; with b1 != 0 it is torch's FFN of a zero row."""
    rng = _rng(47)
    T, d, f, E, k = 12, 4, 6, 3, 1
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d)) * 3
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    res = o.forward_padded(x, w, None, w1, np.zeros_like(b1), w2, b2, k, 2.0)  # cap = 8
    cap = res["cap"]
    assert cap == 8
    empty = np.nonzero(res["row_token"] < 0)[0]
    assert len(empty) == E * cap - T * k
    for r in empty:
        assert np.array_equal(res["Y"][r], b2[r // cap])
    res = o.forward_padded(x, w, None, w1, b1, w2, b2, k, 2.0)
    for r in np.nonzero(res["row_token"] < 0)[0]:
        e = r // cap
        want = _torch_ffn(np.zeros((1, d)), w1[e], b1[e], w2[e], b2[e])[0]
        assert np.max(np.abs(res["Y"][r] - want)) < 1e-14


def check_padded_same_layer(o):
    """Computing the empty slots changes nothing the layer returns: same routing, same kept
    assignments, same output as the compact layout (to float64 rounding of the batched
    products), and each filled buffer row is torch's FFN of its token."""
    rng = _rng(53)
    T, d, f, E, k = 20, 6, 8, 5, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    for C in (0.5, 1.25):
        a = o.forward(x, w, None, w1, b1, w2, b2, k, C)
        p = o.forward_padded(x, w, None, w1, b1, w2, b2, k, C)
        assert np.array_equal(a["slot_of"] >= 0, p["slot_of"] >= 0)
        assert np.max(np.abs(a["out"] - p["out"])) < 1e-13
        cap = p["cap"]
        for r in np.nonzero(p["row_token"] >= 0)[0]:
            e, t = r // cap, p["row_token"][r]
            assert np.max(np.abs(p["Y"][r] - _torch_ffn(x[t:t + 1], w1[e], b1[e], w2[e], b2[e])[0])) < 1e-13
        # the kept assignment of rank r of expert e sits in row e * cap + r
        for t in range(T):
            for c in range(k):
                if a["slot_of"][t, c] >= 0:
                    e = a["ids"][t, c]
                    assert p["slot_of"][t, c] == e * cap + a["slot_of"][t, c] - a["offsets"][e]


# ----------------------------------------------------------------------------- gated expert
def _torch_gated(x_rows, w13, w2):
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    f = np.asarray(w13).shape[0] // 2
    g = F.linear(t(x_rows), t(w13)[:f])
    u = F.linear(t(x_rows), t(w13)[f:])
    return F.linear(F.silu(g) * u, t(w2)).numpy()


def check_gated_closed_forms(o):
    """SiLU(ln 3) = (3/4) ln 3, so with one input, gate and up rows of 1 and W2 = 1 the
    expert returns (3/4) (ln 3)^2; a zero gate gives exactly zero (SiLU(0) = 0)."""
    x = np.array([[math.log(3.0)]])
    y = o.expert_ffn_gated(x, np.array([[1.0], [1.0]]), np.array([[1.0]]))
    assert abs(y[0, 0] - 0.75 * math.log(3.0) ** 2) < 1e-15
    rng = _rng(59)
    d, f = 5, 3
    w13 = rng.standard_normal((2 * f, d)); w13[:f] = 0.0
    y = o.expert_ffn_gated(rng.standard_normal((4, d)), w13, rng.standard_normal((d, f)))
    assert np.array_equal(y, np.zeros_like(y))
    # gate and up halves are not interchangeable: a negative gate with a positive up differs
    x = np.array([[-2.0]])
    y = o.expert_ffn_gated(x, np.array([[1.0], [-1.0]]), np.array([[1.0]]))  # g = -2, u = 2
    assert abs(y[0, 0] - (-2.0 / (1.0 + math.exp(2.0))) * 2.0) < 1e-15


def check_gated_vs_torch(o):
    """The gated expert against torch's float64 linear and SiLU, and the whole gated layer
    against a per-token recomputation with that reference."""
    rng = _rng(61)
    T, d, f, E, k = 16, 6, 5, 4, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w13 = rng.standard_normal((E, 2 * f, d)) / math.sqrt(d)
    w2 = rng.standard_normal((E, d, f)) / math.sqrt(f)
    for e in range(E):
        got = o.expert_ffn_gated(x, w13[e], w2[e])
        assert np.max(np.abs(got - _torch_gated(x, w13[e], w2[e]))) < 1e-13
    res = o.forward_gated(x, w, None, w13, w2, k, 1.0)
    for t in range(T):
        want = x[t].copy()
        for c in range(k):
            if res["slot_of"][t, c] >= 0:
                e = res["ids"][t, c]
                want = want + float(res["gates"][t, c]) * _torch_gated(x[t:t + 1], w13[e], w2[e])[0]
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13


# ----------------------------------------------------------------------------- dropless flow
def check_pairs_hand_example(o):
    """Three tokens, top-2 over three experts, sorted by hand: pair p = t*2 + c.
    ids [[1, 0], [0, 2], [2, 1]] -> expert 0 gets pairs 1, 2; expert 1 pairs 0, 5; expert 2
    pairs 3, 4; GEMM 1 reads token rows p // 2."""
    d = o.dispatch_pairs(np.array([[1, 0], [0, 2], [2, 1]], dtype=np.int32), 3)
    assert list(d["counts"]) == [2, 2, 2]
    assert list(d["offsets"]) == [0, 2, 4, 6]
    assert list(d["sorted_pairs"]) == [1, 2, 0, 5, 3, 4]
    assert list(d["row_token"]) == [0, 1, 0, 2, 1, 2]
    # an expert nobody picked has an empty range
    d = o.dispatch_pairs(np.array([[3], [0], [3]], dtype=np.int32), 4)
    assert list(d["offsets"]) == [0, 1, 1, 1, 3] and list(d["sorted_pairs"]) == [1, 0, 2]


def check_pairs_invariants(o):
    """Counting-sort facts on random ids: a permutation of all pairs, experts in
    non-decreasing order, ascending pairs inside each expert, counts = bincount."""
    rng = _rng(67)
    for T, k, E in ((37, 3, 5), (64, 2, 8), (5, 4, 4)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        d = o.dispatch_pairs(ids, E)
        sp = np.asarray(d["sorted_pairs"], dtype=np.int64)
        assert np.array_equal(np.sort(sp), np.arange(T * k))
        e_of = ids.reshape(-1)[sp]
        assert np.all(np.diff(e_of) >= 0)
        assert np.array_equal(d["counts"], np.bincount(ids.reshape(-1), minlength=E))
        for e in range(E):
            seg = sp[d["offsets"][e]:d["offsets"][e + 1]]
            assert np.all(ids.reshape(-1)[seg] == e) and np.all(np.diff(seg) > 0)
        assert np.array_equal(d["row_token"], sp // k)


def check_moe_sum(o):
    """moe_sum adds rows t*k .. t*k + k - 1: numpy's reshape to [T, k, d] and sum over k."""
    rng = _rng(71)
    T, k, d = 7, 3, 5
    rows = rng.standard_normal((T * k, d))
    res = rng.standard_normal((T, d))
    assert np.max(np.abs(o.moe_sum(rows, k) - rows.reshape(T, k, d).sum(axis=1))) < 1e-14
    assert np.max(np.abs(o.moe_sum(rows, k, res) - res - rows.reshape(T, k, d).sum(axis=1))) < 1e-14


def check_dropless_flow_vs_torch(o):
    """Each pair row is topk_weight * expert(x[t]) and each token leaves as x[t] plus its k
    pair rows, against a per-token recomputation with torch's float64 layers (plain and
    gated experts); skewed router bias so one expert holds most pairs (nothing drops)."""
    rng = _rng(73)
    T, d, f, E, k = 14, 6, 7, 4, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    b = np.array([3.0, 0.0, -1.0, 0.5])
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    res = o.forward_dropless(x, w, b, w1, b1, w2, b2, k)
    assert int(np.max(res["counts"])) > T * k // E  # skewed: a capacity of T*k/E would drop
    for t in range(T):
        want = x[t].copy()
        for c in range(k):
            e = res["ids"][t, c]
            y = float(res["gates"][t, c]) * _torch_ffn(x[t:t + 1], w1[e], b1[e], w2[e], b2[e])[0]
            assert np.max(np.abs(res["pair_rows"][t * k + c] - y)) < 1e-13
            want = want + y
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13
    w13 = rng.standard_normal((E, 2 * f, d)) / math.sqrt(d)
    w2g = rng.standard_normal((E, d, f)) / math.sqrt(f)
    res = o.forward_dropless_gated(x, w, b, w13, w2g, k)
    for t in range(T):
        want = x[t].copy()
        for c in range(k):
            e = res["ids"][t, c]
            want = want + float(res["gates"][t, c]) * _torch_gated(x[t:t + 1], w13[e], w2g[e])[0]
        assert np.max(np.abs(res["out"][t] - want)) < 1e-13


def check_dropless_is_capacity_without_drops(o):
    """With a capacity that holds every pair (C = E gives cap = T*k) the capacity layer drops
    nothing, and the dropless flow returns its output; pair row t*k + c is the gate times the
    capacity layer's expert output in slot slot_of[t, c]."""
    rng = _rng(79)
    T, d, f, E, k = 18, 5, 6, 5, 3
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    a = o.forward(x, w, None, w1, b1, w2, b2, k, float(E))
    p = o.forward_dropless(x, w, None, w1, b1, w2, b2, k)
    assert not a["drop_mask"].any()
    assert np.array_equal(a["ids"], p["ids"]) and np.array_equal(a["counts"], p["counts"])
    assert np.max(np.abs(a["out"] - p["out"])) < 1e-13
    for t in range(T):
        for c in range(k):
            want = float(a["gates"][t, c]) * a["Y"][a["slot_of"][t, c]]
            assert np.max(np.abs(p["pair_rows"][t * k + c] - want)) < 1e-13


# ----------------------------------------------------------------------------- batch scheduler
def check_schedule_diagram(o):
    """The diagram's pool: 8 tokens, top-1 over 4 experts, two batches of 4 in which every
    expert takes one token.  After scheduling, each batch activates 2 experts with 2 tokens
    each, for every order of the second batch's experts (the transcription does not fix it)."""
    with open(GOLDEN_SCHED) as fh:
        g = json.load(fh)["facts"]
    B = g["pool"]["batch_size"]
    for perm in itertools.permutations(range(4)):
        ids = np.array(g["batch1_experts"]["value"] + list(perm), dtype=np.int32)[:, None]
        s = o.schedule_batches(ids, B)
        assert [list(b) for b in s["orig_batches"]] == g["original_batches"]["value"]
        assert list(s["orig_active"]) == [g["original_active_per_batch"]["value"]] * 2
        assert B // g["original_active_per_batch"]["value"] == g["original_tokens_per_expert"]["value"]
        assert list(s["active"]) == [g["optimized_active_per_batch"]["value"]] * 2
        for b in s["batches"]:
            _, per = np.unique(ids[b, 0], return_counts=True)
            assert list(per) == [g["optimized_tokens_per_expert"]["value"]] * 2
        assert sorted(int(t) for t in s["order"]) == list(range(8))


def check_schedule_bruteforce(o):
    """Random pools (top-1 .. top-3): the order is a permutation, tokens sharing an expert set
    are contiguous in it, sets appear in ascending tuple order with ascending token index
    inside, and the active counts are the set sizes counted directly; for top-1 the total
    active experts is at most (experts used) + (batches) - 1."""
    rng = _rng(83)
    for T, B, E, k in ((24, 4, 5, 1), (48, 8, 6, 2), (60, 12, 7, 3), (16, 16, 3, 1), (30, 1, 4, 2)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        s = o.schedule_batches(ids, B)
        order = [int(t) for t in s["order"]]
        assert sorted(order) == list(range(T))
        keys = [tuple(sorted(ids[t])) for t in order]
        for i in range(T - 1):
            assert keys[i] < keys[i + 1] or (keys[i] == keys[i + 1] and order[i] < order[i + 1])
        for j, b in enumerate(s["batches"]):
            assert list(b) == order[j * B:(j + 1) * B]
            assert s["active"][j] == len(set(ids[b].ravel().tolist()))
        for j in range(T // B):
            assert s["orig_active"][j] == len(set(ids[j * B:(j + 1) * B].ravel().tolist()))
        if k == 1:
            assert int(s["active"].sum()) <= len(set(ids.ravel().tolist())) + T // B - 1


def check_batches_output(o):
    """Capacity at least the batch size: nothing drops and every token leaves as x plus its
    gate-weighted experts (torch float64, per token), grouped or not.  A smaller capacity is
    applied per batch: each batch's output is the capacity layer run on that batch alone."""
    rng = _rng(89)
    T, B, d, f, E, k = 24, 6, 5, 7, 4, 2
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    w1, b1, w2, b2 = _rand_weights(rng, E, d, f)
    C = float(E) / k  # capacity = B
    for cons in (False, True):
        res = o.forward_batches(x, w, None, w1, b1, w2, b2, k, C, B, cons)
        assert res["cap"] == B and res["n_kept"] == T * k
        for t in range(T):
            want = x[t].copy()
            for c in range(k):
                e = res["ids"][t, c]
                want = want + float(res["gates"][t, c]) * _torch_ffn(x[t:t + 1], w1[e], b1[e], w2[e], b2[e])[0]
            assert np.max(np.abs(res["out"][t] - want)) < 1e-13
    res = o.forward_batches(x, w, None, w1, b1, w2, b2, k, 0.5, B, True)
    assert res["cap"] == 1
    for b in res["batches"]:
        one = o.forward(x[b], w, None, w1, b1, w2, b2, k, 0.5)
        assert np.max(np.abs(res["out"][b] - one["out"])) < 1e-13


ALL_CHECKS = [
    check_capacity_page, check_capacity_closed_forms, check_softmax_closed_forms,
    check_router_logits_exact, check_topk_bruteforce, check_gates_unrenormalised,
    check_gates_rounded_before_topk,
    check_worked_example_dispatch, check_dispatch_exhaustive, check_dispatch_invariants,
    check_permutation_equivariance, check_silu_closed_forms, check_expert_ffn_vs_torch,
    check_worked_example_outputs, check_dense_special_case, check_dropless_per_token,
    check_all_experts, check_capacity_zero, check_padded_worked_example,
    check_padded_empty_rows, check_padded_same_layer, check_gated_closed_forms,
    check_gated_vs_torch, check_pairs_hand_example, check_pairs_invariants, check_moe_sum,
    check_dropless_flow_vs_torch, check_dropless_is_capacity_without_drops,
    check_schedule_diagram, check_schedule_bruteforce, check_batches_output,
]
