"""The GPU-vs-oracle comparison rules of tests/parity.py, on the CPU: the route comparison is
bit-exact except where the float64 rounding bound certifies a difference."""
import numpy as np
import pytest

import oracle.moe_oracle as O
import parity as P


def _route(seed=0, T=300, d=64, E=8, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d)) / 8
    return x, w, O.route(x, w, None, k)


def test_identical_routing_passes():
    x, w, r = _route()
    info = P.compare_route(r["ids"], r["gates"], r, x=x, w=w)
    assert info == {"mismatched_tokens": [], "certified": 0, "max_gate_ulp": 0}


def test_bound_is_small_and_positive():
    x, w, r = _route()
    rho = P.route_bound(r, x, w)
    assert np.all(rho > 0) and np.all(rho < 1e-11)


@pytest.mark.parametrize("what", ["swap_ids", "gate_up_one_ulp", "gate_down_one_ulp",
                                  "other_expert", "no_bound"])
def test_uncertified_differences_fail(what):
    x, w, r = _route(seed=1)
    ids, gates = r["ids"].copy(), r["gates"].copy()
    t = 7
    if what == "swap_ids":
        ids[t] = ids[t][::-1]
        gates[t] = gates[t][::-1]
    elif what == "gate_up_one_ulp":
        gates[t, 0] = np.nextafter(gates[t, 0], np.float32(1))
    elif what == "gate_down_one_ulp":
        gates[t, 1] = np.nextafter(gates[t, 1], np.float32(0))
    elif what == "other_expert":
        e = [e for e in range(8) if e not in ids[t]][0]
        ids[t, 1] = e
        gates[t, 1] = r["gates_all"][t, e]
    else:
        gates[t, 0] = np.nextafter(gates[t, 0], np.float32(1))
        with pytest.raises(AssertionError):
            P.compare_route(ids, gates, r)
        return
    with pytest.raises(AssertionError):
        P.compare_route(ids, gates, r, x=x, w=w)


def _midpoint_case():
    """One token, two experts, probabilities 0.5 + 2^-25 and 0.5 - 2^-25.  The first lies exactly
    on the midpoint between the fp32 values 0.5 and 0.5 + 2^-24 (round to nearest even gives
    0.5); an evaluation a hair above rounds up instead, which the bound must admit."""
    p = np.array([[0.5 + 2.0 ** -25, 0.5 - 2.0 ** -25]])
    L = np.log(p)
    g32 = p.astype(np.float32)
    ids, gates = O.top_k(g32, 2)
    oref = {"logits": L, "probs": p, "gates_all": g32, "ids": ids, "gates": gates}
    x = np.array([[1.0, 1.0]])
    w = L.T.copy()[:, :1].repeat(2, axis=1) / 2  # any inputs of the logits' size
    return oref, x, w


def test_certified_midpoint_is_accepted_and_reported():
    oref, x, w = _midpoint_case()
    assert float(oref["gates"][0, 0]) == 0.5
    up = np.float32(0.5 + 2.0 ** -24)
    info = P.compare_route(oref["ids"], np.array([[up, oref["gates"][0, 1]]], np.float32), oref,
                           x=x, w=w)
    assert info["certified"] == 1 and info["max_gate_ulp"] == 1


def test_certified_midpoint_still_checks_the_order():
    oref, x, w = _midpoint_case()
    up = np.float32(0.5 + 2.0 ** -24)
    # the admissible gate is there, but the choices are out of order
    with pytest.raises(AssertionError):
        P.compare_route(oref["ids"][:, ::-1].copy(),
                        np.array([[oref["gates"][0, 1], up]], np.float32), oref, x=x, w=w)
    # a two-ulp move is never admissible
    with pytest.raises(AssertionError):
        P.compare_route(oref["ids"], np.array([[np.nextafter(up, np.float32(1)),
                                                oref["gates"][0, 1]]], np.float32), oref, x=x, w=w)


def test_elementwise_diagnostic():
    ref = np.array([0.0, 1.0, -2.0])
    got = np.array([1e-3, 1.01, -2.0])
    # |1e-3 - 0| / (0 + 1e-3) = 1 dominates; the normalised error is 0.01 / 2
    assert P.elementwise_rel(got, ref) == pytest.approx(1.0, rel=1e-12)
    assert P.max_abs_rel(got, ref) == pytest.approx(0.01 / 2.0)
