"""Comparison rules between the HIP path and the CPU oracle.

  * integers (expert ids, counts, offsets, slots, row tokens, drop masks): exact;
  * gates and expert ids: exact, except for a token where the oracle's float64 probability of
    some expert lies so close to the midpoint between two fp32 values that a different but
    equally valid float64 evaluation can round it the other way.  "Close" is a proven bound,
    not a tolerance (route_bound): both sides sum the same exact products of the router
    inputs in float64 in different orders and evaluate the same softmax.  Such a token is
    accepted only if every GPU gate is one of the roundings the bound admits, the chosen set
    is the top-k of some admissible gate vector, and it is counted and reported;
  * floats: max|gpu - ref| / max|ref| <= 2e-2 (bf16 storage, fp32 accumulation) or 1e-5
    (fp32), per tensor; the element-wise max|gpu - ref| / (|ref| + 1e-3) is reported beside it;
  * rows of tokens with no kept choice: bit-identical to x.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-5}
U64 = 2.0 ** -53  # unit roundoff of float64


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a tensor (int16 for bf16, int32 for fp32)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return num
    return num / den


def elementwise_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """Diagnostic: max over elements of |got - ref| / (|ref| + 1e-3)."""
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)))


def route_bound(oref: dict, x64: np.ndarray, w64: np.ndarray, b=None) -> np.ndarray:
    """Per token, a bound rho such that any two float64 evaluations of the softmax
    probabilities that follow the oracle's definition differ by at most 2 rho p, relative.

    Each side forms L_e = sum_j x_j w_ej + b_e from exact products (a bf16 or fp32 product is
    exact in float64) with d additions in its own order, so |L_e - exact| <= gamma_{d+1} A_e,
    A_e = sum_j |x_j w_ej| + |b_e|, gamma_n = n u / (1 - n u) (recursive summation in any
    order).  A perturbation dL of the logits moves ln p_e by dL_e - sum p_e' dL_e', at most
    2 max|dL|.  Evaluating p = exp(L - m) / sum exp(L - m) adds the rounding of L - m (|L - m|
    u), exp's own error (at most 1 ulp each side), the sum of E terms (gamma_E) and the
    division (u).  rho bounds one side's relative error against the exact value; it is
    doubled for the safety of first-order terms."""
    x64 = np.asarray(x64, np.float64); w64 = np.asarray(w64, np.float64)
    A = np.abs(x64) @ np.abs(w64).T
    if b is not None:
        A = A + np.abs(np.asarray(b, np.float64))[None, :]
    n = x64.shape[1] + 1
    gamma = n * U64 / (1 - n * U64)
    L = oref["logits"]
    E = L.shape[1]
    spread = np.max(np.abs(L - L.max(axis=1, keepdims=True)), axis=1)
    rho = 2.0 * gamma * A.max(axis=1) + (spread + E + 6) * 2 * U64
    return 2.0 * rho


def _fp32_neighbours(g: np.float32):
    return (np.nextafter(g, np.float32(-np.inf)), np.nextafter(g, np.float32(np.inf)))


def _admissible(p: float, rho: float) -> list:
    """fp32 values a float64 evaluation within 2 rho p (relative) of p can round to."""
    g = np.float32(p)
    out = [g]
    for nb in _fp32_neighbours(g):
        mid = (float(g) + float(nb)) / 2.0
        if abs(p - mid) <= 2.0 * rho * abs(p):
            out.append(nb)
    return out


def compare_route(ids_gpu, gates_gpu, oref, x=None, w=None, b=None) -> dict:
    """Top-k ids and gates of the GPU against the oracle, bit for bit.

    A token whose ids or gates differ is accepted only when the difference is certified by
    route_bound (x, w, b are the router inputs in float64; without them no difference is
    accepted): every GPU gate must be an admissible fp32 rounding of its expert's probability,
    the choices must be in (gate descending, expert ascending) order, and every expert left out
    must be able to sort after the last choice with some admissible gate.  Returns the
    mismatched (certified) tokens and the largest gate difference in fp32 ulps."""
    ids_gpu = np.asarray(ids_gpu); gates_gpu = np.asarray(gates_gpu, np.float32)
    ids_ref, gates_ref, probs = oref["ids"], oref["gates"], oref["probs"]
    T, k = ids_ref.shape
    E = probs.shape[1]
    assert ids_gpu.shape == (T, k) and gates_gpu.shape == (T, k)
    bad = np.nonzero(np.any(ids_gpu != ids_ref, axis=1) |
                     np.any(gates_gpu.view(np.uint32) != gates_ref.view(np.uint32), axis=1))[0]
    rho = route_bound(oref, x, w, b) if (len(bad) and x is not None) else None
    for t in bad:
        assert rho is not None, (f"token {t}: ids {ids_gpu[t]} gates {gates_gpu[t]} against "
                                 f"{ids_ref[t]} {gates_ref[t]} (no bound given)")
        ch = [int(e) for e in ids_gpu[t]]
        assert all(0 <= e < E for e in ch) and len(set(ch)) == k, f"token {t}: ids {ch}"
        adm = {e: _admissible(float(probs[t, e]), float(rho[t])) for e in range(E)}
        for c, e in enumerate(ch):
            assert gates_gpu[t, c] in adm[e], (
                f"token {t}: gate {gates_gpu[t, c]!r} of expert {e} is not an admissible "
                f"rounding of p = {probs[t, e]!r} (bound {rho[t]:.2e})")
        for c in range(k - 1):
            a, bb = (gates_gpu[t, c], ch[c]), (gates_gpu[t, c + 1], ch[c + 1])
            assert a[0] > bb[0] or (a[0] == bb[0] and a[1] < bb[1]), f"token {t}: order {ch}"
        g_last, e_last = gates_gpu[t, k - 1], ch[k - 1]
        for e in range(E):
            if e in ch:
                continue
            lo = min(adm[e])
            assert lo < g_last or (lo == g_last and e > e_last), (
                f"token {t}: expert {e} (p = {probs[t, e]!r}) must have been chosen over "
                f"{ch} (gates {gates_gpu[t]})")
    # gate differences in fp32 ulps, against the rounding of the chosen expert's probability
    ref_g = probs[np.arange(T)[:, None], np.clip(ids_gpu, 0, E - 1)].astype(np.float32)
    ulp = np.abs(gates_gpu.view(np.int32).astype(np.int64) - ref_g.view(np.int32).astype(np.int64))
    return {"mismatched_tokens": [int(t) for t in bad], "certified": int(len(bad)),
            "max_gate_ulp": int(ulp.max()) if ulp.size else 0}


def compare_dispatch(gpu: dict, dref: dict, max_rows: int | None = None):
    """Exact equality of every integer output of the dispatch step."""
    assert np.array_equal(to_np(gpu["counts"]), dref["counts"]), "expert counts"
    if "offsets" in gpu:
        assert np.array_equal(to_np(gpu["offsets"]), dref["offsets"]), "expert offsets"
    assert np.array_equal(to_np(gpu["slot_of"]), dref["slot_of"]), "slot_of"
    assert np.array_equal(to_np(gpu["drop_mask"]), dref["drop_mask"]), "drop_mask"
    if "row_token" in gpu:
        n = dref["n_kept"]
        assert np.array_equal(to_np(gpu["row_token"])[:n], dref["row_token"]), "row_token"
