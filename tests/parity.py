"""Comparison rules between the HIP path and the CPU oracle.

  * integers (expert ids, counts, offsets, slots, row tokens, drop masks): exact;
  * gates: exact, except where the oracle's fp64 probability lies within fp64 rounding noise
    of the midpoint between two fp32 values (the decision cannot be reproduced without the
    same summation order); such a case must also be a 1-ulp difference and is reported;
  * floats: max|gpu - ref| / max|ref| <= 2e-2 (bf16 storage, fp32 accumulation) or 1e-5
    (fp32), per tensor;
  * rows of tokens with no kept choice: bit-identical to x.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-5}
# fp64 logits are summed in a different order on the two sides (and exp may differ in the
# last ulp): allow a relative gap of this size to the fp32 rounding midpoint
AMBIGUITY_REL = 1e-12


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


def _ambiguous(p64: float, g_a: np.float32, g_b: np.float32) -> bool:
    """True if g_a and g_b are adjacent fp32 values and p64 sits at their midpoint within
    fp64 noise."""
    a, b = sorted([float(g_a), float(g_b)])
    if np.nextafter(np.float32(a), np.float32(np.inf)) != np.float32(b):
        return False
    mid = (a + b) / 2.0
    return abs(p64 - mid) <= AMBIGUITY_REL * abs(p64)


def compare_route(ids_gpu, gates_gpu, oref) -> dict:
    """Exact comparison of top-k ids/gates with certified-ambiguity accounting.

    Returns {"mismatched_tokens": [...], "ambiguous": n}; raises AssertionError on any
    difference that is not a certified fp32 rounding tie."""
    ids_gpu = np.asarray(ids_gpu); gates_gpu = np.asarray(gates_gpu)
    ids_ref, gates_ref, probs = oref["ids"], oref["gates"], oref["probs"]
    bad = np.nonzero(np.any(ids_gpu != ids_ref, axis=1) |
                     np.any(gates_gpu.view(np.uint32) != gates_ref.view(np.uint32), axis=1))[0]
    n_amb = 0
    for t in bad:
        # every GPU gate must be a correct or certified-ambiguous rounding of its probability
        for c in range(ids_gpu.shape[1]):
            e = int(ids_gpu[t, c])
            g_or = np.float32(probs[t, e])
            g = np.float32(gates_gpu[t, c])
            if g != g_or:
                assert _ambiguous(float(probs[t, e]), g, g_or), \
                    f"token {t}: gate of expert {e} is {g!r}, oracle {g_or!r} (p={probs[t, e]!r})"
                n_amb += 1
        # the chosen set must be a valid top-k of the GPU's (certified) gates: every chosen
        # gate is >= every unchosen oracle gate within one fp32 ulp
        chosen = set(int(e) for e in ids_gpu[t])
        others = [float(oref["gates_all"][t, e]) for e in range(probs.shape[1]) if e not in chosen]
        if others:
            lo = float(np.min(gates_gpu[t]))
            assert lo >= np.nextafter(np.float32(max(others)), np.float32(-np.inf)), \
                f"token {t}: chosen {ids_gpu[t]} vs oracle {ids_ref[t]}"
    assert len(bad) <= max(2, ids_ref.shape[0] // 10000), f"{len(bad)} tokens differ in routing"
    return {"mismatched_tokens": [int(t) for t in bad], "ambiguous": n_amb}


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
