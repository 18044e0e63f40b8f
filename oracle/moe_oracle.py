"""Plain CPU oracle for the forward pass of a capacity-limited Mixture-of-Experts layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check of the
entry module and the CPU-baseline leg of the benchmark may import or call this module.
The product path (the HIP library and its Python binding) never touches it, and this
module imports nothing from the product package.

Everything here is written from the pages' description of the method, in float64,
in the order the pages give the steps, with no blocking, fusion or reordering beyond
what a library primitive (matmul, sort) does internally:

  * "Expert Networks > Worked Example: Expert Specialization" (mbrenndoerfer.com):
    top-1 routing of 8 tokens to 4 experts, capacity from the capacity factor
    rounded down, the lowest-confidence token of an overloaded expert dropped, the
    expert FFN as up-projection, SiLU, down-projection, and the output of a kept
    token as the residual plus the confidence-weighted expert output; a dropped
    token leaves the layer unchanged.
  * "Some Tokens Do Not Get In" (getbasislab.com), sections "Why there is a buffer"
    and "Past the edge": t*k token slots, one fixed buffer per expert sized by the
    capacity factor, tokens placed in some order, overflow tokens take the residual
    path and reach the next layer exactly as they entered.
  * "Dynamic Token Routing AI" (freenetmedia.pl), "How it works": a gating network
    scores each token and selects the expert(s).
  * "Token Routing Optimization in Batch Processing" (subtext diagram): a Token Scheduler
    that regroups the tokens of several batches, leaving each token's routing unchanged, so
    that each new batch activates fewer experts with more tokens per active expert.
  * The fused-MoE flow diagram (monishver11.github.io, moe-vllm flow): the dropless
    pair-order flow (GEMM 1 reads token row p // top_k and writes pair row p, GEMM 2
    scales pair row p by its top-k weight, moe_sum adds a token's top_k consecutive
    rows) and the gated expert (GEMM 1 of width 2 d_ff, then SiLU x mul).

Where the pages leave a step open, the reading taken is stated in the docstring of
the function that takes it (softmax over all experts, unrenormalised top-k gates,
fill order gate-descending then token then choice, float64 logits of exact products).

Every floating-point input is taken as float64 holding the exact value of the stored
(bf16 or fp32) number; the caller does that conversion.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "capacity",
    "router_logits",
    "softmax",
    "gates_fp32",
    "top_k",
    "route",
    "dispatch",
    "silu",
    "expert_ffn",
    "expert_ffn_slots",
    "combine",
    "forward",
    "expert_ffn_gated",
    "expert_ffn_slots_gated",
    "forward_gated",
    "dispatch_padded",
    "expert_ffn_padded",
    "forward_padded",
    "forward_with_routing",
    "dispatch_pairs",
    "moe_sum",
    "forward_dropless_with_routing",
    "forward_dropless",
    "forward_dropless_gated",
    "schedule_batches",
    "active_experts",
    "forward_batches",
]


def capacity(T: int, top_k: int, n_experts: int, capacity_factor: float) -> int:
    """Per-expert slot budget: floor(C * T * k / E), computed as an exact rational.

    Worked Example (capacity paragraph): C = 1.25, 8 tokens over 4 experts gives 2.5,
    which is rounded down to 2.  "Some Tokens Do Not Get In", "Why there is a buffer":
    the number of slots to fill is t times k, spread over the experts with slack set by
    the capacity factor.  No lower clamp: the budget may be 0.
    """
    if T < 0 or top_k < 1 or n_experts < 1 or capacity_factor < 0:
        raise ValueError("bad capacity arguments")
    return math.floor(Fraction(capacity_factor) * T * top_k / n_experts)


def router_logits(x: np.ndarray, w_router: np.ndarray, b_router: np.ndarray | None) -> np.ndarray:
    """Router scores L[t, e] = sum_j x[t, j] * W_r[e, j] + b_r[e], in float64.

    "Dynamic Token Routing AI", "How it works": the gating network scores each token.
    The pages leave the score function open; it is read as a linear map plus an
    optional per-expert bias.  Products of two bf16 or two fp32 values are exact in
    float64, so only the summation rounds.
    """
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if b_router is not None:
        L = L + np.asarray(b_router, dtype=np.float64)[None, :]
    return L


def softmax(L: np.ndarray) -> np.ndarray:
    """Row-wise softmax over all experts, float64: exp(L - max) / sum(exp(L - max)).

    The pages call the gate a router confidence (Worked Example, trace of token 0); it is
    read as the softmax probability over all E experts.
    """
    m = L.max(axis=1, keepdims=True)
    z = np.exp(L - m)
    return z / z.sum(axis=1, keepdims=True)


def gates_fp32(p: np.ndarray) -> np.ndarray:
    """Round the float64 probabilities once to float32 (round to nearest even)."""
    return p.astype(np.float32)


def top_k(g32: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Pick the k experts with the largest fp32 gate; ties go to the lower expert index.

    Choice c = 0 is the largest gate.  The gate values are returned as they are, with no
    renormalisation over the chosen k (the Worked Example scales the expert output by the
    router confidence itself).
    """
    T, E = g32.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, E]")
    e_idx = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> descending gate, then ascending expert index
    order = np.lexsort((e_idx, -g32.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    gates = np.take_along_axis(g32, ids, axis=1).astype(np.float32)
    return ids, gates


def route(x, w_router, b_router, k):
    """Router step: logits, softmax probabilities, fp32 gates, top-k ids and gates."""
    L = router_logits(x, w_router, b_router)
    p = softmax(L)
    g32 = gates_fp32(p)
    ids, gates = top_k(g32, k)
    return {"logits": L, "probs": p, "gates_all": g32, "ids": ids, "gates": gates}


def dispatch(ids: np.ndarray, gates: np.ndarray, n_experts: int, cap: int) -> dict:
    """Fill each expert's fixed buffer and mark the overflow as dropped.

    Worked Example (capacity paragraph): the token with the lowest router confidence among
    an overloaded expert's tokens is the one that does not fit.  "Some Tokens Do Not Get
    In", "Past the edge": tokens take their expert's slots in some order and the first one
    to find the buffer full is turned away.  The order is read as: gate descending, then
    token index ascending, then choice rank ascending, over all choice ranks together.

    Slots are numbered compactly: expert e owns slots [off[e], off[e] + kept[e]) with
    off[e] = sum of kept[e'] for e' < e, and the assignment of rank r gets slot off[e] + r.
    """
    T, k = ids.shape
    per_expert: list[list[tuple[float, int, int]]] = [[] for _ in range(n_experts)]
    for t in range(T):
        for c in range(k):
            e = int(ids[t, c])
            if not 0 <= e < n_experts:
                raise ValueError(f"expert id {e} out of range")
            per_expert[e].append((float(gates[t, c]), t, c))

    counts = np.array([len(a) for a in per_expert], dtype=np.int32)
    kept = np.minimum(counts, cap).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(kept)

    slot_of = np.full((T, k), -1, dtype=np.int32)
    rank = np.full((T, k), -1, dtype=np.int64)
    row_token = np.full(int(offsets[-1]), -1, dtype=np.int32)
    for e in range(n_experts):
        ordered = sorted(per_expert[e], key=lambda a: (-a[0], a[1], a[2]))
        for r, (_, t, c) in enumerate(ordered):
            rank[t, c] = r
            if r < cap:
                s = int(offsets[e]) + r
                slot_of[t, c] = s
                row_token[s] = t
    drop_mask = (slot_of < 0).astype(np.uint8)
    return {
        "counts": counts,
        "kept": kept,
        "offsets": offsets,
        "slot_of": slot_of,
        "rank": rank,
        "row_token": row_token,
        "drop_mask": drop_mask,
        "n_kept": int(offsets[-1]),
    }


def silu(h: np.ndarray) -> np.ndarray:
    """SiLU(h) = h * sigmoid(h), evaluated without overflow for large |h|."""
    h = np.asarray(h, dtype=np.float64)
    e = np.exp(-np.abs(h))
    sig = np.where(h >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return h * sig


def expert_ffn(x_rows: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray) -> np.ndarray:
    """One expert on a batch of rows: y = W2 . SiLU(W1 . x + b1) + b2, float64.

    Worked Example (trace of token 0): up-projection d_model -> d_ff with bias, SiLU
    element-wise, down-projection d_ff -> d_model with bias.  W1 is [d_ff, d_model] and W2
    is [d_model, d_ff], so W1 . x is the matrix-vector product the trace writes.
    """
    h = x_rows @ np.asarray(w1, dtype=np.float64).T + np.asarray(b1, dtype=np.float64)[None, :]
    a = silu(h)
    return a @ np.asarray(w2, dtype=np.float64).T + np.asarray(b2, dtype=np.float64)[None, :]


def expert_ffn_slots(x, row_token, offsets, w1, b1, w2, b2, slots=None) -> np.ndarray:
    """Expert outputs per slot: Y[s] = FFN_e(x[row_token[s]]) for the expert e owning slot s.

    With `slots` given, only those slots are computed (in the given order); this is what the
    large configurations use to check sampled rows.  Weights are indexed per expert, so a
    caller may pass lazily converted per-expert arrays (anything supporting w1[e]).
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    n_kept = int(offsets[-1])
    if slots is None:
        slots = np.arange(n_kept)
    slots = np.asarray(slots, dtype=np.int64)
    d = x.shape[1]
    out = np.zeros((len(slots), d), dtype=np.float64)
    expert_of = np.searchsorted(offsets, slots, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if len(sel) == 0:
            continue
        rows = np.asarray(x, dtype=np.float64)[np.asarray(row_token)[slots[sel]]]
        out[sel] = expert_ffn(rows, w1[e], b1[e], w2[e], b2[e])
    return out


def combine(x: np.ndarray, gates: np.ndarray, slot_of: np.ndarray, Y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """out[t] = x[t] + sum over kept choices c (ascending) of gates[t, c] * Y[slot_of[t, c]].

    Worked Example: a kept token's output is its residual plus the confidence-scaled
    expert output; the dropped token's output is its input plus nothing.  With k > 1 the
    kept choices are summed and the gates are not renormalised when some choice drops.
    Returns the float64 output and a mask of tokens with no kept choice; for those rows
    the layer output is the input itself, bit for bit ("Past the edge": the token reaches
    the next layer exactly as it entered).
    """
    x64 = np.asarray(x, dtype=np.float64)
    out = x64.copy()
    T, k = slot_of.shape
    for c in range(k):
        kept = slot_of[:, c] >= 0
        if np.any(kept):
            out[kept] = out[kept] + gates[kept, c].astype(np.float64)[:, None] * Y[slot_of[kept, c]]
    all_dropped = np.all(slot_of < 0, axis=1)
    return out, all_dropped


def forward_with_routing(x, ids, gates, cap, n_experts, w1, b1, w2, b2) -> dict:
    """Layer forward from a given routing (ids, gates): dispatch, expert FFN, combine."""
    disp = dispatch(ids, gates, n_experts, cap)
    Y = expert_ffn_slots(x, disp["row_token"], disp["offsets"], w1, b1, w2, b2)
    out, all_dropped = combine(x, gates, disp["slot_of"], Y)
    res = dict(disp)
    res.update({"ids": ids, "gates": gates, "cap": cap, "Y": Y, "out": out, "all_dropped": all_dropped})
    return res


def forward(x, w_router, b_router, w1, b1, w2, b2, k: int, capacity_factor: float) -> dict:
    """Whole layer: route, capacity, dispatch, expert FFN, combine."""
    T = x.shape[0]
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    cap = capacity(T, k, E, capacity_factor)
    res = forward_with_routing(x, r["ids"], r["gates"], cap, E, w1, b1, w2, b2)
    res.update({"logits": r["logits"], "probs": r["probs"], "gates_all": r["gates_all"]})
    return res


def dispatch_padded(ids: np.ndarray, gates: np.ndarray, n_experts: int, cap: int) -> dict:
    """The fixed per-expert buffers themselves ("Some Tokens Do Not Get In", "Why there is a
    buffer": every expert gets a buffer of `cap` token slots whether it fills it or not).

    Expert e's buffer is rows e*cap .. e*cap + cap - 1; its r-th kept assignment in the fill
    order (the ranking of `dispatch`) sits in row e*cap + r; rows past its kept count are
    empty (token -1).  Returns slot_of [T, k] (buffer row or -1) and row_token [E*cap]."""
    d = dispatch(ids, gates, n_experts, cap)
    T, k = ids.shape
    slot_of = np.full((T, k), -1, dtype=np.int64)
    row_token = np.full(n_experts * cap, -1, dtype=np.int64)
    for t in range(T):
        for c in range(k):
            s = int(d["slot_of"][t, c])
            if s < 0:
                continue
            e = int(ids[t, c])
            r = s - int(d["offsets"][e])
            slot_of[t, c] = e * cap + r
            row_token[e * cap + r] = t
    return {"slot_of": slot_of, "row_token": row_token, "counts": d["counts"],
            "n_kept": d["n_kept"], "compact": d}


def expert_ffn_padded(x, row_token, n_experts, cap, w1, b1, w2, b2, rows=None) -> np.ndarray:
    """Expert output of every buffer row (or of the listed `rows`): FFN_e of the row's token,
    and of an all-zero input row for an empty slot, which the fixed buffer computes anyway."""
    row_token = np.asarray(row_token)
    if rows is None:
        rows = np.arange(n_experts * cap)
    rows = np.asarray(rows, dtype=np.int64)
    d = x.shape[1]
    out = np.zeros((len(rows), d), dtype=np.float64)
    if cap == 0 or len(rows) == 0:
        return out
    expert_of = rows // cap
    for e in range(n_experts):
        sel = np.nonzero(expert_of == e)[0]
        if len(sel) == 0:
            continue
        tok = row_token[rows[sel]]
        inp = np.zeros((len(sel), d), dtype=np.float64)
        has = tok >= 0
        inp[has] = np.asarray(x, dtype=np.float64)[tok[has]]
        out[sel] = expert_ffn(inp, w1[e], b1[e], w2[e], b2[e])
    return out


def forward_padded(x, w_router, b_router, w1, b1, w2, b2, k: int, capacity_factor: float) -> dict:
    """Whole layer with the fixed buffers computed whole: route, capacity, fill the buffers,
    expert FFN of every buffer row, combine from the buffer rows.  The output is the layer's
    output (empty rows are never combined); Y holds every buffer row."""
    T = x.shape[0]
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    cap = capacity(T, k, E, capacity_factor)
    d = dispatch_padded(r["ids"], r["gates"], E, cap)
    Y = expert_ffn_padded(x, d["row_token"], E, cap, w1, b1, w2, b2)
    out, all_dropped = combine(x, r["gates"], d["slot_of"], Y)
    return {"ids": r["ids"], "gates": r["gates"], "cap": cap, "slot_of": d["slot_of"],
            "row_token": d["row_token"], "counts": d["counts"], "Y": Y, "out": out,
            "all_dropped": all_dropped}


def expert_ffn_gated(x_rows: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Gated expert of the fused-MoE flow diagram (moe-vllm flow): GEMM 1 writes 2f values
    per row, the SiLU x mul box turns them into f, GEMM 2 follows; no biases are drawn.
    Reading taken: the first f outputs of GEMM 1 are the gate, the last f the up projection.

        g = W_gate x,  u = W_up x,  a = SiLU(g) * u,  y = W2 a
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    f = w13.shape[0] // 2
    g = x_rows @ w13[:f].T
    u = x_rows @ w13[f:].T
    a = silu(g) * u
    return a @ np.asarray(w2, dtype=np.float64).T


def expert_ffn_slots_gated(x, row_token, offsets, w13, w2, slots=None) -> np.ndarray:
    """expert_ffn_slots with the gated expert."""
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    if slots is None:
        slots = np.arange(int(offsets[-1]))
    slots = np.asarray(slots, dtype=np.int64)
    out = np.zeros((len(slots), x.shape[1]), dtype=np.float64)
    expert_of = np.searchsorted(offsets, slots, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if len(sel):
            rows = np.asarray(x, dtype=np.float64)[np.asarray(row_token)[slots[sel]]]
            out[sel] = expert_ffn_gated(rows, w13[e], w2[e])
    return out


def forward_gated(x, w_router, b_router, w13, w2, k: int, capacity_factor: float) -> dict:
    """Whole layer with gated experts: route, capacity, dispatch, gated expert FFN, combine."""
    T = x.shape[0]
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    cap = capacity(T, k, E, capacity_factor)
    disp = dispatch(r["ids"], r["gates"], E, cap)
    Y = expert_ffn_slots_gated(x, disp["row_token"], disp["offsets"], w13, w2)
    out, all_dropped = combine(x, r["gates"], disp["slot_of"], Y)
    res = dict(disp)
    res.update({"ids": r["ids"], "gates": r["gates"], "cap": cap, "Y": Y, "out": out,
                "all_dropped": all_dropped, "logits": r["logits"], "probs": r["probs"],
                "gates_all": r["gates_all"]})
    return res


# ----------------------------------------------------------------------------- dropless flow
def dispatch_pairs(ids: np.ndarray, n_experts: int) -> dict:
    """Group the (token, choice) pairs by expert with no capacity at all.

    Fused-MoE flow diagram (moe-vllm flow), note on the GEMM boxes: both GEMMs walk a list
    of pair indices sorted by expert, so every block of rows uses one expert's weights.
    Pair p = t * top_k + c is the c-th choice of token t (the diagram's pair order).
    Reading taken: within an expert the pairs keep ascending p (a stable sort by expert).

    Returns counts [E], offsets [E+1] (exclusive prefix of the counts), sorted_pairs [T*k]
    (expert e's pairs at offsets[e] .. offsets[e+1] - 1) and row_token = sorted_pairs // k,
    the token row GEMM 1 reads for each of them.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if np.any((flat < 0) | (flat >= n_experts)):
        raise ValueError("expert id out of range")
    groups = [np.nonzero(flat == e)[0] for e in range(n_experts)]  # ascending p
    counts = np.array([len(g) for g in groups], dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = (np.concatenate(groups) if groups else np.zeros(0, np.int64)).astype(np.int32)
    return {"counts": counts, "offsets": offsets, "sorted_pairs": sorted_pairs,
            "row_token": (sorted_pairs // k).astype(np.int32)}


def moe_sum(rows: np.ndarray, k: int, residual: np.ndarray | None = None) -> np.ndarray:
    """moe_sum box of the flow diagram: token t's output is the sum of pair rows
    t*k .. t*k + k - 1 (pair order back to token order), plus the residual when given."""
    rows = np.asarray(rows, dtype=np.float64)
    T = rows.shape[0] // k
    out = np.zeros((T, rows.shape[1])) if residual is None else np.asarray(residual, np.float64).copy()
    for t in range(T):
        for c in range(k):
            out[t] = out[t] + rows[t * k + c]
    return out


def forward_dropless_with_routing(x, ids, gates, n_experts, expert) -> dict:
    """Dropless pair-order flow from a given routing; `expert(e, x_rows)` is one expert on a
    batch of token rows.

    Fused-MoE flow diagram: GEMM 1 reads token row p // top_k and writes pair row p; every
    step up to GEMM 2 stays in pair order; GEMM 2 writes pair row p multiplied by
    topk_weights[p]; moe_sum adds the top_k rows of each token.  No pair is ever dropped.
    Reading taken: the layer's output adds the residual as the worked example's tokens do
    (x plus the confidence-weighted expert outputs), so with capacity for every pair this is
    the capacity layer's output; the top-k weights are the unrenormalised gates.
    """
    x64 = np.asarray(x, dtype=np.float64)
    T, k = ids.shape
    disp = dispatch_pairs(ids, n_experts)
    weights = np.asarray(gates, dtype=np.float64).reshape(-1)  # topk_weights[p]
    rows = np.zeros((T * k, x64.shape[1]))                      # cache3, pair order
    off = disp["offsets"]
    for e in range(n_experts):
        pairs = disp["sorted_pairs"][off[e]:off[e + 1]].astype(np.int64)
        if len(pairs) == 0:
            continue
        y = expert(e, x64[pairs // k])           # GEMM 1 reads row p // top_k ... GEMM 2
        rows[pairs] = weights[pairs][:, None] * y  # GEMM 2 writes row p, times topk_weights[p]
    out = moe_sum(rows, k, residual=x64)
    res = dict(disp)
    res.update({"ids": ids, "gates": gates, "pair_rows": rows, "out": out})
    return res


def forward_dropless(x, w_router, b_router, w1, b1, w2, b2, k: int) -> dict:
    """Whole dropless layer with the plain expert (up-projection, SiLU, down-projection)."""
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    res = forward_dropless_with_routing(
        x, r["ids"], r["gates"], E, lambda e, rows: expert_ffn(rows, w1[e], b1[e], w2[e], b2[e]))
    res.update({"logits": r["logits"], "probs": r["probs"], "gates_all": r["gates_all"]})
    return res


def forward_dropless_gated(x, w_router, b_router, w13, w2, k: int) -> dict:
    """Whole dropless layer with the gated expert: the flow diagram end to end."""
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    res = forward_dropless_with_routing(
        x, r["ids"], r["gates"], E, lambda e, rows: expert_ffn_gated(rows, w13[e], w2[e]))
    res.update({"logits": r["logits"], "probs": r["probs"], "gates_all": r["gates_all"]})
    return res


# ----------------------------------------------------------------------------- batch consolidation
def active_experts(ids: np.ndarray, batches) -> np.ndarray:
    """Number of distinct experts the tokens of each batch are routed to (the experts a batch
    "activates" in the Token Routing Optimization diagram)."""
    ids = np.asarray(ids)
    return np.array([len({int(e) for t in b for e in ids[t]}) for b in batches], dtype=np.int32)


def schedule_batches(ids: np.ndarray, batch_size: int) -> dict:
    """Token Scheduler of "Token Routing Optimization in Batch Processing" (subtext diagram).

    The diagram keeps token-level routing as it is and changes only which tokens travel
    together: two batches that each activate every expert with one token per expert become two
    batches that each activate half the experts with two tokens per expert.  The pages give no
    algorithm; the reading taken is the plainest one that reproduces the diagram: order the
    tokens by the set of experts they are routed to (their k ids sorted ascending, compared as
    tuples), ties by token index, and cut the ordered list into consecutive batches of the
    original size.  Tokens sharing an expert set then travel together.

    ids [T, k] with T a multiple of batch_size.  Returns order [T] (new position -> token),
    the new and the original batches (lists of token arrays), and their active-expert counts.
    """
    ids = np.asarray(ids)
    T = ids.shape[0]
    if batch_size < 1 or T % batch_size:
        raise ValueError("the pool must hold whole batches")
    keys = [tuple(sorted(int(e) for e in ids[t])) for t in range(T)]
    order = np.array(sorted(range(T), key=lambda t: (keys[t], t)), dtype=np.int32)
    M = T // batch_size
    new = [order[b * batch_size:(b + 1) * batch_size] for b in range(M)]
    orig = [np.arange(b * batch_size, (b + 1) * batch_size) for b in range(M)]
    return {"order": order, "batches": new, "orig_batches": orig,
            "active": active_experts(ids, new), "orig_active": active_experts(ids, orig)}


def forward_batches(x, w_router, b_router, w1, b1, w2, b2, k: int, capacity_factor: float,
                    batch_size: int, consolidate: bool) -> dict:
    """A pool of batches through the capacity layer, one batch at a time: route every token
    (routing is per token, so it does not depend on the batch), regroup the batches with
    schedule_batches when `consolidate`, then run dispatch, expert FFN and combine on each
    batch with the capacity of a batch of batch_size tokens.  out is in the pool's token
    order.  With a capacity of at least batch_size nothing can drop, and the output does not
    depend on the grouping."""
    T = x.shape[0]
    E = w_router.shape[0]
    r = route(x, w_router, b_router, k)
    sched = schedule_batches(r["ids"], batch_size)
    batches = sched["batches"] if consolidate else sched["orig_batches"]
    cap = capacity(batch_size, k, E, capacity_factor)
    x64 = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x64)
    n_kept = 0
    for b in batches:
        res = forward_with_routing(x64[b], r["ids"][b], r["gates"][b], cap, E, w1, b1, w2, b2)
        out[b] = res["out"]
        n_kept += res["n_kept"]
    return {"ids": r["ids"], "gates": r["gates"], "logits": r["logits"], "probs": r["probs"],
            "gates_all": r["gates_all"], "order": sched["order"], "batches": batches,
            "active": sched["active"] if consolidate else sched["orig_active"],
            "cap": cap, "n_kept": n_kept, "out": out}
