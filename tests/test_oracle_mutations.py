"""Plant plausible mistakes in copies of the oracle's steps; each must fail some pin.

This shows the pins in tests/pins.py are strong enough that a dropped term, a wrong sign,
a wrong index or a transposed operand in the oracle would not go unnoticed.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle.moe_oracle as O
import pins

_orig = {name: getattr(O, name) for name in O.__all__}


def _cap_ceil(T, k, E, C):
    return math.ceil(Fraction(C) * T * k / E)


def _cap_no_k(T, k, E, C):
    return math.floor(Fraction(C) * T / E)


def _cap_float(T, k, E, C):
    return math.floor(C * T * k / E)


def _logits_transposed(x, w, b):
    L = np.asarray(x, np.float64) @ np.asarray(w, np.float64)
    return L + np.asarray(b)[None, :] if b is not None else L


def _logits_no_bias(x, w, b):
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def _softmax_no_norm(L):
    return np.exp(L - L.max(axis=1, keepdims=True))


def _softmax_wrong_axis(L):
    z = np.exp(L - L.max(axis=1, keepdims=True))
    return z / z.sum(axis=0, keepdims=True)


def _topk_tie_high(g32, k):
    T, E = g32.shape
    e_idx = np.broadcast_to(-np.arange(E), (T, E))
    order = np.lexsort((e_idx, -g32.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    return ids, np.take_along_axis(g32, ids, axis=1)


def _gates_unrounded(p):
    return np.asarray(p, np.float64)  # top-k on the float64 probabilities


def _topk_renorm(g32, k):
    ids, gates = _orig["top_k"](g32, k)
    return ids, (gates / gates.sum(axis=1, keepdims=True)).astype(np.float32)


def _topk_ascending(g32, k):
    T, E = g32.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), g32.astype(np.float64)), axis=1)
    ids = order[:, :k].astype(np.int32)
    return ids, np.take_along_axis(g32, ids, axis=1)


def _make_dispatch(sort_key=None, offsets_from_counts=False, keep_rule=None):
    def dispatch(ids, gates, n_experts, cap):
        T, k = ids.shape
        per = [[] for _ in range(n_experts)]
        for t in range(T):
            for c in range(k):
                per[int(ids[t, c])].append((float(gates[t, c]), t, c))
        counts = np.array([len(a) for a in per], dtype=np.int32)
        kept = np.minimum(counts, cap)
        offsets = np.zeros(n_experts + 1, dtype=np.int32)
        offsets[1:] = np.cumsum(counts if offsets_from_counts else kept)
        slot_of = np.full((T, k), -1, dtype=np.int32)
        row_token = np.full(int(offsets[-1]), -1, dtype=np.int32)
        for e in range(n_experts):
            ordered = sorted(per[e], key=sort_key or (lambda a: (-a[0], a[1], a[2])))
            for r, (_, t, c) in enumerate(ordered):
                if (keep_rule or (lambda r, cap: r < cap))(r, cap):
                    s = int(offsets[e]) + r
                    slot_of[t, c] = s
                    if s < len(row_token):
                        row_token[s] = t
        return {"counts": counts, "kept": kept, "offsets": offsets, "slot_of": slot_of,
                "rank": None, "row_token": row_token, "drop_mask": (slot_of < 0).astype(np.uint8),
                "n_kept": int(offsets[-1])}
    return dispatch


def _silu_sigmoid(h):
    return 1.0 / (1.0 + np.exp(-np.asarray(h, np.float64)))


def _silu_relu(h):
    return np.maximum(np.asarray(h, np.float64), 0.0)


def _silu_sign(h):
    h = np.asarray(h, np.float64)
    return h / (1.0 + np.exp(h))


def _ffn_no_b1(x, w1, b1, w2, b2):
    return O.silu(x @ np.asarray(w1).T) @ np.asarray(w2).T + np.asarray(b2)[None, :]


def _ffn_no_b2(x, w1, b1, w2, b2):
    return O.silu(x @ np.asarray(w1).T + np.asarray(b1)[None, :]) @ np.asarray(w2).T


def _ffn_act_after_down(x, w1, b1, w2, b2):
    return O.silu((x @ np.asarray(w1).T + np.asarray(b1)[None, :]) @ np.asarray(w2).T + np.asarray(b2)[None, :])


def _combine_no_residual(x, gates, slot_of, Y):
    out, dropped = _orig["combine"](np.zeros_like(np.asarray(x, np.float64)), gates, slot_of, Y)
    out[dropped] = np.asarray(x, np.float64)[dropped]
    return out, dropped


def _combine_first_gate(x, gates, slot_of, Y):
    g = np.repeat(gates[:, :1], gates.shape[1], axis=1)
    return _orig["combine"](x, g, slot_of, Y)


def _combine_no_gate(x, gates, slot_of, Y):
    return _orig["combine"](x, np.ones_like(gates), slot_of, Y)


def _combine_signed(x, gates, slot_of, Y):
    return _orig["combine"](x, -gates, slot_of, Y)


def _combine_plus_zero(x, gates, slot_of, Y):
    out, dropped = _orig["combine"](x, gates, slot_of, Y)
    return out + 0.0, dropped  # turns -0.0 into +0.0 on the residual path


def _ffn_padded_minus_one_index(x, row_token, n_experts, cap, w1, b1, w2, b2, rows=None):
    # an empty slot's -1 used as an index: the last token's row instead of a zero row
    if rows is None:
        rows = np.arange(n_experts * cap)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), x.shape[1]))
    for j, r in enumerate(rows):
        e = r // cap
        out[j] = O.expert_ffn(np.asarray(x, np.float64)[[row_token[r]]], w1[e], b1[e], w2[e], b2[e])[0]
    return out


def _dispatch_padded_reversed(ids, gates, n_experts, cap):
    d = _orig["dispatch_padded"](ids, gates, n_experts, cap)
    rt = d["row_token"].copy()
    so = d["slot_of"].copy()
    for e in range(n_experts):
        blk = rt[e * cap:(e + 1) * cap]
        n = int((blk >= 0).sum())
        rt[e * cap:e * cap + n] = blk[:n][::-1]
    for t in range(so.shape[0]):
        for c in range(so.shape[1]):
            s = so[t, c]
            if s >= 0:
                e = s // cap
                n = int((d["row_token"][e * cap:(e + 1) * cap] >= 0).sum())
                so[t, c] = e * cap + (n - 1 - (s - e * cap))
    d.update(row_token=rt, slot_of=so)
    return d


def _dispatch_padded_compact_rows(ids, gates, n_experts, cap):
    # buffer rows at the compact offsets instead of e * cap
    d = _orig["dispatch_padded"](ids, gates, n_experts, cap)
    comp = d["compact"]
    rt = np.full(n_experts * cap, -1, dtype=np.int64)
    n = int(comp["n_kept"])
    rt[:n] = comp["row_token"][:n]
    d.update(row_token=rt, slot_of=comp["slot_of"].astype(np.int64))
    return d


def _gated_halves_swapped(x_rows, w13, w2):
    f = np.asarray(w13).shape[0] // 2
    return _orig["expert_ffn_gated"](x_rows, np.concatenate([w13[f:], w13[:f]]), w2)


def _gated_no_up(x_rows, w13, w2):
    f = np.asarray(w13).shape[0] // 2
    x_rows = np.asarray(x_rows, np.float64)
    return O.silu(x_rows @ np.asarray(w13)[:f].T) @ np.asarray(w2).T


def _gated_silu_after_mul(x_rows, w13, w2):
    f = np.asarray(w13).shape[0] // 2
    x_rows = np.asarray(x_rows, np.float64)
    return O.silu((x_rows @ np.asarray(w13)[:f].T) * (x_rows @ np.asarray(w13)[f:].T)) @ np.asarray(w2).T


def _pairs_descending(ids, n_experts):
    d = _orig["dispatch_pairs"](ids, n_experts)
    sp = d["sorted_pairs"].copy()
    for e in range(n_experts):
        sp[d["offsets"][e]:d["offsets"][e + 1]] = sp[d["offsets"][e]:d["offsets"][e + 1]][::-1]
    d.update(sorted_pairs=sp, row_token=sp // ids.shape[1])
    return d


def _pairs_row_mod(ids, n_experts):
    d = _orig["dispatch_pairs"](ids, n_experts)
    d.update(row_token=d["sorted_pairs"] % ids.shape[1])
    return d


def _moe_sum_token_major(rows, k, residual=None):
    # rows taken as [k, T] (choice-major) instead of pair order t*k + c
    rows = np.asarray(rows, np.float64)
    T = rows.shape[0] // k
    out = np.zeros((T, rows.shape[1])) if residual is None else np.asarray(residual, np.float64).copy()
    for t in range(T):
        for c in range(k):
            out[t] = out[t] + rows[c * T + t]
    return out


def _moe_sum_no_residual(rows, k, residual=None):
    return _orig["moe_sum"](rows, k)


def _make_dropless(read_row=None, weight=True, weight_by_position=False):
    def fwd(x, ids, gates, n_experts, expert):
        x64 = np.asarray(x, np.float64)
        T, k = ids.shape
        disp = O.dispatch_pairs(ids, n_experts)
        wts = np.asarray(gates, np.float64).reshape(-1)
        rows = np.zeros((T * k, x64.shape[1]))
        off = disp["offsets"]
        for e in range(n_experts):
            pairs = disp["sorted_pairs"][off[e]:off[e + 1]].astype(np.int64)
            if len(pairs) == 0:
                continue
            src = (read_row or (lambda p, k: p // k))(pairs, k)
            y = expert(e, x64[src])
            if weight:
                w = wts[np.arange(off[e], off[e + 1])] if weight_by_position else wts[pairs]
                y = w[:, None] * y
            rows[pairs] = y
        out = O.moe_sum(rows, k, residual=x64)
        res = dict(disp)
        res.update({"ids": ids, "gates": gates, "pair_rows": rows, "out": out})
        return res
    return fwd


def _sched_choice_order(ids, batch_size):
    # keys in choice order instead of as sets: (a, b) and (b, a) are kept apart
    ids = np.asarray(ids)
    T = ids.shape[0]
    order = np.array(sorted(range(T), key=lambda t: (tuple(int(e) for e in ids[t]), t)), np.int32)
    M = T // batch_size
    new = [order[j * batch_size:(j + 1) * batch_size] for j in range(M)]
    orig = [np.arange(j * batch_size, (j + 1) * batch_size) for j in range(M)]
    return {"order": order, "batches": new, "orig_batches": orig,
            "active": O.active_experts(ids, new), "orig_active": O.active_experts(ids, orig)}


def _sched_no_tiebreak(ids, batch_size):
    # equal expert sets in descending token order
    d = _orig["schedule_batches"](ids, batch_size)
    ids = np.asarray(ids)
    T = ids.shape[0]
    keys = [tuple(sorted(int(e) for e in ids[t])) for t in range(T)]
    order = np.array(sorted(range(T), key=lambda t: (keys[t], -t)), np.int32)
    new = [order[j * batch_size:(j + 1) * batch_size] for j in range(T // batch_size)]
    d.update(order=order, batches=new, active=O.active_experts(ids, new))
    return d


def _sched_round_robin(ids, batch_size):
    # deal the ordered tokens round-robin over the batches instead of in consecutive runs
    d = _orig["schedule_batches"](ids, batch_size)
    M = len(d["batches"])
    new = [d["order"][j::M] for j in range(M)]
    d.update(batches=new, active=O.active_experts(ids, new))
    return d


def _active_counts_assignments(ids, batches):
    return np.array([len([e for t in b for e in np.asarray(ids)[t]]) for b in batches], np.int32)


def _batches_pool_capacity(x, w_router, b_router, w1, b1, w2, b2, k, C, batch_size, consolidate):
    # the capacity of the whole pool applied to every batch
    res = _orig["forward_batches"](x, w_router, b_router, w1, b1, w2, b2, k, C, batch_size,
                                   consolidate)
    T, E = x.shape[0], w_router.shape[0]
    cap = O.capacity(T, k, E, C)
    out = np.zeros_like(res["out"])
    for b in res["batches"]:
        out[b] = O.forward_with_routing(x[b], res["ids"][b], res["gates"][b], cap, E, w1, b1, w2,
                                        b2)["out"]
    res.update(out=out, cap=cap)
    return res


MUTATIONS = {
    "schedule_keys_in_choice_order": {"schedule_batches": _sched_choice_order},
    "schedule_ties_descending": {"schedule_batches": _sched_no_tiebreak},
    "schedule_round_robin_batches": {"schedule_batches": _sched_round_robin},
    "active_counts_assignments": {"active_experts": _active_counts_assignments},
    "batches_use_pool_capacity": {"forward_batches": _batches_pool_capacity},
    "pairs_descending_within_expert": {"dispatch_pairs": _pairs_descending},
    "pairs_row_token_mod_k": {"dispatch_pairs": _pairs_row_mod},
    "moe_sum_choice_major_rows": {"moe_sum": _moe_sum_token_major},
    "moe_sum_drops_residual": {"moe_sum": _moe_sum_no_residual},
    "dropless_reads_row_p_mod_k": {
        "forward_dropless_with_routing": _make_dropless(read_row=lambda p, k: p % k)},
    "dropless_unweighted_rows": {"forward_dropless_with_routing": _make_dropless(weight=False)},
    "dropless_weight_by_sorted_position": {
        "forward_dropless_with_routing": _make_dropless(weight_by_position=True)},
    "gated_halves_swapped": {"expert_ffn_gated": _gated_halves_swapped},
    "gated_up_dropped": {"expert_ffn_gated": _gated_no_up},
    "gated_silu_after_product": {"expert_ffn_gated": _gated_silu_after_mul},
    "padded_empty_slot_uses_last_token": {"expert_ffn_padded": _ffn_padded_minus_one_index},
    "padded_buffer_order_reversed": {"dispatch_padded": _dispatch_padded_reversed},
    "padded_rows_at_compact_offsets": {"dispatch_padded": _dispatch_padded_compact_rows},
    "capacity_ceil": {"capacity": _cap_ceil},
    "capacity_without_k": {"capacity": _cap_no_k},
    "capacity_float_arith": {"capacity": _cap_float},
    "router_transposed_operand": {"router_logits": _logits_transposed},
    "router_dropped_bias": {"router_logits": _logits_no_bias},
    "softmax_no_denominator": {"softmax": _softmax_no_norm},
    "softmax_wrong_axis": {"softmax": _softmax_wrong_axis},
    "gates_not_rounded_to_fp32": {"gates_fp32": _gates_unrounded},
    "topk_ties_to_higher_expert": {"top_k": _topk_tie_high},
    "topk_renormalised": {"top_k": _topk_renorm},
    "topk_smallest": {"top_k": _topk_ascending},
    "fill_ascending_gate": {"dispatch": _make_dispatch(sort_key=lambda a: (a[0], a[1], a[2]))},
    "fill_ties_late_token_first": {"dispatch": _make_dispatch(sort_key=lambda a: (-a[0], -a[1], a[2]))},
    "fill_choice_before_token": {"dispatch": _make_dispatch(sort_key=lambda a: (-a[0], a[2], a[1]))},
    "fill_token_order_only": {"dispatch": _make_dispatch(sort_key=lambda a: (a[1], a[2]))},
    "offsets_from_counts": {"dispatch": _make_dispatch(offsets_from_counts=True)},
    "keep_off_by_one": {"dispatch": _make_dispatch(keep_rule=lambda r, cap: r <= cap)},
    "silu_is_sigmoid": {"silu": _silu_sigmoid},
    "silu_is_relu": {"silu": _silu_relu},
    "silu_sign_flip": {"silu": _silu_sign},
    "ffn_dropped_b1": {"expert_ffn": _ffn_no_b1},
    "ffn_dropped_b2": {"expert_ffn": _ffn_no_b2},
    "ffn_activation_misplaced": {"expert_ffn": _ffn_act_after_down},
    "combine_no_residual": {"combine": _combine_no_residual},
    "combine_first_gate_for_all": {"combine": _combine_first_gate},
    "combine_ignores_gate": {"combine": _combine_no_gate},
    "combine_negated_gate": {"combine": _combine_signed},
    "combine_plus_zero": {"combine": _combine_plus_zero},
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name].items():
        monkeypatch.setattr(O, attr, fn)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(O)
        except Exception:  # an assertion or a crash: either way the mistake shows
            failed.append(check.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
