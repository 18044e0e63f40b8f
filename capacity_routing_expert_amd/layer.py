"""Device-side convenience around the C interface: upload a workload, allocate outputs and
workspace with torch, and call the staged or whole-layer entry points.  Allocation and
marshalling only; all layer arithmetic runs in libmoe."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def to_device(arr: np.ndarray | None, dtype: str, device) -> torch.Tensor | None:
    """bf16 bit patterns (uint16) become torch.bfloat16; float32 stays float32."""
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    if arr.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def upload(inputs: dict, device="cuda:0") -> dict:
    dt = inputs["dtype"]
    return {k: to_device(inputs[k], dt if k != "b_router" else "f32", device)
            for k in ("x", "w_router", "b_router", "w1", "b1", "w2", "b2")}


def shape_of(dev: dict, top_k: int, capacity: int) -> B.MoeShape:
    x, w2 = dev["x"], dev["w2"]
    dtype = B.MOE_BF16 if x.dtype == torch.bfloat16 else B.MOE_F32
    # d_ff is the activation width: W2 [E, d_model, d_ff] for both expert kinds (a dict from
    # pack_weights states it, its packed w2 being padded)
    return B.make_shape(x.shape[0], x.shape[1], dev.get("d_ff", w2.shape[2]), w2.shape[0], top_k,
                        capacity, dtype, dev.get("weight_layout", B.MOE_WEIGHTS_ROW_MAJOR))


def pack_weights(dev: dict) -> dict:
    """A copy of the device dict with w1 and w2 packed by moe_pack_weights (a one-time
    preparation of the weights).  Each packed array sits in a tensor of shape
    [E, rows, cols rounded up to 32]; the dict records the layout and d_ff."""
    out = dict(dev)
    shape = shape_of(dev, 1, 0)
    for name in ("w1", "w2"):
        w = dev[name]
        E, rows, cols = w.shape
        wp = torch.empty((E, rows, (cols + 31) // 32 * 32), dtype=w.dtype, device=w.device)
        B.moe_pack_weights(shape, w, wp)
        out[name] = wp
    out["weight_layout"] = B.MOE_WEIGHTS_PACKED
    out["d_ff"] = dev["w2"].shape[2]
    return out


def workspace(shape: B.MoeShape, device="cuda:0") -> torch.Tensor:
    return torch.empty(max(B.workspace_bytes(shape), 256), dtype=torch.uint8, device=device)


def layer_forward(dev: dict, top_k: int, capacity: int, ws: torch.Tensor | None = None,
                  events=None) -> dict:
    """Whole layer in one call; returns out and the routing/dispatch outputs."""
    shape = shape_of(dev, top_k, capacity)
    device = dev["x"].device
    T, E = shape.T, shape.n_experts
    ws = workspace(shape, device) if ws is None else ws
    res = {
        "out": torch.empty_like(dev["x"]),
        "ids": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "gates": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "slot_of": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "drop_mask": torch.empty((T, top_k), dtype=torch.uint8, device=device),
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
    }
    args = (shape, dev["x"], dev["w_router"], dev["b_router"], dev["w1"], dev["b1"], dev["w2"],
            dev["b2"], res["out"])
    kw = dict(topk_ids=res["ids"], topk_gates=res["gates"], slot_of=res["slot_of"],
              drop_mask=res["drop_mask"], expert_counts=res["counts"], ws=ws)
    if events is None:
        B.moe_layer_forward(*args, **kw)
    else:
        B.moe_layer_forward_profiled(*args, events, **kw)
    return res


def layer_forward_padded(dev: dict, top_k: int, capacity: int, ws: torch.Tensor | None = None,
                         events=None, want_rows: bool = True) -> dict:
    """The padded fixed-buffer layout in one call: as layer_forward, plus `y_rows`
    [n_experts * capacity, d_model] (every buffer row's expert output) when want_rows."""
    shape = shape_of(dev, top_k, capacity)
    device = dev["x"].device
    T, E = shape.T, shape.n_experts
    if ws is None:
        ws = torch.empty(max(B.workspace_bytes_padded(shape), 256), dtype=torch.uint8,
                         device=device)
    res = {
        "out": torch.empty_like(dev["x"]),
        "ids": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "gates": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "slot_of": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "drop_mask": torch.empty((T, top_k), dtype=torch.uint8, device=device),
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
        "y_rows": torch.empty((E * capacity, shape.d_model), dtype=dev["x"].dtype,
                              device=device) if want_rows else None,
    }
    B.moe_layer_forward_padded(shape, dev["x"], dev["w_router"], dev["b_router"], dev["w1"],
                               dev["b1"], dev["w2"], dev["b2"], res["out"], topk_ids=res["ids"],
                               topk_gates=res["gates"], slot_of=res["slot_of"],
                               drop_mask=res["drop_mask"], expert_counts=res["counts"],
                               y_rows=res["y_rows"], ws=ws, events=events)
    return res


def layer_forward_gated(dev: dict, top_k: int, capacity: int, ws: torch.Tensor | None = None,
                        events=None) -> dict:
    """Whole layer with gated experts (dev["w1"] is W13 [E, 2 d_ff, d_model], no biases)."""
    shape = shape_of(dev, top_k, capacity)
    device = dev["x"].device
    T, E = shape.T, shape.n_experts
    ws = workspace(shape, device) if ws is None else ws
    res = {
        "out": torch.empty_like(dev["x"]),
        "ids": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "gates": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "slot_of": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "drop_mask": torch.empty((T, top_k), dtype=torch.uint8, device=device),
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
    }
    B.moe_layer_forward_gated(shape, dev["x"], dev["w_router"], dev["b_router"], dev["w1"],
                              dev["w2"], res["out"], topk_ids=res["ids"], topk_gates=res["gates"],
                              slot_of=res["slot_of"], drop_mask=res["drop_mask"],
                              expert_counts=res["counts"], ws=ws, events=events)
    return res


def route(dev: dict, top_k: int, capacity: int, ws=None, want_logits=False) -> dict:
    shape = shape_of(dev, top_k, capacity)
    device = dev["x"].device
    T, E = shape.T, shape.n_experts
    ws = workspace(shape, device) if ws is None else ws
    ids = torch.empty((T, top_k), dtype=torch.int32, device=device)
    gates = torch.empty((T, top_k), dtype=torch.float32, device=device)
    logits = torch.empty((T, E), dtype=torch.float32, device=device) if want_logits else None
    B.moe_route(shape, dev["x"], dev["w_router"], dev["b_router"], ids, gates, logits, ws)
    return {"ids": ids, "gates": gates, "logits": logits}


def dispatch(shape: B.MoeShape, ids: torch.Tensor, gates: torch.Tensor, ws=None,
             x: torch.Tensor | None = None) -> dict:
    """moe_dispatch; with `x`, also the token rows in slot order (`x_routed`)."""
    device = ids.device
    T, k, E = shape.T, shape.top_k, shape.n_experts
    ws = workspace(shape, device) if ws is None else ws
    rows = max(B.max_kept_rows(shape), 0)
    res = {
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
        "offsets": torch.empty((E + 1,), dtype=torch.int32, device=device),
        "slot_of": torch.empty((T, k), dtype=torch.int32, device=device),
        "row_token": torch.empty((rows,), dtype=torch.int32, device=device),
        "drop_mask": torch.empty((T, k), dtype=torch.uint8, device=device),
    }
    if x is not None:
        res["x_routed"] = torch.empty((rows, shape.d_model), dtype=x.dtype, device=device)
    B.moe_dispatch(shape, ids, gates, res["counts"], res["offsets"], res["slot_of"],
                   res["row_token"], res["drop_mask"], ws, x=x, x_routed=res.get("x_routed"))
    return res


def expert_ffn(shape: B.MoeShape, dev: dict, row_token, offsets, ws=None) -> torch.Tensor:
    device = dev["x"].device
    ws = workspace(shape, device) if ws is None else ws
    y = torch.empty((max(B.max_kept_rows(shape), 0), shape.d_model), dtype=dev["x"].dtype,
                    device=device)
    B.moe_expert_ffn(shape, dev["x"], row_token, offsets, dev["w1"], dev["b1"], dev["w2"],
                     dev["b2"], y, ws)
    return y


def combine(shape: B.MoeShape, x, gates, slot_of, y_rows) -> torch.Tensor:
    out = torch.empty_like(x)
    B.moe_combine(shape, x, gates, slot_of, y_rows, out)
    return out


# ---------------------------------------------------------------- dropless pair-order flow
def workspace_dropless(shape: B.MoeShape, device="cuda:0") -> torch.Tensor:
    return torch.empty(max(B.workspace_bytes_dropless(shape), 256), dtype=torch.uint8,
                       device=device)


def layer_forward_dropless(dev: dict, top_k: int, ws: torch.Tensor | None = None, events=None,
                           gated: bool = False, want_rows: bool = True) -> dict:
    """Dropless pair-order layer in one call (capacity unused); with `gated`, dev["w1"] is W13.
    Returns out, ids, gates, counts and, when want_rows, pair_rows [T * k, d_model]."""
    shape = shape_of(dev, top_k, 0)
    device = dev["x"].device
    T, E = shape.T, shape.n_experts
    ws = workspace_dropless(shape, device) if ws is None else ws
    res = {
        "out": torch.empty_like(dev["x"]),
        "ids": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "gates": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
        "pair_rows": torch.empty((T * top_k, shape.d_model), dtype=dev["x"].dtype,
                                 device=device) if want_rows else None,
    }
    kw = dict(topk_ids=res["ids"], topk_gates=res["gates"], expert_counts=res["counts"],
              pair_rows=res["pair_rows"], ws=ws, events=events)
    if gated:
        B.moe_layer_forward_dropless_gated(shape, dev["x"], dev["w_router"], dev["b_router"],
                                           dev["w1"], dev["w2"], res["out"], **kw)
    else:
        B.moe_layer_forward_dropless(shape, dev["x"], dev["w_router"], dev["b_router"],
                                     dev["w1"], dev["b1"], dev["w2"], dev["b2"], res["out"], **kw)
    return res


def dispatch_pairs(shape: B.MoeShape, ids: torch.Tensor, ws=None) -> dict:
    device = ids.device
    N, E = shape.T * shape.top_k, shape.n_experts
    ws = workspace_dropless(shape, device) if ws is None else ws
    res = {
        "counts": torch.empty((E,), dtype=torch.int32, device=device),
        "offsets": torch.empty((E + 1,), dtype=torch.int32, device=device),
        "sorted_pairs": torch.empty((N,), dtype=torch.int32, device=device),
        "row_token": torch.empty((N,), dtype=torch.int32, device=device),
    }
    B.moe_dispatch_pairs(shape, ids, res["counts"], res["offsets"], res["sorted_pairs"],
                         res["row_token"], ws)
    return res


def expert_ffn_pairs(shape: B.MoeShape, dev: dict, disp: dict, weights: torch.Tensor, ws=None,
                     gated: bool = False) -> torch.Tensor:
    device = dev["x"].device
    ws = workspace_dropless(shape, device) if ws is None else ws
    rows = torch.empty((shape.T * shape.top_k, shape.d_model), dtype=dev["x"].dtype,
                       device=device)
    B.moe_expert_ffn_pairs(shape, dev["x"], disp["sorted_pairs"], disp["row_token"],
                           disp["offsets"], dev["w1"], None if gated else dev["b1"], dev["w2"],
                           None if gated else dev["b2"], weights, rows, ws, gated=gated)
    return rows


def moe_sum(shape: B.MoeShape, x, ids, pair_rows) -> torch.Tensor:
    out = torch.empty((shape.T, shape.d_model), dtype=pair_rows.dtype, device=pair_rows.device)
    B.moe_sum(shape, x, ids, pair_rows, out)
    return out


# ---------------------------------------------------------------- batch consolidation
def layer_forward_batches(dev: dict, top_k: int, capacity: int, batch_size: int,
                          consolidate: bool, ws: torch.Tensor | None = None,
                          events=None) -> dict:
    """The pool dev["x"] ([n_batches * batch_size, d]) as batches of batch_size tokens, one after
    another, regrouped by the Token Scheduler when `consolidate`.  Returns out (pool order),
    ids, gates, order (consolidating only) and the active experts of each batch as run."""
    x = dev["x"]
    device = x.device
    T = x.shape[0]
    if T % batch_size:
        raise ValueError("the pool must hold whole batches")
    M = T // batch_size
    w2 = dev["w2"]
    dtype = B.MOE_BF16 if x.dtype == torch.bfloat16 else B.MOE_F32
    shape = B.make_shape(batch_size, x.shape[1], dev.get("d_ff", w2.shape[2]), w2.shape[0], top_k,
                         capacity, dtype, dev.get("weight_layout", B.MOE_WEIGHTS_ROW_MAJOR))
    if ws is None:
        ws = torch.empty(max(B.workspace_bytes_batches(shape, M), 256), dtype=torch.uint8,
                         device=device)
    res = {
        "out": torch.empty_like(x),
        "ids": torch.empty((T, top_k), dtype=torch.int32, device=device),
        "gates": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "order": torch.empty((T,), dtype=torch.int32, device=device) if consolidate else None,
        "batch_experts": torch.empty((M,), dtype=torch.int32, device=device),
    }
    B.moe_layer_forward_batches(shape, M, consolidate, x, dev["w_router"], dev["b_router"],
                                dev["w1"], dev["b1"], dev["w2"], dev["b2"], res["out"],
                                topk_ids=res["ids"], topk_gates=res["gates"], order=res["order"],
                                batch_experts=res["batch_experts"], ws=ws, events=events)
    return res


def schedule_batches(ids: torch.Tensor, batch_size: int, n_experts: int) -> dict:
    T, k = ids.shape
    M = T // batch_size
    shape = B.make_shape(batch_size, 8, 8, n_experts, k, 0, B.MOE_BF16)
    res = {"order": torch.empty((T,), dtype=torch.int32, device=ids.device),
           "batch_experts": torch.empty((M,), dtype=torch.int32, device=ids.device),
           "orig_batch_experts": torch.empty((M,), dtype=torch.int32, device=ids.device)}
    B.moe_schedule_batches(shape, M, ids, res["order"], res["batch_experts"],
                           res["orig_batch_experts"])
    return res
