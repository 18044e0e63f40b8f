"""Thin ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module only turns torch tensors into
device pointers, picks torch's current stream, checks the dtype, device, contiguity and size
(number of elements against what the shape needs) of every tensor it is handed, and raises on
a non-OK status.  torch is imported before the library is
loaded so that both use torch's HIP runtime (one runtime per process).

The library is loaded on first use; if it has not been built the call raises, there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_WEIGHTS_ROW_MAJOR, MOE_WEIGHTS_PACKED = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_DEVICE"}

EXPORTS = ("moe_capacity", "moe_workspace_bytes", "moe_max_kept_rows", "moe_status_string",
           "moe_last_error", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
           "moe_layer_forward", "moe_layer_forward_profiled", "moe_workspace_bytes_padded",
           "moe_layer_forward_padded", "moe_layer_forward_gated", "moe_workspace_bytes_dropless",
           "moe_dispatch_pairs", "moe_expert_ffn_pairs", "moe_sum", "moe_layer_forward_dropless",
           "moe_layer_forward_dropless_gated", "moe_workspace_bytes_batches",
           "moe_schedule_batches", "moe_layer_forward_batches", "moe_packed_weights_bytes",
           "moe_pack_weights", "moe_set_gemm_timing", "moe_set_stage_timing",
           "moe_layer_forward_noalloc")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m capacity_routing_expert_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        SP = ctypes.POINTER(MoeShape)
        L.moe_capacity.argtypes = [I64, I32, I32, ctypes.c_double]
        L.moe_capacity.restype = I32
        L.moe_workspace_bytes.argtypes = [SP]
        L.moe_workspace_bytes.restype = SZ
        L.moe_max_kept_rows.argtypes = [SP]
        L.moe_max_kept_rows.restype = I64
        L.moe_status_string.argtypes = [I32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_route.argtypes = [SP, P, P, P, P, P, P, P, SZ, P]
        L.moe_dispatch.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn.argtypes = [SP, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_combine.argtypes = [SP, P, P, P, P, P, P]
        L.moe_layer_forward.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_layer_forward_profiled.argtypes = L.moe_layer_forward.argtypes + [P]
        # moe_layer_forward's arguments without ws and ws_bytes
        L.moe_layer_forward_noalloc.argtypes = [SP] + [P] * 13 + [P]
        L.moe_workspace_bytes_padded.argtypes = [SP]
        L.moe_workspace_bytes_padded.restype = SZ
        # shape, x, w_router, b_router, w1, b1, w2, b2, out, ids, gates, slot_of, drop, counts,
        # y_rows, ws, ws_bytes, stream, events
        L.moe_layer_forward_padded.argtypes = [SP] + [P] * 15 + [SZ, P, P]
        # shape, x, w_router, b_router, w13, w2, out, ids, gates, slot_of, drop, counts, ws,
        # ws_bytes, stream, events
        L.moe_layer_forward_gated.argtypes = [SP] + [P] * 12 + [SZ, P, P]
        L.moe_workspace_bytes_dropless.argtypes = [SP]
        L.moe_workspace_bytes_dropless.restype = SZ
        L.moe_dispatch_pairs.argtypes = [SP, P, P, P, P, P, P, SZ, P]
        # shape, x, sorted_pairs, row_token, offsets, w1, b1, w2, b2, weights, gated, pair_rows,
        # ws, ws_bytes, stream
        L.moe_expert_ffn_pairs.argtypes = [SP] + [P] * 9 + [I32, P, P, SZ, P]
        L.moe_sum.argtypes = [SP, P, P, P, P, P]
        # shape, x, w_router, b_router, w1, b1, w2, b2, out, ids, gates, counts, pair_rows, ws,
        # ws_bytes, stream, events
        L.moe_layer_forward_dropless.argtypes = [SP] + [P] * 13 + [SZ, P, P]
        # shape, x, w_router, b_router, w13, w2, out, ids, gates, counts, pair_rows, ws,
        # ws_bytes, stream, events
        L.moe_layer_forward_dropless_gated.argtypes = [SP] + [P] * 11 + [SZ, P, P]
        L.moe_packed_weights_bytes.argtypes = [SP, I32, I32]
        L.moe_packed_weights_bytes.restype = SZ
        L.moe_pack_weights.argtypes = [SP, P, I32, I32, P, P]
        L.moe_pack_weights.restype = I32
        L.moe_workspace_bytes_batches.argtypes = [SP, I32]
        L.moe_workspace_bytes_batches.restype = SZ
        L.moe_schedule_batches.argtypes = [SP, I32, P, P, P, P, P]
        # shape, n_batches, consolidate, x, w_router, b_router, w1, b1, w2, b2, out, ids, gates,
        # order, batch_experts, ws, ws_bytes, stream, events
        L.moe_layer_forward_batches.argtypes = [SP, I32, I32] + [P] * 13 + [SZ, P, P]
        L.moe_set_gemm_timing.argtypes = [P]
        L.moe_set_gemm_timing.restype = I32
        L.moe_set_stage_timing.argtypes = [P]
        L.moe_set_stage_timing.restype = I32
        for name in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                     "moe_layer_forward", "moe_layer_forward_profiled", "moe_layer_forward_padded",
                     "moe_layer_forward_noalloc",
                     "moe_layer_forward_gated", "moe_dispatch_pairs", "moe_expert_ffn_pairs",
                     "moe_sum", "moe_layer_forward_dropless", "moe_layer_forward_dropless_gated",
                     "moe_schedule_batches", "moe_layer_forward_batches"):
            getattr(L, name).restype = I32
        _lib = L
    return _lib


def make_shape(T: int, d_model: int, d_ff: int, n_experts: int, top_k: int, capacity: int,
               dtype: int, weight_layout: int = MOE_WEIGHTS_ROW_MAJOR) -> MoeShape:
    return MoeShape(int(T), int(d_model), int(d_ff), int(n_experts), int(top_k), int(capacity),
                    int(dtype), int(weight_layout))


def capacity(T: int, top_k: int, n_experts: int, capacity_factor: float) -> int:
    return int(lib().moe_capacity(int(T), int(top_k), int(n_experts), float(capacity_factor)))


def workspace_bytes(shape: MoeShape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def workspace_bytes_padded(shape: MoeShape) -> int:
    return int(lib().moe_workspace_bytes_padded(ctypes.byref(shape)))


def workspace_bytes_dropless(shape: MoeShape) -> int:
    return int(lib().moe_workspace_bytes_dropless(ctypes.byref(shape)))


def max_kept_rows(shape: MoeShape) -> int:
    return int(lib().moe_max_kept_rows(ctypes.byref(shape)))


def last_error() -> str:
    return lib().moe_last_error().decode()


def _ptr(t: torch.Tensor | None, name: str, dtype=None, device=None,
         numel: int | None = None) -> ctypes.c_void_p | None:
    """Device pointer of `t` after checking its dtype, device, contiguity and that it holds at
    least `numel` elements (the library writes or reads that many through the raw pointer)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the shape needs {numel}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _n(shape: MoeShape) -> dict:
    """Element counts the shape needs per argument kind."""
    T, d, f, E, k = int(shape.T), int(shape.d_model), int(shape.d_ff), int(shape.n_experts), int(shape.top_k)
    rows = max(int(max_kept_rows(shape)), 0)
    return {"x": T * d, "wr": E * d, "E": E, "E1": E + 1, "Tk": T * k, "TE": T * E,
            "rows": rows, "yrows": rows * d, "f": f, "d": d, "T": T, "k": k}


def _w(shape: MoeShape, rows: int, cols: int) -> int:
    """Elements of one expert weight array of [E, rows, cols] in the shape's layout."""
    E = int(shape.n_experts)
    if shape.weight_layout == MOE_WEIGHTS_PACKED and shape.dtype == MOE_BF16:
        return E * ((cols + 31) // 32) * rows * 32
    return E * rows * cols  # row-major (other layouts and dtypes are refused by the library)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where, last_error())


def _dtype_of(shape: MoeShape):
    return torch.bfloat16 if shape.dtype == MOE_BF16 else torch.float32


def moe_route(shape, x, w_router, b_router, topk_ids, topk_gates, logits, ws, stream=None):
    dt, n = _dtype_of(shape), _n(shape)
    _check(lib().moe_route(ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
                           _ptr(w_router, "w_router", dt, numel=n["wr"]),
                           _ptr(b_router, "b_router", torch.float32, numel=n["E"]),
                           _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
                           _ptr(topk_gates, "topk_gates", torch.float32, numel=n["Tk"]),
                           _ptr(logits, "logits", torch.float32, numel=n["TE"]),
                           _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "moe_route")


def moe_dispatch(shape, topk_ids, topk_gates, expert_counts, expert_offsets, slot_of, row_token,
                 drop_mask, ws, x=None, x_routed=None, stream=None):
    """x and x_routed (optional, together): the token rows copied into slot order."""
    dt, n = _dtype_of(shape), _n(shape)
    _check(lib().moe_dispatch(ctypes.byref(shape),
                              _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
                              _ptr(topk_gates, "topk_gates", torch.float32, numel=n["Tk"]),
                              _ptr(expert_counts, "expert_counts", torch.int32, numel=n["E"]),
                              _ptr(expert_offsets, "expert_offsets", torch.int32, numel=n["E1"]),
                              _ptr(slot_of, "slot_of", torch.int32, numel=n["Tk"]),
                              _ptr(row_token, "row_token", torch.int32, numel=n["rows"])
                              if row_token.numel() else None,
                              _ptr(drop_mask, "drop_mask", torch.uint8, numel=n["Tk"]),
                              _ptr(x, "x", dt, numel=n["x"]),
                              _ptr(x_routed, "x_routed", dt, numel=n["yrows"])
                              if x_routed is not None and x_routed.numel() else None,
                              _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "moe_dispatch")


def moe_expert_ffn(shape, x, row_token, expert_offsets, w1, b1, w2, b2, y_rows, ws, stream=None):
    dt, n = _dtype_of(shape), _n(shape)
    f, d = n["f"], n["d"]
    _check(lib().moe_expert_ffn(ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
                                _ptr(row_token, "row_token", torch.int32, numel=n["rows"])
                                if row_token.numel() else None,
                                _ptr(expert_offsets, "expert_offsets", torch.int32, numel=n["E1"]),
                                _ptr(w1, "w1", dt, numel=_w(shape, f, d)),
                                _ptr(b1, "b1", dt, numel=n["E"] * f),
                                _ptr(w2, "w2", dt, numel=_w(shape, d, f)),
                                _ptr(b2, "b2", dt, numel=n["E"] * d),
                                _ptr(y_rows, "y_rows", dt, numel=n["yrows"]) if y_rows.numel() else None,
                                _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "moe_expert_ffn")


def moe_combine(shape, x, topk_gates, slot_of, y_rows, out, stream=None):
    dt, n = _dtype_of(shape), _n(shape)
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
                             _ptr(topk_gates, "topk_gates", torch.float32, numel=n["Tk"]),
                             _ptr(slot_of, "slot_of", torch.int32, numel=n["Tk"]),
                             _ptr(y_rows, "y_rows", dt, numel=n["yrows"]) if y_rows.numel() else None,
                             _ptr(out, "out", dt, numel=n["x"]), _stream(stream)), "moe_combine")


def _forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                  slot_of, drop_mask, expert_counts, ws, gated=False):
    dt, n = _dtype_of(shape), _n(shape)
    f, d, E = n["f"], n["d"], n["E"]
    return [ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
            _ptr(w_router, "w_router", dt, numel=n["wr"]),
            _ptr(b_router, "b_router", torch.float32, numel=E),
            _ptr(w1, "w1", dt, numel=_w(shape, 2 * f if gated else f, d)),
            _ptr(b1, "b1", dt, numel=E * f), _ptr(w2, "w2", dt, numel=_w(shape, d, f)),
            _ptr(b2, "b2", dt, numel=E * d), _ptr(out, "out", dt, numel=n["x"]),
            _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
            _ptr(topk_gates, "topk_gates", torch.float32, numel=n["Tk"]),
            _ptr(slot_of, "slot_of", torch.int32, numel=n["Tk"]),
            _ptr(drop_mask, "drop_mask", torch.uint8, numel=n["Tk"]),
            _ptr(expert_counts, "expert_counts", torch.int32, numel=E), _ptr(ws, "ws", torch.uint8),
            ws.numel() if ws is not None else 0]


def moe_layer_forward(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids=None,
                      topk_gates=None, slot_of=None, drop_mask=None, expert_counts=None, ws=None,
                      stream=None):
    args = _forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                         slot_of, drop_mask, expert_counts, ws)
    _check(lib().moe_layer_forward(*args, _stream(stream)), "moe_layer_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_layer_forward_noalloc(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids=None,
                              topk_gates=None, slot_of=None, drop_mask=None, expert_counts=None,
                              stream=None):
    """moe_layer_forward with the library's fixed device scratch as its workspace (no
    allocation anywhere in the call)."""
    args = _forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                         slot_of, drop_mask, expert_counts, None)
    _check(lib().moe_layer_forward_noalloc(*args[:-2], _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_layer_forward_profiled(shape, x, w_router, b_router, w1, b1, w2, b2, out, events,
                               topk_ids=None, topk_gates=None, slot_of=None, drop_mask=None,
                               expert_counts=None, ws=None, stream=None):
    """`events`: 6 torch.cuda.Event(enable_timing=True) objects, already recorded once (so the
    underlying hipEvent_t exists)."""
    handles = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])
    args = _forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                         slot_of, drop_mask, expert_counts, ws)
    _check(lib().moe_layer_forward_profiled(*args, _stream(stream), handles),
           "moe_layer_forward_profiled")


def moe_set_gemm_timing(events):
    """Arms kernel timing of the two expert GEMMs for the next layer or expert-FFN call on this
    thread: `events` are 4 torch.cuda.Event(enable_timing=True) objects (or None in place of
    one GEMM's pair), already recorded once (so the underlying hipEvent_t exists), receiving
    the up-projection's start and end and the down-projection's start and end; None
    disarms."""
    if events is None:
        _check(lib().moe_set_gemm_timing(None), "moe_set_gemm_timing")
        return
    handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(ev.cuda_event if ev is not None else None)
                                      for ev in events])
    _check(lib().moe_set_gemm_timing(handles), "moe_set_gemm_timing")


def moe_set_stage_timing(events):
    """Arms kernel timing of the router and the combine for the next layer call on this thread:
    `events` are 4 torch.cuda.Event(enable_timing=True) objects (or None in place of one
    kernel's pair), already recorded once, receiving the router kernel's start and end and the
    combine kernel's start and end; None disarms."""
    if events is None:
        _check(lib().moe_set_stage_timing(None), "moe_set_stage_timing")
        return
    handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(ev.cuda_event if ev is not None else None)
                                      for ev in events])
    _check(lib().moe_set_stage_timing(handles), "moe_set_stage_timing")


def moe_layer_forward_padded(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids=None,
                             topk_gates=None, slot_of=None, drop_mask=None, expert_counts=None,
                             y_rows=None, ws=None, events=None, stream=None):
    """The padded fixed-buffer layout; `y_rows` [n_experts * capacity, d_model] optional;
    `events` None or 6 recorded torch.cuda.Event(enable_timing=True)."""
    dt = _dtype_of(shape)
    args = _forward_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                         slot_of, drop_mask, expert_counts, ws)
    handles = None
    if events is not None:
        handles = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])
    y = (_ptr(y_rows, "y_rows", dt, numel=int(shape.n_experts) * int(shape.capacity) * int(shape.d_model))
         if y_rows is not None and y_rows.numel() else None)
    # the padded call takes y_rows before the workspace
    _check(lib().moe_layer_forward_padded(*args[:-2], y, args[-2], args[-1], _stream(stream),
                                          handles), "moe_layer_forward_padded")


def moe_layer_forward_gated(shape, x, w_router, b_router, w13, w2, out, topk_ids=None,
                            topk_gates=None, slot_of=None, drop_mask=None, expert_counts=None,
                            ws=None, events=None, stream=None):
    """Gated experts: w13 [E, 2 d_ff, d_model] (gate rows first), w2 [E, d_model, d_ff], no
    biases; bf16 only.  `events` None or 6 recorded torch.cuda.Event(enable_timing=True)."""
    handles = None
    if events is not None:
        handles = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])
    a = _forward_args(shape, x, w_router, b_router, w13, None, w2, None, out, topk_ids,
                      topk_gates, slot_of, drop_mask, expert_counts, ws, gated=True)
    # the gated call has no biases: shape, x, w_router, b_router, w13, w2, out, ...
    _check(lib().moe_layer_forward_gated(*a[:5], a[6], *a[8:], _stream(stream), handles),
           "moe_layer_forward_gated")


def _events(events, n=6):
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"expected {n} events, got {len(events)}")
    return (ctypes.c_void_p * n)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])


def moe_dispatch_pairs(shape, topk_ids, expert_counts, expert_offsets, sorted_pairs, row_token,
                       ws, stream=None):
    n = _n(shape)
    _check(lib().moe_dispatch_pairs(ctypes.byref(shape),
                                    _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
                                    _ptr(expert_counts, "expert_counts", torch.int32, numel=n["E"]),
                                    _ptr(expert_offsets, "expert_offsets", torch.int32,
                                         numel=n["E1"]),
                                    _ptr(sorted_pairs, "sorted_pairs", torch.int32, numel=n["Tk"]),
                                    _ptr(row_token, "row_token", torch.int32, numel=n["Tk"]),
                                    _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "moe_dispatch_pairs")


def moe_expert_ffn_pairs(shape, x, sorted_pairs, row_token, expert_offsets, w1, b1, w2, b2,
                         topk_weights, pair_rows, ws, gated=False, stream=None):
    """gated: w1 is w13 [E, 2 d_ff, d_model] and b1, b2 are ignored (pass None)."""
    dt, n = _dtype_of(shape), _n(shape)
    f, d, E = n["f"], n["d"], n["E"]
    _check(lib().moe_expert_ffn_pairs(
        ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
        _ptr(sorted_pairs, "sorted_pairs", torch.int32, numel=n["Tk"]),
        _ptr(row_token, "row_token", torch.int32, numel=n["Tk"]),
        _ptr(expert_offsets, "expert_offsets", torch.int32, numel=n["E1"]),
        _ptr(w1, "w1", dt, numel=_w(shape, 2 * f if gated else f, d)),
        _ptr(b1, "b1", dt, numel=E * f), _ptr(w2, "w2", dt, numel=_w(shape, d, f)),
        _ptr(b2, "b2", dt, numel=E * d),
        _ptr(topk_weights, "topk_weights", torch.float32, numel=n["Tk"]), int(bool(gated)),
        _ptr(pair_rows, "pair_rows", dt, numel=n["Tk"] * d), _ptr(ws, "ws", torch.uint8),
        ws.numel(), _stream(stream)), "moe_expert_ffn_pairs")


def moe_sum(shape, x, topk_ids, pair_rows, out, stream=None):
    """out[t] = (x[t] +) the sum of pair rows t*k .. t*k + k - 1; x and topk_ids may be None."""
    dt, n = _dtype_of(shape), _n(shape)
    _check(lib().moe_sum(ctypes.byref(shape), _ptr(x, "x", dt, numel=n["x"]),
                         _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
                         _ptr(pair_rows, "pair_rows", dt, numel=n["Tk"] * n["d"]),
                         _ptr(out, "out", dt, numel=n["x"]), _stream(stream)), "moe_sum")


def _dropless_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                   expert_counts, pair_rows, ws, gated):
    dt, n = _dtype_of(shape), _n(shape)
    f, d, E = n["f"], n["d"], n["E"]
    return [_ptr(x, "x", dt, numel=n["x"]), _ptr(w_router, "w_router", dt, numel=n["wr"]),
            _ptr(b_router, "b_router", torch.float32, numel=E),
            _ptr(w1, "w1", dt, numel=_w(shape, 2 * f if gated else f, d)),
            _ptr(b1, "b1", dt, numel=E * f), _ptr(w2, "w2", dt, numel=_w(shape, d, f)),
            _ptr(b2, "b2", dt, numel=E * d), _ptr(out, "out", dt, numel=n["x"]),
            _ptr(topk_ids, "topk_ids", torch.int32, numel=n["Tk"]),
            _ptr(topk_gates, "topk_gates", torch.float32, numel=n["Tk"]),
            _ptr(expert_counts, "expert_counts", torch.int32, numel=E),
            _ptr(pair_rows, "pair_rows", dt, numel=n["Tk"] * d), _ptr(ws, "ws", torch.uint8),
            ws.numel()]


def moe_layer_forward_dropless(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids=None,
                               topk_gates=None, expert_counts=None, pair_rows=None, ws=None,
                               events=None, stream=None):
    """Dropless pair-order layer; `pair_rows` [T * k, d_model] optional; `events` None or 6
    recorded torch.cuda.Event(enable_timing=True)."""
    a = _dropless_args(shape, x, w_router, b_router, w1, b1, w2, b2, out, topk_ids, topk_gates,
                       expert_counts, pair_rows, ws, False)
    _check(lib().moe_layer_forward_dropless(ctypes.byref(shape), *a, _stream(stream),
                                            _events(events)), "moe_layer_forward_dropless")


def moe_layer_forward_dropless_gated(shape, x, w_router, b_router, w13, w2, out, topk_ids=None,
                                     topk_gates=None, expert_counts=None, pair_rows=None,
                                     ws=None, events=None, stream=None):
    a = _dropless_args(shape, x, w_router, b_router, w13, None, w2, None, out, topk_ids,
                       topk_gates, expert_counts, pair_rows, ws, True)
    # no biases: x, w_router, b_router, w13, w2, out, ...
    _check(lib().moe_layer_forward_dropless_gated(ctypes.byref(shape), *a[:4], a[5], *a[7:],
                                                  _stream(stream), _events(events)),
           "moe_layer_forward_dropless_gated")


def workspace_bytes_batches(batch_shape: MoeShape, n_batches: int) -> int:
    return int(lib().moe_workspace_bytes_batches(ctypes.byref(batch_shape), int(n_batches)))


def moe_schedule_batches(batch_shape, n_batches, topk_ids, order, batch_experts=None,
                         orig_batch_experts=None, stream=None):
    Tp = int(batch_shape.T) * int(n_batches)
    _check(lib().moe_schedule_batches(
        ctypes.byref(batch_shape), int(n_batches),
        _ptr(topk_ids, "topk_ids", torch.int32, numel=Tp * int(batch_shape.top_k)),
        _ptr(order, "order", torch.int32, numel=Tp),
        _ptr(batch_experts, "batch_experts", torch.int32, numel=int(n_batches)),
        _ptr(orig_batch_experts, "orig_batch_experts", torch.int32, numel=int(n_batches)),
        _stream(stream)), "moe_schedule_batches")


def moe_layer_forward_batches(batch_shape, n_batches, consolidate, x, w_router, b_router, w1, b1,
                              w2, b2, out, topk_ids=None, topk_gates=None, order=None,
                              batch_experts=None, ws=None, events=None, stream=None):
    """A pool of n_batches batches of batch_shape.T tokens, one batch after another, regrouped
    by the Token Scheduler when `consolidate`; `events` None or 5 recorded
    torch.cuda.Event(enable_timing=True)."""
    dt, n = _dtype_of(batch_shape), _n(batch_shape)
    M = int(n_batches)
    Tp = n["T"] * M
    f, d, E = n["f"], n["d"], n["E"]
    _check(lib().moe_layer_forward_batches(
        ctypes.byref(batch_shape), M, int(bool(consolidate)), _ptr(x, "x", dt, numel=Tp * d),
        _ptr(w_router, "w_router", dt, numel=n["wr"]),
        _ptr(b_router, "b_router", torch.float32, numel=E),
        _ptr(w1, "w1", dt, numel=_w(batch_shape, f, d)), _ptr(b1, "b1", dt, numel=E * f),
        _ptr(w2, "w2", dt, numel=_w(batch_shape, d, f)), _ptr(b2, "b2", dt, numel=E * d),
        _ptr(out, "out", dt, numel=Tp * d),
        _ptr(topk_ids, "topk_ids", torch.int32, numel=Tp * n["k"]),
        _ptr(topk_gates, "topk_gates", torch.float32, numel=Tp * n["k"]),
        _ptr(order, "order", torch.int32, numel=Tp),
        _ptr(batch_experts, "batch_experts", torch.int32, numel=M), _ptr(ws, "ws", torch.uint8),
        ws.numel(), _stream(stream), _events(events, 5)), "moe_layer_forward_batches")


def packed_weights_bytes(shape: MoeShape, rows: int, cols: int) -> int:
    return int(lib().moe_packed_weights_bytes(ctypes.byref(shape), int(rows), int(cols)))


def moe_pack_weights(shape, w, w_packed, stream=None):
    """w [E, rows, cols] bf16 -> w_packed (at least moe_packed_weights_bytes bytes)."""
    E, rows, cols = w.shape
    if w_packed.numel() * w_packed.element_size() < packed_weights_bytes(shape, rows, cols):
        raise ValueError("w_packed is too small")
    _check(lib().moe_pack_weights(ctypes.byref(shape), _ptr(w, "w", torch.bfloat16), int(rows),
                                  int(cols), _ptr(w_packed, "w_packed"), _stream(stream)),
           "moe_pack_weights")
