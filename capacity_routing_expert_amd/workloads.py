"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and stores them (float32, or bf16 bit patterns
rounded to nearest even); it holds none of the layer's arithmetic.  The same host
arrays feed both the HIP library and the CPU oracle.

Draw order for every workload, from numpy's PCG64 seeded with the workload's seed:
x, router weights, router bias (when the workload has one), then for each expert in
turn W1[e], b1[e], W2[e], b2[e].  "N(0, s)" below means standard deviation s.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    name: str          # descriptive name with sizes
    seed: int
    T: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    capacity_factor: float
    dtype: str         # "f32" or "bf16"
    router_bias: str   # "none" | "normal" | "zipf" | "hot"
    weight_bias_std: float | None  # None -> N(0, 1/sqrt(fan_in)) for biases too
    expert: str = "ffn"  # "ffn": W2 SiLU(W1 x + b1) + b2; "gated": W2 (SiLU(W_gate x) * W_up x)
    batch_size: int = 0  # > 0: T is a pool of T / batch_size batches run one after another


WORKLOADS = {
    # 8 tokens, d_model 4, d_ff 8, 4 experts, top-1, capacity factor 1.25 (capacity 2), fp32
    "worked_example": Workload("worked_example", "worked_example_fp32_T8_d4_f8_E4_top1", 0,
                               8, 4, 8, 4, 1, 1.25, "f32", "none", None),
    # bf16, T 4096, d 2048, d_ff 8192, 8 experts, top-2, C 1.25 (capacity 1280)
    "mid": Workload("mid", "mid_bf16_T4096_d2048_f8192_E8_top2_C1.25", 1,
                    4096, 2048, 8192, 8, 2, 1.25, "bf16", "normal", 0.02),
    # bf16, T 16384, d 2048, d_ff 1408, 64 experts, top-6, C 1.0 (capacity 1536), log-Zipf bias
    "fine": Workload("fine", "fine_bf16_T16384_d2048_f1408_E64_top6_C1.0", 2,
                     16384, 2048, 1408, 64, 6, 1.0, "bf16", "zipf", 0.02),
    # bf16, T 64, d 2048, d_ff 8192, 8 experts, top-2, C 4.0 (capacity 64 = T, no drops)
    "decode": Workload("decode", "decode_bf16_T64_d2048_f8192_E8_top2_C4.0", 3,
                       64, 2048, 8192, 8, 2, 4.0, "bf16", "none", 0.02),
    # bf16, T 32768, d 4096, d_ff 14336, 8 experts, top-2, C 2.0 (capacity 16384), +2.5 hot expert
    "collapse": Workload("collapse", "collapse_bf16_T32768_d4096_f14336_E8_top2_C2.0", 4,
                         32768, 4096, 14336, 8, 2, 2.0, "bf16", "hot", 0.02),
    # gated experts with the fused-MoE flow diagram's widths (d_model 2048, GEMM 1 out 2 x 768),
    # the mid layer's routing: bf16, T 4096, 8 experts, top-2, C 1.25 (capacity 1280), no biases
    "gated": Workload("gated", "gated_bf16_T4096_d2048_f768_E8_top2_C1.25", 5,
                      4096, 2048, 768, 8, 2, 1.25, "bf16", "normal", None, "gated"),
    # a pool of 8 decode batches for the Token Scheduler: each batch is the decode layer's
    # (64 tokens, d 2048, d_ff 8192, 8 experts, top-2, C 4.0, capacity 64 per batch)
    "decode_pool": Workload("decode_pool", "decode_pool_bf16_8x64_d2048_f8192_E8_top2_C4.0", 6,
                            512, 2048, 8192, 8, 2, 4.0, "bf16", "none", 0.02, "ffn", 64),
    # one GPU's share of the collapse layer under expert parallelism over 8 GPUs: the hot
    # expert's owner receives its 16384 kept rows (capacity 16384) and runs that one expert's
    # FFN on them (d_model 4096, d_ff 14336); x holds the received rows, in receive order
    "ep8_hot_shard": Workload("ep8_hot_shard", "collapse_ep8_hot_expert_shard_bf16_rows16384_"
                              "d4096_f14336_E1", 7, 16384, 4096, 14336, 1, 1, 1.0, "bf16", "none",
                              0.02),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_float64(arr: np.ndarray | None, dtype: str) -> np.ndarray | None:
    """Exact float64 value of a stored array (bf16 bit patterns or float32)."""
    if arr is None:
        return None
    if dtype == "bf16" and arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_inputs(wl: Workload | str, seed: int | None = None, T: int | None = None) -> dict:
    """Draw the inputs of a workload.

    Returns a dict with x [T, d], w_router [E, d], b_router [E] float32 or None, and
    w1 [E, f, d], b1 [E, f], w2 [E, d, f], b2 [E, d] in the workload's storage type
    (float32, or uint16 bf16 bit patterns); the router bias is always float32.
    `T` overrides the token count (weights are drawn after x, so they change with it).
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    seed = wl.seed if seed is None else seed
    T = wl.T if T is None else T
    d, f, E = wl.d_model, wl.d_ff, wl.n_experts
    rng = np.random.Generator(np.random.PCG64(seed))

    x = _normal(rng, (T, d), 1.0)
    if wl.key == "worked_example":
        w_router = _normal(rng, (E, d), 0.5)
    else:
        w_router = _normal(rng, (E, d), 1.0 / math.sqrt(d))

    if wl.router_bias == "none":
        b_router = None
    elif wl.router_bias == "normal":
        b_router = rng.standard_normal(E).astype(np.float32)
    elif wl.router_bias == "zipf":
        # log of a Zipf(s = 1.1) pmf over a seeded permutation of the experts; the
        # normaliser cancels in the softmax, so rank r gets -1.1 * ln r
        perm = rng.permutation(E)
        b_router = np.zeros(E, dtype=np.float32)
        for r in range(1, E + 1):
            b_router[perm[r - 1]] = np.float32(-1.1 * math.log(r))
    elif wl.router_bias == "hot":
        hot = int(rng.integers(E))
        b_router = np.zeros(E, dtype=np.float32)
        b_router[hot] = np.float32(2.5)
    else:
        raise ValueError(wl.router_bias)

    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    if wl.expert == "gated":
        # per expert: W13[e] [2f, d] (gate rows, then up rows), then W2[e] [d, f]; no biases
        w1 = np.empty((E, 2 * f, d), dtype=sdt)
        w2 = np.empty((E, d, f), dtype=sdt)
        for e in range(E):
            w1[e] = _store(_normal(rng, (2 * f, d), 1.0 / math.sqrt(d)), wl.dtype)
            w2[e] = _store(_normal(rng, (d, f), 1.0 / math.sqrt(f)), wl.dtype)
        return {"x": _store(x, wl.dtype), "w_router": _store(w_router, wl.dtype),
                "b_router": b_router, "w1": w1, "b1": None, "w2": w2, "b2": None,
                "dtype": wl.dtype, "T": T, "workload": wl}
    w1 = np.empty((E, f, d), dtype=sdt)
    b1 = np.empty((E, f), dtype=sdt)
    w2 = np.empty((E, d, f), dtype=sdt)
    b2 = np.empty((E, d), dtype=sdt)
    b1_std = wl.weight_bias_std if wl.weight_bias_std is not None else 1.0 / math.sqrt(d)
    b2_std = wl.weight_bias_std if wl.weight_bias_std is not None else 1.0 / math.sqrt(f)
    for e in range(E):
        w1[e] = _store(_normal(rng, (f, d), 1.0 / math.sqrt(d)), wl.dtype)
        b1[e] = _store(_normal(rng, (f,), b1_std), wl.dtype)
        w2[e] = _store(_normal(rng, (d, f), 1.0 / math.sqrt(f)), wl.dtype)
        b2[e] = _store(_normal(rng, (d,), b2_std), wl.dtype)

    return {
        "x": _store(x, wl.dtype),
        "w_router": _store(w_router, wl.dtype),
        "b_router": b_router,
        "w1": w1, "b1": b1, "w2": w2, "b2": b2,
        "dtype": wl.dtype, "T": T, "workload": wl,
    }


def make_shape_inputs(T: int, d: int, f: int, E: int, dtype: str, seed: int,
                      router_bias_std: float = 0.0, bias_std: float = 0.02,
                      x_values: tuple | None = None, gated: bool = False) -> dict:
    """Inputs of an arbitrary small shape for randomized tests.

    With `x_values` given, x and the router weights are drawn from that finite set of
    values (used to force exact gate ties).  With `gated`, w1 is W13 [E, 2f, d] (gate rows
    first) and there are no biases.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if x_values is not None:
        vals = np.asarray(x_values, dtype=np.float32)
        x = vals[rng.integers(len(vals), size=(T, d))]
        w_router = vals[rng.integers(len(vals), size=(E, d))]
    else:
        x = _normal(rng, (T, d), 1.0)
        w_router = _normal(rng, (E, d), 1.0 / math.sqrt(d))
    b_router = (rng.standard_normal(E).astype(np.float32) * np.float32(router_bias_std)
                if router_bias_std > 0 else None)
    sdt = np.uint16 if dtype == "bf16" else np.float32
    if gated:
        w1 = np.empty((E, 2 * f, d), dtype=sdt)
        w2 = np.empty((E, d, f), dtype=sdt)
        for e in range(E):
            w1[e] = _store(_normal(rng, (2 * f, d), 1.0 / math.sqrt(d)), dtype)
            w2[e] = _store(_normal(rng, (d, f), 1.0 / math.sqrt(f)), dtype)
        return {"x": _store(x, dtype), "w_router": _store(w_router, dtype), "b_router": b_router,
                "w1": w1, "b1": None, "w2": w2, "b2": None, "dtype": dtype, "T": T}
    w1 = np.empty((E, f, d), dtype=sdt)
    b1 = np.empty((E, f), dtype=sdt)
    w2 = np.empty((E, d, f), dtype=sdt)
    b2 = np.empty((E, d), dtype=sdt)
    for e in range(E):
        w1[e] = _store(_normal(rng, (f, d), 1.0 / math.sqrt(d)), dtype)
        b1[e] = _store(_normal(rng, (f,), bias_std), dtype)
        w2[e] = _store(_normal(rng, (d, f), 1.0 / math.sqrt(f)), dtype)
        b2[e] = _store(_normal(rng, (d,), bias_std), dtype)
    return {"x": _store(x, dtype), "w_router": _store(w_router, dtype), "b_router": b_router,
            "w1": w1, "b1": b1, "w2": w2, "b2": b2, "dtype": dtype, "T": T}
