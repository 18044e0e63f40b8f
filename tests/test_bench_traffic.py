"""bench.py's reading of rocprofv3 counter rows into per-launch HBM bytes of the expert GEMMs
(host logic only: synthetic counter rows, no profiler and no GPU)."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _rows(per_step, copy_kib, steps=3):
    """Dispatch-ordered rows of `steps` layer calls, then a small and a 1 GiB copy."""
    rows, i = [("k_pack_weights", 64, 5.0)], 0
    for _ in range(steps):
        rows += [("k_route_mfma4<...>", 4096, 1.0), ("k_dispatch_runs", 16, 2.0),
                 ("k_dispatch_merge", 64, 3.0), ("k_grouped_gemm<...>", 9999, per_step[0]),
                 ("k_grouped_gemm_loaders<...>", 8888, per_step[1]), ("k_combine_bf16", 512, 7.0)]
    # dispatch-only calls (no GEMM) must not shift the GEMM assignment
    rows += [("k_route_mfma4<...>", 4096, 1.0), ("k_dispatch_runs", 16, 2.0)]
    rows += [("__amd_rocclr_copyBuffer", 1024, 11.0), ("__amd_rocclr_copyBuffer", 1 << 24, copy_kib)]
    out = []
    for name, grid, v in rows:
        out.append((i, name, grid, v))
        i += 1
    return out


def test_pmc_gemm_traffic_scales_by_copy():
    b = _bench()
    gib_kib = float(1 << 20)
    vals = {"FETCH_SIZE": _rows((1000.0, 400.0), gib_kib / 2),  # counter reads half for the copy
            "WRITE_SIZE": _rows((300.0, 100.0), gib_kib)}
    r = b.pmc_gemm_traffic(vals)
    assert r["fetch_scale"] == pytest.approx(2.0) and r["write_scale"] == pytest.approx(1.0)
    assert r["expert_up"] == pytest.approx((1000.0 * 2 + 300.0) * 1024)
    assert r["expert_down"] == pytest.approx((400.0 * 2 + 100.0) * 1024)


def test_pmc_gemm_traffic_missing_copy_or_gemm_is_none():
    b = _bench()
    rows = _rows((1.0, 2.0), 1024.0)
    no_copy = [r for r in rows if not r[1].startswith("__amd")]
    assert b.pmc_gemm_traffic({"FETCH_SIZE": no_copy, "WRITE_SIZE": rows}) is None
    no_gemm = [r for r in rows if "k_grouped_gemm" not in r[1]]
    assert b.pmc_gemm_traffic({"FETCH_SIZE": rows, "WRITE_SIZE": no_gemm}) is None


def test_warm_up_runs_min_steps_then_until_the_time_floor():
    """bench.warm_up: at least min_steps steps, then on (in groups of 8, each ended by a sync)
    until min_ms of wall time have passed."""
    import time
    b = _bench()
    calls = {"step": 0, "sync": 0}

    def step():
        calls["step"] += 1

    def sync():
        calls["sync"] += 1

    r = b.warm_up(step, 5, 0.0, sync)  # no time floor: the first multiple of 8 past 5 steps
    assert r["steps"] == calls["step"] == 8 and calls["sync"] >= 1

    calls["step"] = 0
    t0 = time.perf_counter()

    def slow_step():
        calls["step"] += 1
        time.sleep(0.002)

    r = b.warm_up(slow_step, 1, 30.0, sync)
    assert (time.perf_counter() - t0) * 1e3 >= 30.0 and r["ms"] >= 30.0
    assert r["steps"] == calls["step"] and r["steps"] % 8 == 0
