"""Structural invariants of the launch planner (``rlscan_plan``) over random
shapes, estimators and launch overrides, on the CPU (the planner runs on the
host; nothing is launched).

Whatever the heuristics choose, every plan must describe tiles that the
kernels can run and that cover the call exactly:

* tile capacity = 4 elements x rounds x threads, with rounds in {1, 2, 4}
  and 64-512 threads; one or two waves only with one round; Retrace one
  round of at most four waves;
* packed mapping: each tile holds whole rows (a span that is a multiple of
  T and of 4, within the capacity), or all rows when they fit one tile, and
  the tiles cover exactly the N rows;
* look-back mapping: the span is the capacity and the tiles cover exactly
  the N*T elements;
* the grid never exceeds the tiles, and equals them unless capped;
* without an override, rows that fit one tile are packed into it, and a
  packed plan fills at least 3/4 of its tiles unless there is only one.
"""
import math

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from linear_recurrence_scan_coefficient_amd import rlscan

ESTS = ["gae", "vtrace", "retrace", "lambda_returns", "discounted_returns", "eligibility_traces",
        "episodic_prefix_sum"]
MAX_GRID = (1 << 23) - 1


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        rlscan.library()
    except OSError as e:  # pragma: no cover - the library is built by build()
        pytest.fail(f"librlscan.so does not load: {e}")
    yield
    rlscan.rlscan_set_launch_override()


def _check(est, N, T, A, p, mapping_override, grid_cap):
    R, threads, cap = p["rounds"], p["threads"], p["tile_elems"]
    span, tiles, grid = p["tile_span"], p["tiles"], p["grid"]
    ctx = (est, N, T, A, mapping_override, grid_cap, p)
    assert R in (1, 2, 4), ctx
    assert threads in (64, 128, 256, 512), ctx
    assert cap == 4 * R * threads, ctx
    if threads < 256:
        assert R == 1, ctx
    if est == "retrace":
        assert R == 1 and threads <= 256, ctx
    NT = N * T
    if p["mapping"] == rlscan.MAP_PACKED:
        assert mapping_override != rlscan.MAP_LOOKBACK, ctx
        if NT <= cap and tiles == 1:
            assert span == cap, ctx
        else:
            assert 0 < span <= cap and span % T == 0 and span % 4 == 0, ctx
            rows = span // T
            assert tiles == math.ceil(N / rows), ctx
            if mapping_override == rlscan.MAP_AUTO:
                assert tiles == 1 or 4 * span >= 3 * cap, ctx
    else:
        assert p["mapping"] == rlscan.MAP_LOOKBACK, ctx
        assert span == cap and tiles == math.ceil(NT / cap), ctx
        if mapping_override == rlscan.MAP_AUTO:
            assert NT > cap, ctx  # rows that fit one tile are packed into it
    assert 1 <= grid <= tiles, ctx
    want = min(tiles, MAX_GRID, grid_cap if grid_cap > 0 else tiles)
    assert grid == want, ctx


shapes = st.tuples(st.integers(1, 1 << 16), st.integers(1, 1 << 16)).filter(
    lambda s: s[0] * s[1] <= 1 << 30)


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(est=st.sampled_from(ESTS), shape=shapes, A=st.integers(1, 18))
def test_default_plans(est, shape, A):
    N, T = shape
    rlscan.rlscan_set_launch_override()
    _check(est, N, T, A, rlscan.rlscan_plan(est, N, T, A), rlscan.MAP_AUTO, 0)


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(est=st.sampled_from(ESTS), shape=shapes, A=st.integers(1, 18),
       mapping=st.sampled_from([rlscan.MAP_AUTO, rlscan.MAP_PACKED, rlscan.MAP_LOOKBACK]),
       rounds=st.sampled_from([0, 1, 2, 4]), waves=st.sampled_from([0, 1, 2, 4, 8]),
       grid_cap=st.sampled_from([0, 1, 7, 256, 4096]))
def test_overridden_plans(est, shape, A, mapping, rounds, waves, grid_cap):
    N, T = shape
    rlscan.rlscan_set_launch_override(mapping, rounds, waves, grid_cap)
    try:
        p = rlscan.rlscan_plan(est, N, T, A)
    finally:
        rlscan.rlscan_set_launch_override()
    _check(est, N, T, A, p, mapping, grid_cap)
    if rounds and est != "retrace" and not (waves and waves < 4 and rounds != 1):
        assert p["rounds"] == rounds, (est, N, T, p)


@pytest.mark.parametrize("est", ESTS)
def test_benchmark_shapes_plan_as_documented(est):
    """The named workloads' shapes: 4096 x 128 and the 2^20 x 32 large
    batch pack; 8 x 2^20 looks back; every plan obeys the invariants."""
    rlscan.rlscan_set_launch_override()
    for N, T, mapping in ((4096, 128, rlscan.MAP_PACKED), (1 << 20, 32, rlscan.MAP_PACKED),
                          (8, 1 << 20, rlscan.MAP_LOOKBACK), (64, 512, rlscan.MAP_PACKED)):
        p = rlscan.rlscan_plan(est, N, T, 6)
        assert p["mapping"] == mapping, (est, N, T, p)
        _check(est, N, T, 6, p, rlscan.MAP_AUTO, 0)
