"""rlscan_gae_noalloc (GAE with its look-back scratch in a fixed per-GPU
array, for callers that cannot allocate) against rlscan_gae_carry, the entry
point it is a variant of, both called through the C ABI on the same seeded
inputs.  Two look-back calls in a row, the second smaller, so the second
runs on the array as the first left it; then a packed call."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from reference import RTOL, assert_parity, oracle_outputs  # noqa: E402

pytestmark = pytest.mark.gpu


def _gae_inputs(N, T, seed):
    from linear_recurrence_scan_coefficient_amd import device, workloads
    w = workloads.custom(N, T, gamma=0.99, lam=0.95, term_p=0.002, trunc_mode="independent",
                         trunc_p=0.002)
    inputs = workloads.inputs_for("gae", w, seed=seed)
    carry = workloads.rng_for(seed, "values").standard_normal(N).astype(np.float32)
    return w, inputs, device.upload(inputs), torch.from_numpy(carry).cuda()


def _both(d, carry, N, T):
    from linear_recurrence_scan_coefficient_amd import rlscan
    outs = {}
    for name, fn in (("carry", rlscan.rlscan_gae), ("noalloc", rlscan.rlscan_gae_noalloc)):
        adv = torch.empty((N, T), dtype=torch.float32, device="cuda")
        co = torch.empty((N,), dtype=torch.float32, device="cuda")
        fn(d["rewards"], d["values"], d["bootstrap_value"], d["terminated"], d["truncated"],
           d["bootstrap_values"], adv, 0.99, 0.95, carry_in=carry, carry_out=co)
        outs[name] = (adv, co)
    torch.cuda.synchronize()
    return {k: (a.cpu().numpy(), c.cpu().numpy()) for k, (a, c) in outs.items()}


def _close(got, want, label):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64)) / (1.0 + np.abs(want))
    assert np.isfinite(got).all(), label
    assert float(err.max()) <= RTOL, f"{label}: max rel err {float(err.max()):.3e}"


@pytest.mark.parametrize("shapes", [((8, 1 << 17), (3, 5003))])
def test_noalloc_matches_carry_entry_point(shapes):
    from linear_recurrence_scan_coefficient_amd import rlscan
    rlscan.rlscan_set_launch_override()
    before = rlscan.rlscan_lookback_timeouts()
    for i, (N, T) in enumerate(shapes):
        print(f"noalloc call {i}: GAE {N}x{T}", flush=True)
        plan = rlscan.rlscan_plan("gae", N, T)
        assert plan["mapping"] == rlscan.MAP_LOOKBACK and plan["tiles"] > 1
        w, inputs, d, carry = _gae_inputs(N, T, seed=40 + i)
        got = _both(d, carry, N, T)
        _close(got["noalloc"][0], got["carry"][0], f"{N}x{T} advantages")
        _close(got["noalloc"][1], got["carry"][1], f"{N}x{T} carry_out")
    assert rlscan.rlscan_lookback_timeouts() == before


def test_noalloc_packed_and_plain_match_oracle():
    """A packed call (no scratch) and a look-back call without carry, both
    against the oracle as well."""
    from linear_recurrence_scan_coefficient_amd import rlscan
    rlscan.rlscan_set_launch_override()
    for N, T in ((64, 128), (2, 40000)):
        print(f"noalloc vs oracle: GAE {N}x{T}", flush=True)
        w, inputs, d, _ = _gae_inputs(N, T, seed=7)
        adv = torch.empty((N, T), dtype=torch.float32, device="cuda")
        rlscan.rlscan_gae_noalloc(d["rewards"], d["values"], d["bootstrap_value"],
                                  d["terminated"], d["truncated"], d["bootstrap_values"], adv,
                                  0.99, 0.95)
        torch.cuda.synchronize()
        assert_parity({"advantages": adv.cpu().numpy()}, oracle_outputs("gae", inputs, w),
                      f"noalloc {N}x{T}")


# the refused capture at the end leaves its graph empty, as it should
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_noalloc_lookback_calls_captured_into_a_graph():
    """Look-back calls of rlscan_gae_noalloc captured into a HIP graph (each
    records a clear of its status words before its scan): three replays,
    with eager calls of the library on the same array between them, each
    matching the eager rlscan_gae_carry results; a capture that would need
    tickets is refused."""
    from linear_recurrence_scan_coefficient_amd import rlscan
    rlscan.rlscan_set_launch_override()
    before = rlscan.rlscan_lookback_timeouts()
    cases = []
    for i, (N, T) in enumerate(((8, 1 << 17), (3, 5003))):
        assert rlscan.rlscan_plan("gae", N, T)["mapping"] == rlscan.MAP_LOOKBACK
        w, inputs, d, carry = _gae_inputs(N, T, seed=60 + i)
        want = _both(d, carry, N, T)["carry"]
        adv = torch.empty((N, T), dtype=torch.float32, device="cuda")
        co = torch.empty((N,), dtype=torch.float32, device="cuda")
        cases.append((N, T, d, carry, adv, co, want))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for N, T, d, carry, adv, co, _ in cases:
            rlscan.rlscan_gae_noalloc(d["rewards"], d["values"], d["bootstrap_value"],
                                      d["terminated"], d["truncated"], d["bootstrap_values"], adv,
                                      0.99, 0.95, carry_in=carry, carry_out=co)
    _, _, d_other, carry_other = _gae_inputs(5, 7001, seed=70)
    for replay in range(3):
        for *_, adv, co, _ in cases:
            adv.fill_(float("nan"))
            co.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"noalloc graph replay {replay}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for N, T, _, _, adv, co, want in cases:
            _close(adv.cpu().numpy(), want[0], f"replay {replay} {N}x{T} advantages")
            _close(co.cpu().numpy(), want[1], f"replay {replay} {N}x{T} carry_out")
        # eager look-back work on the same array (and the allocating path)
        # between the replays
        got = _both(d_other, carry_other, 5, 7001)
        _close(got["noalloc"][0], got["carry"][0], f"eager call after replay {replay}")
    del g
    # workgroups looping over tiles (tickets) cannot be replayed: refused
    N, T, d, carry, adv, co, _ = cases[1]
    rlscan.rlscan_set_launch_override(grid_cap=2)
    g2 = torch.cuda.CUDAGraph()
    try:
        with pytest.raises(rlscan.RlscanError) as err:
            with torch.cuda.graph(g2):
                rlscan.rlscan_gae_noalloc(d["rewards"], d["values"], d["bootstrap_value"],
                                          d["terminated"], d["truncated"],
                                          d["bootstrap_values"], adv, 0.99, 0.95)
        assert err.value.status == rlscan.RLSCAN_ERR_CAPTURE
    finally:
        rlscan.rlscan_set_launch_override()
    torch.cuda.synchronize()
    assert rlscan.rlscan_lookback_timeouts() == before
