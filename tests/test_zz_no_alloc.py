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
