"""GPU parity for calls of more than 2^31 elements, where element indices and
byte offsets no longer fit 32 bits.

Three calls, each of about 2^31 + 2^11 elements:
  * eligibility traces on 2^24 + 3 rows of 128 steps (whole rows per tile),
    float flags;
  * GAE on 2 rows of 2^30 + 1024 steps (rows spread over tiles joined by
    the decoupled look-back), one-byte flags;
  * the episodic prefix sum on the same shape, one-byte flags, int64 out.

Inputs are drawn on the device from a seeded torch generator.  Every element
is checked against its estimator's recursion (recurrence_residuals; exact for
the prefix sum).  Sampled windows -- around element 2^31, at the row edges
and in the ragged last tile -- are checked against the float64 oracle: each
window is cut from the rest of its row by a forced episode boundary (a
terminated flag at its last step for GAE, a done at its first step for the
forward scans) or by the row's own edge, so the oracle computes its outputs
exactly from the window's inputs alone.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest

from reference import assert_parity
import recurrence_residuals as rr

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from linear_recurrence_scan_coefficient_amd import rlscan  # noqa: E402

GAMMA, LAM = 0.999, 0.97
BIG = 1 << 31
LONG = (2, (1 << 30) + 1024)   # the second row holds element 2^31
PACKED = ((1 << 24) + 3, 128)  # element 2^31 starts row 2^24
WINDOW = 40000                 # about ten 4096-element tiles


@pytest.fixture(autouse=True)
def _release():
    rlscan.rlscan_set_launch_override()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _need(gb):
    free, _ = torch.cuda.mem_get_info()
    if free < gb * 1e9:
        pytest.skip(f"needs {gb} GB of free device memory, {free / 1e9:.0f} GB free")


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _bernoulli(shape, p, g, dtype):
    return (torch.rand(shape, generator=g, device="cuda") < p).to(dtype)


def _host(t):
    return t.cpu().numpy()


def test_gae_beyond_2_31_elements_lookback():
    N, T = LONG
    assert N * T > BIG
    _need(45)
    g = _gen(1)
    rewards = torch.randn(N, T, generator=g, device="cuda")
    values = torch.randn(N, T, generator=g, device="cuda")
    boot = torch.randn(N, generator=g, device="cuda")
    term = _bernoulli((N, T), 1e-4, g, torch.uint8)
    t_big = BIG - T  # element 2^31 in row 1
    windows = [(1, t_big - WINDOW // 2, t_big + WINDOW // 2),  # crosses 2^31
               (1, T - 30000, T),                               # ragged last tile
               (0, T - 30000, T),                               # end of row 0
               (1, 0, 30000)]                                   # start of row 1
    for n, t0, t1 in windows:
        if t1 < T:
            term[n, t1 - 1] = 1  # cuts the window from the rest of its row
    adv = torch.empty(N, T, device="cuda")
    print(f"[large] gae {N}x{T} ({N * T} elements)", flush=True)
    rlscan.rlscan_gae(rewards, values, boot, term, None, None, adv, GAMMA, LAM)
    torch.cuda.synchronize()
    assert rlscan.rlscan_lookback_timeouts() == 0
    ratio, where = rr.gae_residual(adv, rewards, values, term, boot, GAMMA, LAM)
    assert ratio <= 1.0, f"recursion residual {ratio:.3g} of the bound at {where}"
    for n, t0, t1 in windows:
        want = oracle.gae(_host(rewards[n:n + 1, t0:t1]), _host(values[n:n + 1, t0:t1]),
                          _host(term[n:n + 1, t0:t1]).astype(np.float32), gamma=GAMMA,
                          lam=LAM, bootstrap_value=_host(boot[n:n + 1]))
        assert_parity({"advantages": _host(adv[n:n + 1, t0:t1])}, {"advantages": want},
                      f"gae row {n} [{t0}, {t1})")


def test_prefix_sum_beyond_2_31_elements_lookback():
    N, T = LONG
    _need(45)
    g = _gen(2)
    x = torch.randint(-8, 9, (N, T), generator=g, device="cuda", dtype=torch.int32)
    dones = _bernoulli((N, T), 1e-4, g, torch.uint8)
    t_big = BIG - T
    windows = [(1, t_big - WINDOW // 2, t_big + WINDOW // 2), (1, T - 30000, T),
               (0, T - 30000, T), (1, 0, 30000)]
    for n, t0, t1 in windows:
        if t0 > 0:
            dones[n, t0] = 1  # the scan restarts at the window's first step
    out = torch.empty(N, T, device="cuda", dtype=torch.int64)
    print(f"[large] episodic_prefix_sum {N}x{T} ({N * T} elements)", flush=True)
    rlscan.rlscan_episodic_prefix_sum(x, dones, out)
    torch.cuda.synchronize()
    assert rlscan.rlscan_lookback_timeouts() == 0
    bad, first = rr.prefix_sum_mismatches(out, x, dones)
    assert bad == 0, f"{bad} elements break the recursion, first at {first}"
    for n, t0, t1 in windows:
        want = oracle.episodic_prefix_sum(_host(x[n:n + 1, t0:t1]),
                                          _host(dones[n:n + 1, t0:t1]).astype(np.float32))
        assert_parity({"out": _host(out[n:n + 1, t0:t1])}, {"out": want},
                      f"prefix row {n} [{t0}, {t1})")


def test_eligibility_traces_beyond_2_31_elements_packed():
    N, T = PACKED
    assert N * T > BIG
    _need(45)
    g = _gen(3)
    x = torch.randn(N, T, generator=g, device="cuda")
    dones = _bernoulli((N, T), 0.01, g, torch.float32)
    out = torch.empty(N, T, device="cuda")
    print(f"[large] eligibility_traces {N}x{T} ({N * T} elements)", flush=True)
    rlscan.rlscan_eligibility_traces(x, dones, out, GAMMA, LAM)
    torch.cuda.synchronize()
    ratio, where = rr.traces_residual(out, x, dones, GAMMA, LAM)
    assert ratio <= 1.0, f"recursion residual {ratio:.3g} of the bound at {where}"
    rows = [0, 1, (1 << 24) - 2, (1 << 24) - 1, 1 << 24, (1 << 24) + 1, N - 1]
    idx = torch.tensor(rows, device="cuda")
    want = oracle.eligibility_traces(_host(x[idx]), _host(dones[idx]), gamma=GAMMA, lam=LAM)
    assert_parity({"traces": _host(out[idx])}, {"traces": want}, f"rows {rows}")
