"""The recurrence-residual checks used at sizes beyond the oracle's reach,
tried on the CPU: the oracle's own results pass them, in pieces of any size,
and plausible mistakes planted in those results fail them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import recurrence_residuals as rr


def _inputs(N, T, seed=0, p=0.05):
    g = np.random.default_rng(seed)
    return dict(
        rewards=g.standard_normal((N, T)).astype(np.float32),
        values=g.standard_normal((N, T)).astype(np.float32),
        terminated=(g.random((N, T)) < p).astype(np.float32),
        bootstrap_value=g.standard_normal(N).astype(np.float32),
        x=g.standard_normal((N, T)).astype(np.float32),
        xi=g.integers(-8, 9, (N, T)).astype(np.int32),
        dones=(g.random((N, T)) < p).astype(np.float32))


def _gae(d, gamma=0.97, lam=0.9):
    return oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=gamma, lam=lam,
                      bootstrap_value=d["bootstrap_value"])


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


@pytest.mark.parametrize("piece", [1 << 25, 5, 64, 300])
@pytest.mark.parametrize("N,T", [(7, 40), (3, 257), (2, 1000)])
def test_oracle_results_pass(monkeypatch, piece, N, T):
    monkeypatch.setattr(rr, "PIECE", piece)
    d = _inputs(N, T, seed=N * T)
    adv = _gae(d).astype(np.float32)
    ratio, _ = rr.gae_residual(_t(adv), _t(d["rewards"]), _t(d["values"]),
                               _t(d["terminated"]), _t(d["bootstrap_value"]), 0.97, 0.9)
    assert ratio < 0.1
    tr = oracle.eligibility_traces(d["x"], d["dones"], gamma=0.97, lam=0.9).astype(np.float32)
    ratio, _ = rr.traces_residual(_t(tr), _t(d["x"]), _t(d["dones"]), 0.97, 0.9)
    assert ratio < 0.1
    ps = oracle.episodic_prefix_sum(d["xi"], d["dones"])
    assert rr.prefix_sum_mismatches(_t(ps), _t(d["xi"]), _t(d["dones"] != 0)) == (0, None)


@pytest.mark.parametrize("piece", [1 << 25, 64])
def test_planted_mistakes_fail(monkeypatch, piece):
    monkeypatch.setattr(rr, "PIECE", piece)
    N, T = 3, 500
    d = _inputs(N, T, seed=11)
    r, v, term, boot = (_t(d[k]) for k in ("rewards", "values", "terminated",
                                             "bootstrap_value"))

    def gae_ratio(adv):
        return rr.gae_residual(_t(adv.astype(np.float32)), r, v, term, boot, 0.97, 0.9)

    good = _gae(d)
    one = good.copy()
    one[1, 321] += 1e-2 * (1 + abs(one[1, 321]))  # one element off by 100x the bar
    ratio, where = gae_ratio(one)
    assert ratio > 1 and where in ((1, 321), (1, 320))
    assert gae_ratio(_gae(d, lam=0.8))[0] > 1  # lambda dropped to 0.8
    no_boot = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.97, lam=0.9)
    assert gae_ratio(no_boot)[0] > 1  # bootstrap value ignored
    flipped = dict(d, values=-d["values"])
    assert gae_ratio(_gae(flipped))[0] > 1  # sign of V

    x, dn = _t(d["x"]), _t(d["dones"])
    shifted = np.zeros_like(d["dones"])
    shifted[:, 1:] = d["dones"][:, :-1]  # reset read at d_{t-1}
    tr = oracle.eligibility_traces(d["x"], shifted, gamma=0.97, lam=0.9).astype(np.float32)
    assert rr.traces_residual(_t(tr), x, dn, 0.97, 0.9)[0] > 1

    ps = oracle.episodic_prefix_sum(d["xi"], d["dones"])
    xi = _t(d["xi"])
    bad = ps.copy()
    bad[2, 499] += 1
    assert rr.prefix_sum_mismatches(_t(bad), xi, dn) == (1, (2, 499))
    ps_shift = oracle.episodic_prefix_sum(d["xi"], shifted)
    assert rr.prefix_sum_mismatches(_t(ps_shift), xi, dn)[0] > 0
