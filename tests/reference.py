"""Oracle outputs for an estimator call, keyed like the GPU outputs, and the
parity check used by every GPU test."""
from __future__ import annotations

import numpy as np

import oracle

# |gpu - ref| <= RTOL * (1 + |ref|) for every float32 output element, against
# the float64 oracle; integer outputs must be identical.
RTOL = 1e-4


def oracle_outputs(estimator: str, inputs: dict, w) -> dict:
    d = inputs
    g, lam = w.gamma, w.lam
    if estimator == "gae":
        return {"advantages": oracle.gae(
            d["rewards"], d["values"], d["terminated"], gamma=g, lam=lam,
            bootstrap_value=d.get("bootstrap_value"), truncated=d.get("truncated"),
            bootstrap_values=d.get("bootstrap_values"))}
    if estimator == "lambda_returns":
        return {"returns": oracle.lambda_returns(
            d["rewards"], d["values"], d["terminated"], gamma=g, lam=lam,
            bootstrap_value=d.get("bootstrap_value"), truncated=d.get("truncated"),
            bootstrap_values=d.get("bootstrap_values"))}
    if estimator == "discounted_returns":
        return {"returns": oracle.discounted_returns(
            d["rewards"], d["terminated"], gamma=g, bootstrap_value=d.get("bootstrap_value"),
            truncated=d.get("truncated"), bootstrap_values=d.get("bootstrap_values"))}
    if estimator == "vtrace":
        vs, pg = oracle.vtrace(
            d["rewards"], d["values"], d["log_rhos"], d["terminated"], gamma=g,
            rho_bar=w.rho_bar, c_bar=w.c_bar, bootstrap_value=d.get("bootstrap_value"),
            truncated=d.get("truncated"), bootstrap_values=d.get("bootstrap_values"))
        return {"vs": vs, "pg_advantages": pg}
    if estimator == "retrace":
        return {"targets": oracle.retrace(
            d["rewards"], d["next_q_values_all"], d["next_target_probs"], d["actions"],
            d["behaviour_probs"], d["terminated"], d["truncated"], gamma=g, lam=lam)}
    if estimator == "eligibility_traces":
        return {"traces": oracle.eligibility_traces(d["x"], d["dones"], gamma=g, lam=lam)}
    if estimator == "episodic_prefix_sum":
        return {"out": oracle.episodic_prefix_sum(d["x"], d["dones"])}
    raise ValueError(estimator)


def assert_parity(got: dict, want: dict, label: str = ""):
    assert set(got) == set(want), (sorted(got), sorted(want))
    for k, ref in want.items():
        out = got[k]
        assert out.shape == ref.shape, f"{label} {k}: shape {out.shape} vs {ref.shape}"
        if np.issubdtype(ref.dtype, np.integer):
            assert out.dtype == np.int64, f"{label} {k}: dtype {out.dtype}"
            bad = np.flatnonzero(out != ref)
            assert bad.size == 0, (f"{label} {k}: {bad.size} integer mismatches, first at "
                                   f"{np.unravel_index(bad[0], ref.shape)}: "
                                   f"{out.flat[bad[0]]} vs {ref.flat[bad[0]]}")
        else:
            err = np.abs(out.astype(np.float64) - ref) / (1.0 + np.abs(ref))
            finite = np.isfinite(out).all()
            worst = float(err.max()) if err.size else 0.0
            if not finite or worst > RTOL:
                i = int(np.nanargmax(np.where(np.isfinite(err), err, np.inf)))
                raise AssertionError(
                    f"{label} {k}: max rel err {worst:.3e} > {RTOL:.0e} at "
                    f"{np.unravel_index(i, ref.shape)}: gpu {out.flat[i]!r} ref {ref.flat[i]!r}")
