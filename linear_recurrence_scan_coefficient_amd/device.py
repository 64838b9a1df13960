"""Device-side plumbing for the binding: host arrays to GPU tensors, output
allocation, and a uniform call of any estimator by name.

Marshalling only -- every step of the computation runs in librlscan.
"""
from __future__ import annotations

import numpy as np
import torch

from . import rlscan
from .workloads import Workload

OUTPUTS = {
    "gae": (("advantages", torch.float32),),
    "lambda_returns": (("returns", torch.float32),),
    "discounted_returns": (("returns", torch.float32),),
    "vtrace": (("vs", torch.float32), ("pg_advantages", torch.float32)),
    "retrace": (("targets", torch.float32),),
    "eligibility_traces": (("traces", torch.float32),),
    "episodic_prefix_sum": (("out", torch.int64),),
}


# each estimator's inputs in the order of its plain C entry point (the order
# of an rlscan_call's `in` array)
INPUT_ORDER = {
    "gae": ("rewards", "values", "bootstrap_value", "terminated", "truncated", "bootstrap_values"),
    "lambda_returns": ("rewards", "values", "bootstrap_value", "terminated", "truncated",
                       "bootstrap_values"),
    "discounted_returns": ("rewards", "bootstrap_value", "terminated", "truncated",
                           "bootstrap_values"),
    "vtrace": ("rewards", "values", "bootstrap_value", "log_rhos", "terminated", "truncated",
               "bootstrap_values"),
    "retrace": ("rewards", "next_q_values_all", "next_target_probs", "actions",
                "behaviour_probs", "terminated", "truncated"),
    "eligibility_traces": ("x", "dones"),
    "episodic_prefix_sum": ("x", "dones"),
}


def upload(inputs: dict, device="cuda") -> dict:
    return {k: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(device))
            for k, v in inputs.items()}


def alloc_outputs(estimator: str, N: int, T: int, device="cuda") -> dict:
    return {name: torch.empty((N, T), dtype=dt, device=device)
            for name, dt in OUTPUTS[estimator]}


def call(estimator: str, d: dict, out: dict, w: Workload, stream=None):
    """Enqueues one estimator call on `stream` (default: current stream)."""
    g, lam = w.gamma, w.lam
    if estimator == "gae":
        rlscan.rlscan_gae(d["rewards"], d["values"], d.get("bootstrap_value"), d["terminated"],
                          d.get("truncated"), d.get("bootstrap_values"), out["advantages"],
                          g, lam, stream)
    elif estimator == "lambda_returns":
        rlscan.rlscan_lambda_returns(d["rewards"], d["values"], d.get("bootstrap_value"),
                                     d["terminated"], d.get("truncated"),
                                     d.get("bootstrap_values"), out["returns"], g, lam, stream)
    elif estimator == "discounted_returns":
        rlscan.rlscan_discounted_returns(d["rewards"], d.get("bootstrap_value"), d["terminated"],
                                         d.get("truncated"), d.get("bootstrap_values"),
                                         out["returns"], g, stream)
    elif estimator == "vtrace":
        rlscan.rlscan_vtrace(d["rewards"], d["values"], d.get("bootstrap_value"), d["log_rhos"],
                             d["terminated"], d.get("truncated"), d.get("bootstrap_values"),
                             out["vs"], out["pg_advantages"], g, w.rho_bar, w.c_bar, stream)
    elif estimator == "retrace":
        rlscan.rlscan_retrace(d["rewards"], d["next_q_values_all"], d["next_target_probs"],
                              d["actions"], d["behaviour_probs"], d["terminated"], d["truncated"],
                              out["targets"], g, lam, stream)
    elif estimator == "eligibility_traces":
        rlscan.rlscan_eligibility_traces(d["x"], d["dones"], out["traces"], g, lam, stream)
    elif estimator == "episodic_prefix_sum":
        rlscan.rlscan_episodic_prefix_sum(d["x"], d["dones"], out["out"], stream)
    else:
        raise ValueError(f"unknown estimator {estimator!r}")
    return out


def run(estimator: str, inputs: dict, w: Workload, device="cuda") -> dict:
    """Uploads host inputs, runs one call, returns host (numpy) outputs."""
    d = upload(inputs, device)
    N, T = w.N, w.T
    out = alloc_outputs(estimator, N, T, device)
    call(estimator, d, out, w)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}
