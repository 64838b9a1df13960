"""Seeded synthetic inputs for the credit-assignment estimators.

This module holds no arithmetic of the estimators themselves: it only draws
random inputs (numpy ``PCG64``) with the shapes and distributions of the
workloads the pages benchmark, so that the GPU path and the float64 oracle
read the very same float32 host arrays.

Every array is drawn from its own stream, keyed by ``(seed, stream id)``, so
an array's values do not depend on which other arrays were requested.

Workloads (named by what they are and their sizes):

``gae_64x512``
    The README's usage example shape (64 envs x 512 steps, gamma 0.99,
    lambda 0.95) with rewards, values ~ N(0, 1), a per-row bootstrap value
    ~ N(0, 1) standing for V[T], terminated ~ Bernoulli(0.01), no truncation.
``production_4096x128``
    All seven estimators at 4096 envs x 128 steps (the README's
    production-regime headline shape), gamma 0.99, lambda 0.95,
    terminated ~ Bernoulli(1/200), no truncation; V-trace log-ratios
    ~ N(0, 0.5^2) with rho_bar = c_bar = 1; Retrace with A = 6 actions,
    next-state Q ~ N(0, 1), target policy softmax(N(0, 1) logits), taken
    actions uniform in [0, 6), behaviour probability ~ U(0.05, 1) and an
    all-zero truncated tensor; traces x ~ N(0, 1), dones ~ Bernoulli(0.01);
    prefix sum int32 x uniform in [-8, 8], dones ~ Bernoulli(0.01).
``truncation_4096x128``
    As above for GAE, V-trace, Retrace, TD(lambda) and discounted returns,
    but each step draws u ~ U(0, 1): u < 0.005 terminates, 0.005 <= u < 0.010
    truncates with a bootstrap value ~ N(0, 1) at that step.
``sweep_<N>x<T>``
    GAE, V-trace and discounted returns, distributions as in the production
    workload, at (16384, 32), (4096, 128), (1024, 512), (256, 2048),
    (64, 8192), (16, 32768): 2^19 elements each.
``long_8x1048576``
    GAE, V-trace, discounted returns and the prefix sum at 8 x 2^20,
    gamma 0.999, lambda 0.97, terminated and truncated each
    ~ Bernoulli(1e-4) drawn independently (so a step may carry both),
    bootstrap values ~ N(0, 1); prefix sum dones ~ Bernoulli(1e-4).
``large_batch_1048576x32``
    A supplementary large-batch case, not one of the shapes above: GAE,
    V-trace and discounted returns at 2^20 x 32 (2^25 elements, the packed
    mapping at a size where HBM bandwidth, not launch latency, bounds the
    call), distributions as in the production workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

ESTIMATORS = ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns",
              "eligibility_traces", "episodic_prefix_sum")

_STREAM_IDS = {
    "rewards": 1, "values": 2, "bootstrap_value": 3, "terminated": 4, "truncated": 5,
    "bootstrap_values": 6, "log_rhos": 7, "next_q": 8, "logits": 9, "actions": 10,
    "behaviour_probs": 11, "trace_x": 12, "trace_dones": 13, "prefix_x": 14,
    "prefix_dones": 15, "flag_u": 16,
}


def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for one named array."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed),
                                                                      _STREAM_IDS[name]])))


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    T: int
    estimators: tuple = ESTIMATORS
    gamma: float = 0.99
    lam: float = 0.95
    term_p: float = 1.0 / 200.0
    # "none": no truncated tensor; "exclusive": one uniform draw per step
    # decides terminated / truncated / neither; "independent": two Bernoullis.
    trunc_mode: str = "none"
    trunc_p: float = 0.0
    excl_term_below: float = 0.005
    excl_trunc_below: float = 0.010
    done_p: float = 0.01
    A: int = 6
    rho_bar: float = 1.0
    c_bar: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def elements(self) -> int:
        return self.N * self.T


SWEEP_SHAPES = ((16384, 32), (4096, 128), (1024, 512), (256, 2048), (64, 8192), (16, 32768))


def _presets():
    p = {
        "gae_64x512": Workload("gae_64x512", 64, 512, ("gae",), term_p=0.01),
        "production_4096x128": Workload("production_4096x128", 4096, 128),
        "truncation_4096x128": Workload(
            "truncation_4096x128", 4096, 128,
            ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns"),
            trunc_mode="exclusive"),
        "long_8x1048576": Workload(
            "long_8x1048576", 8, 1 << 20,
            ("gae", "vtrace", "discounted_returns", "episodic_prefix_sum"),
            gamma=0.999, lam=0.97, term_p=1e-4, trunc_mode="independent", trunc_p=1e-4,
            done_p=1e-4),
        "large_batch_1048576x32": Workload(
            "large_batch_1048576x32", 1 << 20, 32,
            ("gae", "vtrace", "discounted_returns")),
    }
    for n, t in SWEEP_SHAPES:
        name = f"sweep_{n}x{t}"
        p[name] = Workload(name, n, t, ("gae", "vtrace", "discounted_returns"))
    return p


WORKLOADS = _presets()


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def custom(N: int, T: int, **kw) -> Workload:
    return Workload(kw.pop("name", f"custom_{N}x{T}"), N, T, **kw)


# ------------------------------------------------------------------ draws
def _normal(seed, name, shape, scale=1.0):
    return (scale * rng_for(seed, name).standard_normal(shape)).astype(np.float32)


def _bernoulli(seed, name, shape, p):
    return (rng_for(seed, name).random(shape) < p).astype(np.float32)


def episode_flags(w: Workload, seed: int = 0):
    """(terminated, truncated_or_None, bootstrap_values_or_None)."""
    shape = (w.N, w.T)
    if w.trunc_mode == "none":
        return _bernoulli(seed, "terminated", shape, w.term_p), None, None
    if w.trunc_mode == "exclusive":
        u = rng_for(seed, "flag_u").random(shape)
        term = (u < w.excl_term_below).astype(np.float32)
        trunc = ((u >= w.excl_term_below) & (u < w.excl_trunc_below)).astype(np.float32)
    elif w.trunc_mode == "independent":
        term = _bernoulli(seed, "terminated", shape, w.term_p)
        trunc = _bernoulli(seed, "truncated", shape, w.trunc_p)
    else:
        raise ValueError(f"unknown trunc_mode {w.trunc_mode!r}")
    return term, trunc, _normal(seed, "bootstrap_values", shape)


def value_inputs(w: Workload, seed: int = 0) -> dict:
    """Inputs of GAE, TD(lambda), discounted returns (and the shared part of V-trace)."""
    shape = (w.N, w.T)
    term, trunc, bvals = episode_flags(w, seed)
    return {
        "rewards": _normal(seed, "rewards", shape),
        "values": _normal(seed, "values", shape),
        "bootstrap_value": _normal(seed, "bootstrap_value", (w.N,)),
        "terminated": term,
        "truncated": trunc,
        "bootstrap_values": bvals,
    }


def vtrace_inputs(w: Workload, seed: int = 0) -> dict:
    d = value_inputs(w, seed)
    d["log_rhos"] = _normal(seed, "log_rhos", (w.N, w.T), scale=0.5)
    return d


def retrace_inputs(w: Workload, seed: int = 0) -> dict:
    shape = (w.N, w.T)
    term, trunc, _ = episode_flags(w, seed)
    if trunc is None:
        trunc = np.zeros(shape, np.float32)
    logits = rng_for(seed, "logits").standard_normal((w.N, w.T, w.A))
    logits -= logits.max(axis=-1, keepdims=True)
    probs = np.exp(logits)
    probs /= probs.sum(axis=-1, keepdims=True)
    return {
        "rewards": _normal(seed, "rewards", shape),
        "next_q_values_all": _normal(seed, "next_q", (w.N, w.T, w.A)),
        "next_target_probs": probs.astype(np.float32),
        "actions": rng_for(seed, "actions").integers(0, w.A, size=shape).astype(np.int32),
        "behaviour_probs": rng_for(seed, "behaviour_probs").uniform(0.05, 1.0, shape)
                                                          .astype(np.float32),
        "terminated": term,
        "truncated": trunc,
    }


def trace_inputs(w: Workload, seed: int = 0) -> dict:
    shape = (w.N, w.T)
    return {"x": _normal(seed, "trace_x", shape),
            "dones": _bernoulli(seed, "trace_dones", shape, w.done_p)}


def prefix_inputs(w: Workload, seed: int = 0) -> dict:
    shape = (w.N, w.T)
    x = rng_for(seed, "prefix_x").integers(-8, 9, size=shape).astype(np.int32)
    return {"x": x, "dones": _bernoulli(seed, "prefix_dones", shape, w.done_p)}


def inputs_for(estimator: str, w: Workload, seed: int = 0) -> dict:
    if estimator in ("gae", "lambda_returns"):
        return value_inputs(w, seed)
    if estimator == "discounted_returns":
        d = value_inputs(w, seed)
        d.pop("values")
        return d
    if estimator == "vtrace":
        return vtrace_inputs(w, seed)
    if estimator == "retrace":
        return retrace_inputs(w, seed)
    if estimator == "eligibility_traces":
        return trace_inputs(w, seed)
    if estimator == "episodic_prefix_sum":
        return prefix_inputs(w, seed)
    raise ValueError(f"unknown estimator {estimator!r}")
