"""The float64 oracle against its pins (CPU only).

Three groups:
  1. every pin in ``oracle_pins.PINS`` on the real oracle build;
  2. the (a, b) coefficient table of every estimator, solved by the plain
     recurrence, reproduces the estimator's own defining loop -- this checks,
     without a GPU, the reformulation that the GPU kernels implement;
  3. mutation checks: a plausible mistake planted in a copy of the oracle's
     source (on the CPU) must make at least one pin fail.
"""
from __future__ import annotations

import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
from oracle_pins import (PINS, close, cut_array, f32, small_retrace_inputs,
                         small_value_inputs, vhat_array)

ALL_PINS = [(group, fn) for group, fns in PINS.items() for fn in fns]


@pytest.mark.parametrize("group,pin", ALL_PINS, ids=[f"{g}-{f.__name__}" for g, f in ALL_PINS])
def test_pin(group, pin, olib):
    pin(olib)


# --------------------------------------------------------------- (a, b) table
def _next_values(d):
    vn = np.zeros(d["rewards"].shape)
    vn[:, :-1] = d["values"][:, 1:]
    return vn


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_coefficient_tables_reproduce_estimators(seed, olib):
    g, l = f32(0.97), f32(0.9)
    d = small_value_inputs(100 + seed, N=6, T=70, term_p=0.05, trunc_p=0.05)
    cuts = cut_array(d)
    vh = vhat_array(d)
    r = d["rewards"].astype(np.float64)
    v = d["values"].astype(np.float64)
    vn = _next_values(d)
    kw = dict(bootstrap_value=d["bootstrap_value"], truncated=d["truncated"],
              bootstrap_values=d["bootstrap_values"], lib=olib)

    # GAE: a = 0 at a cut else gamma*lambda; b = TD error
    a = np.where(cuts, 0.0, g * l)
    b = r + g * np.where(cuts, vh, vn) - v
    close(oracle.linear_recurrence(a, b, True, olib),
          oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=g, lam=l, **kw))

    # TD(lambda)
    b = np.where(cuts, r + g * vh, r + g * (1 - l) * vn)
    close(oracle.linear_recurrence(a, b, True, olib),
          oracle.lambda_returns(d["rewards"], d["values"], d["terminated"], gamma=g, lam=l,
                                **kw))

    # discounted returns
    a = np.where(cuts, 0.0, g)
    b = np.where(cuts, r + g * vh, r)
    close(oracle.linear_recurrence(a, b, True, olib),
          oracle.discounted_returns(d["rewards"], d["terminated"], gamma=g, **kw))

    # V-trace: the scan gives u = vs - V; pg reads u one step ahead
    lr = (0.6 * np.random.default_rng(seed).standard_normal(r.shape)).astype(np.float32)
    rb, cb = f32(1.2), f32(0.9)
    ratio = np.exp(lr.astype(np.float64))
    rho, c = np.minimum(rb, ratio), np.minimum(cb, ratio)
    a = np.where(cuts, 0.0, g * c)
    b = rho * (r + g * np.where(cuts, vh, vn) - v)
    u = oracle.linear_recurrence(a, b, True, olib)
    un = np.zeros_like(u)
    un[:, :-1] = u[:, 1:]
    vs, pg = oracle.vtrace(d["rewards"], d["values"], lr, d["terminated"], gamma=g,
                           rho_bar=rb, c_bar=cb, **kw)
    close(v + u, vs)
    close(rho * (r + g * np.where(cuts, vh, vn + un) - v), pg)


@pytest.mark.parametrize("seed", [0, 1])
def test_retrace_coefficient_table(seed, olib):
    g, l = f32(0.99), f32(0.95)
    d = small_retrace_inputs(200 + seed, N=5, T=64, A=6, term_p=0.05, trunc_p=0.05)
    N, T, A = d["next_q"].shape
    term = d["terminated"] != 0
    cuts = term | (d["truncated"] != 0)
    cuts[:, -1] = True
    eq = (d["next_pi"].astype(np.float64) * d["next_q"]).sum(-1)
    an = np.zeros((N, T), np.int64)
    an[:, :-1] = d["actions"][:, 1:]
    mun = np.ones((N, T))
    mun[:, :-1] = d["mu"][:, 1:]
    ii, tt = np.arange(N)[:, None], np.arange(T)[None, :]
    q_sel = d["next_q"][ii, tt, an].astype(np.float64)
    p_sel = d["next_pi"][ii, tt, an].astype(np.float64)
    cprime = l * np.minimum(1.0, p_sel / mun)
    r = d["rewards"].astype(np.float64)
    a = np.where(cuts, 0.0, g * cprime)
    b = np.where(cuts, r + g * np.where(term, 0.0, eq), r + g * (eq - cprime * q_sel))
    close(oracle.linear_recurrence(a, b, True, olib),
          oracle.retrace(d["rewards"], d["next_q"], d["next_pi"], d["actions"], d["mu"],
                         d["terminated"], d["truncated"], gamma=g, lam=l, lib=olib))


def test_forward_coefficient_tables(olib):
    rng = np.random.default_rng(7)
    N, T = 5, 90
    x = rng.standard_normal((N, T)).astype(np.float32)
    dn = (rng.random((N, T)) < 0.05).astype(np.float32)
    g, l = f32(0.99), f32(0.9)
    reset = dn != 0
    reset[:, 0] = True
    a = np.where(reset, 0.0, g * l)
    close(oracle.linear_recurrence(a, x, False, olib),
          oracle.eligibility_traces(x, dn, gamma=g, lam=l, lib=olib))
    xi = rng.integers(-8, 9, (N, T)).astype(np.int32)
    got = oracle.linear_recurrence(np.where(reset, 0.0, 1.0), xi, False, olib)
    assert np.array_equal(got.astype(np.int64), oracle.episodic_prefix_sum(xi, dn, lib=olib))


# --------------------------------------------------------------- mutations
MUTATIONS = [
    ("operator", "*b_out = aL * bE + bL;", "*b_out = aE * bL + bE;"),
    ("operator", "state = a[i] * state + b[i];", "state = b[i] * state + a[i];"),
    ("gae", "const double delta = (double)rewards[i] + gamma * v_next - (double)values[i];",
     "const double delta = (double)rewards[i] + v_next - (double)values[i];"),
    ("gae", "const double adv = delta + gamma * lambda * carry;",
     "const double adv = delta + gamma * carry;"),
    ("gae", "is_cut(terminated, truncated, i, t, T, continues) ? 0.0 : next_adv;",
     "is_cut(terminated, NULL, i, t, T, continues) ? 0.0 : next_adv;"),
    ("gae", "if (is_set(terminated, i)) return 0.0;\n    if (is_set(truncated, i)) return "
            "(double)bootstrap_values[i];",
     "if (is_set(truncated, i)) return (double)bootstrap_values[i];\n    "
     "if (is_set(terminated, i)) return 0.0;"),
    ("gae", "if (t == T - 1) return bootstrap_value ? (double)bootstrap_value[n] : 0.0;",
     "if (t == T - 1) return 0.0;"),
    ("lambda_returns", "(1.0 - lambda) * v_next", "lambda * v_next"),
    ("lambda_returns", "g = (double)rewards[i] + gamma * v_next;", "g = (double)rewards[i] + v_next;"),
    ("discounted_returns", "follow = next_ret;", "follow = gamma * next_ret;"),
    ("discounted_returns", "follow = next_state_value(NULL,", "follow = 0.0 * next_state_value(NULL,"),
    ("vtrace", "gamma * c * next_u", "gamma * rho * next_u"),
    ("vtrace", "const double follow = cut ? v_next : next_vs;",
     "const double follow = cut ? v_next : next_u;"),
    ("vtrace", "(ratio < c_bar ? ratio : c_bar)", "(ratio < c_bar ? ratio : 1.0)"),
    ("vtrace", "const double c = lambda * (", "const double c = ("),
    ("vtrace", "const double rho_pg = ratio < rho_bar_pg ? ratio : rho_bar_pg;",
     "const double rho_pg = ratio < rho_bar ? ratio : rho_bar;"),
    ("vtrace", "pg_advantages[i] = rho_pg *", "pg_advantages[i] = rho *"),
    ("retrace", "next_actions[n] : actions[i + 1];", "next_actions[n] : actions[i];"),
    ("retrace", "(double)behaviour_probs[i + 1]", "(double)behaviour_probs[i]"),
    ("retrace", "g = (double)rewards[i];\n", "g = (double)rewards[i] + gamma * eq;\n"),
    ("retrace", "const double c = lambda * (ratio < 1.0 ? ratio : 1.0);",
     "const double c = lambda * ratio;"),
    ("eligibility_traces", "(is_set(dones, i) ? 0.0 : gamma * lambda * prev)",
     "((t > 0 && is_set(dones, i - 1)) ? 0.0 : gamma * lambda * prev)"),
    ("episodic_prefix_sum", "(is_set(dones, i) ? 0 : prev)", "prev"),
    # the carry arguments (streaming one rollout through several calls)
    ("gae", "(t == T - 1 && !continues)", "(t == T - 1)"),
    ("gae", "double next_adv = carry_of(carry_in, n);", "double next_adv = 0.0;"),
    ("gae", "if (carry_out) carry_out[n] = advantages[n * T];",
     "if (carry_out) carry_out[n] = advantages[n * T + 1];"),
    ("lambda_returns", "double next_ret = carry_of(carry_in, n);  /* G_T */\n        for "
                       "(int64_t t = T - 1; t >= 0; --t) {\n            const int64_t i = n * T "
                       "+ t;\n            const double v_next",
     "double next_ret = 0.0;\n        for (int64_t t = T - 1; t >= 0; --t) {\n            "
     "const int64_t i = n * T + t;\n            const double v_next"),
    ("discounted_returns", "carry_out[n] = returns[n * T];\n    }\n}\n\n/* ----------------"
                           "-------------------------------------------------------- *\n * V-trace",
     "carry_out[n] = returns[n * T + T - 1];\n    }\n}\n\n/* ----------------"
     "-------------------------------------------------------- *\n * V-trace"),
    ("vtrace", "next_vs - v_T", "next_vs"),
    ("retrace", "(double)next_behaviour_probs[n]", "(double)behaviour_probs[i]"),
    ("eligibility_traces", "double prev = carry_of(carry_in, n);", "double prev = 0.0;"),
    ("episodic_prefix_sum", "int64_t prev = carry_in ? carry_in[n] : 0;", "int64_t prev = 0;"),
    ("episodic_prefix_sum_float", "(double)x[i] + (is_set(dones, i) ? 0.0 : prev)",
     "(double)x[i] + prev"),
    ("episodic_prefix_sum_float", "double prev = carry_of(carry_in, n);  /* y_{-1} */",
     "double prev = 0.0;  /* y_{-1} */"),
    ("episodic_prefix_sum_float",
     "? 0.0 : prev);\n            out[i] = y;\n            prev = y;\n        }\n        if "
     "(carry_out) carry_out[n] = out[n * T + T - 1];",
     "? 0.0 : prev);\n            out[i] = y;\n            prev = y;\n        }\n        if "
     "(carry_out) carry_out[n] = out[n * T];"),
]


@pytest.mark.parametrize("group,search,replace", MUTATIONS,
                         ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTATIONS)])
def test_planted_mistake_is_caught(group, search, replace):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert search in src, f"mutation anchor not found: {search!r}"
    mutated = src.replace(search, replace, 1)
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        c_path = os.path.join(tmp, "oracle_mut.c")
        so_path = os.path.join(tmp, "liboracle_mut.so")
        with open(c_path, "w") as f:
            f.write(mutated)
        oracle.build(src=c_path, out=so_path)
        lib = oracle.load_library(path=so_path)
        failures = 0
        for pin in PINS[group]:
            try:
                pin(lib)
            except (AssertionError, ValueError):
                failures += 1
        assert failures > 0, f"no {group} pin caught the planted mistake {replace!r}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
