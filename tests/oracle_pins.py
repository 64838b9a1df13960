"""Pins of the float64 oracle to things other than itself.

Each pin takes a loaded oracle library (so the mutation tests can hand it a
deliberately broken build) and raises AssertionError on a mismatch.  The
expected values come from:
  - explicit-sum brute force in exact rational arithmetic (``fractions``),
    which unrolls each estimator's recursion into its closed sum;
  - closed forms and special cases (lambda = 0, lambda = 1, rho = c = 1,
    constant reward, one-hot target policy, all-done, no-done);
  - library routines (``scipy.signal.lfilter`` for discounted sums,
    ``numpy.cumsum`` for prefix sums);
  - identities between estimators (TD(lambda) = GAE + V, ...);
  - the algebra of the (a, b) operator (associativity, identity).

The readings of points the pages leave open (flag precedence, the index of
the done flag, the bootstrap inputs) are those stated in oracle.c; the pins
check the arithmetic under those readings.
"""
from __future__ import annotations

import math
from fractions import Fraction as F

import numpy as np
from scipy.signal import lfilter

import oracle

TOL = 1e-12


def close(got, want, tol=TOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want) / (1.0 + np.abs(want))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"max rel err {worst:.3e} > {tol:.1e}"


def f32(x):
    return float(np.float32(x))


def fr(x):
    return F(float(x))


# ------------------------------------------------------------ small inputs
def small_value_inputs(seed, N=3, T=11, term_p=0.15, trunc_p=0.15, with_trunc=True,
                       with_boot=True):
    rng = np.random.default_rng(seed)
    d = {
        "rewards": rng.standard_normal((N, T)).astype(np.float32),
        "values": rng.standard_normal((N, T)).astype(np.float32),
        "bootstrap_value": rng.standard_normal(N).astype(np.float32) if with_boot else None,
        "terminated": (rng.random((N, T)) < term_p).astype(np.float32),
        "truncated": None,
        "bootstrap_values": None,
    }
    if with_trunc:
        d["truncated"] = (rng.random((N, T)) < trunc_p).astype(np.float32)
        d["bootstrap_values"] = rng.standard_normal((N, T)).astype(np.float32)
        # make sure some step carries both flags (terminated must win)
        d["terminated"][0, 2] = 1.0
        d["truncated"][0, 2] = 1.0
    return d


def flag(arr, n, t):
    return arr is not None and arr[n, t] != 0


def cut(d, n, t):
    T = d["rewards"].shape[1]
    return flag(d["terminated"], n, t) or flag(d["truncated"], n, t) or t == T - 1


def first_cut(d, n, t):
    e = t
    while not cut(d, n, e):
        e += 1
    return e


def vhat(d, n, t, values_key="values"):
    """Exact successor value seen from a step that is a chain cut (or V_{t+1})."""
    T = d["rewards"].shape[1]
    if flag(d["terminated"], n, t):
        return F(0)
    if flag(d["truncated"], n, t):
        return fr(d["bootstrap_values"][n, t])
    if t == T - 1:
        return fr(d["bootstrap_value"][n]) if d["bootstrap_value"] is not None else F(0)
    return fr(d[values_key][n, t + 1])


def vhat_array(d):
    """Float64 [N,T] of the successor value used at chain cuts."""
    N, T = d["rewards"].shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            if cut(d, n, t):
                out[n, t] = float(vhat(d, n, t))
    return out


def cut_array(d):
    N, T = d["rewards"].shape
    return np.array([[cut(d, n, t) for t in range(T)] for n in range(N)])


def mc_return_lfilter(rewards, vhat_cut, cuts, gamma):
    """Discounted sum of rewards up to the next cut, plus the discounted
    successor value there, via scipy's IIR filter over reversed segments."""
    N, T = rewards.shape
    out = np.empty((N, T))
    for n in range(N):
        start = 0
        for e in np.flatnonzero(cuts[n]):
            seg = rewards[n, start:e + 1][::-1].astype(np.float64)
            y, _ = lfilter([1.0], [1.0, -gamma], seg, zi=[gamma * vhat_cut[n, e]])
            out[n, start:e + 1] = y[::-1]
            start = e + 1
    return out


def oracle_kw(d, keys=("bootstrap_value", "truncated", "bootstrap_values")):
    return {k: d[k] for k in keys}


# ------------------------------------------------------------ operator
def pin_operator_associative(lib):
    rng = np.random.default_rng(1)
    # small integers: every product and sum is exact in float64
    for _ in range(2000):
        x, y, z = (tuple(float(v) for v in rng.integers(-50, 50, 2)) for _ in range(3))
        left = oracle.compose(oracle.compose(x, y, lib), z, lib)
        right = oracle.compose(x, oracle.compose(y, z, lib), lib)
        assert left == right, (x, y, z, left, right)
    for _ in range(10000):
        x, y, z = (tuple(rng.standard_normal(2)) for _ in range(3))
        left = oracle.compose(oracle.compose(x, y, lib), z, lib)
        right = oracle.compose(x, oracle.compose(y, z, lib), lib)
        close(left, right, 1e-14)
    for _ in range(5000):
        x, y, z = ((int(rng.integers(0, 2)), int(rng.integers(-2**40, 2**40)))
                   for _ in range(3))
        left = oracle.compose_i64(oracle.compose_i64(x, y, lib), z, lib)
        right = oracle.compose_i64(x, oracle.compose_i64(y, z, lib), lib)
        assert left == right


def pin_operator_identity_and_meaning(lib):
    rng = np.random.default_rng(2)
    for _ in range(1000):
        e = tuple(float(v) for v in rng.integers(-100, 100, 2))
        assert oracle.compose(e, (1.0, 0.0), lib) == e
        assert oracle.compose((1.0, 0.0), e, lib) == e
        # composition means "apply the right step first, then the left one"
        L, R = (tuple(float(v) for v in rng.integers(-20, 20, 2)) for _ in range(2))
        x = float(rng.integers(-20, 20))
        a, b = oracle.compose(L, R, lib)
        assert a * x + b == L[0] * (R[0] * x + R[1]) + L[1]
    # not commutative
    assert oracle.compose((2.0, 3.0), (5.0, 7.0), lib) != oracle.compose((5.0, 7.0), (2.0, 3.0), lib)
    assert oracle.compose_i64((1, 5), (0, 9), lib) == (0, 14)
    assert oracle.compose_i64((0, 5), (1, 9), lib) == (0, 5)


def pin_linear_recurrence_brute(lib):
    rng = np.random.default_rng(3)
    N, T = 4, 9
    a = rng.standard_normal((N, T))
    a[rng.random((N, T)) < 0.2] = 0.0
    b = rng.standard_normal((N, T))
    for reverse in (False, True):
        want = np.zeros((N, T))
        for n in range(N):
            for t in range(T):
                ks = range(t, T) if reverse else range(t, -1, -1)
                s = F(0)
                for k in ks:
                    # x_t = sum_k (prod of a strictly between t and k, from t) b_k
                    prod = F(1)
                    steps = range(t, k) if reverse else range(t, k, -1)
                    for j in steps:
                        prod *= fr(a[n, j])
                    s += prod * fr(b[n, k])
                want[n, t] = float(s)
        close(oracle.linear_recurrence(a, b, reverse, lib), want)


# ------------------------------------------------------------ GAE
def gae_brute(d, gamma, lam):
    g, l = fr(f32(gamma)), fr(f32(lam))
    N, T = d["rewards"].shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = first_cut(d, n, t)
            s = F(0)
            for k in range(t, e + 1):
                delta = fr(d["rewards"][n, k]) + g * vhat(d, n, k) - fr(d["values"][n, k])
                s += (g * l) ** (k - t) * delta
            out[n, t] = float(s)
    return out


def pin_gae_brute(lib):
    for seed, trunc, boot in ((10, True, True), (11, False, True), (12, True, False)):
        d = small_value_inputs(seed, with_trunc=trunc, with_boot=boot)
        got = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.9, lam=0.8,
                         lib=lib, **oracle_kw(d))
        close(got, gae_brute(d, 0.9, 0.8))


def pin_gae_lambda0_is_td_error(lib):
    d = small_value_inputs(13, N=5, T=40)
    g = f32(0.97)
    got = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.97, lam=0.0,
                     lib=lib, **oracle_kw(d))
    vnext = np.zeros_like(got)
    vnext[:, :-1] = d["values"][:, 1:]
    cuts = cut_array(d)
    vnext = np.where(cuts, vhat_array(d), vnext)
    close(got, d["rewards"] + g * vnext - d["values"].astype(np.float64))


def pin_gae_lambda1_is_mc_return_minus_value(lib):
    d = small_value_inputs(14, N=5, T=60)
    g = f32(0.95)
    got = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.95, lam=1.0,
                     lib=lib, **oracle_kw(d))
    mc = mc_return_lfilter(d["rewards"], vhat_array(d), cut_array(d), g)
    close(got, mc - d["values"], 1e-11)


def pin_gae_terminated_wins(lib):
    d = small_value_inputs(15, N=2, T=12, with_trunc=True)
    d["truncated"][:] = 0
    d["terminated"][:] = 0
    d["terminated"][1, 5] = 1
    base = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.9, lam=0.9,
                      lib=lib, **oracle_kw(d))
    d["truncated"][1, 5] = 1
    both = oracle.gae(d["rewards"], d["values"], d["terminated"], gamma=0.9, lam=0.9,
                      lib=lib, **oracle_kw(d))
    assert np.array_equal(base, both)
    # and at that step no bootstrap at all: A = r - V
    assert both[1, 5] == float(d["rewards"][1, 5]) - float(d["values"][1, 5])


# ------------------------------------------------------------ TD(lambda)
def lambda_brute(d, gamma, lam):
    g, l = fr(f32(gamma)), fr(f32(lam))
    N, T = d["rewards"].shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = first_cut(d, n, t)
            full = sum(g ** (k - t) * fr(d["rewards"][n, k]) for k in range(t, e + 1))
            full += g ** (e - t + 1) * vhat(d, n, e)
            mix = F(0)
            for m in range(1, e - t + 1):   # m-step returns that stop before the cut
                gm = sum(g ** k * fr(d["rewards"][n, t + k]) for k in range(m))
                gm += g ** m * fr(d["values"][n, t + m])
                mix += l ** (m - 1) * gm
            out[n, t] = float((1 - l) * mix + l ** (e - t) * full)
    return out


def pin_lambda_returns_brute(lib):
    for seed, trunc in ((20, True), (21, False)):
        d = small_value_inputs(seed, with_trunc=trunc)
        got = oracle.lambda_returns(d["rewards"], d["values"], d["terminated"], gamma=0.9,
                                    lam=0.7, lib=lib, **oracle_kw(d))
        close(got, lambda_brute(d, 0.9, 0.7))


def pin_lambda_returns_is_gae_plus_values(lib):
    d = small_value_inputs(22, N=6, T=80)
    kw = dict(gamma=0.99, lam=0.95, lib=lib, **oracle_kw(d))
    td = oracle.lambda_returns(d["rewards"], d["values"], d["terminated"], **kw)
    adv = oracle.gae(d["rewards"], d["values"], d["terminated"], **kw)
    close(td, adv + d["values"], 1e-11)


def pin_lambda_returns_limits(lib):
    d = small_value_inputs(23, N=4, T=50)
    g = f32(0.9)
    one = oracle.lambda_returns(d["rewards"], d["values"], d["terminated"], gamma=0.9,
                                lam=1.0, lib=lib, **oracle_kw(d))
    close(one, mc_return_lfilter(d["rewards"], vhat_array(d), cut_array(d), g), 1e-11)
    zero = oracle.lambda_returns(d["rewards"], d["values"], d["terminated"], gamma=0.9,
                                 lam=0.0, lib=lib, **oracle_kw(d))
    vnext = np.zeros_like(zero)
    vnext[:, :-1] = d["values"][:, 1:]
    vnext = np.where(cut_array(d), vhat_array(d), vnext)
    close(zero, d["rewards"] + g * vnext)


# ------------------------------------------------------------ discounted
def discounted_brute(d, gamma):
    g = fr(f32(gamma))
    N, T = d["rewards"].shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            e = first_cut(d, n, t)
            s = sum(g ** (k - t) * fr(d["rewards"][n, k]) for k in range(t, e + 1))
            out[n, t] = float(s + g ** (e - t + 1) * vhat(d, n, e))
    return out


def pin_discounted_brute(lib):
    for seed, trunc, boot in ((30, True, True), (31, False, False), (32, True, False)):
        d = small_value_inputs(seed, with_trunc=trunc, with_boot=boot)
        got = oracle.discounted_returns(d["rewards"], d["terminated"], gamma=0.85, lib=lib,
                                        **oracle_kw(d))
        close(got, discounted_brute(d, 0.85))


def pin_discounted_constant_reward(lib):
    N, T, c = 3, 200, 1.5
    g = f32(0.99)
    r = np.full((N, T), c, np.float32)
    got = oracle.discounted_returns(r, np.zeros((N, T), np.float32), gamma=0.99, lib=lib)
    t = np.arange(T)
    close(got, np.broadcast_to(c * (1 - g ** (T - t)) / (1 - g), (N, T)), 1e-12)


def pin_discounted_lfilter(lib):
    d = small_value_inputs(33, N=5, T=300, term_p=0.02, trunc_p=0.02)
    got = oracle.discounted_returns(d["rewards"], d["terminated"], gamma=0.999, lib=lib,
                                    **oracle_kw(d))
    close(got, mc_return_lfilter(d["rewards"], vhat_array(d), cut_array(d), f32(0.999)), 1e-11)


# ------------------------------------------------------------ V-trace
def vtrace_brute(d, gamma, rho_bar, c_bar, lam=1.0, rho_bar_pg=None):
    """IMPALA's explicit sum for vs (trace coefficients lambda*min(c_bar, ratio))
    and the policy-gradient advantage with weight min(rho_bar_pg, ratio)."""
    g = fr(f32(gamma))
    N, T = d["rewards"].shape
    def clip(level, n, t):
        ratio = F(math.exp(float(d["log_rhos"][n, t])))
        return ratio if math.isinf(level) else min(fr(f32(level)), ratio)

    rho = [[clip(rho_bar, n, t) for t in range(T)] for n in range(N)]
    c = [[fr(f32(lam)) * clip(c_bar, n, t) for t in range(T)] for n in range(N)]
    pg_level = rho_bar if rho_bar_pg is None else rho_bar_pg
    rho_pg = [[clip(pg_level, n, t) for t in range(T)] for n in range(N)]
    vs = [[None] * T for _ in range(N)]
    for n in range(N):
        for s in range(T):
            e = first_cut(d, n, s)
            acc, prod = F(0), F(1)
            for t in range(s, e + 1):
                delta = rho[n][t] * (fr(d["rewards"][n, t]) + g * vhat(d, n, t)
                                     - fr(d["values"][n, t]))
                acc += g ** (t - s) * prod * delta
                prod *= c[n][t]
            vs[n][s] = fr(d["values"][n, s]) + acc
    pg = np.zeros((N, T))
    for n in range(N):
        for s in range(T):
            follow = vhat(d, n, s) if cut(d, n, s) else vs[n][s + 1]
            pg[n, s] = float(rho_pg[n][s] * (fr(d["rewards"][n, s]) + g * follow
                                             - fr(d["values"][n, s])))
    return np.array([[float(v) for v in row] for row in vs]), pg


def pin_vtrace_brute(lib):
    for seed, trunc, clip in ((40, True, (1.0, 1.0)), (41, False, (1.5, 0.8)),
                              (42, True, (math.inf, math.inf))):
        d = small_value_inputs(seed, with_trunc=trunc)
        d["log_rhos"] = (0.7 * np.random.default_rng(seed).standard_normal(
            d["rewards"].shape)).astype(np.float32)
        vs, pg = oracle.vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                               gamma=0.9, rho_bar=clip[0], c_bar=clip[1], lib=lib,
                               **oracle_kw(d))
        want_vs, want_pg = vtrace_brute(d, 0.9, *clip)
        close(vs, want_vs)
        close(pg, want_pg)


def pin_vtrace_on_policy_is_discounted_return(lib):
    d = small_value_inputs(43, N=4, T=90)
    # log ratios >= 0, so rho = c = 1 with rho_bar = c_bar = 1
    d["log_rhos"] = np.abs(np.random.default_rng(43).standard_normal(
        d["rewards"].shape)).astype(np.float32)
    g = f32(0.97)
    vs, pg = oracle.vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                           gamma=0.97, lib=lib, **oracle_kw(d))
    mc = mc_return_lfilter(d["rewards"], vhat_array(d), cut_array(d), g)
    close(vs, mc, 1e-11)
    follow = np.zeros_like(mc)
    follow[:, :-1] = mc[:, 1:]
    follow = np.where(cut_array(d), vhat_array(d), follow)
    close(pg, d["rewards"] + g * follow - d["values"], 1e-11)


def pin_vtrace_no_trace_is_one_step(lib):
    d = small_value_inputs(44, N=3, T=30)
    d["log_rhos"] = (0.5 * np.random.default_rng(44).standard_normal(
        d["rewards"].shape)).astype(np.float32)
    g = f32(0.9)
    vs, _ = oracle.vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                          gamma=0.9, rho_bar=1.0, c_bar=0.0, lib=lib, **oracle_kw(d))
    rho = np.minimum(1.0, np.exp(d["log_rhos"].astype(np.float64)))
    vnext = np.zeros_like(vs)
    vnext[:, :-1] = d["values"][:, 1:]
    vnext = np.where(cut_array(d), vhat_array(d), vnext)
    close(vs, d["values"] + rho * (d["rewards"] + g * vnext - d["values"]))


def _vtrace_inputs(seed, scale=0.7, **kw):
    d = small_value_inputs(seed, **kw)
    d["log_rhos"] = (scale * np.random.default_rng(seed).standard_normal(
        d["rewards"].shape)).astype(np.float32)
    return d


def pin_vtrace_lambda_and_pg_clip_brute(lib):
    """IMPALA's lambda variant and a separate policy-gradient truncation
    level, against the explicit sum in exact rationals."""
    for seed, trunc, (rho_bar, c_bar, lam, rho_bar_pg) in (
            (45, True, (1.0, 1.0, 0.8, 0.5)),
            (46, False, (1.5, 0.9, 0.3, math.inf)),
            (47, True, (math.inf, 1.2, 0.95, 2.0))):
        d = _vtrace_inputs(seed, with_trunc=trunc)
        vs, pg = oracle.vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                               gamma=0.9, rho_bar=rho_bar, c_bar=c_bar, lam=lam,
                               rho_bar_pg=rho_bar_pg, lib=lib, **oracle_kw(d))
        want_vs, want_pg = vtrace_brute(d, 0.9, rho_bar, c_bar, lam, rho_bar_pg)
        close(vs, want_vs)
        close(pg, want_pg)


def pin_vtrace_lambda_zero_is_one_step(lib):
    """lambda = 0 switches the traces off: vs_t = V_t + rho_t*(r_t + gamma*Vhat_{t+1} - V_t)."""
    d = _vtrace_inputs(48, 0.5, N=3, T=30)
    g = f32(0.9)
    vs, _ = oracle.vtrace(d["rewards"], d["values"], d["log_rhos"], d["terminated"],
                          gamma=0.9, rho_bar=1.0, c_bar=1.0, lam=0.0, lib=lib, **oracle_kw(d))
    rho = np.minimum(1.0, np.exp(d["log_rhos"].astype(np.float64)))
    vnext = np.zeros_like(vs)
    vnext[:, :-1] = d["values"][:, 1:]
    vnext = np.where(cut_array(d), vhat_array(d), vnext)
    close(vs, d["values"] + rho * (d["rewards"] + g * vnext - d["values"]))


def pin_vtrace_lambda_scales_c_bar(lib):
    """Where every ratio is at least c_bar, c_t = lambda*c_bar for every t, which
    is the plain form with truncation level lambda*c_bar (lambda = 0.5, so the
    product is exact in float32)."""
    d = _vtrace_inputs(49, 0.5, N=3, T=60)
    d["log_rhos"] = (np.abs(d["log_rhos"]) + np.float32(math.log(0.8) + 1e-3)).astype(
        np.float32)
    kw = dict(gamma=0.95, rho_bar=1.0, lib=lib, **oracle_kw(d))
    args = (d["rewards"], d["values"], d["log_rhos"], d["terminated"])
    vs_l, pg_l = oracle.vtrace(*args, c_bar=0.8, lam=0.5, **kw)
    vs_c, pg_c = oracle.vtrace(*args, c_bar=0.4, **kw)
    close(vs_l, vs_c, 1e-14)
    close(pg_l, pg_c, 1e-14)
    vs_1, _ = oracle.vtrace(*args, c_bar=0.8, **kw)
    assert np.abs(vs_1 - vs_l).max() > 1e-3  # lambda does act


def pin_vtrace_pg_clip_only_rescales_pg(lib):
    """rho_bar_pg leaves vs unchanged and multiplies each pg_t by
    min(rho_bar_pg, ratio_t) / min(rho_bar, ratio_t)."""
    d = _vtrace_inputs(50, 1.0, N=3, T=40)
    args = (d["rewards"], d["values"], d["log_rhos"], d["terminated"])
    kw = dict(gamma=0.97, rho_bar=1.0, c_bar=1.0, lam=0.9, lib=lib, **oracle_kw(d))
    vs_a, pg_a = oracle.vtrace(*args, **kw)
    vs_b, pg_b = oracle.vtrace(*args, rho_bar_pg=0.6, **kw)
    assert np.array_equal(vs_a, vs_b)
    ratio = np.exp(d["log_rhos"].astype(np.float64))
    close(pg_b, pg_a * np.minimum(f32(0.6), ratio) / np.minimum(1.0, ratio), 1e-13)


# ------------------------------------------------------------ Retrace
def small_retrace_inputs(seed, N=3, T=10, A=4, term_p=0.15, trunc_p=0.15):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((N, T, A))
    p = np.exp(logits)
    p /= p.sum(-1, keepdims=True)
    d = {
        "rewards": rng.standard_normal((N, T)).astype(np.float32),
        "next_q": rng.standard_normal((N, T, A)).astype(np.float32),
        "next_pi": p.astype(np.float32),
        "actions": rng.integers(0, A, (N, T)).astype(np.int32),
        "mu": rng.uniform(0.05, 1.0, (N, T)).astype(np.float32),
        "terminated": (rng.random((N, T)) < term_p).astype(np.float32),
        "truncated": (rng.random((N, T)) < trunc_p).astype(np.float32),
    }
    d["terminated"][0, 3] = d["truncated"][0, 3] = 1.0
    return d


def call_retrace(d, gamma, lam, lib):
    return oracle.retrace(d["rewards"], d["next_q"], d["next_pi"], d["actions"], d["mu"],
                          d["terminated"], d["truncated"], gamma=gamma, lam=lam, lib=lib)


def retrace_brute(d, gamma, lam):
    g, l = fr(f32(gamma)), fr(f32(lam))
    N, T = d["rewards"].shape
    A = d["next_q"].shape[2]

    def eq(n, t):
        return sum(fr(d["next_pi"][n, t, a]) * fr(d["next_q"][n, t, a]) for a in range(A))

    def x(n, t):
        return fr(d["rewards"][n, t]) + (F(0) if flag(d["terminated"], n, t) else g * eq(n, t))

    def c(n, i):
        a = d["actions"][n, i]
        return l * min(F(1), fr(d["next_pi"][n, i - 1, a]) / fr(d["mu"][n, i]))

    out = np.zeros((N, T))
    for n in range(N):
        for s in range(T):
            e = first_cut(d, n, s)
            total, prod = x(n, s), F(1)
            for t in range(s + 1, e + 1):
                prod *= c(n, t)
                total += g ** (t - s) * prod * (x(n, t)
                                                - fr(d["next_q"][n, t - 1, d["actions"][n, t]]))
            out[n, s] = float(total)
    return out


def pin_retrace_brute(lib):
    for seed, A in ((50, 4), (51, 6), (52, 1)):
        d = small_retrace_inputs(seed, A=A)
        close(call_retrace(d, 0.9, 0.8, lib), retrace_brute(d, 0.9, 0.8))


def pin_retrace_lambda0(lib):
    d = small_retrace_inputs(53, N=4, T=40, A=6)
    g = f32(0.99)
    got = call_retrace(d, 0.99, 0.0, lib)
    eq = (d["next_pi"].astype(np.float64) * d["next_q"]).sum(-1)
    close(got, d["rewards"] + g * (1 - d["terminated"]) * eq)


def pin_retrace_onehot_on_policy(lib):
    """lambda = 1, mu = 1 and a target policy that puts all its mass on the
    action taken next: every trace coefficient is 1 and the target is the
    discounted return, bootstrapped by E_pi Q at a truncation/row end and by
    0 at a termination."""
    d = small_retrace_inputs(54, N=4, T=60, A=5, term_p=0.05, trunc_p=0.05)
    N, T, A = d["next_q"].shape
    d["mu"][:] = 1.0
    p = np.zeros((N, T, A), np.float32)
    nxt = np.concatenate([d["actions"][:, 1:], d["actions"][:, :1]], axis=1)
    p[np.arange(N)[:, None], np.arange(T)[None, :], nxt] = 1.0
    d["next_pi"] = p
    g = f32(0.95)
    got = call_retrace(d, 0.95, 1.0, lib)
    cuts = (d["terminated"] != 0) | (d["truncated"] != 0)
    cuts[:, -1] = True
    eq = d["next_q"][np.arange(N)[:, None], np.arange(T)[None, :], nxt].astype(np.float64)
    boot = np.where(d["terminated"] != 0, 0.0, eq)
    close(got, mc_return_lfilter(d["rewards"], boot, cuts, g), 1e-11)


# ------------------------------------------------------------ traces
def pin_eligibility_brute(lib):
    rng = np.random.default_rng(60)
    N, T = 4, 12
    x = rng.standard_normal((N, T)).astype(np.float32)
    dn = (rng.random((N, T)) < 0.25).astype(np.float32)
    gl = fr(f32(0.9)) * fr(f32(0.8))
    want = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            s = t
            while s > 0 and dn[n, s] == 0:
                s -= 1
            want[n, t] = float(sum(gl ** (t - k) * fr(x[n, k]) for k in range(s, t + 1)))
    close(oracle.eligibility_traces(x, dn, gamma=0.9, lam=0.8, lib=lib), want)


def pin_eligibility_limits(lib):
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3, 100)).astype(np.float32)
    none = np.zeros_like(x)
    close(oracle.eligibility_traces(x, none, gamma=1.0, lam=1.0, lib=lib),
          np.cumsum(x.astype(np.float64), axis=1), 1e-12)
    assert np.array_equal(oracle.eligibility_traces(x, np.ones_like(x), gamma=0.9, lam=0.9,
                                                    lib=lib), x.astype(np.float64))
    g = f32(0.5)
    close(oracle.eligibility_traces(x, none, gamma=0.5, lam=1.0, lib=lib),
          lfilter([1.0], [1.0, -g], x.astype(np.float64), axis=1))


# ------------------------------------------------------------ prefix sum
def segment_cumsum(x, dones):
    out = np.empty(x.shape, np.int64)
    for n in range(x.shape[0]):
        starts = sorted(set([0] + list(np.flatnonzero(dones[n] != 0))))
        ends = starts[1:] + [x.shape[1]]
        for s, e in zip(starts, ends):
            out[n, s:e] = np.cumsum(x[n, s:e], dtype=np.int64)
    return out


def pin_prefix_sum(lib):
    rng = np.random.default_rng(70)
    x = rng.integers(-8, 9, (5, 300)).astype(np.int32)
    d = (rng.random((5, 300)) < 0.03).astype(np.float32)
    assert np.array_equal(oracle.episodic_prefix_sum(x, d, lib=lib), segment_cumsum(x, d))
    none = np.zeros_like(d)
    assert np.array_equal(oracle.episodic_prefix_sum(x, none, lib=lib),
                          np.cumsum(x, axis=1, dtype=np.int64))
    assert np.array_equal(oracle.episodic_prefix_sum(x, np.ones_like(d), lib=lib),
                          x.astype(np.int64))
    big = np.full((1, 4), 2**31 - 1, np.int32)
    assert oracle.episodic_prefix_sum(big, np.zeros((1, 4), np.float32), lib=lib)[0, -1] \
        == 4 * (2**31 - 1)


def segment_cumsum_float(x, dones):
    out = np.empty(x.shape, np.float64)
    for n in range(x.shape[0]):
        starts = sorted(set([0] + list(np.flatnonzero(dones[n] != 0))))
        ends = starts[1:] + [x.shape[1]]
        for s, e in zip(starts, ends):
            out[n, s:e] = np.cumsum(x[n, s:e].astype(np.float64))
    return out


def pin_prefix_sum_float(lib):
    """Float values: per-episode numpy.cumsum in float64; all-done is x; no
    done is the whole-row cumsum; a carry enters only the first episode."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    d = (rng.random((5, 300)) < 0.03).astype(np.float32)
    close(oracle.episodic_prefix_sum_float(x, d, lib=lib), segment_cumsum_float(x, d), 1e-14)
    none = np.zeros_like(d)
    close(oracle.episodic_prefix_sum_float(x, none, lib=lib),
          np.cumsum(x.astype(np.float64), axis=1), 1e-14)
    assert np.array_equal(oracle.episodic_prefix_sum_float(x, np.ones_like(d), lib=lib),
                          x.astype(np.float64))
    ci = rng.standard_normal(5).astype(np.float32)
    got, co = oracle.episodic_prefix_sum_float(x, d, carry_in=ci, return_carry=True, lib=lib)
    want = segment_cumsum_float(x, d)
    for n in range(5):
        first = np.flatnonzero(d[n] != 0)
        stop = first[0] if first.size else 300
        want[n, :stop] += np.float64(ci[n])
    close(got, want, 1e-13)
    assert np.array_equal(co, got[:, -1])


# ------------------------------------------------------------ carry (chunking)
# Streaming one rollout through several calls must give the whole-rollout
# result: the chunk after a split point is computed first (reverse
# estimators) and hands its edge output to the chunk before it as carry_in;
# forward estimators hand it the other way.  The whole-rollout oracle is
# pinned by the brute-force and closed-form pins above, so these pin the
# carry arguments to it.  The carry crosses the call in float32 (as on the
# GPU), hence the tolerance; a dropped or misplaced carry errs by O(1).
CARRY_TOL = 1e-6


def split_points(T):
    return (1, 2, T // 2, T - 1)


def _force_edge_flags(d, T1):
    """Make the step just before the split terminated in row 0 and
    truncated in row 1, so the carry must be ignored there."""
    if d.get("terminated") is not None:
        d["terminated"][0, T1 - 1] = 1.0
    if d.get("truncated") is not None:
        d["truncated"][1, T1 - 1] = 1.0


def _cols(d, lo, hi):
    out = {}
    for k, v in d.items():
        if v is None or k == "bootstrap_value":
            out[k] = v
        elif isinstance(v, np.ndarray) and v.ndim >= 2:
            out[k] = np.ascontiguousarray(v[:, lo:hi])
        else:
            out[k] = v
    return out


def _reverse_chunk_pin(lib, fn, keys, d, gamma_kw, two_outputs=False):
    T = d["rewards"].shape[1]
    whole = fn(**{k: d[k] for k in keys}, **gamma_kw, lib=lib)
    for T1 in split_points(T):
        late = _cols(d, T1, T)
        early = _cols(d, 0, T1)
        res_late = fn(**{k: late[k] for k in keys}, **gamma_kw, return_carry=True, lib=lib)
        carry = res_late[-1].astype(np.float32)
        if "values" in d:  # V at the split point is the early chunk's bootstrap
            early["bootstrap_value"] = np.ascontiguousarray(d["values"][:, T1])
        res_early = fn(**{k: early[k] for k in keys}, **gamma_kw, carry_in=carry,
                       return_carry=True, lib=lib)
        outs_whole = whole if two_outputs else (whole,)
        for i, w in enumerate(outs_whole):
            got = np.concatenate([res_early[i], res_late[i]], axis=1)
            close(got, w, CARRY_TOL)
        close(res_early[-1], res_early[0][:, 0], 0.0)  # carry_out is the t = 0 output


def _reverse_data(seed, with_values=True):
    d = small_value_inputs(seed, N=3, T=12)
    if not with_values:
        d.pop("values")
    return d


def pin_gae_chunked(lib):
    for T1 in (5,):
        d = _reverse_data(41)
        _force_edge_flags(d, T1)
        _reverse_chunk_pin(lib, oracle.gae, ("rewards", "values", "terminated",
                                             "bootstrap_value", "truncated",
                                             "bootstrap_values"), d,
                           dict(gamma=0.97, lam=0.9))
    _reverse_chunk_pin(lib, oracle.gae, ("rewards", "values", "terminated", "bootstrap_value",
                                         "truncated", "bootstrap_values"), _reverse_data(42),
                       dict(gamma=0.97, lam=0.9))


def pin_lambda_returns_chunked(lib):
    d = _reverse_data(43)
    _force_edge_flags(d, 6)
    _reverse_chunk_pin(lib, oracle.lambda_returns, ("rewards", "values", "terminated",
                                                    "bootstrap_value", "truncated",
                                                    "bootstrap_values"), d,
                       dict(gamma=0.95, lam=0.8))


def pin_discounted_chunked(lib):
    d = _reverse_data(44)
    _force_edge_flags(d, 6)
    # the split point's V_T is not an input of discounted returns: the early
    # chunk continues straight into the carried return
    _reverse_chunk_pin(lib, oracle.discounted_returns,
                       ("rewards", "terminated", "bootstrap_value", "truncated",
                        "bootstrap_values"), {k: v for k, v in d.items() if k != "values"},
                       dict(gamma=0.93))


def pin_vtrace_chunked(lib):
    d = _reverse_data(45)
    _force_edge_flags(d, 6)
    rng = np.random.default_rng(46)
    d["log_rhos"] = (0.5 * rng.standard_normal(d["rewards"].shape)).astype(np.float32)
    _reverse_chunk_pin(lib, oracle.vtrace, ("rewards", "values", "log_rhos", "terminated",
                                            "bootstrap_value", "truncated",
                                            "bootstrap_values"), d,
                       dict(gamma=0.96, rho_bar=1.0, c_bar=0.9), two_outputs=True)


def pin_retrace_chunked(lib):
    d = small_retrace_inputs(47, N=3, T=12)
    T = 12
    whole = call_retrace(d, 0.95, 0.85, lib)
    for T1 in split_points(T):
        e = {k: np.ascontiguousarray(v[:, :T1]) for k, v in d.items()}
        l = {k: np.ascontiguousarray(v[:, T1:]) for k, v in d.items()}
        if T1 == T // 2:
            e["terminated"][0, -1] = 1.0
            e["truncated"][1, -1] = 1.0
            dd = {k: v.copy() for k, v in d.items()}
            dd["terminated"][0, T1 - 1] = dd["truncated"][1, T1 - 1] = 1.0
            ref = call_retrace(dd, 0.95, 0.85, lib)
        else:
            ref = whole
        tl, carry = oracle.retrace(l["rewards"], l["next_q"], l["next_pi"], l["actions"],
                                   l["mu"], l["terminated"], l["truncated"], gamma=0.95,
                                   lam=0.85, return_carry=True, lib=lib)
        te, co = oracle.retrace(e["rewards"], e["next_q"], e["next_pi"], e["actions"], e["mu"],
                                e["terminated"], e["truncated"], gamma=0.95, lam=0.85,
                                carry_in=carry.astype(np.float32),
                                next_actions=d["actions"][:, T1],
                                next_behaviour_probs=d["mu"][:, T1], return_carry=True,
                                lib=lib)
        close(np.concatenate([te, tl], axis=1), ref, CARRY_TOL)
        close(co, te[:, 0], 0.0)


def pin_eligibility_chunked(lib):
    rng = np.random.default_rng(48)
    x = rng.standard_normal((3, 12)).astype(np.float32)
    dones = (rng.random((3, 12)) < 0.2).astype(np.float32)
    whole = oracle.eligibility_traces(x, dones, gamma=0.9, lam=0.8, lib=lib)
    for T1 in split_points(12):
        dd = dones.copy()
        if T1 == 6:
            dd[0, T1] = 1.0  # the later chunk's first step drops the carry
        ref = oracle.eligibility_traces(x, dd, gamma=0.9, lam=0.8, lib=lib)
        e, co = oracle.eligibility_traces(x[:, :T1], dd[:, :T1], gamma=0.9, lam=0.8,
                                          return_carry=True, lib=lib)
        l = oracle.eligibility_traces(np.ascontiguousarray(x[:, T1:]),
                                      np.ascontiguousarray(dd[:, T1:]), gamma=0.9, lam=0.8,
                                      carry_in=co.astype(np.float32), lib=lib)
        close(np.concatenate([e, l], axis=1), ref, CARRY_TOL)
        close(co, e[:, -1], 0.0)
    assert np.array_equal(whole, oracle.eligibility_traces(x, dones, gamma=0.9, lam=0.8,
                                                           lib=lib))


def pin_prefix_sum_chunked(lib):
    rng = np.random.default_rng(49)
    x = rng.integers(-8, 9, (3, 12)).astype(np.int32)
    dones = (rng.random((3, 12)) < 0.2).astype(np.float32)
    for T1 in split_points(12):
        dd = dones.copy()
        if T1 == 6:
            dd[1, T1] = 1.0
        ref = segment_cumsum(x, dd)
        e, co = oracle.episodic_prefix_sum(x[:, :T1], dd[:, :T1], return_carry=True, lib=lib)
        l = oracle.episodic_prefix_sum(np.ascontiguousarray(x[:, T1:]),
                                       np.ascontiguousarray(dd[:, T1:]), carry_in=co, lib=lib)
        assert np.array_equal(np.concatenate([e, l], axis=1), ref)
        assert np.array_equal(co, e[:, -1])


PINS = {
    "operator": [pin_operator_associative, pin_operator_identity_and_meaning,
                 pin_linear_recurrence_brute],
    "gae": [pin_gae_brute, pin_gae_lambda0_is_td_error,
            pin_gae_lambda1_is_mc_return_minus_value, pin_gae_terminated_wins,
            pin_gae_chunked],
    "lambda_returns": [pin_lambda_returns_brute, pin_lambda_returns_is_gae_plus_values,
                       pin_lambda_returns_limits, pin_lambda_returns_chunked],
    "discounted_returns": [pin_discounted_brute, pin_discounted_constant_reward,
                           pin_discounted_lfilter, pin_discounted_chunked],
    "vtrace": [pin_vtrace_brute, pin_vtrace_on_policy_is_discounted_return,
               pin_vtrace_no_trace_is_one_step, pin_vtrace_chunked,
               pin_vtrace_lambda_and_pg_clip_brute, pin_vtrace_lambda_zero_is_one_step,
               pin_vtrace_lambda_scales_c_bar, pin_vtrace_pg_clip_only_rescales_pg],
    "retrace": [pin_retrace_brute, pin_retrace_lambda0, pin_retrace_onehot_on_policy,
                pin_retrace_chunked],
    "eligibility_traces": [pin_eligibility_brute, pin_eligibility_limits,
                           pin_eligibility_chunked],
    "episodic_prefix_sum": [pin_prefix_sum, pin_prefix_sum_chunked],
    "episodic_prefix_sum_float": [pin_prefix_sum_float],
}
