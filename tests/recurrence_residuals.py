"""Checks of a computed result against its own recurrence, element by element,
at sizes the oracle cannot take whole.

Each estimator's output satisfies one step of its defining recursion
(rl-triton README, section Kernels: GAE's advantage recursion, the
eligibility-trace recursion with its done reset, the episodic prefix sum).
Given the inputs and the output, the step's residual is computed in float64
(int64 for the prefix sum) with torch on whatever device holds the tensors,
in pieces of bounded size.

Bound for float outputs: if every element x_t meets the parity bar
|x_t - ref_t| <= rtol * (1 + |ref_t|), the residual of a step
x_t - b_t - a_t * x_prev (|a_t| <= 1) is at most
rtol * (2 + |x_t| + |x_prev|) up to second-order terms; a residual above that
means some element misses the bar.  The prefix sum's residual must be zero.
The checks find a wrong element anywhere, but not a uniform error that every
step shares (a wrong gamma, say): the sampled oracle windows cover that.
"""
from __future__ import annotations

import torch

PIECE = 1 << 25  # elements per piece


def _pieces(N: int, T: int):
    """(r0, r1, t0, t1) blocks of at most PIECE elements covering [N, T]."""
    if T <= PIECE:
        rows = max(1, PIECE // T)
        for r0 in range(0, N, rows):
            yield r0, min(N, r0 + rows), 0, T
    else:
        for r in range(N):
            for t0 in range(0, T, PIECE):
                yield r, r + 1, t0, min(T, t0 + PIECE)


def _flag(f, r0, r1, t0, t1):
    return f[r0:r1, t0:t1] != 0


def _next(x, r0, r1, t0, t1, last):
    """x[:, t+1] for t in [t0, t1); `last` ([rows] float64) stands in at t = T-1."""
    T = x.shape[1]
    if t1 < T:
        return x[r0:r1, t0 + 1:t1 + 1].double()
    return torch.cat([x[r0:r1, t0 + 1:T].double(), last[:, None]], dim=1)


def _prev(x, r0, r1, t0, t1, dtype):
    """x[:, t-1] for t in [t0, t1), with 0 at t = 0."""
    head = (x[r0:r1, t0 - 1:t0].to(dtype) if t0 > 0
            else torch.zeros(r1 - r0, 1, dtype=dtype, device=x.device))
    return torch.cat([head, x[r0:r1, t0:t1 - 1].to(dtype)], dim=1)


def _worst(res, bound):
    ratio = (res.abs() / bound).flatten()
    i = int(torch.argmax(ratio))
    return float(ratio[i]), i


def gae_residual(adv, rewards, values, terminated, bootstrap_value, gamma, lam, rtol=1e-4):
    """Largest |residual| / bound of A_t = delta_t + gamma*lam*(1 - cut_t)*A_{t+1}
    over every element (no truncation: cut_t is terminated_t or t = T-1), and
    where it is, as (ratio, (row, t))."""
    N, T = adv.shape
    g, gl = float(gamma), float(gamma) * float(lam)
    worst, where = 0.0, None
    for r0, r1, t0, t1 in _pieces(N, T):
        a = adv[r0:r1, t0:t1].double()
        zero = torch.zeros(r1 - r0, dtype=torch.float64, device=adv.device)
        a_next = _next(adv, r0, r1, t0, t1, zero)
        boot = (bootstrap_value[r0:r1].double() if bootstrap_value is not None else zero)
        v_next = _next(values, r0, r1, t0, t1, boot)
        term = _flag(terminated, r0, r1, t0, t1)
        t_idx = torch.arange(t0, t1, device=adv.device)
        cut = term | (t_idx == T - 1)[None, :]
        v_hat = torch.where(term, torch.zeros_like(v_next), v_next)
        delta = rewards[r0:r1, t0:t1].double() + g * v_hat - values[r0:r1, t0:t1].double()
        res = a - delta - gl * torch.where(cut, torch.zeros_like(a_next), a_next)
        ratio, i = _worst(res, rtol * (2.0 + a.abs() + a_next.abs()))
        if ratio > worst:
            worst, where = ratio, (r0 + i // (t1 - t0), t0 + i % (t1 - t0))
    return worst, where


def traces_residual(traces, x, dones, gamma, lam, rtol=1e-4):
    """Largest |residual| / bound of e_t = x_t + gamma*lam*(1 - d_t)*e_{t-1}
    (e_{-1} = 0), and where it is."""
    N, T = traces.shape
    gl = float(gamma) * float(lam)
    worst, where = 0.0, None
    for r0, r1, t0, t1 in _pieces(N, T):
        e = traces[r0:r1, t0:t1].double()
        prev = _prev(traces, r0, r1, t0, t1, torch.float64)
        d = _flag(dones, r0, r1, t0, t1)
        res = e - x[r0:r1, t0:t1].double() - gl * torch.where(d, torch.zeros_like(prev), prev)
        ratio, i = _worst(res, rtol * (2.0 + e.abs() + prev.abs()))
        if ratio > worst:
            worst, where = ratio, (r0 + i // (t1 - t0), t0 + i % (t1 - t0))
    return worst, where


def prefix_sum_mismatches(out, x, dones):
    """Elements where y_t != x_t + (1 - d_t)*y_{t-1} (y_{-1} = 0), int64, and
    the first of them as (row, t) or None."""
    N, T = out.shape
    bad, first = 0, None
    for r0, r1, t0, t1 in _pieces(N, T):
        y = out[r0:r1, t0:t1]
        prev = _prev(out, r0, r1, t0, t1, torch.int64)
        d = _flag(dones, r0, r1, t0, t1)
        want = x[r0:r1, t0:t1].long() + torch.where(d, torch.zeros_like(prev), prev)
        wrong = (y != want).flatten()
        k = int(wrong.sum())
        if k and first is None:
            i = int(torch.nonzero(wrong)[0])
            first = (r0 + i // (t1 - t0), t0 + i % (t1 - t0))
        bad += k
    return bad, first
