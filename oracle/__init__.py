"""Float64 CPU oracle for the seven credit-assignment estimators.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  The arithmetic
lives in ``oracle.c`` (plain sequential C loops, one per estimator, each
citing the passage it follows); this module only compiles it, loads it with
ctypes and marshals numpy arrays.

Every float input is passed exactly as the float32 array the GPU receives and
every parameter (gamma, lambda, clip levels) as the same float32 value, which
the C code widens to double.  Outputs are float64 (int64 for the prefix sum).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load_library(path: str = _LIB_PATH, rebuild: bool = False):
    """Load (building first if absent) and declare the C signatures."""
    global _lib
    if _lib is not None and path == _LIB_PATH and not rebuild:
        return _lib
    if rebuild or not os.path.exists(path) or (
            path == _LIB_PATH and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    lib.oracle_op_compose.argtypes = [ctypes.c_double] * 4 + [_f64p, _f64p]
    lib.oracle_op_compose.restype = None
    lib.oracle_op_compose_i64.argtypes = [_i64] * 4 + [_i64p, _i64p]
    lib.oracle_op_compose_i64.restype = None
    lib.oracle_linear_recurrence.argtypes = [_i64, _i64, ctypes.c_int, _f64p, _f64p, _f64p]
    lib.oracle_linear_recurrence.restype = None
    # every estimator: ..., carry_in (or NULL), outputs..., carry_out (or NULL)
    lib.oracle_gae.argtypes = [_i64, _i64, _f32, _f32] + [_f32p] * 7 + [_f64p, _f64p]
    lib.oracle_gae.restype = None
    lib.oracle_lambda_returns.argtypes = [_i64, _i64, _f32, _f32] + [_f32p] * 7 + [_f64p, _f64p]
    lib.oracle_lambda_returns.restype = None
    lib.oracle_discounted_returns.argtypes = [_i64, _i64, _f32] + [_f32p] * 6 + [_f64p, _f64p]
    lib.oracle_discounted_returns.restype = None
    lib.oracle_vtrace.argtypes = ([_i64, _i64, _f32, _f32, _f32, _f32, _f32] + [_f32p] * 8
                                  + [_f64p, _f64p, _f64p])
    lib.oracle_vtrace.restype = None
    lib.oracle_retrace.argtypes = ([_i64, _i64, _i64, _f32, _f32, _f32p, _f32p, _f32p, _i32p]
                                   + [_f32p] * 4 + [_i32p, _f32p, _f64p, _f64p])
    lib.oracle_retrace.restype = ctypes.c_int
    lib.oracle_eligibility_traces.argtypes = [_i64, _i64, _f32, _f32, _f32p, _f32p, _f32p,
                                              _f64p, _f64p]
    lib.oracle_eligibility_traces.restype = None
    lib.oracle_episodic_prefix_sum.argtypes = [_i64, _i64, _i32p, _f32p, _i64p, _i64p, _i64p]
    lib.oracle_episodic_prefix_sum.restype = None
    lib.oracle_episodic_prefix_sum_float.argtypes = [_i64, _i64, _f32p, _f32p, _f32p, _f64p,
                                                     _f64p]
    lib.oracle_episodic_prefix_sum_float.restype = None
    if path == _LIB_PATH:
        _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling
def _f32_in(x, shape=None):
    if x is None:
        return None, None
    arr = np.ascontiguousarray(x, dtype=np.float32)
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {arr.shape}")
    return arr, arr.ctypes.data_as(_f32p)


def _ptr(pair):
    return pair[1]


def _shape2(x):
    arr = np.asarray(x)
    if arr.ndim != 2:
        raise ValueError("expected a [N, T] array")
    return arr.shape


def _param(v) -> float:
    """The float32 value the GPU receives, as a Python float."""
    return float(np.float32(v))


def compose(left, right, lib=None):
    """(aL, bL) o (aE, bE) in float64: apply `right` first, then `left`."""
    lib = lib or load_library()
    a, b = ctypes.c_double(), ctypes.c_double()
    lib.oracle_op_compose(float(left[0]), float(left[1]), float(right[0]), float(right[1]),
                          ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def compose_i64(left, right, lib=None):
    lib = lib or load_library()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    lib.oracle_op_compose_i64(int(left[0]), int(left[1]), int(right[0]), int(right[1]),
                              ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def linear_recurrence(a, b, reverse: bool, lib=None):
    """Sequential x_t = a_t x_{t+-1} + b_t per row, float64, zero initial state."""
    lib = lib or load_library()
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    if a.shape != b.shape or a.ndim != 2:
        raise ValueError("a and b must be [N, T] arrays of equal shape")
    out = np.empty_like(a)
    N, T = a.shape
    lib.oracle_linear_recurrence(N, T, int(bool(reverse)), a.ctypes.data_as(_f64p),
                                 b.ctypes.data_as(_f64p), out.ctypes.data_as(_f64p))
    return out


def _reverse_inputs(rewards, values, bootstrap_value, terminated, truncated,
                    bootstrap_values):
    N, T = _shape2(rewards)
    r = _f32_in(rewards, (N, T))
    v = _f32_in(values, (N, T)) if values is not None else (None, None)
    bv = _f32_in(bootstrap_value, (N,))
    term = _f32_in(terminated, (N, T))
    trunc = _f32_in(truncated, (N, T))
    bvals = _f32_in(bootstrap_values, (N, T))
    if trunc[0] is not None and bvals[0] is None:
        raise ValueError("bootstrap_values is required when truncated is given")
    return N, T, r, v, bv, term, trunc, bvals


# Carry (streaming one rollout through several calls; see oracle.c):
# `carry_in` [N] is the output just past the chunk (t = T reverse, t = -1
# forward), or None for whole rollouts; with return_carry=True the call also
# returns carry_out [N], the output at the chunk's other edge.
def _carry_in(carry_in, N):
    return _f32_in(carry_in, (N,))


def _with_carry(result, carry_out, return_carry):
    if not return_carry:
        return result
    return (*result, carry_out) if isinstance(result, tuple) else (result, carry_out)


def gae(rewards, values, terminated, *, gamma, lam, bootstrap_value=None,
        truncated=None, bootstrap_values=None, carry_in=None, return_carry=False, lib=None):
    lib = lib or load_library()
    N, T, r, v, bv, term, trunc, bvals = _reverse_inputs(
        rewards, values, bootstrap_value, terminated, truncated, bootstrap_values)
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    lib.oracle_gae(N, T, _param(gamma), _param(lam), _ptr(r), _ptr(v), _ptr(bv), _ptr(term),
                   _ptr(trunc), _ptr(bvals), _ptr(_carry_in(carry_in, N)),
                   out.ctypes.data_as(_f64p), co.ctypes.data_as(_f64p))
    return _with_carry(out, co, return_carry)


def lambda_returns(rewards, values, terminated, *, gamma, lam, bootstrap_value=None,
                   truncated=None, bootstrap_values=None, carry_in=None, return_carry=False,
                   lib=None):
    lib = lib or load_library()
    N, T, r, v, bv, term, trunc, bvals = _reverse_inputs(
        rewards, values, bootstrap_value, terminated, truncated, bootstrap_values)
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    lib.oracle_lambda_returns(N, T, _param(gamma), _param(lam), _ptr(r), _ptr(v), _ptr(bv),
                              _ptr(term), _ptr(trunc), _ptr(bvals),
                              _ptr(_carry_in(carry_in, N)), out.ctypes.data_as(_f64p),
                              co.ctypes.data_as(_f64p))
    return _with_carry(out, co, return_carry)


def discounted_returns(rewards, terminated, *, gamma, bootstrap_value=None, truncated=None,
                       bootstrap_values=None, carry_in=None, return_carry=False, lib=None):
    lib = lib or load_library()
    N, T, r, _, bv, term, trunc, bvals = _reverse_inputs(
        rewards, None, bootstrap_value, terminated, truncated, bootstrap_values)
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    lib.oracle_discounted_returns(N, T, _param(gamma), _ptr(r), _ptr(bv), _ptr(term),
                                  _ptr(trunc), _ptr(bvals), _ptr(_carry_in(carry_in, N)),
                                  out.ctypes.data_as(_f64p), co.ctypes.data_as(_f64p))
    return _with_carry(out, co, return_carry)


def vtrace(rewards, values, log_rhos, terminated, *, gamma, rho_bar=1.0, c_bar=1.0,
           bootstrap_value=None, truncated=None, bootstrap_values=None, carry_in=None,
           return_carry=False, lam=1.0, rho_bar_pg=None, lib=None):
    """Returns (vs, pg_advantages), both float64 [N, T] (and carry_out, the
    vs at t = 0, with return_carry); carry_in is vs at t = T.  lam scales
    every trace coefficient c_t; rho_bar_pg (None: rho_bar) truncates the
    policy-gradient weight."""
    lib = lib or load_library()
    N, T, r, v, bv, term, trunc, bvals = _reverse_inputs(
        rewards, values, bootstrap_value, terminated, truncated, bootstrap_values)
    lr = _f32_in(log_rhos, (N, T))
    vs = np.empty((N, T), np.float64)
    pg = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    pg_clip = rho_bar if rho_bar_pg is None else rho_bar_pg
    lib.oracle_vtrace(N, T, _param(gamma), _param(lam), _param(rho_bar), _param(c_bar),
                      _param(pg_clip), _ptr(r), _ptr(v),
                      _ptr(bv), _ptr(lr), _ptr(term), _ptr(trunc), _ptr(bvals),
                      _ptr(_carry_in(carry_in, N)), vs.ctypes.data_as(_f64p),
                      pg.ctypes.data_as(_f64p), co.ctypes.data_as(_f64p))
    return _with_carry((vs, pg), co, return_carry)


def retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
            terminated, truncated, *, gamma, lam, carry_in=None, next_actions=None,
            next_behaviour_probs=None, return_carry=False, lib=None):
    """With carry_in (G at t = T), next_actions [N] and next_behaviour_probs
    [N] are a_T and mu(a_T | x_T) of the chunk that follows."""
    lib = lib or load_library()
    N, T = _shape2(rewards)
    q = np.ascontiguousarray(next_q_values_all, dtype=np.float32)
    if q.ndim != 3 or q.shape[:2] != (N, T):
        raise ValueError("next_q_values_all must be [N, T, A]")
    A = q.shape[2]
    p = _f32_in(next_target_probs, (N, T, A))
    acts = np.ascontiguousarray(actions, dtype=np.int32)
    if acts.shape != (N, T):
        raise ValueError("actions must be [N, T]")
    r = _f32_in(rewards, (N, T))
    mu = _f32_in(behaviour_probs, (N, T))
    term = _f32_in(terminated, (N, T))
    trunc = _f32_in(truncated, (N, T))
    if term[0] is None or trunc[0] is None:
        raise ValueError("retrace takes both terminated and truncated")
    ci = _carry_in(carry_in, N)
    na = nmu = None
    if ci[0] is not None:
        if next_actions is None or next_behaviour_probs is None:
            raise ValueError("carry_in needs next_actions and next_behaviour_probs")
        na = np.ascontiguousarray(next_actions, dtype=np.int32).reshape(N)
        nmu = _f32_in(next_behaviour_probs, (N,))
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    rc = lib.oracle_retrace(N, T, A, _param(gamma), _param(lam), _ptr(r),
                            q.ctypes.data_as(_f32p), _ptr(p), acts.ctypes.data_as(_i32p),
                            _ptr(mu), _ptr(term), _ptr(trunc), _ptr(ci),
                            na.ctypes.data_as(_i32p) if na is not None else None,
                            _ptr(nmu) if nmu is not None else None,
                            out.ctypes.data_as(_f64p), co.ctypes.data_as(_f64p))
    if rc != 0:
        raise ValueError("an action lies outside [0, A)")
    return _with_carry(out, co, return_carry)


def eligibility_traces(x, dones, *, gamma, lam, carry_in=None, return_carry=False, lib=None):
    lib = lib or load_library()
    N, T = _shape2(x)
    xs = _f32_in(x, (N, T))
    d = _f32_in(dones, (N, T))
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    lib.oracle_eligibility_traces(N, T, _param(gamma), _param(lam), _ptr(xs), _ptr(d),
                                  _ptr(_carry_in(carry_in, N)), out.ctypes.data_as(_f64p),
                                  co.ctypes.data_as(_f64p))
    return _with_carry(out, co, return_carry)


def episodic_prefix_sum(x, dones, *, carry_in=None, return_carry=False, lib=None):
    lib = lib or load_library()
    N, T = _shape2(x)
    xs = np.ascontiguousarray(x, dtype=np.int32)
    d = _f32_in(dones, (N, T))
    ci = None
    if carry_in is not None:
        ci = np.ascontiguousarray(carry_in, dtype=np.int64).reshape(N)
    out = np.empty((N, T), np.int64)
    co = np.empty(N, np.int64)
    lib.oracle_episodic_prefix_sum(N, T, xs.ctypes.data_as(_i32p), _ptr(d),
                                   ci.ctypes.data_as(_i64p) if ci is not None else None,
                                   out.ctypes.data_as(_i64p), co.ctypes.data_as(_i64p))
    return _with_carry(out, co, return_carry)


def episodic_prefix_sum_float(x, dones, *, carry_in=None, return_carry=False, lib=None):
    """Float-valued episodic prefix sum, float64 [N, T]; carry_in is y at
    t = -1, carry_out y at t = T - 1."""
    lib = lib or load_library()
    N, T = _shape2(x)
    xs = _f32_in(x, (N, T))
    d = _f32_in(dones, (N, T))
    out = np.empty((N, T), np.float64)
    co = np.empty(N, np.float64)
    lib.oracle_episodic_prefix_sum_float(N, T, _ptr(xs), _ptr(d), _ptr(_carry_in(carry_in, N)),
                                         out.ctypes.data_as(_f64p), co.ctypes.data_as(_f64p))
    return _with_carry(out, co, return_carry)
