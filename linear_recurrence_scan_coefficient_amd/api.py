"""PyTorch-facing calls with the pages' call shape: each takes [num_envs,
seq_len] device tensors, allocates its outputs and returns them, e.g.

    advantages = compute_gae(rewards, values, terminateds, gamma=0.99, lambda_=0.95)

The names and the (rewards, values, terminateds, gamma, lambda_) shape follow
the rl-triton README, sections "Kernels" (one compute_* function per
estimator) and "Usage" (compute_gae on [64, 512] float tensors, returning
the advantages).  The optional truncation arguments follow its section
"Performance" (terminations, time-limit truncations and bootstrap values for
GAE, V-trace, TD(lambda) and discounted returns; Retrace takes both flags and
no bootstrap tensor; traces and the prefix sum take a single dones flag).

Argument marshalling only: every computation runs in librlscan's HIP kernels
through the C ABI (`rlscan.rlscan_*`).  Inputs must already be on the GPU;
there is no CPU path.  Flags (set iff != 0) given as float32 take the
float-flag kernels and bool / uint8 flags the one-byte-flag kernels, both
without any conversion; flags of other dtypes, or a mix of float32 and
one-byte flags in one call, are first turned into bool (one elementwise
pass).  Non-contiguous inputs are made contiguous, and the call runs on the
current stream, or on `stream`: such a call first waits for the current
stream (where its temporaries and outputs are made) and marks every tensor
it uses as used by `stream`; the caller waits for `stream` before reading
the outputs elsewhere.  gamma and lambda_ default to the values of
the README's usage example.

Streaming one rollout through several calls (the README's chunked fallback
for long sequences, Kernels table, last column): every call takes
`carry_in` [num_envs], the output just past this chunk (t = T for the
reverse estimators, whose later chunks go first; t = -1 for traces and the
prefix sum), and with `return_carry=True` also returns carry_out [num_envs],
the output at the chunk's other edge -- the next call's carry_in.  V at
t = T is `bootstrap_value`; compute_retrace also needs `next_actions` and
`next_behaviour_probs` [num_envs] of the chunk that follows.

Several calls in one launch: inside `with grouped():` the compute_* calls
return their (not yet written) outputs at once and are run together as one
`rlscan_group` launch when the block ends, on the stream current then.
Calls that take or return a carry, or name a stream of their own, and the
float-valued prefix sum run at once as usual.  If the collected calls cannot share a launch (rows longer
than a grouped tile, unaligned tensors, Retrace with an action count other
than 4, 6 or 8), they run one by one instead.
"""
from __future__ import annotations

import threading

import torch

from . import rlscan

__all__ = [
    "compute_gae", "compute_vtrace", "compute_retrace", "compute_lambda_returns",
    "compute_discounted_returns", "compute_eligibility_traces", "compute_episodic_prefix_sum",
    "grouped",
]

_local = threading.local()


class grouped:
    """Collects the compute_* calls made in its block (on this thread) and
    runs them as one grouped launch when the block ends."""

    def __init__(self, stream=None):
        self.stream = stream
        self.calls = []  # (GroupCall, the same call made alone)

    def __enter__(self):
        stack = getattr(_local, "groups", None)
        if stack is None:
            stack = _local.groups = []
        stack.append(self)
        return self

    def __exit__(self, exc_type, exc, tb):
        _local.groups.pop()
        if exc_type is None:
            self.launch()
        return False

    def launch(self):
        calls, self.calls = self.calls, []
        if not calls:
            return
        tensors = [t for g, _ in calls for part in g.keep for t in part]

        def run(stream):
            try:
                rlscan.rlscan_group([g for g, _ in calls], stream)
            except rlscan.RlscanError as e:
                if e.status != rlscan.RLSCAN_ERR_PARAM:
                    raise
                for _, alone in calls:  # not groupable: the same calls one by one
                    alone(stream)

        _on_stream(run, self.stream, tensors)


def _as_stream(stream):
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_stream(fn, stream, tensors):
    """Runs `fn(stream)`.  Inputs, temporaries and outputs were made on the
    current stream; a launch on another stream first waits for the current
    one, and every tensor is marked as used by that stream so that the
    caching allocator does not hand its memory out again before that
    stream's work is done."""
    if stream is None:
        fn(None)
        return
    s = _as_stream(stream)
    cur = torch.cuda.current_stream(s.device)
    if s == cur:
        fn(s)
        return
    s.wait_stream(cur)
    fn(s)
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            t.record_stream(s)


def _submit(estimator, ins, outs, params, alone, stream, carry, extra=()):
    """Runs `alone(stream)` now, or defers the call to the innermost active
    `grouped` block (plain calls on the current stream only).  `extra`: the
    call's other tensors (carries, Retrace's next-chunk arrays)."""
    stack = getattr(_local, "groups", None)
    if stack and not carry and stream is None:
        stack[-1].calls.append((rlscan.GroupCall(estimator, ins, outs, **params), alone))
    else:
        _on_stream(alone, stream, (*ins, *outs, *extra))


def _device_tensor(t, name, dtype=torch.float32, flag=False):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got device {t.device}); rlscan has no "
                         "CPU path")
    if t.dtype != dtype:
        if not flag:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
        t = t.to(dtype)  # a flag: any dtype, set iff nonzero
    return t.contiguous()


_BYTE = (torch.bool, torch.uint8)


def _flags(**flags):
    """The call's flag tensors, all float32 or all one-byte (bool / uint8)."""
    given = {k: t for k, t in flags.items() if t is not None}
    for k, t in given.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{k} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{k} must be on the GPU (got device {t.device}); rlscan has no "
                             "CPU path")
    def kind(t):
        return "float32" if t.dtype == torch.float32 else ("byte" if t.dtype in _BYTE else "other")

    kinds = {kind(t) for t in given.values()}
    if kinds in ({"float32"}, {"byte"}):
        out = {k: t.contiguous() for k, t in given.items()}
    else:  # any other dtype, or a mix: one byte per flag
        out = {k: (t if t.dtype in _BYTE else t != 0).contiguous() for k, t in given.items()}
    return [out.get(k) for k in flags]


def _carry_out(wanted, N, device, dtype=torch.float32):
    return torch.empty((N,), dtype=dtype, device=device) if wanted else None


def _check_2d(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a [num_envs, seq_len] tensor, got shape "
                         f"{tuple(t.shape)}")
    return t.shape


def compute_gae(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *,
                bootstrap_value=None, truncateds=None, bootstrap_values=None, carry_in=None,
                return_carry=False, stream=None):
    """Advantages A_t = delta_t + gamma*lambda*(1 - cut_t)*A_{t+1} [N, T]
    (README, Kernels: compute_gae).  bootstrap_value [N] is V at t = T
    (None: 0); truncateds [N, T] with bootstrap_values [N, T] handle
    time-limit truncation."""
    r = _device_tensor(rewards, "rewards")
    N, T = _check_2d(r, "rewards")
    out = torch.empty((N, T), dtype=torch.float32, device=r.device)
    co = _carry_out(return_carry, N, r.device)
    term, trunc = _flags(terminateds=terminateds, truncateds=truncateds)
    ins = (r, _device_tensor(values, "values"), _device_tensor(bootstrap_value, "bootstrap_value"),
           term, trunc, _device_tensor(bootstrap_values, "bootstrap_values"))
    ci = _device_tensor(carry_in, "carry_in")
    _submit("gae", ins, (out,), dict(gamma=float(gamma), lam=float(lambda_)),
            lambda st: rlscan.rlscan_gae(*ins, out, float(gamma), float(lambda_), st,
                                         carry_in=ci, carry_out=co),
            stream, ci is not None or co is not None, (ci, co))
    return (out, co) if return_carry else out


def compute_lambda_returns(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *,
                           bootstrap_value=None, truncateds=None, bootstrap_values=None,
                           carry_in=None, return_carry=False, stream=None):
    """TD(lambda) returns [N, T] (README, Kernels: compute_lambda_returns)."""
    r = _device_tensor(rewards, "rewards")
    N, T = _check_2d(r, "rewards")
    out = torch.empty((N, T), dtype=torch.float32, device=r.device)
    co = _carry_out(return_carry, N, r.device)
    term, trunc = _flags(terminateds=terminateds, truncateds=truncateds)
    ins = (r, _device_tensor(values, "values"), _device_tensor(bootstrap_value, "bootstrap_value"),
           term, trunc, _device_tensor(bootstrap_values, "bootstrap_values"))
    ci = _device_tensor(carry_in, "carry_in")
    _submit("lambda_returns", ins, (out,), dict(gamma=float(gamma), lam=float(lambda_)),
            lambda st: rlscan.rlscan_lambda_returns(*ins, out, float(gamma), float(lambda_), st,
                                                    carry_in=ci, carry_out=co),
            stream, ci is not None or co is not None, (ci, co))
    return (out, co) if return_carry else out


def compute_discounted_returns(rewards, terminateds, gamma=0.99, *, bootstrap_value=None,
                               truncateds=None, bootstrap_values=None, carry_in=None,
                               return_carry=False, stream=None):
    """Discounted reward-to-go [N, T] (README, Kernels:
    compute_discounted_returns)."""
    r = _device_tensor(rewards, "rewards")
    N, T = _check_2d(r, "rewards")
    out = torch.empty((N, T), dtype=torch.float32, device=r.device)
    co = _carry_out(return_carry, N, r.device)
    term, trunc = _flags(terminateds=terminateds, truncateds=truncateds)
    ins = (r, _device_tensor(bootstrap_value, "bootstrap_value"), term, trunc,
           _device_tensor(bootstrap_values, "bootstrap_values"))
    ci = _device_tensor(carry_in, "carry_in")
    _submit("discounted_returns", ins, (out,), dict(gamma=float(gamma)),
            lambda st: rlscan.rlscan_discounted_returns(*ins, out, float(gamma), st, carry_in=ci,
                                                        carry_out=co),
            stream, ci is not None or co is not None, (ci, co))
    return (out, co) if return_carry else out


def compute_vtrace(rewards, values, log_rhos, terminateds, gamma=0.99, rho_bar=1.0, c_bar=1.0,
                   *, bootstrap_value=None, truncateds=None, bootstrap_values=None,
                   carry_in=None, return_carry=False, lambda_=None, rho_bar_pg=None,
                   stream=None):
    """V-trace targets vs and policy-gradient advantages [N, T] each, as a
    tuple (README, Kernels: compute_vtrace).  log_rhos = log pi - log mu.
    carry_in / carry_out are vs values.  IMPALA's options: lambda_ scales
    every trace coefficient c_t (None: 1) and rho_bar_pg truncates the
    policy-gradient weight (None: rho_bar)."""
    r = _device_tensor(rewards, "rewards")
    N, T = _check_2d(r, "rewards")
    vs = torch.empty((N, T), dtype=torch.float32, device=r.device)
    pg = torch.empty((N, T), dtype=torch.float32, device=r.device)
    co = _carry_out(return_carry, N, r.device)
    term, trunc = _flags(terminateds=terminateds, truncateds=truncateds)
    ins = (r, _device_tensor(values, "values"), _device_tensor(bootstrap_value, "bootstrap_value"),
           _device_tensor(log_rhos, "log_rhos"), term, trunc,
           _device_tensor(bootstrap_values, "bootstrap_values"))
    ci = _device_tensor(carry_in, "carry_in")
    lam = None if lambda_ is None else float(lambda_)
    pgc = None if rho_bar_pg is None else float(rho_bar_pg)
    _submit("vtrace", ins, (vs, pg),
            dict(gamma=float(gamma), lam=1.0 if lam is None else lam, rho_bar=float(rho_bar),
                 c_bar=float(c_bar), rho_bar_pg=pgc),
            lambda st: rlscan.rlscan_vtrace(*ins, vs, pg, float(gamma), float(rho_bar),
                                            float(c_bar), st, carry_in=ci, carry_out=co,
                                            lam=lam, rho_bar_pg=pgc),
            stream, ci is not None or co is not None, (ci, co))
    return (vs, pg, co) if return_carry else (vs, pg)


def compute_retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                    terminateds, truncateds, gamma=0.99, lambda_=0.95, *, carry_in=None,
                    next_actions=None, next_behaviour_probs=None, return_carry=False,
                    stream=None):
    """Retrace(lambda) targets [N, T] (README, Kernels: compute_retrace).
    next_q_values_all and next_target_probs are [N, T, A] at each step's
    successor state; actions [N, T] are the taken actions (int32, or any
    integer dtype, converted); behaviour_probs [N, T] is mu of the taken
    action.  Both flags are required (README, Performance)."""
    r = _device_tensor(rewards, "rewards")
    N, T = _check_2d(r, "rewards")
    if truncateds is None:
        raise ValueError("compute_retrace takes terminateds and truncateds, both required")
    a = actions
    if isinstance(a, torch.Tensor) and a.dtype != torch.int32 and not a.dtype.is_floating_point:
        a = a.to(torch.int32)
    na = next_actions
    if isinstance(na, torch.Tensor) and na.dtype != torch.int32 and not na.dtype.is_floating_point:
        na = na.to(torch.int32)
    out = torch.empty((N, T), dtype=torch.float32, device=r.device)
    co = _carry_out(return_carry, N, r.device)
    term, trunc = _flags(terminateds=terminateds, truncateds=truncateds)
    ins = (r, _device_tensor(next_q_values_all, "next_q_values_all"),
           _device_tensor(next_target_probs, "next_target_probs"),
           _device_tensor(a, "actions", torch.int32),
           _device_tensor(behaviour_probs, "behaviour_probs"), term, trunc)
    ci = _device_tensor(carry_in, "carry_in")
    nat = _device_tensor(na, "next_actions", torch.int32)
    nbp = _device_tensor(next_behaviour_probs, "next_behaviour_probs")
    _submit("retrace", ins, (out,), dict(gamma=float(gamma), lam=float(lambda_)),
            lambda st: rlscan.rlscan_retrace(*ins, out, float(gamma), float(lambda_), st,
                                             carry_in=ci, carry_out=co, next_actions=nat,
                                             next_behaviour_probs=nbp),
            stream, ci is not None or co is not None, (ci, co, nat, nbp))
    return (out, co) if return_carry else out


def compute_eligibility_traces(x, dones, gamma=0.99, lambda_=0.95, *, carry_in=None,
                               return_carry=False, stream=None):
    """Forward traces e_t = x_t + gamma*lambda*(1 - d_t)*e_{t-1} [N, T]
    (README, Kernels: compute_eligibility_traces)."""
    xx = _device_tensor(x, "x")
    N, T = _check_2d(xx, "x")
    out = torch.empty((N, T), dtype=torch.float32, device=xx.device)
    co = _carry_out(return_carry, N, xx.device)
    ins = (xx, _flags(dones=dones)[0])
    ci = _device_tensor(carry_in, "carry_in")
    _submit("eligibility_traces", ins, (out,), dict(gamma=float(gamma), lam=float(lambda_)),
            lambda st: rlscan.rlscan_eligibility_traces(*ins, out, float(gamma), float(lambda_),
                                                        st, carry_in=ci, carry_out=co),
            stream, ci is not None or co is not None, (ci, co))
    return (out, co) if return_carry else out


def compute_episodic_prefix_sum(x, dones, *, carry_in=None, return_carry=False, stream=None):
    """Cumulative sum restarted where dones is set (README, Kernels:
    compute_episodic_prefix_sum).  Integer x: exact int64 output [N, T]; x is
    int32, narrower integer dtypes are widened, int64 is refused (it would
    not fit).  float32 x: float32 output, summed in float32 in the scan's
    order (float dones only)."""
    if isinstance(x, torch.Tensor) and x.dtype == torch.float32:
        xx = _device_tensor(x, "x")
        N, T = _check_2d(xx, "x")
        out = torch.empty((N, T), dtype=torch.float32, device=xx.device)
        co = _carry_out(return_carry, N, xx.device)
        d = _device_tensor(dones, "dones", torch.float32, flag=True)
        ci = _device_tensor(carry_in, "carry_in")
        _on_stream(lambda st: rlscan.rlscan_episodic_prefix_sum_f32(xx, d, out, st, carry_in=ci,
                                                                     carry_out=co),
                   stream, (xx, d, out, ci, co))
        return (out, co) if return_carry else out
    xx = x
    if isinstance(xx, torch.Tensor) and xx.dtype in (torch.bool, torch.uint8, torch.int8,
                                                     torch.int16):
        xx = xx.to(torch.int32)
    xx = _device_tensor(xx, "x", torch.int32)
    N, T = _check_2d(xx, "x")
    out = torch.empty((N, T), dtype=torch.int64, device=xx.device)
    co = _carry_out(return_carry, N, xx.device, torch.int64)
    ins = (xx, _flags(dones=dones)[0])
    ci = _device_tensor(carry_in, "carry_in", torch.int64)
    _submit("episodic_prefix_sum", ins, (out,), {},
            lambda st: rlscan.rlscan_episodic_prefix_sum(*ins, out, st, carry_in=ci,
                                                         carry_out=co),
            stream, ci is not None or co is not None, (ci, co))
    return (out, co) if return_carry else out
