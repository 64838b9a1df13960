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

import ctypes
import struct
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
        # the rlscan_call array, packed straight from the calls' tensors
        # (already checked by their compute_* call)
        buf = bytearray(_CALL_SIZE * len(calls))
        for k, c in enumerate(calls):
            ins = [0 if t is None else t.data_ptr() for t in c.ins]
            outs = [0 if t is None else t.data_ptr() for t in c.outs]
            struct.pack_into(_CALL_FMT, buf, k * _CALL_SIZE, c.est, c.flags, c.N, c.T, c.A,
                             *c.params, 0.0, *ins, *([0] * (8 - len(ins))), *outs,
                             *([0] * (2 - len(outs))))
        arr = (rlscan.Call * len(calls)).from_buffer(buf)
        first = calls[0].outs[0]

        def run(stream):
            rc = _lib().rlscan_group(arr, len(calls), _raw_stream(stream, first))
            if rc == rlscan.RLSCAN_ERR_PARAM:
                for c in calls:  # not groupable: the same calls one by one
                    c.alone(stream)
            else:
                _check(rc)

        several = _several_gpus()
        if self.stream is None and not several:
            run(None)
            return
        tensors = [t for c in calls for t in (*c.ins, *c.outs) if t is not None]
        index = first.get_device()
        if several:
            _one_device(index, tensors)
        with _on_device(index):
            _on_stream(run, self.stream, tensors)


# The layout of rlscan_call (include/rlscan.h): estimator, flags, N, T, A,
# gamma, lam, rho_bar, c_bar, rho_bar_pg, reserved, inp[8], out[2].
_CALL_FMT = "@iiqqqffffff8P2P"
_CALL_SIZE = struct.calcsize(_CALL_FMT)
assert _CALL_SIZE == ctypes.sizeof(rlscan.Call)


class _Deferred:
    """A compute_* call held by a `grouped` block until it ends."""
    __slots__ = ("est", "flags", "N", "T", "A", "params", "ins", "outs", "alone")

    def __init__(self, estimator, ins, outs, params, alone, byte):
        self.est = rlscan.ESTIMATOR_IDS[estimator]
        self.flags = rlscan.CALL_BYTE_FLAGS if byte else 0
        self.N, self.T = ins[0].shape
        self.A = ins[1].shape[2] if estimator == "retrace" else 1
        rho_bar = params.get("rho_bar", 1.0)
        rbpg = params.get("rho_bar_pg")
        self.params = (params.get("gamma", 0.99), params.get("lam", 0.95), rho_bar,
                       params.get("c_bar", 1.0), rho_bar if rbpg is None else rbpg)
        self.ins, self.outs, self.alone = ins, outs, alone


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


_gpus = None


def _several_gpus():
    """Whether more than one GPU is visible (with one, every device tensor
    is on the current device and the checks below have nothing to find)."""
    global _gpus
    if _gpus is None:
        _gpus = torch.cuda.device_count()
    return _gpus > 1


def _one_device(index, tensors):
    """Every tensor of a call on the GPU of index `index`."""
    for t in tensors:
        if t is not None and t.get_device() != index:
            raise ValueError(f"every tensor of a call must be on cuda:{index}, got one on "
                             f"{t.device}")


class _on_device:
    """Makes GPU `index` current for the block (the library launches on, and
    takes its scratch from, the current device)."""

    def __init__(self, index):
        self.index, self.prev = index, None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.index:
            self.prev = cur
            torch.cuda.set_device(self.index)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def _submit(estimator, ins, outs, params, alone, stream, carry, extra=(), byte=False):
    """Runs `alone(stream)` now, or defers the call to the innermost active
    `grouped` block (plain calls on the current stream only).  `extra`: the
    call's other tensors (carries, Retrace's next-chunk arrays); `byte`: its
    flags are one byte each."""
    several = _several_gpus()
    if several:
        index = outs[0].get_device()
        _one_device(index, (*ins, *extra))
        if isinstance(stream, torch.cuda.Stream) and stream.device.index != index:
            raise ValueError(f"stream is on {stream.device}, the tensors on cuda:{index}")
    stack = getattr(_local, "groups", None)
    if stack and not carry and stream is None:
        stack[-1].calls.append(_Deferred(estimator, ins, outs, params, alone, byte))
    elif stream is None and not several:
        alone(None)
    elif several:
        with _on_device(index):
            _on_stream(alone, stream, (*ins, *outs, *extra))
    else:
        _on_stream(alone, stream, (*ins, *outs, *extra))


# ------------------------------------------------------------------ marshalling
# One pass over each tensor: device, dtype, shape, contiguity; then the C
# entry point is called with raw pointers.  (The binding module rlscan.py
# checks the same things again; these calls skip that second pass: it cost
# about as much as the kernel of a 4096 x 128 call.)
_F32 = torch.float32
_I32 = torch.int32
_BYTE = (torch.bool, torch.uint8)
_clib = None


def _lib():
    global _clib
    if _clib is None:
        _clib = rlscan.library()
    return _clib


def _check(rc):
    if rc != rlscan.RLSCAN_OK:
        raise rlscan.RlscanError(rc, rlscan.status_string(rc))


def _gpu(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got device {t.device}); rlscan has no "
                         "CPU path")
    return t


def _tensor(t, name, shape, dtype=_F32):
    """A device tensor of `dtype` and `shape`, made contiguous; None stays
    None."""
    if t is None:
        return None
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is dtype and t.shape == shape):
        _gpu(t, name)  # raises for a non-tensor or a host tensor
        if t.dtype is not dtype:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t if t.is_contiguous() else t.contiguous()


def _rows(t, name, dtype=_F32):
    """The first [num_envs, seq_len] tensor of a call: its shape sets N, T."""
    _gpu(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be a [num_envs, seq_len] tensor, got shape "
                         f"{tuple(t.shape)}")
    return _tensor(t, name, t.shape, dtype)


def _flags(shape, *named):
    """The call's flag tensors (name, tensor pairs), all float32 or all one
    byte (bool / uint8): as given when they already are, else each turned
    into bool (set iff != 0).  Returns (tensors, one_byte)."""
    # the common case: contiguous float32 device flags of the right shape
    fast = []
    for n, t in named:
        if t is None:
            fast.append(None)
        elif (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is _F32 and
              t.shape == shape and t.is_contiguous()):
            fast.append(t)
        else:
            break
    else:
        return fast, False
    given = [(n, t) for n, t in named if t is not None]
    for n, t in given:
        _gpu(t, n)
        if t.shape != shape:
            raise ValueError(f"{n} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if all(t.dtype is _F32 for _, t in given):
        byte = False
    elif all(t.dtype in _BYTE for _, t in given):
        byte = True
    else:  # any other dtype, or a mix: one byte per flag
        given = [(n, t if t.dtype in _BYTE else t != 0) for n, t in given]
        byte = True
    out = dict((n, t if t.is_contiguous() else t.contiguous()) for n, t in given)
    return [out.get(n) for n, _ in named], byte


def _p(t):
    return None if t is None else t.data_ptr()


def _raw_stream(stream, t):
    """The HIP stream handle of `stream` (None: the current stream of t's
    device)."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(t.get_device())
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def compute_gae(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *,
                bootstrap_value=None, truncateds=None, bootstrap_values=None, carry_in=None,
                return_carry=False, stream=None):
    """Advantages A_t = delta_t + gamma*lambda*(1 - cut_t)*A_{t+1} [N, T]
    (README, Kernels: compute_gae).  bootstrap_value [N] is V at t = T
    (None: 0); truncateds [N, T] with bootstrap_values [N, T] handle
    time-limit truncation."""
    r = _rows(rewards, "rewards")
    N, T = r.shape
    (term, trunc), byte = _flags(r.shape, ("terminateds", terminateds), ("truncateds", truncateds))
    ins = (r, _tensor(values, "values", r.shape), _tensor(bootstrap_value, "bootstrap_value", (N,)),
           term, trunc, _tensor(bootstrap_values, "bootstrap_values", r.shape))
    ci = _tensor(carry_in, "carry_in", (N,))
    out = torch.empty_like(r)
    co = r.new_empty((N,)) if return_carry else None
    g, lam = float(gamma), float(lambda_)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, r)
        if byte:
            _check(lib.rlscan_gae_u8(*P, _p(ci), out.data_ptr(), _p(co), N, T, g, lam, h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_gae_carry(*P, _p(ci), out.data_ptr(), _p(co), N, T, g, lam, h))
        else:
            _check(lib.rlscan_gae(*P, out.data_ptr(), N, T, g, lam, h))
    _submit("gae", ins, (out,), dict(gamma=g, lam=lam), alone, stream,
            ci is not None or co is not None, (ci, co), byte)
    return (out, co) if return_carry else out


def compute_lambda_returns(rewards, values, terminateds, gamma=0.99, lambda_=0.95, *,
                           bootstrap_value=None, truncateds=None, bootstrap_values=None,
                           carry_in=None, return_carry=False, stream=None):
    """TD(lambda) returns [N, T] (README, Kernels: compute_lambda_returns)."""
    r = _rows(rewards, "rewards")
    N, T = r.shape
    (term, trunc), byte = _flags(r.shape, ("terminateds", terminateds), ("truncateds", truncateds))
    ins = (r, _tensor(values, "values", r.shape), _tensor(bootstrap_value, "bootstrap_value", (N,)),
           term, trunc, _tensor(bootstrap_values, "bootstrap_values", r.shape))
    ci = _tensor(carry_in, "carry_in", (N,))
    out = torch.empty_like(r)
    co = r.new_empty((N,)) if return_carry else None
    g, lam = float(gamma), float(lambda_)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, r)
        if byte:
            _check(lib.rlscan_lambda_returns_u8(*P, _p(ci), out.data_ptr(), _p(co), N, T, g, lam,
                                                h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_lambda_returns_carry(*P, _p(ci), out.data_ptr(), _p(co), N, T, g,
                                                   lam, h))
        else:
            _check(lib.rlscan_lambda_returns(*P, out.data_ptr(), N, T, g, lam, h))
    _submit("lambda_returns", ins, (out,), dict(gamma=g, lam=lam), alone, stream,
            ci is not None or co is not None, (ci, co), byte)
    return (out, co) if return_carry else out


def compute_discounted_returns(rewards, terminateds, gamma=0.99, *, bootstrap_value=None,
                               truncateds=None, bootstrap_values=None, carry_in=None,
                               return_carry=False, stream=None):
    """Discounted reward-to-go [N, T] (README, Kernels:
    compute_discounted_returns)."""
    r = _rows(rewards, "rewards")
    N, T = r.shape
    (term, trunc), byte = _flags(r.shape, ("terminateds", terminateds), ("truncateds", truncateds))
    ins = (r, _tensor(bootstrap_value, "bootstrap_value", (N,)), term, trunc,
           _tensor(bootstrap_values, "bootstrap_values", r.shape))
    ci = _tensor(carry_in, "carry_in", (N,))
    out = torch.empty_like(r)
    co = r.new_empty((N,)) if return_carry else None
    g = float(gamma)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, r)
        if byte:
            _check(lib.rlscan_discounted_returns_u8(*P, _p(ci), out.data_ptr(), _p(co), N, T, g,
                                                    h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_discounted_returns_carry(*P, _p(ci), out.data_ptr(), _p(co), N, T,
                                                       g, h))
        else:
            _check(lib.rlscan_discounted_returns(*P, out.data_ptr(), N, T, g, h))
    _submit("discounted_returns", ins, (out,), dict(gamma=g), alone, stream,
            ci is not None or co is not None, (ci, co), byte)
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
    r = _rows(rewards, "rewards")
    N, T = r.shape
    (term, trunc), byte = _flags(r.shape, ("terminateds", terminateds), ("truncateds", truncateds))
    ins = (r, _tensor(values, "values", r.shape), _tensor(bootstrap_value, "bootstrap_value", (N,)),
           _tensor(log_rhos, "log_rhos", r.shape), term, trunc,
           _tensor(bootstrap_values, "bootstrap_values", r.shape))
    ci = _tensor(carry_in, "carry_in", (N,))
    vs, pg = torch.empty_like(r), torch.empty_like(r)
    co = r.new_empty((N,)) if return_carry else None
    g, rb, cb = float(gamma), float(rho_bar), float(c_bar)
    ex = lambda_ is not None or rho_bar_pg is not None
    lam = 1.0 if lambda_ is None else float(lambda_)
    rbpg = rb if rho_bar_pg is None else float(rho_bar_pg)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, r)
        o = (vs.data_ptr(), pg.data_ptr())
        if byte:
            _check(lib.rlscan_vtrace_u8(*P, _p(ci), *o, _p(co), N, T, g, lam, rb, cb, rbpg, h))
        elif ex:
            _check(lib.rlscan_vtrace_ex(*P, _p(ci), *o, _p(co), N, T, g, lam, rb, cb, rbpg, h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_vtrace_carry(*P, _p(ci), *o, _p(co), N, T, g, rb, cb, h))
        else:
            _check(lib.rlscan_vtrace(*P, *o, N, T, g, rb, cb, h))
    _submit("vtrace", ins, (vs, pg),
            dict(gamma=g, lam=lam, rho_bar=rb, c_bar=cb, rho_bar_pg=rbpg), alone, stream,
            ci is not None or co is not None, (ci, co), byte)
    return (vs, pg, co) if return_carry else (vs, pg)


def _int32(t, name, shape):
    """Integer indices as int32 (any integer dtype, narrowed or widened)."""
    if t is None:
        return None
    _gpu(t, name)
    if t.dtype is not _I32 and not t.dtype.is_floating_point:
        t = t.to(_I32)
    return _tensor(t, name, shape, _I32)


def compute_retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                    terminateds, truncateds, gamma=0.99, lambda_=0.95, *, carry_in=None,
                    next_actions=None, next_behaviour_probs=None, return_carry=False,
                    stream=None):
    """Retrace(lambda) targets [N, T] (README, Kernels: compute_retrace).
    next_q_values_all and next_target_probs are [N, T, A] at each step's
    successor state; actions [N, T] are the taken actions (int32, or any
    integer dtype, converted); behaviour_probs [N, T] is mu of the taken
    action.  Both flags are required (README, Performance)."""
    r = _rows(rewards, "rewards")
    N, T = r.shape
    if truncateds is None:
        raise ValueError("compute_retrace takes terminateds and truncateds, both required")
    q = _gpu(next_q_values_all, "next_q_values_all")
    if q.dim() != 3 or q.shape[:2] != r.shape:
        raise ValueError(f"next_q_values_all must be a [N, T, A] tensor, got shape "
                         f"{tuple(q.shape)}")
    A = q.shape[2]
    (term, trunc), byte = _flags(r.shape, ("terminateds", terminateds), ("truncateds", truncateds))
    ins = (r, _tensor(q, "next_q_values_all", q.shape),
           _tensor(next_target_probs, "next_target_probs", q.shape),
           _int32(actions, "actions", r.shape), _tensor(behaviour_probs, "behaviour_probs", r.shape),
           term, trunc)
    ci = _tensor(carry_in, "carry_in", (N,))
    nat = _int32(next_actions, "next_actions", (N,))
    nbp = _tensor(next_behaviour_probs, "next_behaviour_probs", (N,))
    out = torch.empty_like(r)
    co = r.new_empty((N,)) if return_carry else None
    g, lam = float(gamma), float(lambda_)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, r)
        if byte or ci is not None or co is not None:
            fn = lib.rlscan_retrace_u8 if byte else lib.rlscan_retrace_carry
            _check(fn(*P, _p(ci), _p(nat), _p(nbp), out.data_ptr(), _p(co), N, T, A, g, lam, h))
        else:
            _check(lib.rlscan_retrace(*P, out.data_ptr(), N, T, A, g, lam, h))
    _submit("retrace", ins, (out,), dict(gamma=g, lam=lam), alone, stream,
            ci is not None or co is not None, (ci, co, nat, nbp), byte)
    return (out, co) if return_carry else out


def compute_eligibility_traces(x, dones, gamma=0.99, lambda_=0.95, *, carry_in=None,
                               return_carry=False, stream=None):
    """Forward traces e_t = x_t + gamma*lambda*(1 - d_t)*e_{t-1} [N, T]
    (README, Kernels: compute_eligibility_traces)."""
    xx = _rows(x, "x")
    N, T = xx.shape
    (d,), byte = _flags(xx.shape, ("dones", dones))
    ins = (xx, d)
    ci = _tensor(carry_in, "carry_in", (N,))
    out = torch.empty_like(xx)
    co = xx.new_empty((N,)) if return_carry else None
    g, lam = float(gamma), float(lambda_)

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, xx)
        if byte:
            _check(lib.rlscan_eligibility_traces_u8(*P, _p(ci), out.data_ptr(), _p(co), N, T, g,
                                                    lam, h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_eligibility_traces_carry(*P, _p(ci), out.data_ptr(), _p(co), N, T,
                                                       g, lam, h))
        else:
            _check(lib.rlscan_eligibility_traces(*P, out.data_ptr(), N, T, g, lam, h))
    _submit("eligibility_traces", ins, (out,), dict(gamma=g, lam=lam), alone, stream,
            ci is not None or co is not None, (ci, co), byte)
    return (out, co) if return_carry else out


def compute_episodic_prefix_sum(x, dones, *, carry_in=None, return_carry=False, stream=None):
    """Cumulative sum restarted where dones is set (README, Kernels:
    compute_episodic_prefix_sum).  Integer x: exact int64 output [N, T]; x is
    int32, narrower integer dtypes are widened, int64 is refused (it would
    not fit).  float32 x: float32 output, summed in float32 in the scan's
    order (float dones only)."""
    if isinstance(x, torch.Tensor) and x.dtype is _F32:
        xx = _rows(x, "x")
        N, T = xx.shape
        d = _gpu(dones, "dones")
        d = _tensor(d if d.dtype is _F32 else (d != 0).to(_F32), "dones", xx.shape)
        ci = _tensor(carry_in, "carry_in", (N,))
        out = torch.empty_like(xx)
        co = xx.new_empty((N,)) if return_carry else None

        def alone_f32(st):
            _check(_lib().rlscan_episodic_prefix_sum_f32(
                xx.data_ptr(), d.data_ptr(), _p(ci), out.data_ptr(), _p(co), N, T,
                _raw_stream(st, xx)))
        _on_stream(alone_f32, stream, (xx, d, out, ci, co))
        return (out, co) if return_carry else out
    xx = x
    if isinstance(xx, torch.Tensor) and xx.dtype in (torch.bool, torch.uint8, torch.int8,
                                                     torch.int16):
        xx = _gpu(xx, "x").to(_I32)
    xx = _rows(xx, "x", _I32)
    N, T = xx.shape
    (d,), byte = _flags(xx.shape, ("dones", dones))
    ins = (xx, d)
    ci = _tensor(carry_in, "carry_in", (N,), torch.int64)
    out = torch.empty((N, T), dtype=torch.int64, device=xx.device)
    co = torch.empty((N,), dtype=torch.int64, device=xx.device) if return_carry else None

    def alone(st):
        lib, P, h = _lib(), [_p(t) for t in ins], _raw_stream(st, xx)
        if byte:
            _check(lib.rlscan_episodic_prefix_sum_u8(*P, _p(ci), out.data_ptr(), _p(co), N, T, h))
        elif ci is not None or co is not None:
            _check(lib.rlscan_episodic_prefix_sum_carry(*P, _p(ci), out.data_ptr(), _p(co), N, T,
                                                        h))
        else:
            _check(lib.rlscan_episodic_prefix_sum(*P, out.data_ptr(), N, T, h))
    _submit("episodic_prefix_sum", ins, (out,), {}, alone, stream,
            ci is not None or co is not None, (ci, co), byte)
    return (out, co) if return_carry else out
