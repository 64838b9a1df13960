"""Thin ctypes binding of librlscan's C ABI (argument marshalling only).

Each ``rlscan_*`` function here has the name and argument order of the C
entry point declared in ``include/rlscan.h``; tensors replace raw device
pointers and N, T (and A) are read from their shapes.  Outputs are
caller-provided tensors, exactly as in C.  All computation runs in the HIP
kernels of librlscan; this module has no fallback path: if the library is
missing or fails to load, every call raises.

PyTorch supplies device memory and the current stream only.  ``torch`` is
imported before the library is loaded, so librlscan binds to the same HIP
runtime as PyTorch.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

LIB_PATH = _build.LIB_PATH

RLSCAN_OK = 0
RLSCAN_ERR_NULL = -1
RLSCAN_ERR_SHAPE = -2
RLSCAN_ERR_PARAM = -3
RLSCAN_ERR_ALIAS = -4
RLSCAN_ERR_HIP = -5
RLSCAN_ERR_ALLOC = -6
RLSCAN_ERR_CAPTURE = -7
RLSCAN_ERR_SCRATCH = -8

MAP_AUTO, MAP_PACKED, MAP_LOOKBACK = 0, 1, 2
FLAG_TICKETS = 1
FLAG_GROUP_INTERLEAVED = 2  # rlscan_group: deal workgroups to the calls' tiles in turn
FLAG_LOOKBACK_GIVE_UP = 4  # tests: every look-back wait gives up (poisoned outputs)

ESTIMATOR_IDS = {
    "gae": 0, "lambda_returns": 1, "discounted_returns": 2, "vtrace": 3, "retrace": 4,
    "eligibility_traces": 5, "episodic_prefix_sum": 6,
}

EXPORTED = (
    "rlscan_gae", "rlscan_lambda_returns", "rlscan_discounted_returns", "rlscan_vtrace",
    "rlscan_retrace", "rlscan_eligibility_traces", "rlscan_episodic_prefix_sum",
    "rlscan_status_string", "rlscan_version", "rlscan_release_scratch", "rlscan_plan",
    "rlscan_set_launch_override", "rlscan_lookback_timeouts", "rlscan_launch_floor",
    "rlscan_stream_copy",
    "rlscan_gae_carry", "rlscan_lambda_returns_carry", "rlscan_discounted_returns_carry",
    "rlscan_vtrace_carry", "rlscan_retrace_carry", "rlscan_eligibility_traces_carry",
    "rlscan_episodic_prefix_sum_carry",
    "rlscan_vtrace_ex", "rlscan_episodic_prefix_sum_f32",
    "rlscan_gae_u8", "rlscan_lambda_returns_u8", "rlscan_discounted_returns_u8",
    "rlscan_vtrace_u8", "rlscan_retrace_u8", "rlscan_eligibility_traces_u8",
    "rlscan_episodic_prefix_sum_u8", "rlscan_group", "rlscan_gae_noalloc", "rlscan_stream_mix",
    "rlscan_stream_mix_arrays",
    "rlscan_set_xcd_run",
)


class RlscanError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"rlscan error {status}: {message}")
        self.status = status


class Call(ctypes.Structure):
    """rlscan_call: one estimator call of a grouped launch."""
    _fields_ = [("estimator", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("N", ctypes.c_int64), ("T", ctypes.c_int64), ("A", ctypes.c_int64),
                ("gamma", ctypes.c_float), ("lam", ctypes.c_float),
                ("rho_bar", ctypes.c_float), ("c_bar", ctypes.c_float),
                ("rho_bar_pg", ctypes.c_float), ("reserved", ctypes.c_float),
                ("inp", ctypes.c_void_p * 8), ("out", ctypes.c_void_p * 2)]


CALL_BYTE_FLAGS = 1
# positions of the flag tensors among each estimator's inputs
_FLAG_SLOTS = {"gae": (3, 4), "lambda_returns": (3, 4), "discounted_returns": (2, 3),
               "vtrace": (4, 5), "retrace": (5, 6), "eligibility_traces": (1,),
               "episodic_prefix_sum": (1,)}


class PlanInfo(ctypes.Structure):
    _fields_ = [("mapping", ctypes.c_int32), ("rounds", ctypes.c_int32),
                ("tile_elems", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("threads", ctypes.c_int32),
                ("tile_span", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def _declare(lib):
    lib.rlscan_gae.argtypes = [_vp] * 7 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_lambda_returns.argtypes = [_vp] * 7 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_discounted_returns.argtypes = [_vp] * 6 + [_i64, _i64, _f32, _vp]
    lib.rlscan_vtrace.argtypes = [_vp] * 9 + [_i64, _i64, _f32, _f32, _f32, _vp]
    lib.rlscan_retrace.argtypes = [_vp] * 8 + [_i64, _i64, _i64, _f32, _f32, _vp]
    lib.rlscan_eligibility_traces.argtypes = [_vp] * 3 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_episodic_prefix_sum.argtypes = [_vp] * 3 + [_i64, _i64, _vp]
    lib.rlscan_gae_carry.argtypes = [_vp] * 9 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_lambda_returns_carry.argtypes = [_vp] * 9 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_discounted_returns_carry.argtypes = [_vp] * 8 + [_i64, _i64, _f32, _vp]
    lib.rlscan_vtrace_carry.argtypes = [_vp] * 11 + [_i64, _i64, _f32, _f32, _f32, _vp]
    lib.rlscan_retrace_carry.argtypes = [_vp] * 12 + [_i64, _i64, _i64, _f32, _f32, _vp]
    lib.rlscan_eligibility_traces_carry.argtypes = [_vp] * 5 + [_i64, _i64, _f32, _f32, _vp]
    lib.rlscan_episodic_prefix_sum_carry.argtypes = [_vp] * 5 + [_i64, _i64, _vp]
    lib.rlscan_vtrace_ex.argtypes = [_vp] * 11 + [_i64, _i64] + [_f32] * 5 + [_vp]
    lib.rlscan_episodic_prefix_sum_f32.argtypes = [_vp] * 5 + [_i64, _i64, _vp]
    # the *_u8 calls take the argument list of the *_carry calls (V-trace: of
    # rlscan_vtrace_ex) with one-byte flags
    lib.rlscan_gae_u8.argtypes = lib.rlscan_gae_carry.argtypes
    lib.rlscan_lambda_returns_u8.argtypes = lib.rlscan_lambda_returns_carry.argtypes
    lib.rlscan_discounted_returns_u8.argtypes = lib.rlscan_discounted_returns_carry.argtypes
    lib.rlscan_vtrace_u8.argtypes = lib.rlscan_vtrace_ex.argtypes
    lib.rlscan_retrace_u8.argtypes = lib.rlscan_retrace_carry.argtypes
    lib.rlscan_eligibility_traces_u8.argtypes = lib.rlscan_eligibility_traces_carry.argtypes
    lib.rlscan_episodic_prefix_sum_u8.argtypes = lib.rlscan_episodic_prefix_sum_carry.argtypes
    for name in EXPORTED:
        if name.endswith(("_u8", "_ex", "_f32")):
            getattr(lib, name).restype = ctypes.c_int
    for name in ("rlscan_gae", "rlscan_lambda_returns", "rlscan_discounted_returns",
                 "rlscan_vtrace", "rlscan_retrace", "rlscan_eligibility_traces",
                 "rlscan_episodic_prefix_sum", "rlscan_release_scratch"):
        getattr(lib, name).restype = ctypes.c_int
        if name != "rlscan_release_scratch":
            getattr(lib, name + "_carry").restype = ctypes.c_int
    lib.rlscan_gae_noalloc.argtypes = lib.rlscan_gae_carry.argtypes
    lib.rlscan_gae_noalloc.restype = ctypes.c_int
    lib.rlscan_group.argtypes = [ctypes.POINTER(Call), ctypes.c_int32, _vp]
    lib.rlscan_group.restype = ctypes.c_int
    lib.rlscan_release_scratch.argtypes = []
    lib.rlscan_status_string.argtypes = [ctypes.c_int]
    lib.rlscan_status_string.restype = ctypes.c_char_p
    lib.rlscan_version.argtypes = []
    lib.rlscan_version.restype = ctypes.c_char_p
    lib.rlscan_plan.argtypes = [ctypes.c_int, _i64, _i64, _i64, ctypes.POINTER(PlanInfo)]
    lib.rlscan_plan.restype = ctypes.c_int
    lib.rlscan_set_launch_override.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64,
                                                ctypes.c_int]
    lib.rlscan_set_launch_override.restype = ctypes.c_int
    lib.rlscan_lookback_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.rlscan_lookback_timeouts.restype = ctypes.c_int
    lib.rlscan_launch_floor.argtypes = [_i64, ctypes.c_int32, _vp]
    lib.rlscan_launch_floor.restype = ctypes.c_int
    lib.rlscan_stream_copy.argtypes = [_vp, _vp, _i64, _vp]
    lib.rlscan_stream_copy.restype = ctypes.c_int
    lib.rlscan_set_xcd_run.argtypes = [_i64]
    lib.rlscan_set_xcd_run.restype = ctypes.c_int
    lib.rlscan_stream_mix.argtypes = [_vp, _i64, _vp, _i64, ctypes.c_int32, ctypes.c_int32, _vp]
    lib.rlscan_stream_mix.restype = ctypes.c_int
    lib.rlscan_stream_mix_arrays.argtypes = [_vp, _i64, _vp, _i64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, _vp]
    lib.rlscan_stream_mix_arrays.restype = ctypes.c_int


def library(path: str = LIB_PATH):
    """Loads librlscan.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"librlscan.so not found at {path}; build it first "
            "(python -m linear_recurrence_scan_coefficient_amd.build)")
    lib = ctypes.CDLL(path)
    _declare(lib)
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().rlscan_status_string(int(status)).decode()


def version() -> str:
    return library().rlscan_version().decode()


def _check(status: int):
    if status != RLSCAN_OK:
        raise RlscanError(status, status_string(status))


# ------------------------------------------------------------------ marshalling
_gpus = None


def _several_gpus():
    """Whether more than one GPU is visible (with one, every device tensor is
    on the current device)."""
    global _gpus
    if _gpus is None:
        _gpus = torch.cuda.device_count()
    return _gpus > 1


def _ptr(t, dtype=torch.float32, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() > 0 and t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.numel() > 0 and _several_gpus() and t.get_device() != torch.cuda.current_device():
        raise ValueError(f"{name} must live on the current device (cuda:"
                         f"{torch.cuda.current_device()}), got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _nt(t, name):
    if t is None or t.dim() != 2:
        raise ValueError(f"{name} must be a [N, T] tensor")
    return t.shape


# ------------------------------------------------------------------ entry points
# Every entry point below takes optional carry_in / carry_out [N] tensors
# (streaming one rollout through several calls); with either given it calls
# the *_carry C function, else the plain one.  Flags are float32, or uint8 /
# bool (one byte, set iff != 0) for every flag of the call, which calls the
# *_u8 C function.
def _carry(carry_in, carry_out, N, dtype=torch.float32):
    return (carry_in is not None or carry_out is not None,
            _ptr(carry_in, dtype=dtype, shape=(N,), name="carry_in"),
            _ptr(carry_out, dtype=dtype, shape=(N,), name="carry_out"))


_BYTE_FLAGS = (torch.uint8, torch.bool)


def _byte_flags(flags: dict) -> bool:
    """True if the given flag tensors are one-byte (uint8 or bool), False if
    float32; a mix of the two is refused."""
    kinds = {t.dtype in _BYTE_FLAGS for t in flags.values() if t is not None}
    if len(kinds) > 1:
        raise TypeError(f"flags {sorted(flags)} must all be float32 or all uint8/bool")
    return kinds == {True}


def _flag(t, N, T, name, byte):
    if t is None:
        return None
    if byte:
        if t.dtype not in _BYTE_FLAGS:
            raise TypeError(f"{name} must be uint8 or bool, got {t.dtype}")
        return _ptr(t, dtype=t.dtype, shape=(N, T), name=name)
    return _ptr(t, shape=(N, T), name=name)


def rlscan_gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
               advantages, gamma, lam, stream=None, carry_in=None, carry_out=None):
    N, T = _nt(rewards, "rewards")
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"terminated": terminated, "truncated": truncated})
    ins = (_ptr(rewards, shape=(N, T), name="rewards"), _ptr(values, shape=(N, T), name="values"),
           _ptr(bootstrap_value, shape=(N,), name="bootstrap_value"),
           _flag(terminated, N, T, "terminated", byte), _flag(truncated, N, T, "truncated", byte),
           _ptr(bootstrap_values, shape=(N, T), name="bootstrap_values"))
    out = _ptr(advantages, shape=(N, T), name="advantages")
    lib = library()
    if byte:
        _check(lib.rlscan_gae_u8(*ins, ci, out, co, N, T, gamma, lam, _stream(stream)))
    elif use:
        _check(lib.rlscan_gae_carry(*ins, ci, out, co, N, T, gamma, lam, _stream(stream)))
    else:
        _check(lib.rlscan_gae(*ins, out, N, T, gamma, lam, _stream(stream)))
    return advantages


def rlscan_gae_noalloc(rewards, values, bootstrap_value, terminated, truncated,
                       bootstrap_values, advantages, gamma, lam, stream=None, carry_in=None,
                       carry_out=None):
    """rlscan_gae_carry without any allocation (float32 flags): the look-back
    scratch is the library's fixed per-GPU array."""
    N, T = _nt(rewards, "rewards")
    _, ci, co = _carry(carry_in, carry_out, N)
    _check(library().rlscan_gae_noalloc(
        _ptr(rewards, shape=(N, T), name="rewards"), _ptr(values, shape=(N, T), name="values"),
        _ptr(bootstrap_value, shape=(N,), name="bootstrap_value"),
        _ptr(terminated, shape=(N, T), name="terminated"),
        _ptr(truncated, shape=(N, T), name="truncated"),
        _ptr(bootstrap_values, shape=(N, T), name="bootstrap_values"), ci,
        _ptr(advantages, shape=(N, T), name="advantages"), co, N, T, gamma, lam,
        _stream(stream)))
    return advantages


def rlscan_lambda_returns(rewards, values, bootstrap_value, terminated, truncated,
                          bootstrap_values, returns, gamma, lam, stream=None, carry_in=None,
                          carry_out=None):
    N, T = _nt(rewards, "rewards")
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"terminated": terminated, "truncated": truncated})
    ins = (_ptr(rewards, shape=(N, T), name="rewards"), _ptr(values, shape=(N, T), name="values"),
           _ptr(bootstrap_value, shape=(N,), name="bootstrap_value"),
           _flag(terminated, N, T, "terminated", byte), _flag(truncated, N, T, "truncated", byte),
           _ptr(bootstrap_values, shape=(N, T), name="bootstrap_values"))
    out = _ptr(returns, shape=(N, T), name="returns")
    lib = library()
    if byte:
        _check(lib.rlscan_lambda_returns_u8(*ins, ci, out, co, N, T, gamma, lam,
                                            _stream(stream)))
    elif use:
        _check(lib.rlscan_lambda_returns_carry(*ins, ci, out, co, N, T, gamma, lam,
                                               _stream(stream)))
    else:
        _check(lib.rlscan_lambda_returns(*ins, out, N, T, gamma, lam, _stream(stream)))
    return returns


def rlscan_discounted_returns(rewards, bootstrap_value, terminated, truncated, bootstrap_values,
                              returns, gamma, stream=None, carry_in=None, carry_out=None):
    N, T = _nt(rewards, "rewards")
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"terminated": terminated, "truncated": truncated})
    ins = (_ptr(rewards, shape=(N, T), name="rewards"),
           _ptr(bootstrap_value, shape=(N,), name="bootstrap_value"),
           _flag(terminated, N, T, "terminated", byte), _flag(truncated, N, T, "truncated", byte),
           _ptr(bootstrap_values, shape=(N, T), name="bootstrap_values"))
    out = _ptr(returns, shape=(N, T), name="returns")
    lib = library()
    if byte:
        _check(lib.rlscan_discounted_returns_u8(*ins, ci, out, co, N, T, gamma,
                                                _stream(stream)))
    elif use:
        _check(lib.rlscan_discounted_returns_carry(*ins, ci, out, co, N, T, gamma,
                                                   _stream(stream)))
    else:
        _check(lib.rlscan_discounted_returns(*ins, out, N, T, gamma, _stream(stream)))
    return returns


def rlscan_vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                  bootstrap_values, vs, pg_advantages, gamma, rho_bar, c_bar, stream=None,
                  carry_in=None, carry_out=None, lam=None, rho_bar_pg=None):
    """lam (trace factor) and rho_bar_pg (policy-gradient clip), when either is
    given, call rlscan_vtrace_ex (None: 1 and rho_bar)."""
    N, T = _nt(rewards, "rewards")
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"terminated": terminated, "truncated": truncated})
    ins = (_ptr(rewards, shape=(N, T), name="rewards"), _ptr(values, shape=(N, T), name="values"),
           _ptr(bootstrap_value, shape=(N,), name="bootstrap_value"),
           _ptr(log_rhos, shape=(N, T), name="log_rhos"),
           _flag(terminated, N, T, "terminated", byte), _flag(truncated, N, T, "truncated", byte),
           _ptr(bootstrap_values, shape=(N, T), name="bootstrap_values"))
    outs = (_ptr(vs, shape=(N, T), name="vs"),
            _ptr(pg_advantages, shape=(N, T), name="pg_advantages"))
    lib = library()
    ex = lam is not None or rho_bar_pg is not None
    lam = 1.0 if lam is None else lam
    rho_bar_pg = rho_bar if rho_bar_pg is None else rho_bar_pg
    if byte:
        _check(lib.rlscan_vtrace_u8(*ins, ci, *outs, co, N, T, gamma, lam, rho_bar, c_bar,
                                    rho_bar_pg, _stream(stream)))
    elif ex:
        _check(lib.rlscan_vtrace_ex(*ins, ci, *outs, co, N, T, gamma, lam, rho_bar, c_bar,
                                    rho_bar_pg, _stream(stream)))
    elif use:
        _check(lib.rlscan_vtrace_carry(*ins, ci, *outs, co, N, T, gamma, rho_bar, c_bar,
                                       _stream(stream)))
    else:
        _check(lib.rlscan_vtrace(*ins, *outs, N, T, gamma, rho_bar, c_bar, _stream(stream)))
    return vs, pg_advantages


def rlscan_retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                   terminated, truncated, targets, gamma, lam, stream=None, carry_in=None,
                   carry_out=None, next_actions=None, next_behaviour_probs=None):
    N, T = _nt(rewards, "rewards")
    if next_q_values_all is None or next_q_values_all.dim() != 3:
        raise ValueError("next_q_values_all must be a [N, T, A] tensor")
    A = next_q_values_all.shape[2]
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"terminated": terminated, "truncated": truncated})
    ins = (_ptr(rewards, shape=(N, T), name="rewards"),
           _ptr(next_q_values_all, shape=(N, T, A), name="next_q_values_all"),
           _ptr(next_target_probs, shape=(N, T, A), name="next_target_probs"),
           _ptr(actions, dtype=torch.int32, shape=(N, T), name="actions"),
           _ptr(behaviour_probs, shape=(N, T), name="behaviour_probs"),
           _flag(terminated, N, T, "terminated", byte), _flag(truncated, N, T, "truncated", byte))
    out = _ptr(targets, shape=(N, T), name="targets")
    lib = library()
    if use or byte:
        fn = lib.rlscan_retrace_u8 if byte else lib.rlscan_retrace_carry
        _check(fn(*ins, ci, _ptr(next_actions, dtype=torch.int32, shape=(N,), name="next_actions"),
                  _ptr(next_behaviour_probs, shape=(N,), name="next_behaviour_probs"), out, co,
                  N, T, A, gamma, lam, _stream(stream)))
    else:
        _check(lib.rlscan_retrace(*ins, out, N, T, A, gamma, lam, _stream(stream)))
    return targets


def rlscan_eligibility_traces(x, dones, traces, gamma, lam, stream=None, carry_in=None,
                              carry_out=None):
    N, T = _nt(x, "x")
    use, ci, co = _carry(carry_in, carry_out, N)
    byte = _byte_flags({"dones": dones})
    ins = (_ptr(x, shape=(N, T), name="x"), _flag(dones, N, T, "dones", byte))
    out = _ptr(traces, shape=(N, T), name="traces")
    lib = library()
    if byte:
        _check(lib.rlscan_eligibility_traces_u8(*ins, ci, out, co, N, T, gamma, lam,
                                                _stream(stream)))
    elif use:
        _check(lib.rlscan_eligibility_traces_carry(*ins, ci, out, co, N, T, gamma, lam,
                                                   _stream(stream)))
    else:
        _check(lib.rlscan_eligibility_traces(*ins, out, N, T, gamma, lam, _stream(stream)))
    return traces


def rlscan_episodic_prefix_sum(x, dones, out, stream=None, carry_in=None, carry_out=None):
    N, T = _nt(x, "x")
    use, ci, co = _carry(carry_in, carry_out, N, dtype=torch.int64)
    byte = _byte_flags({"dones": dones})
    ins = (_ptr(x, dtype=torch.int32, shape=(N, T), name="x"), _flag(dones, N, T, "dones", byte))
    o = _ptr(out, dtype=torch.int64, shape=(N, T), name="out")
    lib = library()
    if byte:
        _check(lib.rlscan_episodic_prefix_sum_u8(*ins, ci, o, co, N, T, _stream(stream)))
    elif use:
        _check(lib.rlscan_episodic_prefix_sum_carry(*ins, ci, o, co, N, T, _stream(stream)))
    else:
        _check(lib.rlscan_episodic_prefix_sum(*ins, o, N, T, _stream(stream)))
    return out


def rlscan_episodic_prefix_sum_f32(x, dones, out, stream=None, carry_in=None, carry_out=None):
    """Episodic prefix sum of float32 values x [N, T] into float32 out."""
    N, T = _nt(x, "x")
    _, ci, co = _carry(carry_in, carry_out, N)
    _check(library().rlscan_episodic_prefix_sum_f32(
        _ptr(x, shape=(N, T), name="x"), _ptr(dones, shape=(N, T), name="dones"), ci,
        _ptr(out, shape=(N, T), name="out"), co, N, T, _stream(stream)))
    return out


def _require_byte_flags(**flags):
    if not _byte_flags(flags) or any(t is None for k, t in flags.items() if k != "truncated"):
        raise TypeError(f"{', '.join(flags)} must be uint8 or bool tensors")


# The *_u8 names of the C ABI: the calls above with one-byte flags required.
def rlscan_gae_u8(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
                  advantages, gamma, lam, stream=None, carry_in=None, carry_out=None):
    _require_byte_flags(terminated=terminated, truncated=truncated)
    return rlscan_gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
                      advantages, gamma, lam, stream, carry_in, carry_out)


def rlscan_lambda_returns_u8(rewards, values, bootstrap_value, terminated, truncated,
                             bootstrap_values, returns, gamma, lam, stream=None, carry_in=None,
                             carry_out=None):
    _require_byte_flags(terminated=terminated, truncated=truncated)
    return rlscan_lambda_returns(rewards, values, bootstrap_value, terminated, truncated,
                                 bootstrap_values, returns, gamma, lam, stream, carry_in,
                                 carry_out)


def rlscan_discounted_returns_u8(rewards, bootstrap_value, terminated, truncated,
                                 bootstrap_values, returns, gamma, stream=None, carry_in=None,
                                 carry_out=None):
    _require_byte_flags(terminated=terminated, truncated=truncated)
    return rlscan_discounted_returns(rewards, bootstrap_value, terminated, truncated,
                                     bootstrap_values, returns, gamma, stream, carry_in,
                                     carry_out)


def rlscan_vtrace_ex(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                     bootstrap_values, vs, pg_advantages, gamma, lam, rho_bar, c_bar,
                     rho_bar_pg, stream=None, carry_in=None, carry_out=None):
    return rlscan_vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                         bootstrap_values, vs, pg_advantages, gamma, rho_bar, c_bar, stream,
                         carry_in, carry_out, lam=lam, rho_bar_pg=rho_bar_pg)


def rlscan_vtrace_u8(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                     bootstrap_values, vs, pg_advantages, gamma, lam, rho_bar, c_bar,
                     rho_bar_pg, stream=None, carry_in=None, carry_out=None):
    _require_byte_flags(terminated=terminated, truncated=truncated)
    return rlscan_vtrace_ex(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                            bootstrap_values, vs, pg_advantages, gamma, lam, rho_bar, c_bar,
                            rho_bar_pg, stream, carry_in, carry_out)


def rlscan_retrace_u8(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                      terminated, truncated, targets, gamma, lam, stream=None, carry_in=None,
                      carry_out=None, next_actions=None, next_behaviour_probs=None):
    _require_byte_flags(terminated=terminated, truncated=truncated)
    return rlscan_retrace(rewards, next_q_values_all, next_target_probs, actions,
                          behaviour_probs, terminated, truncated, targets, gamma, lam, stream,
                          carry_in, carry_out, next_actions, next_behaviour_probs)


def rlscan_eligibility_traces_u8(x, dones, traces, gamma, lam, stream=None, carry_in=None,
                                 carry_out=None):
    _require_byte_flags(dones=dones)
    return rlscan_eligibility_traces(x, dones, traces, gamma, lam, stream, carry_in, carry_out)


def rlscan_episodic_prefix_sum_u8(x, dones, out, stream=None, carry_in=None, carry_out=None):
    _require_byte_flags(dones=dones)
    return rlscan_episodic_prefix_sum(x, dones, out, stream, carry_in, carry_out)


class GroupCall:
    """One call of a grouped launch: the estimator's inputs and outputs as
    tensors in the order of its plain entry point (None for an absent
    optional input).  One-byte flags (uint8 / bool) set the byte-flag bit."""

    def __init__(self, estimator, inputs, outputs, gamma=0.99, lam=0.95, rho_bar=1.0,
                 c_bar=1.0, rho_bar_pg=None):
        if estimator not in ESTIMATOR_IDS:
            raise ValueError(f"unknown estimator {estimator!r}")
        if len(inputs) > 8 or len(outputs) > 2:
            raise ValueError("at most 8 inputs and 2 outputs")
        first = inputs[0]
        if first is None or first.dim() != 2:
            raise ValueError("the first input must be a [N, T] tensor")
        N, T = first.shape
        flags = {f"input {i}": inputs[i] for i in _FLAG_SLOTS[estimator] if i < len(inputs)}
        byte = _byte_flags(flags)
        self.keep = (tuple(inputs), tuple(outputs))  # the tensors outlive the launch
        c = Call()
        c.estimator = ESTIMATOR_IDS[estimator]
        c.flags = CALL_BYTE_FLAGS if byte else 0
        c.N, c.T = N, T
        c.A = 1
        if estimator == "retrace":
            q = inputs[1] if len(inputs) > 1 else None
            if q is None or q.dim() != 3:
                raise ValueError("Retrace's next_q_values_all must be a [N, T, A] tensor")
            c.A = q.shape[2]
        c.gamma, c.lam = gamma, lam
        c.rho_bar, c.c_bar = rho_bar, c_bar
        c.rho_bar_pg = rho_bar if rho_bar_pg is None else rho_bar_pg
        for i, t in enumerate(inputs):
            c.inp[i] = None if t is None else _ptr(t, dtype=t.dtype, name=f"input {i}")
        for i, t in enumerate(outputs):
            c.out[i] = None if t is None else _ptr(t, dtype=t.dtype, name=f"output {i}")
        self.call = c


def rlscan_group(calls, stream=None):
    """Runs the GroupCall list `calls` in one kernel launch (rlscan_group)."""
    arr = (Call * len(calls))(*[c.call for c in calls])
    _check(library().rlscan_group(arr, len(calls), _stream(stream)))


def rlscan_release_scratch():
    _check(library().rlscan_release_scratch())


def rlscan_plan(estimator, N, T, A=1) -> dict:
    info = PlanInfo()
    est = ESTIMATOR_IDS[estimator] if isinstance(estimator, str) else int(estimator)
    _check(library().rlscan_plan(est, N, T, A, ctypes.byref(info)))
    return {f[0]: getattr(info, f[0]) for f in PlanInfo._fields_}


def rlscan_set_launch_override(mapping=MAP_AUTO, rounds=0, waves=0, grid_cap=0, flags=0):
    _check(library().rlscan_set_launch_override(int(mapping), int(rounds), int(waves), int(grid_cap),
                                                int(flags)))


def rlscan_set_xcd_run(run=-1):
    """Tiles per XCD run of packed and grouped launches (-1: the library's
    choice, 0: tile = workgroup index)."""
    _check(library().rlscan_set_xcd_run(int(run)))


def rlscan_lookback_timeouts() -> int:
    n = ctypes.c_uint64()
    _check(library().rlscan_lookback_timeouts(ctypes.byref(n)))
    return n.value


def rlscan_launch_floor(grid, threads=256, stream=None):
    _check(library().rlscan_launch_floor(int(grid), int(threads), _stream(stream)))


def rlscan_stream_copy(dst, src, nbytes=None, stream=None):
    """Streaming copy of `nbytes` (default: all of `src`) between two
    contiguous device tensors."""
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    if nbytes > dst.numel() * dst.element_size() or nbytes > src.numel() * src.element_size():
        raise RlscanError(RLSCAN_ERR_SHAPE, "rlscan_stream_copy: nbytes exceeds a tensor")
    _check(library().rlscan_stream_copy(dst.data_ptr(), src.data_ptr(), int(nbytes),
                                        _stream(stream)))


def rlscan_stream_mix_arrays(dst, src, write_bytes=None, read_bytes=None, arrays_in=1,
                             arrays_out=1, words=1, workgroups_per_cu=0, stream=None):
    """Streaming kernel in a scan's access pattern: `src` as `arrays_in`
    arrays, `dst` as `arrays_out` arrays; word i of every output array gets
    the sum of word i of every input array; `words` indices per thread; at
    most `workgroups_per_cu` resident workgroups per CU (0: no cap)."""
    if read_bytes is None:
        read_bytes = src.numel() * src.element_size()
    if write_bytes is None:
        write_bytes = dst.numel() * dst.element_size()
    if read_bytes > src.numel() * src.element_size() or \
            write_bytes > dst.numel() * dst.element_size():
        raise RlscanError(RLSCAN_ERR_SHAPE, "rlscan_stream_mix_arrays: a size exceeds its tensor")
    _check(library().rlscan_stream_mix_arrays(dst.data_ptr(), int(write_bytes), src.data_ptr(),
                                              int(read_bytes), int(arrays_in), int(arrays_out),
                                              int(words), int(workgroups_per_cu),
                                              _stream(stream)))


def rlscan_stream_mix(dst, src, write_bytes=None, read_bytes=None, reads=1, writes=1,
                      stream=None):
    """Streaming kernel reading `read_bytes` of `src` and writing
    `write_bytes` of `dst` (defaults: whole tensors), `reads` and `writes`
    16-byte words per thread."""
    if read_bytes is None:
        read_bytes = src.numel() * src.element_size()
    if write_bytes is None:
        write_bytes = dst.numel() * dst.element_size()
    if read_bytes > src.numel() * src.element_size() or \
            write_bytes > dst.numel() * dst.element_size():
        raise RlscanError(RLSCAN_ERR_SHAPE, "rlscan_stream_mix: a size exceeds its tensor")
    _check(library().rlscan_stream_mix(dst.data_ptr(), int(write_bytes), src.data_ptr(),
                                       int(read_bytes), int(reads), int(writes),
                                       _stream(stream)))
