"""GPU parity of the estimator variants: one-byte flags (every estimator),
V-trace with a trace factor lambda and a separate policy-gradient clip, and
the float-valued episodic prefix sum.

One-byte flags run the same arithmetic as float flags (any nonzero byte
counts as set), so their results equal the float-flag call's on the same
inputs -- bit for bit where the call is deterministic (packed mappings,
integer outputs), to a few ulps where the look-back's combination order
varies between runs -- and are within tolerance of the float64 oracle.  The
V-trace options and the float prefix sum are compared element by element
with their oracle functions; with lambda = 1 and rho_bar_pg = rho_bar the
V-trace call must equal the plain call bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from reference import assert_parity, oracle_outputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from linear_recurrence_scan_coefficient_amd import api, device, rlscan, workloads  # noqa: E402
from linear_recurrence_scan_coefficient_amd.workloads import ESTIMATORS  # noqa: E402

TRUNC = ("gae", "lambda_returns", "discounted_returns", "vtrace", "retrace")
FLAG_KEYS = ("terminated", "truncated", "dones")


@pytest.fixture(autouse=True)
def _reset_override():
    rlscan.rlscan_set_launch_override()
    yield
    rlscan.rlscan_set_launch_override()


@pytest.fixture(scope="module", autouse=True)
def _no_lookback_timeouts():
    yield
    assert rlscan.rlscan_lookback_timeouts() == 0


def case(estimator, N, T, seed, **kw):
    opts = dict(term_p=0.05, done_p=0.05, gamma=0.97, lam=0.9)
    if estimator in TRUNC:
        opts.update(trunc_mode="independent", trunc_p=0.05)
    opts.update(kw)
    w = workloads.custom(N, T, **opts)
    return w, workloads.inputs_for(estimator, w, seed)


def byte_flags(d, seed, dtype=torch.uint8):
    """The flags of `d` (device tensors) as one-byte tensors; set flags get a
    random nonzero byte (bool: True)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = dict(d)
    for k in FLAG_KEYS:
        t = d.get(k)
        if t is None:
            continue
        if dtype == torch.bool:
            out[k] = t != 0
        else:
            vals = torch.randint(1, 256, t.shape, generator=g, dtype=torch.int32).to(t.device)
            out[k] = torch.where(t != 0, vals, torch.zeros_like(vals)).to(torch.uint8)
    return out


def host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def run_both(estimator, w, inputs, seed, dtype=torch.uint8):
    d = device.upload(inputs)
    ref = device.alloc_outputs(estimator, w.N, w.T)
    device.call(estimator, d, ref, w)
    got = device.alloc_outputs(estimator, w.N, w.T)
    device.call(estimator, byte_flags(d, seed, dtype), got, w)
    torch.cuda.synchronize()
    return host(ref), host(got)


def same_results(estimator, w, got, ref, label=""):
    """Bit for bit where the call is deterministic: packed calls, and integer
    outputs.  Float results of look-back calls may differ in the last bits
    between any two runs (the walk composes whichever predecessor tiles are
    ready), so there they agree to a few float32 ulps."""
    packed = rlscan.rlscan_plan(estimator, w.N, w.T, w.A)["mapping"] == rlscan.MAP_PACKED
    for k in ref:
        if packed or np.issubdtype(ref[k].dtype, np.integer):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{estimator} {k} {label}")
        else:
            r = ref[k].astype(np.float64)
            err = np.abs(got[k].astype(np.float64) - r) / (1.0 + np.abs(r))
            assert err.max() <= 1e-5, (estimator, k, label, float(err.max()))


def check_bytes(estimator, w, inputs, seed, label="", dtype=torch.uint8):
    print(f"[variants] byte flags {estimator} {w.N}x{w.T} {label}", flush=True)
    ref, got = run_both(estimator, w, inputs, seed, dtype)
    same_results(estimator, w, got, ref, label)
    assert_parity(got, oracle_outputs(estimator, inputs, w), f"u8 {estimator} {label}")


SHAPES = [(1, 1), (3, 3), (5, 64), (3, 65), (2, 255), (37, 129), (64, 512), (3, 5000),
          (2, 20000)]


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{n}x{t}" for n, t in SHAPES])
def test_byte_flags_match_float_flags(estimator, shape):
    w, inputs = case(estimator, *shape, seed=shape[0] * 31 + shape[1])
    check_bytes(estimator, w, inputs, seed=shape[1])


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_bool_flags(estimator):
    w, inputs = case(estimator, 19, 777, seed=3)
    check_bytes(estimator, w, inputs, seed=3, label="bool", dtype=torch.bool)


MAPPINGS = {"lookback": rlscan.MAP_LOOKBACK, "packed": rlscan.MAP_PACKED}
RW = [(1, 1), (1, 2), (1, 4), (1, 8), (2, 4), (2, 8), (4, 4), (4, 8)]


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("mapping", list(MAPPINGS))
@pytest.mark.parametrize("rounds,waves", RW, ids=[f"R{r}W{w}" for r, w in RW])
def test_byte_flags_across_launch_shapes(estimator, mapping, rounds, waves):
    rlscan.rlscan_set_launch_override(MAPPINGS[mapping], rounds, waves, 0, 0)
    for N, T in ((512, 128), (3, 3001)):
        w, inputs = case(estimator, N, T, seed=N + T + rounds)
        check_bytes(estimator, w, inputs, seed=rounds * 8 + waves,
                    label=f"{mapping} R={rounds} W={waves}")


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("offset", [1, 4])
def test_byte_flags_offset(estimator, offset):
    """Flag tensors starting `offset` bytes into their buffer: 1 takes the
    scalar path, 4 keeps the vector path with a base that is not 16-byte
    aligned."""
    w, inputs = case(estimator, 9, 1500, seed=offset)
    d = device.upload(inputs)
    ref = device.alloc_outputs(estimator, w.N, w.T)
    device.call(estimator, d, ref, w)
    b = byte_flags(d, seed=offset)
    for k in FLAG_KEYS:
        if b.get(k) is not None:
            buf = torch.zeros(b[k].numel() + offset, dtype=torch.uint8, device="cuda")
            view = buf[offset:].view(b[k].shape)
            view.copy_(b[k])
            b[k] = view
    got = device.alloc_outputs(estimator, w.N, w.T)
    print(f"[variants] byte flags offset {offset} {estimator}", flush=True)
    device.call(estimator, b, got, w)
    torch.cuda.synchronize()
    same_results(estimator, w, host(got), host(ref), f"offset {offset}")
    assert_parity(host(got), oracle_outputs(estimator, inputs, w), f"u8 offset {estimator}")


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_byte_flags_with_carry(estimator):
    """The compute_* calls chained over two pieces of each row through the
    carry, with bool flags (which take the one-byte kernels)."""
    w, inputs = case(estimator, 6, 2500, seed=29)
    d = device.upload(inputs)
    whole = device.alloc_outputs(estimator, w.N, w.T)
    device.call(estimator, d, whole, w)
    b = byte_flags(d, seed=29, dtype=torch.bool)
    T1 = 1111
    part = lambda lo, hi: {k: (v[:, lo:hi].contiguous() if v is not None and v.dim() >= 2  # noqa: E731
                               else v) for k, v in b.items()}
    g, lam = w.gamma, w.lam
    print(f"[variants] byte flags carry {estimator}", flush=True)
    if estimator == "eligibility_traces":
        a, z = part(0, T1), part(T1, w.T)
        first, c = api.compute_eligibility_traces(a["x"], a["dones"], g, lam, return_carry=True)
        second = api.compute_eligibility_traces(z["x"], z["dones"], g, lam, carry_in=c)
        got = {"traces": torch.cat([first, second], 1)}
    elif estimator == "episodic_prefix_sum":
        a, z = part(0, T1), part(T1, w.T)
        first, c = api.compute_episodic_prefix_sum(a["x"], a["dones"], return_carry=True)
        second = api.compute_episodic_prefix_sum(z["x"], z["dones"], carry_in=c)
        got = {"out": torch.cat([first, second], 1)}
    elif estimator == "retrace":
        early, late = part(0, T1), part(T1, w.T)
        l, c = api.compute_retrace(late["rewards"], late["next_q_values_all"],
                                   late["next_target_probs"], late["actions"],
                                   late["behaviour_probs"], late["terminated"],
                                   late["truncated"], g, lam, return_carry=True)
        e = api.compute_retrace(early["rewards"], early["next_q_values_all"],
                                early["next_target_probs"], early["actions"],
                                early["behaviour_probs"], early["terminated"],
                                early["truncated"], g, lam, carry_in=c,
                                next_actions=b["actions"][:, T1].contiguous(),
                                next_behaviour_probs=b["behaviour_probs"][:, T1].contiguous())
        got = {"targets": torch.cat([e, l], 1)}
    elif estimator == "vtrace":
        early, late = part(0, T1), part(T1, w.T)
        vb = b["values"][:, T1].contiguous()
        lv, lp, c = api.compute_vtrace(late["rewards"], late["values"], late["log_rhos"],
                                       late["terminated"], g, w.rho_bar, w.c_bar,
                                       bootstrap_value=b.get("bootstrap_value"),
                                       truncateds=late.get("truncated"),
                                       bootstrap_values=late.get("bootstrap_values"),
                                       return_carry=True)
        ev, ep = api.compute_vtrace(early["rewards"], early["values"], early["log_rhos"],
                                    early["terminated"], g, w.rho_bar, w.c_bar,
                                    bootstrap_value=vb, truncateds=early.get("truncated"),
                                    bootstrap_values=early.get("bootstrap_values"), carry_in=c)
        got = {"vs": torch.cat([ev, lv], 1), "pg_advantages": torch.cat([ep, lp], 1)}
    else:
        fn = {"gae": api.compute_gae, "lambda_returns": api.compute_lambda_returns}.get(estimator)
        early, late = part(0, T1), part(T1, w.T)
        if fn is not None:
            vb = b["values"][:, T1].contiguous()
            l, c = fn(late["rewards"], late["values"], late["terminated"], g, lam,
                      bootstrap_value=b.get("bootstrap_value"), truncateds=late.get("truncated"),
                      bootstrap_values=late.get("bootstrap_values"), return_carry=True)
            e = fn(early["rewards"], early["values"], early["terminated"], g, lam,
                   bootstrap_value=vb, truncateds=early.get("truncated"),
                   bootstrap_values=early.get("bootstrap_values"), carry_in=c)
        else:
            l, c = api.compute_discounted_returns(
                late["rewards"], late["terminated"], g, bootstrap_value=b.get("bootstrap_value"),
                truncateds=late.get("truncated"), bootstrap_values=late.get("bootstrap_values"),
                return_carry=True)
            e = api.compute_discounted_returns(
                early["rewards"], early["terminated"], g, truncateds=early.get("truncated"),
                bootstrap_values=early.get("bootstrap_values"), carry_in=c)
        got = {device.OUTPUTS[estimator][0][0]: torch.cat([e, l], 1)}
    got = host(got)
    for k, ref in host(whole).items():
        if np.issubdtype(ref.dtype, np.integer):
            np.testing.assert_array_equal(got[k], ref)
        else:
            r = ref.astype(np.float64)
            err = np.abs(got[k].astype(np.float64) - r) / (1 + np.abs(r))
            assert err.max() <= 1e-4, (k, float(err.max()))


@pytest.mark.parametrize("name", ["long_8x1048576", "production_4096x128"])
def test_byte_flags_benchmark_workloads(name):
    """The benchmark's workloads, in the launch configuration it times, with
    one-byte flags: against the float-flag call and the oracle in full."""
    w = workloads.get(name)
    for est in w.estimators:
        inputs = workloads.inputs_for(est, w, 0)
        ref, got = run_both(est, w, inputs, seed=5)
        same_results(est, w, got, ref, name)
        assert_parity(got, oracle_outputs(est, inputs, w), f"u8 {name} {est}")
        print(f"[variants] {name} byte flags {est} ok", flush=True)


def test_byte_flag_arguments_are_checked():
    d = {k: torch.zeros((2, 8), device="cuda") for k in ("r", "v", "t")}
    out = torch.empty((2, 8), device="cuda")
    mixed = torch.zeros((2, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(TypeError):
        rlscan.rlscan_gae(d["r"], d["v"], None, d["t"], mixed, d["r"], out, 0.9, 0.9)
    with pytest.raises(TypeError):
        rlscan.rlscan_gae_u8(d["r"], d["v"], None, d["t"], None, None, out, 0.9, 0.9)
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_gae_u8(d["r"], d["v"], None, mixed, mixed, None, out, 0.9, 0.9)
    assert e.value.status == rlscan.RLSCAN_ERR_NULL  # truncated without bootstrap_values


# ---------------------------------------------------------------- V-trace options
# lambda = 0, and a lambda so small that lambda*c rounds to 0 in float32, make
# a_t = 0 at steps that are not cuts, where pg_t still reads u_{t+1}
VT_OPTS = [(1.0, None), (0.8, None), (1.0, 0.5), (0.3, 2.0), (0.0, 1.0), (1e-45, None)]


def vtrace_call(d, w, lam, rho_bar_pg, carry_in=None, carry_out=None):
    vs = torch.empty((w.N, w.T), device="cuda")
    pg = torch.empty((w.N, w.T), device="cuda")
    rlscan.rlscan_vtrace_ex(d["rewards"], d["values"], d.get("bootstrap_value"), d["log_rhos"],
                            d["terminated"], d.get("truncated"), d.get("bootstrap_values"), vs,
                            pg, w.gamma, lam, w.rho_bar, w.c_bar,
                            w.rho_bar if rho_bar_pg is None else rho_bar_pg,
                            carry_in=carry_in, carry_out=carry_out)
    return vs, pg


def vtrace_oracle(inputs, w, lam, rho_bar_pg, **kw):
    return oracle.vtrace(inputs["rewards"], inputs["values"], inputs["log_rhos"],
                         inputs["terminated"], gamma=w.gamma, rho_bar=w.rho_bar, c_bar=w.c_bar,
                         lam=lam, rho_bar_pg=rho_bar_pg,
                         bootstrap_value=inputs.get("bootstrap_value"),
                         truncated=inputs.get("truncated"),
                         bootstrap_values=inputs.get("bootstrap_values"), **kw)


@pytest.mark.parametrize("lam,rho_bar_pg", VT_OPTS, ids=[f"l{l}-pg{p}" for l, p in VT_OPTS])
@pytest.mark.parametrize("shape", [(4096, 128), (3, 5000), (37, 129), (1, 1)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_vtrace_options(lam, rho_bar_pg, shape):
    w, inputs = case("vtrace", *shape, seed=shape[1] + int(lam * 10), rho_bar=1.2, c_bar=0.9)
    d = device.upload(inputs)
    print(f"[variants] vtrace lam={lam} rho_bar_pg={rho_bar_pg} {shape}", flush=True)
    vs, pg = vtrace_call(d, w, lam, rho_bar_pg)
    torch.cuda.synchronize()
    want_vs, want_pg = vtrace_oracle(inputs, w, lam, rho_bar_pg)
    assert_parity({"vs": vs.cpu().numpy(), "pg_advantages": pg.cpu().numpy()},
                  {"vs": want_vs, "pg_advantages": want_pg}, f"vtrace_ex {lam} {rho_bar_pg}")


def test_vtrace_options_default_is_the_plain_call():
    w, inputs = case("vtrace", 4096, 128, seed=8, rho_bar=1.5, c_bar=0.7)  # packed
    d = device.upload(inputs)
    plain = device.alloc_outputs("vtrace", w.N, w.T)
    device.call("vtrace", d, plain, w)
    vs, pg = vtrace_call(d, w, 1.0, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vs.cpu().numpy(), plain["vs"].cpu().numpy())
    np.testing.assert_array_equal(pg.cpu().numpy(), plain["pg_advantages"].cpu().numpy())


def test_vtrace_options_with_carry_and_byte_flags():
    w, inputs = case("vtrace", 21, 700, seed=12)
    rng = np.random.default_rng(12)
    inputs["bootstrap_value"] = rng.standard_normal(w.N).astype(np.float32)
    ci = rng.standard_normal(w.N).astype(np.float32)
    lam, rho_bar_pg = 0.7, 0.4
    want_vs, want_pg, want_co = vtrace_oracle(inputs, w, lam, rho_bar_pg, carry_in=ci,
                                              return_carry=True)
    d = byte_flags(device.upload(inputs), seed=12)
    co = torch.empty(w.N, device="cuda")
    vs = torch.empty((w.N, w.T), device="cuda")
    pg = torch.empty((w.N, w.T), device="cuda")
    rlscan.rlscan_vtrace_u8(d["rewards"], d["values"], d["bootstrap_value"], d["log_rhos"],
                            d["terminated"], d["truncated"], d["bootstrap_values"], vs, pg,
                            w.gamma, lam, w.rho_bar, w.c_bar, rho_bar_pg,
                            carry_in=torch.from_numpy(ci).cuda(), carry_out=co)
    torch.cuda.synchronize()
    assert_parity({"vs": vs.cpu().numpy(), "pg_advantages": pg.cpu().numpy(),
                   "carry_out": co.cpu().numpy()},
                  {"vs": want_vs, "pg_advantages": want_pg, "carry_out": want_co},
                  "vtrace u8 carry")


def test_vtrace_option_arguments_are_checked():
    z = torch.zeros((2, 8), device="cuda")
    out = torch.empty((2, 8), device="cuda")
    out2 = torch.empty((2, 8), device="cuda")
    for lam, pgc in ((1.5, 1.0), (-0.1, 1.0), (1.0, 0.0), (1.0, float("nan"))):
        with pytest.raises(rlscan.RlscanError) as e:
            rlscan.rlscan_vtrace_ex(z, z, None, z, z, None, None, out, out2, 0.9, lam, 1.0, 1.0,
                                    pgc)
        assert e.value.status == rlscan.RLSCAN_ERR_PARAM


# ---------------------------------------------------------------- float prefix sum
@pytest.mark.parametrize("shape", [(1, 1), (3, 65), (4096, 128), (37, 129), (3, 5000),
                                   (2, 20000)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_float_prefix_sum(shape):
    N, T = shape
    rng = np.random.default_rng(N * 13 + T)
    x = rng.standard_normal((N, T)).astype(np.float32)
    dones = (rng.random((N, T)) < 0.01).astype(np.float32)
    out = torch.empty((N, T), device="cuda")
    print(f"[variants] float prefix sum {shape}", flush=True)
    rlscan.rlscan_episodic_prefix_sum_f32(torch.from_numpy(x).cuda(),
                                          torch.from_numpy(dones).cuda(), out)
    torch.cuda.synchronize()
    assert_parity({"out": out.cpu().numpy()},
                  {"out": oracle.episodic_prefix_sum_float(x, dones)}, "prefix f32")


def test_float_prefix_sum_carry_and_long_rows():
    """8 x 2^20 with rare dones (|y| grows to hundreds) and a carry."""
    N, T = 8, 1 << 20
    rng = np.random.default_rng(77)
    x = rng.standard_normal((N, T)).astype(np.float32)
    dones = (rng.random((N, T)) < 1e-4).astype(np.float32)
    ci = rng.standard_normal(N).astype(np.float32)
    out = torch.empty((N, T), device="cuda")
    co = torch.empty(N, device="cuda")
    rlscan.rlscan_episodic_prefix_sum_f32(torch.from_numpy(x).cuda(),
                                          torch.from_numpy(dones).cuda(), out,
                                          carry_in=torch.from_numpy(ci).cuda(), carry_out=co)
    torch.cuda.synchronize()
    want, want_co = oracle.episodic_prefix_sum_float(x, dones, carry_in=ci, return_carry=True)
    assert_parity({"out": out.cpu().numpy(), "carry_out": co.cpu().numpy()},
                  {"out": want, "carry_out": want_co}, "prefix f32 long")
