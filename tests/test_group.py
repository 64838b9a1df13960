"""GPU parity of rlscan_group (several estimator calls in one kernel launch)
against the float64 oracle and against the same calls made one by one.

Cases: the seven estimators at the 4096 x 128 production shape, mixed shapes
that need wider tiles, one-byte flags and V-trace's options inside a group,
more calls than one launch takes, graph capture and replay, and the calls a
group refuses (nothing may be written then).  The shape cases run with the
calls' tiles laid out call after call (the default) and interleaved over the
grid."""
from __future__ import annotations

import numpy as np
import pytest

from reference import assert_parity, oracle_outputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from linear_recurrence_scan_coefficient_amd import device, rlscan, workloads  # noqa: E402
from linear_recurrence_scan_coefficient_amd.workloads import ESTIMATORS  # noqa: E402

TRUNC = ("gae", "lambda_returns", "discounted_returns", "vtrace", "retrace")


@pytest.fixture(autouse=True)
def _reset_override():
    rlscan.rlscan_set_launch_override()
    yield
    rlscan.rlscan_set_launch_override()


def case(estimator, N, T, seed, **kw):
    opts = dict(term_p=0.05, done_p=0.05, gamma=0.97, lam=0.9)
    if estimator in TRUNC:
        opts.update(trunc_mode="independent", trunc_p=0.05)
    opts.update(kw)
    w = workloads.custom(N, T, **opts)
    return w, workloads.inputs_for(estimator, w, seed)


FLAG_KEYS = ("terminated", "truncated", "dones")
LAYOUTS = {"contiguous": 0, "interleaved": rlscan.FLAG_GROUP_INTERLEAVED}


def group_call(estimator, d, out, w, **kw):
    ins = tuple(d.get(k) for k in device.INPUT_ORDER[estimator])
    outs = tuple(out[name] for name, _ in device.OUTPUTS[estimator])
    opts = dict(gamma=w.gamma, lam=w.lam, rho_bar=w.rho_bar, c_bar=w.c_bar)
    if estimator == "vtrace":
        opts["lam"] = 1.0
    opts.update(kw)
    return rlscan.GroupCall(estimator, ins, outs, **opts)


def host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def close_to(got, ref, label):
    for k in ref:
        if np.issubdtype(ref[k].dtype, np.integer):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=label)
        else:
            r = ref[k].astype(np.float64)
            err = np.abs(got[k].astype(np.float64) - r) / (1.0 + np.abs(r))
            assert err.max() <= 1e-6, (label, k, float(err.max()))


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("waves", [0, 1, 2, 4])
def test_group_of_the_seven_production_calls(waves, layout):
    """All seven estimators at 4096 x 128 in one launch: the oracle, and the
    same calls made one by one."""
    w = workloads.get("production_4096x128")
    data = {e: device.upload(workloads.inputs_for(e, w, 3)) for e in ESTIMATORS}
    singles, grouped, calls = {}, {}, []
    for e in ESTIMATORS:
        singles[e] = device.alloc_outputs(e, w.N, w.T)
        device.call(e, data[e], singles[e], w)
        grouped[e] = device.alloc_outputs(e, w.N, w.T)
        calls.append(group_call(e, data[e], grouped[e], w))
    rlscan.rlscan_set_launch_override(waves=waves, flags=LAYOUTS[layout])
    print(f"[group] production seven, waves={waves}, {layout}", flush=True)
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    for e in ESTIMATORS:
        got = host(grouped[e])
        close_to(got, host(singles[e]), f"group vs single {e}")
        assert_parity(got, oracle_outputs(e, workloads.inputs_for(e, w, 3), w), f"group {e}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_group_of_mixed_shapes_flags_and_options(layout):
    """Different shapes in one group (the tile grows to hold 512-step rows),
    one-byte flags, Retrace with 4 and 8 actions, V-trace with lambda and a
    policy-gradient clip, a ragged last tile, and three 300-step rows that
    fit only the 1024-element tile as one."""
    specs = [("retrace", 300, 128, dict(A=8)), ("gae", 64, 512, {}),
             ("vtrace", 1000, 32, {}), ("episodic_prefix_sum", 77, 256, {}),
             ("retrace", 129, 64, dict(A=4)), ("discounted_returns", 5, 1, {}),
             ("eligibility_traces", 3, 300, {}), ("lambda_returns", 999, 16, {})]
    calls, outs, want = [], [], []
    for i, (e, N, T, kw) in enumerate(specs):
        w, inputs = case(e, N, T, seed=100 + i, **kw)
        d = device.upload(inputs)
        if i % 2 == 1:  # every other call with one-byte flags
            for k in FLAG_KEYS:
                if d.get(k) is not None:
                    d[k] = (d[k] != 0).to(torch.uint8)
        out = device.alloc_outputs(e, N, T)
        opts = {}
        if e == "vtrace":
            opts = dict(lam=0.8, rho_bar_pg=0.6)
            vs, pg = oracle.vtrace(inputs["rewards"], inputs["values"], inputs["log_rhos"],
                                   inputs["terminated"], gamma=w.gamma, rho_bar=w.rho_bar,
                                   c_bar=w.c_bar, lam=0.8, rho_bar_pg=0.6,
                                   bootstrap_value=inputs.get("bootstrap_value"),
                                   truncated=inputs.get("truncated"),
                                   bootstrap_values=inputs.get("bootstrap_values"))
            want.append({"vs": vs, "pg_advantages": pg})
        else:
            want.append(oracle_outputs(e, inputs, w))
        calls.append(group_call(e, d, out, w, **opts))
        outs.append(out)
    rlscan.rlscan_set_launch_override(flags=LAYOUTS[layout])
    print(f"[group] mixed shapes, {layout}", flush=True)
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    for (e, N, T, _), out, ref in zip(specs, outs, want):
        assert_parity(host(out), ref, f"group mixed {e} {N}x{T}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_group_of_more_calls_than_one_launch_takes(layout):
    calls, outs, want = [], [], []
    for i in range(19):
        e = ESTIMATORS[i % len(ESTIMATORS)]
        w, inputs = case(e, 40 + i, 64, seed=200 + i)
        d = device.upload(inputs)
        out = device.alloc_outputs(e, w.N, w.T)
        calls.append(group_call(e, d, out, w))
        outs.append(out)
        want.append((e, oracle_outputs(e, inputs, w)))
    rlscan.rlscan_set_launch_override(flags=LAYOUTS[layout])
    print(f"[group] 19 calls, {layout}", flush=True)
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    for out, (e, ref) in zip(outs, want):
        assert_parity(host(out), ref, f"group of 19 {e}")


def test_group_graph_capture_and_replay():
    """A grouped launch captured into a HIP graph, replayed several times
    with eager work and synchronisation between replays."""
    w = workloads.get("production_4096x128")
    data = {e: device.upload(workloads.inputs_for(e, w, 4)) for e in ESTIMATORS}
    outs = {e: device.alloc_outputs(e, w.N, w.T) for e in ESTIMATORS}
    calls = [group_call(e, data[e], outs[e], w) for e in ESTIMATORS]
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    ref = {e: host(outs[e]) for e in ESTIMATORS}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for o in outs.values():
            for t in o.values():
                t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            rlscan.rlscan_group(calls, stream=s)
    for rep in range(4):
        for o in outs.values():
            for t in o.values():
                t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e in ESTIMATORS:
            got = host(outs[e])
            for k in ref[e]:
                np.testing.assert_array_equal(got[k], ref[e][k], err_msg=f"replay {rep} {e}")


def test_group_refusals_write_nothing():
    w, inputs = case("gae", 8, 128, seed=9)
    d = device.upload(inputs)
    out = device.alloc_outputs("gae", 8, 128)
    out["advantages"].fill_(5.0)
    ok = group_call("gae", d, out, w)
    # rows of 3000 steps do not fit a tile of at most 1024 elements
    wl, il = case("gae", 2, 3000, seed=10)
    dl = device.upload(il)
    ol = device.alloc_outputs("gae", 2, 3000)
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_group([ok, group_call("gae", dl, ol, wl)])
    assert e.value.status == rlscan.RLSCAN_ERR_PARAM
    # a misaligned input takes the scalar path, which a group does not run
    buf = torch.empty(8 * 128 + 1, device="cuda")
    shifted = buf[1:].view(8, 128)
    shifted.copy_(d["values"])
    dm = dict(d, values=shifted)
    om = device.alloc_outputs("gae", 8, 128)
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_group([ok, group_call("gae", dm, om, w)])
    assert e.value.status == rlscan.RLSCAN_ERR_PARAM
    # Retrace with 5 actions
    wr, ir = case("retrace", 8, 128, seed=11, A=5)
    dr = device.upload(ir)
    orr = device.alloc_outputs("retrace", 8, 128)
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_group([ok, group_call("retrace", dr, orr, wr)])
    assert e.value.status == rlscan.RLSCAN_ERR_PARAM
    # a call reading another call's output
    d2 = dict(d, rewards=out["advantages"])
    o2 = device.alloc_outputs("gae", 8, 128)
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_group([ok, group_call("gae", d2, o2, w)])
    assert e.value.status == rlscan.RLSCAN_ERR_ALIAS
    # a parameter out of range in the second call
    with pytest.raises(rlscan.RlscanError) as e:
        rlscan.rlscan_group([ok, group_call("gae", d, o2, w, gamma=1.5)])
    assert e.value.status == rlscan.RLSCAN_ERR_PARAM
    torch.cuda.synchronize()
    assert bool((out["advantages"] == 5.0).all())


@pytest.mark.parametrize("seed", range(48))
def test_random_groups(seed):
    """Seeded random groups: 1-11 calls of random estimators and shapes whose
    rows fit the group's tile (T a power of two up to 1024, or a single tile),
    float or one-byte flags per call, either grid layout; every output is
    checked against the oracle."""
    rng = np.random.default_rng(70_000 + seed)
    count = int(rng.integers(1, 12))
    calls, outs, want = [], [], []
    for i in range(count):
        e = ESTIMATORS[rng.integers(len(ESTIMATORS))]
        if rng.random() < 0.2:
            N, T = int(rng.integers(1, 4)), int(rng.integers(1, 300))  # one tile
            if N * T > 512:
                N = 1
        else:
            T = int(2 ** rng.integers(0, 11))
            N = int(rng.integers(1, max(2, 40_000 // T)))
        kw = {"A": int(rng.choice([4, 6, 8]))} if e == "retrace" else {}
        w, inputs = case(e, N, T, seed=seed * 100 + i, **kw)
        d = device.upload(inputs)
        if rng.random() < 0.5:
            for k in FLAG_KEYS:
                if d.get(k) is not None:
                    d[k] = (d[k] != 0).to(torch.uint8)
        out = device.alloc_outputs(e, N, T)
        calls.append(group_call(e, d, out, w))
        outs.append((e, N, T, out))
        want.append(oracle_outputs(e, inputs, w))
    layout = list(LAYOUTS)[rng.integers(len(LAYOUTS))]
    rlscan.rlscan_set_launch_override(flags=LAYOUTS[layout])
    print(f"[group] random seed={seed}: {count} calls, {layout}: "
          f"{[(e, N, T) for e, N, T, _ in outs]}", flush=True)
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    for (e, N, T, out), ref in zip(outs, want):
        assert_parity(host(out), ref, f"random group seed={seed} {e} {N}x{T}")
