"""GPU parity: every estimator through the C ABI against the float64 oracle,
element by element, on the same seeded float32 inputs.

Bar: |gpu - ref| <= 1e-4 * (1 + |ref|) for float32 outputs; identical values
for the int64 prefix sum.  Shapes span several tiles with ragged tails, both
launch mappings (whole rows per tile, and rows spread over tiles through the
decoupled look-back), every round count, looping (grid-capped) launches,
misaligned pointers, the degenerate flag patterns, empty inputs and the full
benchmark workloads.
"""
from __future__ import annotations

import numpy as np
import pytest

from reference import assert_parity, oracle_outputs

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from linear_recurrence_scan_coefficient_amd import device, rlscan, workloads  # noqa: E402
from linear_recurrence_scan_coefficient_amd.workloads import ESTIMATORS  # noqa: E402

REVERSE_WITH_TRUNC = ("gae", "lambda_returns", "discounted_returns", "vtrace")


@pytest.fixture(autouse=True)
def _reset_override():
    rlscan.rlscan_set_launch_override()
    rlscan.rlscan_set_xcd_run(-1)
    yield
    rlscan.rlscan_set_launch_override()
    rlscan.rlscan_set_xcd_run(-1)


@pytest.fixture(scope="module", autouse=True)
def _no_lookback_timeouts():
    yield
    assert rlscan.rlscan_lookback_timeouts() == 0


def case(estimator, N, T, seed=0, **kw):
    """A workload with many episode boundaries, truncation included where the
    estimator takes it."""
    opts = dict(term_p=0.05, done_p=0.05, gamma=0.97, lam=0.9)
    if estimator in REVERSE_WITH_TRUNC or estimator == "retrace":
        opts.update(trunc_mode="independent", trunc_p=0.05)
    opts.update(kw)
    w = workloads.custom(N, T, **opts)
    return w, workloads.inputs_for(estimator, w, seed)


def check(estimator, w, inputs, label=""):
    print(f"[parity] {estimator} N={w.N} T={w.T} {label}", flush=True)
    got = device.run(estimator, inputs, w)
    assert_parity(got, oracle_outputs(estimator, inputs, w), f"{estimator} {w.N}x{w.T} {label}")


SHAPES = [(1, 1), (1, 2), (3, 3), (2, 5), (7, 63), (5, 64), (3, 65), (4, 127), (2, 255),
          (2, 256), (3, 257), (2, 1023), (1, 1024), (2, 1025), (1, 4097), (3, 5000), (37, 129),
          (64, 512), (9, 1536), (2, 20000)]


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{n}x{t}" for n, t in SHAPES])
def test_small_shapes(estimator, shape):
    w, inputs = case(estimator, *shape, seed=shape[0] * 7919 + shape[1])
    check(estimator, w, inputs)


MAPPINGS = {
    "lookback": (rlscan.MAP_LOOKBACK, 0),
    "lookback_tickets": (rlscan.MAP_LOOKBACK, rlscan.FLAG_TICKETS),
    "packed": (rlscan.MAP_PACKED, 0),
}


# (rounds, waves) pairs that have kernels: 1 and 2 waves with one round
SHAPES_RW = [(1, 1), (1, 2), (1, 4), (1, 8), (2, 4), (2, 8), (4, 4), (4, 8)]


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("mapping", list(MAPPINGS))
@pytest.mark.parametrize("rounds,waves", SHAPES_RW, ids=[f"R{r}W{w}" for r, w in SHAPES_RW])
def test_mappings_and_rounds(estimator, mapping, rounds, waves):
    m, flags = MAPPINGS[mapping]
    rlscan.rlscan_set_launch_override(m, rounds, waves, 0, flags)
    for N, T in ((512, 128), (40, 4096), (3, 3001)):
        w, inputs = case(estimator, N, T, seed=N + T + rounds)
        plan = rlscan.rlscan_plan(estimator, N, T, w.A)
        check(estimator, w, inputs, f"{mapping} R={rounds} W={waves} plan={plan}")


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("mapping", list(MAPPINGS))
@pytest.mark.parametrize("waves", [1, 4, 8])
def test_grid_capped_loops(estimator, mapping, waves):
    m, flags = MAPPINGS[mapping]
    rlscan.rlscan_set_launch_override(m, 0, waves, 13, flags)
    for N, T in ((256, 128), (5, 9000)):
        w, inputs = case(estimator, N, T, seed=N * T)
        check(estimator, w, inputs, f"{mapping} W={waves} grid_cap=13")


def test_ticket_bases_across_mixed_lookback_launches():
    """Grid-capped (ticketed), ticket-ordered and one-tile-per-workgroup
    look-back calls in turn on one scratch: every ticketed call's tickets
    must start where the last ticketed call's ended."""
    forms = [(0, 0), (5, 0), (0, rlscan.FLAG_TICKETS), (9, rlscan.FLAG_TICKETS), (2, 0),
             (64, 0), (1, 0)]
    for i, (cap, flags) in enumerate(forms * 2):
        N, T = [(3, 5000), (2, 70000), (11, 999)][i % 3]
        est = ["gae", "episodic_prefix_sum", "vtrace"][i % 3]
        rlscan.rlscan_set_launch_override(rlscan.MAP_LOOKBACK, 1, 4, cap, flags)
        w, inputs = case(est, N, T, seed=i)
        check(est, w, inputs, f"mixed look-back launches, call {i} cap={cap} flags={flags}")
    assert rlscan.rlscan_lookback_timeouts() == 0


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_flag_patterns(estimator):
    N, T = 6, 700
    w, inputs = case(estimator, N, T, seed=11)
    flag_keys = [k for k in ("terminated", "truncated", "dones") if inputs.get(k) is not None]
    first = np.zeros((N, T), np.float32)
    first[:, 0] = 1
    last = np.zeros((N, T), np.float32)
    last[:, -1] = 1
    alternating = np.zeros((N, T), np.float32)
    alternating[1::2] = 1
    patterns = {"none": np.zeros((N, T), np.float32), "all": np.ones((N, T), np.float32),
                "first": first, "last": last, "row_alternating": alternating}
    for name, pattern in patterns.items():
        d = dict(inputs)
        for k in flag_keys:
            d[k] = pattern.copy()
        check(estimator, w, d, f"flags={name}")
    if estimator in REVERSE_WITH_TRUNC or estimator == "retrace":
        d = dict(inputs)
        d["terminated"] = np.ones((N, T), np.float32)
        d["truncated"] = np.ones((N, T), np.float32)
        check(estimator, w, d, "both flags everywhere (terminated wins)")


@pytest.mark.parametrize("estimator", REVERSE_WITH_TRUNC)
def test_optional_inputs(estimator):
    w, inputs = case(estimator, 9, 777, seed=5, trunc_mode="none")
    check(estimator, w, inputs, "no truncated tensor")
    d = dict(inputs)
    d["truncated"] = np.zeros((9, 777), np.float32)
    d["bootstrap_values"] = np.full((9, 777), 123.0, np.float32)
    check(estimator, w, d, "all-zero truncated tensor")
    d = dict(inputs)
    d["bootstrap_value"] = None
    check(estimator, w, d, "no per-row bootstrap value")


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_misaligned_pointers(estimator):
    """Inputs and outputs offset by one element: the scalar-load path."""
    N, T = 33, 250
    w, inputs = case(estimator, N, T, seed=3)
    d = device.upload(inputs)
    shifted = {}
    for k, v in d.items():
        if v is None:
            shifted[k] = None
            continue
        buf = torch.empty(v.numel() + 1, dtype=v.dtype, device=v.device)
        view = buf[1:].view(v.shape)
        view.copy_(v)
        shifted[k] = view
    outs = {}
    for name, dt in device.OUTPUTS[estimator]:
        buf = torch.empty(N * T + 1, dtype=dt, device="cuda")
        outs[name] = buf[1:].view(N, T)
    print(f"[parity] misaligned {estimator}", flush=True)
    device.call(estimator, shifted, outs, w)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in outs.items()}
    assert_parity(got, oracle_outputs(estimator, inputs, w), f"misaligned {estimator}")


@pytest.mark.parametrize("A", [1, 3, 4, 5, 6, 8, 18])
def test_retrace_action_counts(A):
    w, inputs = case("retrace", 17, 300, seed=A, A=A)
    check("retrace", w, inputs, f"A={A}")


def test_retrace_out_of_range_actions_do_not_fault():
    w, inputs = case("retrace", 4, 200, seed=9)
    inputs["actions"][:, ::7] = 99
    inputs["actions"][:, 3::7] = -5
    print("[parity] retrace out-of-range actions", flush=True)
    got = device.run("retrace", inputs, w)
    assert got["targets"].shape == (4, 200)


# Degenerate parameters of the method: gamma = 0 or lambda = 0 make every
# step a chain cut (a = 0: no state crosses any step); gamma = lambda = 1
# leaves the recurrence undamped (a = 1: plain episodic sums, the longest
# chains and the largest magnitudes); V-trace with both clips at +inf (plain
# importance weights) or at 1e-3 (traces all but cut).
DEGENERATE = [
    dict(gamma=0.0, lam=0.9), dict(gamma=0.97, lam=0.0), dict(gamma=1.0, lam=1.0),
    dict(gamma=0.97, lam=1.0), dict(gamma=1.0, lam=0.5),
    dict(gamma=0.97, lam=0.9, rho_bar=float("inf"), c_bar=float("inf")),
    dict(gamma=0.97, lam=0.9, rho_bar=1e-3, c_bar=1e-3),
]


@pytest.mark.parametrize("estimator", [e for e in ESTIMATORS if e != "episodic_prefix_sum"])
@pytest.mark.parametrize("params", DEGENERATE,
                         ids=["-".join(f"{k}{v:g}" for k, v in p.items()) for p in DEGENERATE])
@pytest.mark.parametrize("shape", [(64, 128), (2, 5000)], ids=["packed", "lookback"])
def test_degenerate_parameters(estimator, params, shape):
    if "rho_bar" in params and estimator != "vtrace":
        pytest.skip("clip parameters are V-trace's")
    w, inputs = case(estimator, *shape, seed=shape[1] + 17, **params)
    mapping = rlscan.rlscan_plan(estimator, w.N, w.T, w.A)["mapping"]
    assert mapping == (rlscan.MAP_PACKED if shape[1] == 128 else rlscan.MAP_LOOKBACK)
    check(estimator, w, inputs, f"degenerate {params}")


# V-trace whose trace coefficients gamma*c_t can exceed 1 (gamma*lambda*c_bar
# > 1, here c_bar = 2 or +inf): the recurrence expands along an episode.
# With terminated ~ Bernoulli(0.01) (episodes of about 100 steps) the trace
# products reach 10^3 and beyond, and float32 evaluation misses the bar; the
# library runs these calls in its float64 form.  Every mapping and round
# count, one-byte flags, and a long look-back row.
INF = float("inf")
EXPANDING = [dict(c_bar=INF, rho_bar=1.0), dict(c_bar=2.0, rho_bar=1.0),
             dict(c_bar=INF, rho_bar=INF)]
EXPANDING_SHAPES = [((4096, 128), None), ((40, 1000), None), ((3, 5000), None),
                    ((2, 20000), (1, 1)), ((2, 20000), (1, 8)), ((2, 20000), (2, 4)),
                    ((2, 20000), (4, 8)), ((8, 1 << 18), None)]


@pytest.mark.parametrize("params", EXPANDING, ids=["cinf", "c2", "cinf-rhoinf"])
@pytest.mark.parametrize("shape,rw", EXPANDING_SHAPES,
                         ids=[f"{n}x{t}" + (f"-R{rw[0]}W{rw[1]}" if rw else "")
                              for (n, t), rw in EXPANDING_SHAPES])
@pytest.mark.parametrize("byte_flags", [False, True], ids=["f32flags", "u8flags"])
def test_vtrace_expanding_traces(params, shape, rw, byte_flags):
    N, T = shape
    w, inputs = case("vtrace", N, T, seed=T + N, gamma=0.99, term_p=0.01, trunc_p=0.002,
                     **params)
    if rw is not None:
        rlscan.rlscan_set_launch_override(rlscan.MAP_AUTO, *rw)
    print(f"[parity] vtrace expanding {N}x{T} {params} rw={rw} u8={byte_flags}", flush=True)
    d = device.upload(inputs)
    if byte_flags:
        for k in ("terminated", "truncated"):
            d[k] = (d[k] != 0).to(torch.uint8)
    out = device.alloc_outputs("vtrace", N, T)
    device.call("vtrace", d, out, w)
    torch.cuda.synchronize()
    assert_parity({k: v.cpu().numpy() for k, v in out.items()},
                  oracle_outputs("vtrace", inputs, w), f"vtrace expanding {N}x{T} {params}")


def test_vtrace_expanding_traces_options_carry_and_group():
    """The float64 form through rlscan_vtrace_ex (lambda = 0.9: gamma*lambda
    *c_bar still above 1), chained carry calls, and a grouped launch beside
    a float32-form call."""
    import oracle
    w, inputs = case("vtrace", 24, 3000, seed=77, gamma=0.995, term_p=0.01, c_bar=INF,
                     rho_bar=1.5)
    lam, rho_bar_pg = 0.9, 0.8
    d = device.upload(inputs)
    vs = torch.empty((w.N, w.T), device="cuda")
    pg = torch.empty((w.N, w.T), device="cuda")
    rlscan.rlscan_vtrace_ex(d["rewards"], d["values"], d["bootstrap_value"], d["log_rhos"],
                            d["terminated"], d["truncated"], d["bootstrap_values"], vs, pg,
                            w.gamma, lam, w.rho_bar, w.c_bar, rho_bar_pg)
    # the same rollout in three chunks, later chunks first, chained through
    # carry_in / carry_out (vs at the chunk edges)
    cuts = (0, 1100, 2048, w.T)
    cvs = torch.empty((w.N, w.T), device="cuda")
    cpg = torch.empty((w.N, w.T), device="cuda")
    carry = None
    for a, b in reversed(list(zip(cuts[:-1], cuts[1:]))):
        part = {k: (None if v is None else v[:, a:b].contiguous() if v.dim() == 2 else v)
                for k, v in d.items()}
        if b < w.T:  # V at the chunk's end is V_b, the next chunk's first value
            part["bootstrap_value"] = d["values"][:, b].contiguous()
        pvs = torch.empty((w.N, b - a), device="cuda")
        ppg = torch.empty((w.N, b - a), device="cuda")
        co = torch.empty(w.N, device="cuda")
        rlscan.rlscan_vtrace_ex(part["rewards"], part["values"], part["bootstrap_value"],
                                part["log_rhos"], part["terminated"], part["truncated"],
                                part["bootstrap_values"], pvs, ppg, w.gamma, lam, w.rho_bar,
                                w.c_bar, rho_bar_pg, carry_in=carry, carry_out=co)
        cvs[:, a:b] = pvs
        cpg[:, a:b] = ppg
        carry = co
    torch.cuda.synchronize()
    want_vs, want_pg = oracle.vtrace(
        inputs["rewards"], inputs["values"], inputs["log_rhos"], inputs["terminated"],
        gamma=w.gamma, rho_bar=w.rho_bar, c_bar=w.c_bar,
        bootstrap_value=inputs["bootstrap_value"], truncated=inputs["truncated"],
        bootstrap_values=inputs["bootstrap_values"], lam=lam, rho_bar_pg=rho_bar_pg)
    want = {"vs": want_vs, "pg_advantages": want_pg}
    assert_parity({"vs": vs.cpu().numpy(), "pg_advantages": pg.cpu().numpy()}, want,
                  "vtrace_ex expanding")
    # The carry crosses the interface in float32 (vs at the chunk edge), and
    # an expanding recurrence amplifies that rounding like any other: the
    # reference for the chained calls is the oracle chained the same way, its
    # own carry_out rounded to float32 before the chunk below reads it.
    ovs, opg = np.empty((w.N, w.T)), np.empty((w.N, w.T))
    ocarry = None
    for a, b in reversed(list(zip(cuts[:-1], cuts[1:]))):
        part = {k: (None if v is None else v[:, a:b] if v.ndim == 2 else v)
                for k, v in inputs.items()}
        if b < w.T:
            part["bootstrap_value"] = inputs["values"][:, b].copy()
        pv, pp, co = oracle.vtrace(
            part["rewards"], part["values"], part["log_rhos"], part["terminated"],
            gamma=w.gamma, rho_bar=w.rho_bar, c_bar=w.c_bar,
            bootstrap_value=part["bootstrap_value"], truncated=part["truncated"],
            bootstrap_values=part["bootstrap_values"], lam=lam, rho_bar_pg=rho_bar_pg,
            carry_in=ocarry, return_carry=True)
        ovs[:, a:b], opg[:, a:b] = pv, pp
        ocarry = co.astype(np.float32)
    assert_parity({"vs": cvs.cpu().numpy(), "pg_advantages": cpg.cpu().numpy()},
                  {"vs": ovs, "pg_advantages": opg}, "vtrace_ex expanding, chained carry calls")
    # grouped: an expanding call beside a float32-form call
    wg, ig = case("vtrace", 512, 128, seed=78, gamma=0.99, term_p=0.01, c_bar=INF)
    wf, jf = case("vtrace", 256, 128, seed=79, gamma=0.99, term_p=0.01, c_bar=1.0)
    dg, df = device.upload(ig), device.upload(jf)
    og, of = device.alloc_outputs("vtrace", 512, 128), device.alloc_outputs("vtrace", 256, 128)
    calls = [rlscan.GroupCall("vtrace", tuple(x.get(k) for k in device.INPUT_ORDER["vtrace"]),
                              (o["vs"], o["pg_advantages"]), gamma=ww.gamma, lam=1.0,
                              rho_bar=ww.rho_bar, c_bar=ww.c_bar)
             for x, o, ww in ((dg, og, wg), (df, of, wf))]
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    assert_parity({k: v.cpu().numpy() for k, v in og.items()}, oracle_outputs("vtrace", ig, wg),
                  "grouped expanding vtrace")
    assert_parity({k: v.cpu().numpy() for k, v in of.items()}, oracle_outputs("vtrace", jf, wf),
                  "grouped float32-form vtrace")


@pytest.mark.parametrize("reads,writes", [(1, 1), (3, 1), (12, 4), (16, 1), (2, 3)])
def test_stream_mix_kernel(reads, writes):
    """The bandwidth-reference kernel: thread t of workgroup b writes the sum
    of its read words (b*256*reads + u*256 + t) to its write words.  Small
    integer values, so every float32 sum is exact in any order; a ragged
    tail on both sides."""
    g = 37  # workgroups
    nr, nw = g * 256 * reads - 5, g * 256 * writes - 3  # 16-byte words
    src = torch.randint(-8, 9, (g * 256 * reads, 4), device="cuda").float()
    src[nr:] = 0  # past read_bytes: read as zero by the kernel
    dst = torch.full((g * 256 * writes, 4), -1.0, device="cuda")
    rlscan.rlscan_stream_mix(dst, src, write_bytes=nw * 16, read_bytes=nr * 16, reads=reads,
                             writes=writes)
    torch.cuda.synchronize()
    acc = src.view(g, reads, 256, 4).sum(1)  # [g, 256, 4]
    want = acc[:, None].expand(g, writes, 256, 4).reshape(-1, 4).clone()
    want[nw:] = -1.0
    assert torch.equal(dst, want)


@pytest.mark.parametrize("ain,aout,words,cap", [(1, 1, 1, 0), (5, 1, 2, 0), (3, 2, 4, 2),
                                                 (16, 1, 1, 3), (2, 4, 3, 8)])
def test_stream_mix_arrays_kernel(ain, aout, words, cap):
    """The reference kernel in a scan's pattern: word i of every output array
    is the sum of word i of every input array.  Small integers (exact float32
    sums); arrays whose length is not a multiple of a workgroup's span."""
    n_in, n_out = 37 * 256 * words - 5, 37 * 256 * words - 3  # 16-byte words per array
    src = torch.randint(-8, 9, (ain, n_in, 4), device="cuda").float()
    dst = torch.full((aout, n_out, 4), -1.0, device="cuda")
    rlscan.rlscan_stream_mix_arrays(dst, src, arrays_in=ain, arrays_out=aout, words=words,
                                    workgroups_per_cu=cap)
    torch.cuda.synchronize()
    acc = torch.zeros(max(n_in, n_out), 4, device="cuda")
    acc[:n_in] = src.sum(0)
    assert torch.equal(dst, acc[None, :n_out].expand(aout, n_out, 4))


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_empty_inputs(estimator):
    for N, T in ((0, 5), (5, 0), (0, 0)):
        w, inputs = case(estimator, max(N, 1), max(T, 1), seed=1)
        d = device.upload({k: (None if v is None else v[:N, :T] if v.ndim >= 2 else v[:N])
                           for k, v in inputs.items()})
        outs = device.alloc_outputs(estimator, N, T)
        w0 = workloads.custom(N, T, gamma=w.gamma, lam=w.lam)
        device.call(estimator, d, outs, w0)
    torch.cuda.synchronize()


def test_many_lookback_calls_and_scratch_growth():
    """Consecutive look-back calls with varying tile counts (epochs, ticket
    bases and scratch growth), on the default and on a side stream."""
    rlscan.rlscan_set_launch_override(rlscan.MAP_LOOKBACK, 1)
    side = torch.cuda.Stream()
    for i, (N, T) in enumerate([(2, 3000), (50, 999), (1, 70000), (3, 5), (9, 2**17),
                                (2, 3000)] * 3):
        w, inputs = case("gae", N, T, seed=i)
        d = device.upload(inputs)
        out = device.alloc_outputs("gae", N, T)
        stream = side if i % 2 else None
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                device.call("gae", d, out, w)
            torch.cuda.current_stream().wait_stream(stream)
        else:
            device.call("gae", d, out, w)
        torch.cuda.synchronize()
        print(f"[parity] look-back call {i} {N}x{T}", flush=True)
        assert_parity({k: v.cpu().numpy() for k, v in out.items()},
                      oracle_outputs("gae", inputs, w), f"call {i}")
    assert rlscan.rlscan_lookback_timeouts() == 0


def test_prefix_sum_large_magnitudes():
    N, T = 3, 50000
    w = workloads.custom(N, T, done_p=1e-4)
    inputs = workloads.prefix_inputs(w, 0)
    inputs["x"] = np.random.default_rng(0).integers(2**31 - 100, 2**31 - 1, (N, T)).astype(np.int32)
    check("episodic_prefix_sum", w, inputs, "values near int32 max")


@pytest.mark.parametrize("rounds,waves", [(0, 0), (1, 4), (4, 8)])
def test_prefix_sum_mixed_magnitudes(rounds, waves):
    """Blocks of small values between blocks of +-2^30: tile aggregates and
    running sums that fit 32 bits and others that need 64, side by side in
    one look-back window."""
    N, T = 3, (1 << 20) + 123
    w = workloads.custom(N, T, done_p=2e-4)
    inputs = workloads.prefix_inputs(w, 5)
    g = np.random.default_rng(5)
    flat = inputs["x"].reshape(-1)
    kinds = g.integers(0, 3, flat.size // 4096 + 1)
    for k, sign in ((1, 1), (2, -1)):
        idx = np.flatnonzero(np.repeat(kinds == k, 4096)[:flat.size])
        flat[idx] = sign * ((1 << 30) + g.integers(0, 9, idx.size))
    rlscan.rlscan_set_launch_override(rlscan.MAP_LOOKBACK, rounds, waves)
    check("episodic_prefix_sum", w, inputs, f"mixed magnitudes R{rounds}W{waves}")


# ------------------------------------------------------------ full workloads
FULL = [(name, est) for name, wl in workloads.WORKLOADS.items() for est in wl.estimators]


@pytest.mark.parametrize("name,estimator", FULL, ids=[f"{n}-{e}" for n, e in FULL])
def test_benchmark_workloads(name, estimator):
    w = workloads.get(name)
    inputs = workloads.inputs_for(estimator, w, 0)
    check(estimator, w, inputs, name)


def test_graph_capture_of_packed_calls():
    """All seven estimators captured into one HIP graph (packed shapes) and
    replayed several times, with eager work and synchronisations between the
    replays; every replay must reproduce the eager outputs bit for bit."""
    w = workloads.get("production_4096x128")
    host = {e: workloads.inputs_for(e, w, 1) for e in ESTIMATORS}
    dev = {e: device.upload(host[e]) for e in ESTIMATORS}
    eager = {}
    for e in ESTIMATORS:
        out = device.alloc_outputs(e, w.N, w.T)
        device.call(e, dev[e], out, w)
        eager[e] = out
    torch.cuda.synchronize()
    eager = {e: {k: v.clone() for k, v in o.items()} for e, o in eager.items()}
    outs = {e: device.alloc_outputs(e, w.N, w.T) for e in ESTIMATORS}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for e in ESTIMATORS:
            device.call(e, dev[e], outs[e], w)
    for rep in range(3):
        for o in outs.values():
            for v in o.values():
                v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[parity] graph replay {rep}", flush=True)
        for e in ESTIMATORS:
            for k in eager[e]:
                assert torch.equal(outs[e][k], eager[e][k]), (rep, e, k)
        # eager work between replays
        device.call("gae", dev["gae"], eager["gae"], w)
        torch.cuda.synchronize()


# Rollout lengths that divide no tile size: tiles of whole rows whose span
# falls short of the tile (the remaining lanes idle), a multiple of 4
# elements; ragged last tiles (fewer rows); odd T.
PARTIAL = [(4096, 100), (4096, 200), (1024, 96), (2048, 1000), (4096, 20), (1000, 7),
           (333, 25), (77, 37), (130, 124), (9, 300)]


@pytest.mark.parametrize("estimator", ESTIMATORS)
@pytest.mark.parametrize("shape", PARTIAL, ids=[f"{n}x{t}" for n, t in PARTIAL])
def test_packed_rows_that_do_not_divide_the_tile(estimator, shape):
    N, T = shape
    w, inputs = case(estimator, N, T, seed=N + 3 * T)
    plan = rlscan.rlscan_plan(estimator, N, T, w.A)
    assert plan["mapping"] == rlscan.MAP_PACKED, plan
    assert plan["tile_span"] % 4 == 0 and plan["tile_span"] % T == 0 or plan["tiles"] == 1
    print(f"[parity] {estimator} {N}x{T} packed span {plan['tile_span']} of "
          f"{plan['tile_elems']}", flush=True)
    d = device.upload(inputs)
    outs = [device.alloc_outputs(estimator, N, T) for _ in range(2)]
    for out in outs:
        device.call(estimator, d, out, w)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in outs[0].items()}
    assert_parity(got, oracle_outputs(estimator, inputs, w), f"{estimator} {N}x{T} packed")
    for k, v in outs[1].items():  # no look-back: deterministic
        assert torch.equal(v, outs[0][k]), k


@pytest.mark.parametrize("run", [0, 1, 3, 16, 1 << 20])
@pytest.mark.parametrize("shape", [(4096, 100), (333, 128), (64, 8192)],
                         ids=["4096x100", "333x128", "64x8192"])
def test_xcd_tile_order(run, shape):
    """Packed and grouped launches with workgroups taking tiles in runs per
    XCD (a permutation of the tiles; the last, short group of runs keeps
    tile = workgroup index); look-back launches ignore the order."""
    N, T = shape
    rlscan.rlscan_set_xcd_run(run)
    for est in ("gae", "episodic_prefix_sum", "retrace"):
        w, inputs = case(est, N, T, seed=run % 97 + N)
        check(est, w, inputs, f"xcd run {run}")
    if T <= 128:
        w = workloads.custom(N, T, gamma=0.99, lam=0.95, term_p=0.01, done_p=0.02)
        host = {e: workloads.inputs_for(e, w, 5) for e in ESTIMATORS}
        dev = {e: device.upload(host[e]) for e in ESTIMATORS}
        outs = {e: device.alloc_outputs(e, N, T) for e in ESTIMATORS}
        rlscan.rlscan_group([rlscan.GroupCall(e, tuple(dev[e].get(k) for k in
                                                       device.INPUT_ORDER[e]),
                                              tuple(outs[e].values()), gamma=w.gamma,
                                              lam=1.0 if e == "vtrace" else w.lam)
                             for e in ESTIMATORS])
        torch.cuda.synchronize()
        for e in ESTIMATORS:
            assert_parity({k: v.cpu().numpy() for k, v in outs[e].items()},
                          oracle_outputs(e, host[e], w), f"grouped {e} xcd run {run}")


@pytest.mark.parametrize("estimator", ESTIMATORS)
def test_forced_packed_mapping_with_a_sparse_tile(estimator):
    """A packed mapping forced where the rows fill less than 3/4 of a tile
    (one row of 3000 in 4096), two rounds of eight waves."""
    w, inputs = case(estimator, 6, 3000, seed=5)
    rlscan.rlscan_set_launch_override(rlscan.MAP_PACKED, 2, 8)
    plan = rlscan.rlscan_plan(estimator, 6, 3000, w.A)
    want = rlscan.MAP_PACKED if estimator != "retrace" else plan["mapping"]
    assert plan["mapping"] == want
    check(estimator, w, inputs, f"forced packed {plan}")


def test_graph_capture_and_group_of_rows_that_do_not_divide_the_tile():
    """Calls of 4096 x 100 (packed with partly filled tiles) capture into a
    HIP graph, replaying to the eager results bit for bit, and join one
    grouped launch."""
    w = workloads.custom(4096, 100, gamma=0.99, lam=0.95, term_p=1 / 200, done_p=0.01)
    host = {e: workloads.inputs_for(e, w, 3) for e in ESTIMATORS}
    dev = {e: device.upload(host[e]) for e in ESTIMATORS}
    eager = {}
    for e in ESTIMATORS:
        eager[e] = device.alloc_outputs(e, w.N, w.T)
        device.call(e, dev[e], eager[e], w)
    torch.cuda.synchronize()
    for e in ESTIMATORS:
        assert_parity({k: v.cpu().numpy() for k, v in eager[e].items()},
                      oracle_outputs(e, host[e], w), f"{e} 4096x100")
    outs = {e: device.alloc_outputs(e, w.N, w.T) for e in ESTIMATORS}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for e in ESTIMATORS:
            device.call(e, dev[e], outs[e], w)
    for rep in range(3):
        for o in outs.values():
            for v in o.values():
                v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[parity] 4096x100 graph replay {rep}", flush=True)
        for e in ESTIMATORS:
            for k in eager[e]:
                assert torch.equal(outs[e][k], eager[e][k]), (rep, e, k)
        device.call("gae", dev["gae"], outs["gae"], w)  # eager work between replays
        torch.cuda.synchronize()
    grouped = {e: device.alloc_outputs(e, w.N, w.T) for e in ESTIMATORS}
    calls = [rlscan.GroupCall(e, tuple(dev[e].get(k) for k in device.INPUT_ORDER[e]),
                              tuple(grouped[e].values()), gamma=w.gamma,
                              lam=1.0 if e == "vtrace" else w.lam)
             for e in ESTIMATORS]
    rlscan.rlscan_group(calls)
    torch.cuda.synchronize()
    for e in ESTIMATORS:
        assert_parity({k: v.cpu().numpy() for k, v in grouped[e].items()},
                      oracle_outputs(e, host[e], w), f"grouped {e} 4096x100")


# the refused call enqueues nothing, so the captured graph is empty by design
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_lookback_launch_refuses_capture():
    w, inputs = case("gae", 5, 3001, seed=2)
    d = device.upload(inputs)
    out = device.alloc_outputs("gae", 5, 3001)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(rlscan.RlscanError) as err:
        with torch.cuda.graph(g):
            device.call("gae", d, out, w)
    assert err.value.status == rlscan.RLSCAN_ERR_CAPTURE
    torch.cuda.synchronize()


def test_lookback_calls_on_two_streams_without_host_synchronisation():
    """Look-back calls alternating between two streams with no
    synchronisation between them: the library orders look-back launches
    across streams, so every call is correct and no wait times out."""
    rlscan.rlscan_set_launch_override(rlscan.MAP_LOOKBACK)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    jobs = []
    for i in range(12):
        est = ("gae", "episodic_prefix_sum", "vtrace")[i % 3]
        w, inputs = case(est, 4, 200000 + 1000 * i, seed=300 + i)
        d = device.upload(inputs)
        out = device.alloc_outputs(est, w.N, w.T)
        jobs.append((est, w, inputs, d, out))
    torch.cuda.synchronize()
    for i, (est, w, inputs, d, out) in enumerate(jobs):
        with torch.cuda.stream(streams[i % 2]):
            device.call(est, d, out, w)
    torch.cuda.synchronize()
    for i, (est, w, inputs, d, out) in enumerate(jobs):
        print(f"[parity] two streams, call {i}: {est} {w.N}x{w.T}", flush=True)
        assert_parity({k: v.cpu().numpy() for k, v in out.items()},
                      oracle_outputs(est, inputs, w), f"two streams call {i}")
    assert rlscan.rlscan_lookback_timeouts() == 0


def test_calls_from_several_host_threads():
    """Four host threads, each with its own stream, making look-back and
    packed calls at once (the binding releases the interpreter lock during
    each C call): every result is correct and no look-back wait times out."""
    import threading

    jobs = []
    for t in range(4):
        mine = []
        for i, (est, N, T) in enumerate((("gae", 3, 70000), ("vtrace", 64, 128),
                                        ("episodic_prefix_sum", 2, 90000),
                                        ("discounted_returns", 512, 256))):
            w, inputs = case(est, N, T, seed=400 + 10 * t + i)
            mine.append((est, w, inputs, device.upload(inputs),
                         device.alloc_outputs(est, w.N, w.T)))
        jobs.append(mine)
    torch.cuda.synchronize()
    errors = []

    def work(mine):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(3):
                    for est, w, inputs, d, out in mine:
                        device.call(est, d, out, w)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(m,)) for m in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not any(th.is_alive() for th in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for t, mine in enumerate(jobs):
        for est, w, inputs, d, out in mine:
            print(f"[parity] thread {t}: {est} {w.N}x{w.T}", flush=True)
            assert_parity({k: v.cpu().numpy() for k, v in out.items()},
                          oracle_outputs(est, inputs, w), f"thread {t} {est}")
    assert rlscan.rlscan_lookback_timeouts() == 0


def random_case(seed):
    """A seeded random call: estimator, shape (log-uniform, up to ~2e5
    elements), flag rates, truncation mode, gamma and lambda (including the
    exact ends 0 and 1), V-trace clips, Retrace's action count, and a launch
    override (mapping, rounds, waves, grid cap, ticket order)."""
    rng = np.random.default_rng(90_000 + seed)
    est = ESTIMATORS[rng.integers(len(ESTIMATORS))]
    N = int(np.exp(rng.uniform(0, np.log(400))))
    T = int(np.exp(rng.uniform(0, np.log(20000))))
    while N * T > 200_000:
        T = max(1, T // 2)

    def unit():
        return float(rng.choice([0.0, 1.0, rng.uniform(0.5, 1.0), rng.uniform(0.0, 1.0)],
                                p=[0.1, 0.1, 0.5, 0.3]))
    opts = dict(gamma=unit(), lam=unit(), term_p=float(rng.choice([0.0, 1e-3, 0.02, 0.3])),
                done_p=float(rng.choice([0.0, 1e-3, 0.02, 0.3])),
                A=int(rng.choice([1, 3, 4, 6, 8])))
    if est in REVERSE_WITH_TRUNC or est == "retrace":
        opts["trunc_mode"] = str(rng.choice(["none", "independent", "exclusive"]))
        opts["trunc_p"] = float(rng.choice([1e-3, 0.05]))
        if est == "retrace" and opts["trunc_mode"] == "none":
            opts["trunc_mode"] = "independent"
    if est == "vtrace":
        opts["rho_bar"] = float(rng.choice([1.0, 0.5, 2.0, np.inf]))
        opts["c_bar"] = float(rng.choice([1.0, 0.9, 1e-3, 2.0, np.inf]))
        if opts["c_bar"] > 1.0:
            # expanding traces (the float64 form when gamma*c_bar > 1):
            # episodes of at most about 100 steps on average, so that trace
            # products stay within float32's range
            opts["term_p"] = float(rng.choice([0.01, 0.02, 0.3]))
    rounds, waves = SHAPES_RW[rng.integers(len(SHAPES_RW))]
    mapping = int(rng.choice([rlscan.MAP_AUTO, rlscan.MAP_LOOKBACK]))
    grid_cap = int(rng.choice([0, 0, 0, 7, 64]))
    flags = int(rng.choice([0, 0, rlscan.FLAG_TICKETS]))
    if rng.random() < 0.3:  # the planner's own choice
        mapping, rounds, waves, grid_cap, flags = rlscan.MAP_AUTO, 0, 0, 0, 0
    byte_flags = bool(rng.random() < 0.5)  # uint8 flags: the *_u8 entry points
    return est, N, T, opts, (mapping, rounds, waves, grid_cap, flags), byte_flags


@pytest.mark.parametrize("seed", range(256))
def test_random_cases(seed):
    est, N, T, opts, override, byte_flags = random_case(seed)
    w = workloads.custom(N, T, **opts)
    inputs = workloads.inputs_for(est, w, seed)
    rlscan.rlscan_set_launch_override(*override)
    plan = rlscan.rlscan_plan(est, N, T, w.A)
    label = f"random seed={seed} {opts} override={override} u8={byte_flags} plan={plan}"
    print(f"[parity] {est} N={N} T={T} {label}", flush=True)
    d = device.upload(inputs)
    if byte_flags:
        for k in ("terminated", "truncated", "dones"):
            if d.get(k) is not None:
                d[k] = (d[k] != 0).to(torch.uint8)
    out = device.alloc_outputs(est, N, T)
    device.call(est, d, out, w)
    torch.cuda.synchronize()
    assert_parity({k: v.cpu().numpy() for k, v in out.items()}, oracle_outputs(est, inputs, w),
                  f"{est} {N}x{T} {label}")
