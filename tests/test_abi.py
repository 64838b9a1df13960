"""The C ABI without a GPU: the library loads, exports every symbol that
include/rlscan.h declares, and every argument check returns its status
before any HIP call (the fake pointers below are never dereferenced)."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlscan.h")


@pytest.fixture(scope="module")
def lib():
    from linear_recurrence_scan_coefficient_amd import build, rlscan
    if build.is_stale():
        build.build()
    return rlscan.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlscan_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_seven_estimators():
    names = declared_functions()
    for est in ("gae", "vtrace", "retrace", "lambda_returns", "discounted_returns",
                "eligibility_traces", "episodic_prefix_sum"):
        assert f"rlscan_{est}" in names


def test_every_declared_symbol_is_exported(lib):
    from linear_recurrence_scan_coefficient_amd import rlscan
    names = declared_functions()
    for name in names:
        assert hasattr(lib, name), f"{name} declared in rlscan.h but not exported"
    assert sorted(rlscan.EXPORTED) == names


def test_version_and_status_strings(lib):
    from linear_recurrence_scan_coefficient_amd import rlscan
    assert "gfx950" in rlscan.version()
    for code in range(0, -9, -1):
        s = rlscan.status_string(code)
        assert s and s != "unknown rlscan status"
    assert rlscan.status_string(-99) == "unknown rlscan status"


# fake, distinct, 16-byte aligned "device pointers": only compared, never read
P = [0x10000 * (i + 1) for i in range(12)]
OK, NULL, SHAPE, PARAM, ALIAS = 0, -1, -2, -3, -4


def gae(lib, *, ptrs=None, N=4, T=8, gamma=0.99, lam=0.95):
    p = list(ptrs if ptrs is not None else P[:7])
    return lib.rlscan_gae(*p, N, T, gamma, lam, None)


def test_gae_argument_checks(lib):
    assert gae(lib, N=-1) == SHAPE
    assert gae(lib, T=-3) == SHAPE
    assert gae(lib, N=1 << 30, T=1 << 30) == SHAPE
    for bad in (-0.1, 1.5, math.nan, math.inf):
        assert gae(lib, gamma=bad) == PARAM
        assert gae(lib, lam=bad) == PARAM
    # empty: success without touching any pointer
    assert gae(lib, ptrs=[None] * 7, N=0) == OK
    assert gae(lib, ptrs=[None] * 7, T=0) == OK
    # required pointers
    for i in (0, 1, 3, 6):
        p = list(P[:7])
        p[i] = None
        assert gae(lib, ptrs=p) == NULL, i
    p = list(P[:7])
    p[5] = None  # truncated given without bootstrap_values
    assert gae(lib, ptrs=p) == NULL
    # output aliasing any input
    for i in range(6):
        p = list(P[:7])
        p[6] = p[i]
        assert gae(lib, ptrs=p) == ALIAS, i


def test_other_entry_points_argument_checks(lib):
    f = lib
    # lambda returns: same shape as GAE
    assert f.rlscan_lambda_returns(*P[:7], 4, 8, 2.0, 0.5, None) == PARAM
    assert f.rlscan_lambda_returns(P[0], None, *P[2:7], 4, 8, 0.9, 0.5, None) == NULL
    # discounted: values not needed, bootstrap_value optional
    assert f.rlscan_discounted_returns(P[0], None, P[2], None, None, P[0], 4, 8, 0.9, None) == ALIAS
    assert f.rlscan_discounted_returns(P[0], None, P[2], P[3], None, P[5], 4, 8, 0.9, None) == NULL
    assert f.rlscan_discounted_returns(None, None, None, None, None, None, 0, 8, 0.9, None) == OK
    # vtrace: clip levels > 0, +inf allowed (checked as far as the alias test)
    args = P[:9]
    assert f.rlscan_vtrace(*args, 4, 8, 0.9, 0.0, 1.0, None) == PARAM
    assert f.rlscan_vtrace(*args, 4, 8, 0.9, 1.0, -1.0, None) == PARAM
    assert f.rlscan_vtrace(*args, 4, 8, 0.9, math.nan, 1.0, None) == PARAM
    same_out = list(args)
    same_out[8] = same_out[7]
    assert f.rlscan_vtrace(*same_out, 4, 8, 0.9, math.inf, math.inf, None) == ALIAS
    # retrace: both flags required, A >= 1
    assert f.rlscan_retrace(*P[:8], 4, 8, 0, 0.9, 0.9, None) == SHAPE
    assert f.rlscan_retrace(*P[:6], None, P[7], 4, 8, 6, 0.9, 0.9, None) == NULL
    assert f.rlscan_retrace(*P[:7], P[3], 4, 8, 6, 0.9, 0.9, None) == ALIAS
    assert f.rlscan_retrace(*P[:8], 1 << 20, 1 << 20, 1 << 10, 0.9, 0.9, None) == SHAPE
    # traces / prefix sum
    assert f.rlscan_eligibility_traces(P[0], P[1], P[1], 4, 8, 0.9, 0.9, None) == ALIAS
    assert f.rlscan_eligibility_traces(P[0], P[1], P[2], 4, 8, 0.9, -0.1, None) == PARAM
    assert f.rlscan_episodic_prefix_sum(P[0], None, P[2], 4, 8, None) == NULL
    assert f.rlscan_episodic_prefix_sum(P[0], P[1], P[0], 4, 8, None) == ALIAS
    assert f.rlscan_episodic_prefix_sum(None, None, None, 3, 0, None) == OK


def test_plan_mapping_choice(lib):
    from linear_recurrence_scan_coefficient_amd import rlscan
    rlscan.rlscan_set_launch_override()
    # whole rows per tile: packed, no inter-workgroup traffic; one round
    # takes the smallest tile that holds whole rows (two waves for GAE and
    # V-trace, one for the others)
    p = rlscan.rlscan_plan("gae", 4096, 128)
    assert p["mapping"] == rlscan.MAP_PACKED and p["rounds"] == 1
    assert p["tile_elems"] == 512 and p["tiles"] == 1024 and p["grid"] == 1024
    assert p["threads"] == 128
    p = rlscan.rlscan_plan("episodic_prefix_sum", 4096, 128)
    assert p["threads"] == 64 and p["tile_elems"] == 256 and p["tiles"] == 2048
    assert rlscan.rlscan_plan("retrace", 4096, 128, 6)["threads"] == 64
    assert rlscan.rlscan_plan("gae", 16384, 32)["mapping"] == rlscan.MAP_PACKED
    p = rlscan.rlscan_plan("gae", 64, 512)
    assert p["tiles"] == 64 and p["threads"] == 128
    assert rlscan.rlscan_plan("eligibility_traces", 64, 512)["threads"] == 128
    # the smallest tile of up to eight waves that holds whole rows
    assert rlscan.rlscan_plan("gae", 1024, 1024)["threads"] == 256
    p = rlscan.rlscan_plan("discounted_returns", 256, 2048)
    assert p["threads"] == 512 and p["mapping"] == rlscan.MAP_PACKED
    assert p["tile_span"] == p["tile_elems"]
    # rows that divide no tile: the smallest tile whose whole rows fill at
    # least 7/8 of it (3/4 for Retrace and the prefix sum; a span that is a
    # multiple of 4), else the best-filled one if at least 3/4 full; the
    # remaining lanes idle
    for est, N, T, threads, span, tiles in (
            ("gae", 4096, 100, 128, 500, 820), ("episodic_prefix_sum", 4096, 100, 64, 200, 2048),
            ("discounted_returns", 4096, 100, 128, 500, 820),
            ("retrace", 4096, 96, 64, 192, 2048), ("retrace", 4096, 200, 64, 200, 4096),
            ("gae", 4096, 200, 256, 1000, 820), ("discounted_returns", 1024, 96, 128, 480, 205),
            ("retrace", 4096, 20, 64, 240, 342), ("gae", 5, 1000, 256, 1000, 5),
            ("eligibility_traces", 11, 7, 64, 256, 1)):
        p = rlscan.rlscan_plan(est, N, T, 6)
        assert p["mapping"] == rlscan.MAP_PACKED, (est, N, T)
        assert (p["threads"], p["tile_span"], p["tiles"]) == (threads, span, tiles), (est, N, T, p)
    p = rlscan.rlscan_plan("gae", 1000, 7)  # 73 rows of 7 would be 511 elements: 72 rows
    assert p["mapping"] == rlscan.MAP_PACKED and p["tile_span"] == 504 and p["tiles"] == 14
    p = rlscan.rlscan_plan("gae", 2048, 1000)  # two rounds of eight waves: 4 rows of 4096
    assert p["rounds"] == 2 and p["tile_span"] == 4000 and p["tiles"] == 512
    # rows longer than a tile, or filling less than 3/4 of one: look-back,
    # with eight waves (one round)
    p = rlscan.rlscan_plan("gae", 64, 8192)
    assert p["mapping"] == rlscan.MAP_LOOKBACK and p["threads"] == 512 and p["rounds"] == 1
    assert p["tile_span"] == p["tile_elems"]
    p = rlscan.rlscan_plan("gae", 1024, 3000)  # one row of 3000 in a tile of 4096
    assert p["mapping"] == rlscan.MAP_LOOKBACK and p["tiles"] == (1024 * 3000 + 4095) // 4096
    # long rows: four rounds of four waves
    for est, waves in (("discounted_returns", 4), ("episodic_prefix_sum", 4),
                       ("eligibility_traces", 4), ("gae", 4), ("vtrace", 4),
                       ("lambda_returns", 4)):
        big = rlscan.rlscan_plan(est, 8, 1 << 20)
        assert big["mapping"] == rlscan.MAP_LOOKBACK and big["rounds"] == 4, est
        assert big["threads"] == 64 * waves, est
        assert big["tile_elems"] == 256 * waves * 4, est
        assert big["tiles"] == (8 << 20) // big["tile_elems"], est
    # two rounds below 2^22 elements, with eight waves; four from 2^22
    p = rlscan.rlscan_plan("gae", 8, 1 << 18)
    assert p["rounds"] == 2 and p["threads"] == 512
    assert rlscan.rlscan_plan("gae", 8, 1 << 19)["rounds"] == 4
    # a single tile never needs a carry
    assert rlscan.rlscan_plan("gae", 3, 100)["mapping"] == rlscan.MAP_PACKED
    # Retrace runs one round of four waves
    p = rlscan.rlscan_plan("retrace", 8, 1 << 20, 6)
    assert p["rounds"] == 1 and p["threads"] == 256
    # overrides
    rlscan.rlscan_set_launch_override(rlscan.MAP_LOOKBACK, 2, grid_cap=7)
    p = rlscan.rlscan_plan("gae", 4096, 128)
    assert p["mapping"] == rlscan.MAP_LOOKBACK and p["rounds"] == 2 and p["grid"] == 7
    # a forced packed mapping is honoured wherever a tile holds a whole row
    rlscan.rlscan_set_launch_override(rlscan.MAP_PACKED, 2, 8)
    p = rlscan.rlscan_plan("gae", 1024, 3000)
    assert p["mapping"] == rlscan.MAP_PACKED and p["tile_span"] == 3000 and p["tiles"] == 1024
    assert rlscan.rlscan_plan("gae", 4, 5000)["mapping"] == rlscan.MAP_LOOKBACK
    rlscan.rlscan_set_launch_override(waves=8)
    p = rlscan.rlscan_plan("gae", 4096, 128)
    assert p["threads"] == 512 and p["tile_elems"] == 2048 and p["tiles"] == 256
    assert p["mapping"] == rlscan.MAP_PACKED
    assert rlscan.rlscan_plan("retrace", 4096, 128, 6)["threads"] == 256
    # one or two waves exist with one round only
    rlscan.rlscan_set_launch_override(rounds=2, waves=1)
    assert rlscan.rlscan_plan("gae", 4096, 128)["threads"] == 256
    rlscan.rlscan_set_launch_override(rounds=1, waves=1)
    p = rlscan.rlscan_plan("vtrace", 4096, 128)
    assert p["threads"] == 64 and p["tiles"] == 2048
    rlscan.rlscan_set_launch_override()
    with pytest.raises(rlscan.RlscanError):
        rlscan.rlscan_set_launch_override(rounds=3)
    with pytest.raises(rlscan.RlscanError):
        rlscan.rlscan_set_launch_override(waves=6)
    with pytest.raises(rlscan.RlscanError):
        rlscan.rlscan_set_launch_override(flags=8)
    with pytest.raises(rlscan.RlscanError):
        rlscan.rlscan_plan("gae", -1, 5)
    assert rlscan.rlscan_plan("gae", 0, 5)["tiles"] == 0


def test_stream_copy_argument_checks(lib):
    f = lib.rlscan_stream_copy
    assert f(P[1], P[0], 0, None) == OK            # nothing to copy
    assert f(P[1], P[0], 15, None) == SHAPE        # not a multiple of 16
    assert f(P[1], P[0], -16, None) == SHAPE
    assert f(None, P[0], 64, None) == NULL
    assert f(P[1] + 4, P[0], 64, None) == PARAM    # misaligned
    assert f(P[0] + 32, P[0], 64, None) == ALIAS   # overlapping ranges
    assert f(P[0], P[0] + 32, 64, None) == ALIAS


def test_xcd_run_override_checks(lib):
    f = lib.rlscan_set_xcd_run
    assert f(-2) == PARAM and f((1 << 20) + 1) == PARAM
    assert f(0) == OK and f(16) == OK and f(1 << 20) == OK and f(-1) == OK


def test_stream_mix_argument_checks(lib):
    f = lib.rlscan_stream_mix
    assert f(P[1], 0, P[0], 0, 1, 1, None) == OK          # nothing to move
    assert f(P[1], 16, P[0], 15, 1, 1, None) == SHAPE     # not a multiple of 16
    assert f(P[1], -16, P[0], 16, 1, 1, None) == SHAPE
    assert f(P[1], 64, P[0], 64, 0, 1, None) == PARAM     # word counts out of range
    assert f(P[1], 64, P[0], 64, 17, 1, None) == PARAM
    assert f(P[1], 64, P[0], 64, 1, 5, None) == PARAM
    assert f(None, 64, P[0], 64, 1, 1, None) == NULL
    assert f(P[1], 64, None, 64, 1, 1, None) == NULL
    assert f(P[1] + 4, 64, P[0], 64, 1, 1, None) == PARAM  # misaligned
    assert f(P[0] + 32, 64, P[0], 64, 1, 1, None) == ALIAS  # overlapping ranges
    assert f(P[1], 1 << 44, P[0], 16, 1, 1, None) == SHAPE  # grid beyond 2^23 workgroups


def test_stream_mix_arrays_argument_checks(lib):
    f = lib.rlscan_stream_mix_arrays
    assert f(P[1], 0, P[0], 0, 1, 1, 1, 0, None) == OK           # nothing to move
    assert f(P[1], 64, P[0], 48, 2, 1, 1, 0, None) == SHAPE      # 3 words do not split in 2 arrays
    assert f(P[1], 48, P[0], 64, 1, 2, 1, 0, None) == SHAPE
    assert f(P[1], -16, P[0], 16, 1, 1, 1, 0, None) == SHAPE
    assert f(P[1], 64, P[0], 64, 0, 1, 1, 0, None) == PARAM      # counts out of range
    assert f(P[1], 64, P[0], 64 * 17, 17, 1, 1, 0, None) == PARAM
    assert f(P[1], 64, P[0], 64, 1, 5, 1, 0, None) == PARAM
    assert f(P[1], 64, P[0], 64, 1, 1, 5, 0, None) == PARAM
    assert f(P[1], 64, P[0], 64 * 5, 5, 1, 4, 0, None) == PARAM  # 5 arrays x 4 words > 16
    assert f(None, 64, P[0], 64, 1, 1, 1, 0, None) == NULL
    assert f(P[1], 64, None, 64, 1, 1, 1, 0, None) == NULL
    assert f(P[1] + 4, 64, P[0], 64, 1, 1, 1, 0, None) == PARAM  # misaligned
    assert f(P[0] + 32, 64, P[0], 64, 1, 1, 1, 0, None) == ALIAS  # overlapping ranges
    for cap in (-1, 1, 9):                                       # residency cap out of range
        assert f(P[1], 64, P[0], 64, 1, 1, 1, cap, None) == PARAM


def test_launch_floor_argument_checks(lib):
    """Refused on the host before any launch: a grid outside [1, 2^23) or a
    workgroup size that is not a multiple of 64 from 64 to 1024."""
    f = lib.rlscan_launch_floor
    assert f(0, 256, None) == SHAPE
    assert f(1 << 23, 256, None) == SHAPE
    for threads in (0, 32, 100, 1088, -64):
        assert f(16, threads, None) == SHAPE, threads


def test_carry_entry_points_argument_checks(lib):
    f = lib
    # GAE with carry: carry_out may not alias an input or the output
    args = list(P[:9])  # 6 inputs, carry_in, advantages, carry_out
    bad = list(args)
    bad[8] = bad[7]
    assert f.rlscan_gae_carry(*bad, 4, 8, 0.9, 0.9, None) == ALIAS
    bad = list(args)
    bad[8] = bad[6]
    assert f.rlscan_gae_carry(*bad, 4, 8, 0.9, 0.9, None) == ALIAS
    # carry_out alone is allowed to be the only optional pointer given
    assert f.rlscan_gae_carry(*P[:6], None, P[7], P[7], 4, 8, 0.9, 0.9, None) == ALIAS
    # Retrace: a carry_in needs next_actions and next_behaviour_probs
    r = list(P[:7]) + [P[7], None, P[9], P[10], P[11]]
    assert f.rlscan_retrace_carry(*r, 4, 8, 6, 0.9, 0.9, None) == NULL
    r = list(P[:7]) + [P[7], P[8], None, P[10], P[11]]
    assert f.rlscan_retrace_carry(*r, 4, 8, 6, 0.9, 0.9, None) == NULL
    r = list(P[:7]) + [P[7], P[8], P[9], P[10], P[10]]
    assert f.rlscan_retrace_carry(*r, 4, 8, 6, 0.9, 0.9, None) == ALIAS
    # forward estimators
    assert f.rlscan_eligibility_traces_carry(P[0], P[1], P[2], P[3], P[2], 4, 8, 0.9, 0.9,
                                             None) == ALIAS
    assert f.rlscan_episodic_prefix_sum_carry(P[0], P[1], P[2], P[3], P[0], 4, 8, None) == ALIAS
    assert f.rlscan_episodic_prefix_sum_carry(None, None, None, None, None, 0, 8, None) == OK
    # the same parameter checks as the plain calls
    assert f.rlscan_discounted_returns_carry(*P[:8], 4, 8, 1.5, None) == PARAM
    assert f.rlscan_vtrace_carry(*P[:11], 4, 8, 0.9, 0.0, 1.0, None) == PARAM
    assert f.rlscan_lambda_returns_carry(*P[:9], -1, 8, 0.9, 0.9, None) == SHAPE


def test_noalloc_argument_checks(lib):
    """rlscan_gae_noalloc checks its arguments as rlscan_gae_carry does, and
    refuses a look-back plan beyond its fixed array before any HIP call."""
    f = lib.rlscan_gae_noalloc
    SCRATCH = -8
    bad = list(P[:9])
    bad[8] = bad[7]
    assert f(*bad, 4, 8, 0.9, 0.9, None) == ALIAS
    assert f(*P[:9], 4, 8, 1.5, 0.9, None) == PARAM
    assert f(*P[:9], -1, 8, 0.9, 0.9, None) == SHAPE
    assert f(*[None] * 9, 0, 8, 0.9, 0.9, None) == OK
    p = list(P[:9])
    p[0] = None
    assert f(*p, 4, 8, 0.9, 0.9, None) == NULL
    # 2 rows of 2^28 + 4096 steps: 4096-element tiles, 131074 > 65536 of them
    plan = lib.rlscan_plan
    from linear_recurrence_scan_coefficient_amd import rlscan
    info = rlscan.PlanInfo()
    N, T = 2, (1 << 28) + 4096
    assert plan(0, N, T, 1, ctypes.byref(info)) == OK
    assert info.mapping == 2 and info.tiles > 65536
    assert f(*P[:9], N, T, 0.9, 0.9, None) == SCRATCH
    assert rlscan.status_string(SCRATCH) != "unknown rlscan status"


def test_variant_entry_points_argument_checks(lib):
    """V-trace options, the float prefix sum and the one-byte-flag calls:
    their own parameter checks, and the shared ones (nothing is launched:
    every case below returns before any HIP call)."""
    f = lib
    vt = list(P[:11])  # 7 inputs, carry_in, vs, pg, carry_out
    for lam, pg in ((1.5, 1.0), (-0.5, 1.0), (math.nan, 1.0), (0.9, 0.0), (0.9, -2.0),
                    (0.9, math.nan)):
        assert f.rlscan_vtrace_ex(*vt, 4, 8, 0.9, lam, 1.0, 1.0, pg, None) == PARAM
        assert f.rlscan_vtrace_u8(*vt, 4, 8, 0.9, lam, 1.0, 1.0, pg, None) == PARAM
    bad = list(vt)
    bad[9] = bad[8]
    assert f.rlscan_vtrace_ex(*bad, 4, 8, 0.9, 0.9, 1.0, 1.0, math.inf, None) == ALIAS
    assert f.rlscan_vtrace_ex(*[None] * 11, 0, 8, 0.9, 0.9, 1.0, 1.0, 1.0, None) == OK
    # float prefix sum: x, dones, carry_in, out, carry_out
    assert f.rlscan_episodic_prefix_sum_f32(P[0], None, None, P[3], None, 4, 8, None) == NULL
    assert f.rlscan_episodic_prefix_sum_f32(P[0], P[1], None, P[0], None, 4, 8, None) == ALIAS
    assert f.rlscan_episodic_prefix_sum_f32(P[0], P[1], None, P[3], None, -1, 8, None) == SHAPE
    assert f.rlscan_episodic_prefix_sum_f32(None, None, None, None, None, 4, 0, None) == OK
    # one-byte flags: the checks of the *_carry calls
    assert f.rlscan_gae_u8(*P[:9], 4, 8, 1.5, 0.9, None) == PARAM
    assert f.rlscan_gae_u8(P[0], P[1], P[2], None, *P[4:9], 4, 8, 0.9, 0.9, None) == NULL
    assert f.rlscan_lambda_returns_u8(*P[:6], None, P[7], P[7], 4, 8, 0.9, 0.9, None) == ALIAS
    assert f.rlscan_discounted_returns_u8(P[0], None, P[2], P[3], None, None, P[6], None, 4, 8,
                                          0.9, None) == NULL
    r = list(P[:7]) + [P[7], None, P[9], P[10], P[11]]
    assert f.rlscan_retrace_u8(*r, 4, 8, 6, 0.9, 0.9, None) == NULL
    r = list(P[:5]) + [P[5], None] + [None, None, None, P[10], None]
    assert f.rlscan_retrace_u8(*r, 4, 8, 6, 0.9, 0.9, None) == NULL
    assert f.rlscan_eligibility_traces_u8(P[0], P[1], None, P[1], None, 4, 8, 0.9, 0.9,
                                          None) == ALIAS
    assert f.rlscan_episodic_prefix_sum_u8(P[0], None, None, P[3], None, 4, 8, None) == NULL
    assert f.rlscan_episodic_prefix_sum_u8(None, None, None, None, None, 0, 0, None) == OK


def test_group_argument_checks(lib):
    """rlscan_group refusals that return before anything is launched."""
    from linear_recurrence_scan_coefficient_amd.rlscan import Call
    assert lib.rlscan_group(None, 0, None) == OK
    assert lib.rlscan_group(None, -1, None) == SHAPE
    assert lib.rlscan_group(None, 2, None) == NULL

    def call(est, N=4, T=8, ins=P[:6], outs=P[6:7], gamma=0.9):
        c = Call()
        c.estimator, c.N, c.T, c.A = est, N, T, 6
        c.gamma, c.lam, c.rho_bar, c.c_bar, c.rho_bar_pg = gamma, 0.9, 1.0, 1.0, 1.0
        for i, p in enumerate(ins):
            c.inp[i] = p
        for i, p in enumerate(outs):
            c.out[i] = p
        return c

    def group(*calls):
        arr = (Call * len(calls))(*calls)
        return lib.rlscan_group(arr, len(calls), None)

    # one call writes what another reads
    assert group(call(0), call(0, ins=[P[6]] + P[1:6], outs=[P[7]])) == ALIAS
    # rows of 3000 steps fit no grouped tile
    assert group(call(0, N=2, T=3000)) == PARAM
    # unknown estimator
    assert group(call(9)) == PARAM
    # a call's own checks: gamma out of range
    assert group(call(0, gamma=1.5)) == PARAM
    # misaligned pointer: refused while collecting, before any launch
    assert group(call(0, ins=[P[0] + 4] + P[1:6])) == PARAM
    # empty calls are no-ops: a group of them launches nothing
    assert group(call(0, N=0), call(5, T=0, ins=P[8:10], outs=P[10:11])) == OK
