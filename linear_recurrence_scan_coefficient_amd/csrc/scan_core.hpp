// scan_core.hpp -- the (a, b) step type, its composition, and the wave64
// inclusive scan used by every estimator kernel (gfx950, wave64).
//
// A step maps the recurrence state x to a*x + b.  Composition of a step E
// (applied first) with a step L (applied after it) is
//     L o E = (aL*aE, aL*bE + bL),
// associative with identity (1, 0) ("rl-triton: High-Performance Triton GPU
// Kernels for Reinforcement Learning Credit Assignment", abstract: one shared
// associative operator for all seven estimators).  Scans below run in "scan
// order": the order in which the recurrence consumes steps (descending t for
// reverse-time estimators, ascending t for forward-time ones), so one forward
// lane-order scan serves both directions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlscan {

constexpr int kWave = 64;
constexpr int kChunk = 4;  // consecutive elements per lane per round
// A workgroup holds W wave64s (4 or 8, a template parameter of the kernels):
// W*64 threads scanning a tile of W*64*kChunk*R elements.
constexpr int kMaxWaves = 8;

// Floating-point step of one element, as built from the inputs.
struct StepF {
    float a, b;
};

// Composition of many floating-point steps.  The product `a` of many equal
// factors (gamma*lambda, gamma, ...) rounds the same way at every multiply,
// so in float32 its relative error grows linearly with the number of
// factors and then biases every b it scales (at gamma = 0.999 over a few
// thousand steps that reaches the 1e-4 level).  `a` is therefore carried in
// float64, where the same growth stays ~1e-13; `b` stays float32 (its
// roundings are not correlated and do not grow that way).
struct StepD {
    double a;
    float b;
};

// Integer step of the episodic prefix sum: a is 0 (restart) or 1 (carry).
struct StepI {
    uint32_t a;
    int64_t b;
};

// Float64 step, for recurrences whose coefficients can exceed 1 (V-trace
// with gamma*lambda*c_bar > 1).  There the trace products grow along an
// episode, and so does the weight of every earlier rounding: a relative
// error of 1e-8 in one coefficient (one float32 rounding of exp or of a
// TD error) can move a result by 1e-4 of its size.  Coefficients, state and
// epilogue are then all float64, and only the outputs are rounded.
struct StepW {
    double a, b;
};

// The step operations below are host-and-device functions: the CPU model of
// the look-back protocol (tests) composes steps with them too.

// Type that holds compositions of a given element step type.
template <class S> struct AggOf;
template <> struct AggOf<StepF> { using type = StepD; };
template <> struct AggOf<StepI> { using type = StepI; };
template <> struct AggOf<StepW> { using type = StepW; };

__host__ __device__ __forceinline__ StepD identity_step(StepD) { return {1.0, 0.0f}; }
__host__ __device__ __forceinline__ StepI identity_step(StepI) { return {1u, 0}; }
__host__ __device__ __forceinline__ StepF identity_step(StepF) { return {1.0f, 0.0f}; }
__host__ __device__ __forceinline__ StepW identity_step(StepW) { return {1.0, 0.0}; }

__host__ __device__ __forceinline__ StepD promote(StepF s) { return {static_cast<double>(s.a), s.b}; }
__host__ __device__ __forceinline__ StepI promote(StepI s) { return s; }
__host__ __device__ __forceinline__ StepW promote(StepW s) { return s; }

// later o earlier
__host__ __device__ __forceinline__ StepD compose(StepD later, StepD earlier) {
    return {later.a * earlier.a, fmaf(static_cast<float>(later.a), earlier.b, later.b)};
}
__host__ __device__ __forceinline__ StepI compose(StepI later, StepI earlier) {
    return {later.a & earlier.a, later.a ? later.b + earlier.b : later.b};
}
__host__ __device__ __forceinline__ StepW compose(StepW later, StepW earlier) {
    return {later.a * earlier.a, fma(later.a, earlier.b, later.b)};
}

__host__ __device__ __forceinline__ float apply(StepF s, float x) { return fmaf(s.a, x, s.b); }
__host__ __device__ __forceinline__ float apply(StepD s, float x) {
    return fmaf(static_cast<float>(s.a), x, s.b);
}
__host__ __device__ __forceinline__ int64_t apply(StepI s, int64_t x) { return s.a ? x + s.b : s.b; }
__host__ __device__ __forceinline__ double apply(StepW s, double x) { return fma(s.a, x, s.b); }

__host__ __device__ __forceinline__ bool cuts_chain(StepF s) { return s.a == 0.0f; }
__host__ __device__ __forceinline__ bool cuts_chain(StepD s) { return s.a == 0.0; }
__host__ __device__ __forceinline__ bool cuts_chain(StepI s) { return s.a == 0u; }
__host__ __device__ __forceinline__ bool cuts_chain(StepW s) { return s.a == 0.0; }

// ---------------------------------------------------------------- DPP moves
// DPP control words of the GFX9 family (gfx950 included):
//   row_shr:n = 0x110 + n   (lane i reads lane i-n of its 16-lane row)
//   row_bcast:15 = 0x142    (lane 15 of each row feeds the whole next row)
//   row_bcast:31 = 0x143    (lane 31 feeds rows 2 and 3)
// With bound_ctrl off, a lane whose source is outside its row, or whose row
// is masked off, keeps `old` -- here the identity element.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_move(uint32_t old, uint32_t src) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(old), static_cast<int>(src), kCtrl, kRowMask, 0xF, false));
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ StepF dpp_step(StepF s) {
    StepF r;
    r.a = __uint_as_float(dpp_move<kCtrl, kRowMask>(__float_as_uint(1.0f), __float_as_uint(s.a)));
    r.b = __uint_as_float(dpp_move<kCtrl, kRowMask>(0u, __float_as_uint(s.b)));
    return r;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ StepD dpp_step(StepD s) {
    const uint64_t ua = static_cast<uint64_t>(__double_as_longlong(s.a));
    const uint64_t one = static_cast<uint64_t>(__double_as_longlong(1.0));
    const uint32_t lo = dpp_move<kCtrl, kRowMask>(static_cast<uint32_t>(one),
                                                  static_cast<uint32_t>(ua));
    const uint32_t hi = dpp_move<kCtrl, kRowMask>(static_cast<uint32_t>(one >> 32),
                                                  static_cast<uint32_t>(ua >> 32));
    StepD r;
    r.a = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
    r.b = __uint_as_float(dpp_move<kCtrl, kRowMask>(0u, __float_as_uint(s.b)));
    return r;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_move64(uint64_t old, uint64_t src) {
    const uint32_t lo = dpp_move<kCtrl, kRowMask>(static_cast<uint32_t>(old),
                                                  static_cast<uint32_t>(src));
    const uint32_t hi = dpp_move<kCtrl, kRowMask>(static_cast<uint32_t>(old >> 32),
                                                  static_cast<uint32_t>(src >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ StepW dpp_step(StepW s) {
    const uint64_t one = static_cast<uint64_t>(__double_as_longlong(1.0));
    StepW r;
    r.a = __longlong_as_double(static_cast<long long>(
        dpp_move64<kCtrl, kRowMask>(one, static_cast<uint64_t>(__double_as_longlong(s.a)))));
    r.b = __longlong_as_double(static_cast<long long>(
        dpp_move64<kCtrl, kRowMask>(0u, static_cast<uint64_t>(__double_as_longlong(s.b)))));
    return r;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ StepI dpp_step(StepI s) {
    const uint64_t ub = static_cast<uint64_t>(s.b);
    StepI r;
    r.a = dpp_move<kCtrl, kRowMask>(1u, s.a);
    const uint32_t lo = dpp_move<kCtrl, kRowMask>(0u, static_cast<uint32_t>(ub));
    const uint32_t hi = dpp_move<kCtrl, kRowMask>(0u, static_cast<uint32_t>(ub >> 32));
    r.b = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    return r;
}

// Inclusive scan over the 64 lanes of a wave, lane 0 first: on return lane i
// holds s_i o s_{i-1} o ... o s_0.  Hillis-Steele within each 16-lane row
// (four row_shr steps), then two row broadcasts stitch the four rows.
template <class S>
__device__ __forceinline__ S wave_inclusive_scan(S s) {
    s = compose(s, dpp_step<0x111, 0xF>(s));
    s = compose(s, dpp_step<0x112, 0xF>(s));
    s = compose(s, dpp_step<0x114, 0xF>(s));
    s = compose(s, dpp_step<0x118, 0xF>(s));
    s = compose(s, dpp_step<0x142, 0xA>(s));
    s = compose(s, dpp_step<0x143, 0xC>(s));
    return s;
}

// ---------------------------------------------------------------- lane moves
__device__ __forceinline__ float read_lane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int64_t read_lane(int64_t v, int lane) {
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), lane);
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ double read_lane(double v, int lane) {
    return __longlong_as_double(read_lane(static_cast<int64_t>(__double_as_longlong(v)), lane));
}
__device__ __forceinline__ StepD read_lane(StepD s, int lane) {
    return {read_lane(s.a, lane), read_lane(s.b, lane)};
}
__device__ __forceinline__ StepW read_lane(StepW s, int lane) {
    return {read_lane(s.a, lane), read_lane(s.b, lane)};
}
__device__ __forceinline__ StepI read_lane(StepI s, int lane) {
    return {static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(s.a), lane)),
            read_lane(s.b, lane)};
}

// Value of lane i-1 (lane 0 receives `first`), through ds_bpermute.
__device__ __forceinline__ uint32_t lane_before_u32(uint32_t v, int lane, uint32_t first) {
    const int src = (lane > 0 ? lane - 1 : 0) << 2;
    const uint32_t got = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(v)));
    return lane > 0 ? got : first;
}
__device__ __forceinline__ float lane_before(float v, int lane, float first) {
    return __uint_as_float(lane_before_u32(__float_as_uint(v), lane, __float_as_uint(first)));
}
__device__ __forceinline__ int64_t lane_before(int64_t v, int lane, int64_t first) {
    const uint64_t u = static_cast<uint64_t>(v), f = static_cast<uint64_t>(first);
    const uint32_t lo = lane_before_u32(static_cast<uint32_t>(u), lane, static_cast<uint32_t>(f));
    const uint32_t hi = lane_before_u32(static_cast<uint32_t>(u >> 32), lane,
                                        static_cast<uint32_t>(f >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double lane_before(double v, int lane, double first) {
    return __longlong_as_double(static_cast<long long>(
        lane_before(static_cast<int64_t>(__double_as_longlong(v)), lane,
                    static_cast<int64_t>(__double_as_longlong(first)))));
}

}  // namespace rlscan
