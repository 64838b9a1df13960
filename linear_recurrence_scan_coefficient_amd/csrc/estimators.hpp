// estimators.hpp -- on-chip construction of the recurrence steps (a_t, b_t)
// for the seven credit-assignment estimators, and their epilogues.
//
// Each estimator type provides
//   S, V              step type and state type (StepF/float or StepI/int64_t)
//   kReverse          true for reverse-time estimators (x_t depends on x_{t+1})
//   Params            device pointers and scalars of one call
//   Chunk             registers holding one lane's 4-element chunk
//   load<VEC,FULL,CARRY>  read the chunk's inputs (plus the one-element halo just
//                     above the chunk where the step needs values at t+1);
//                     `stage` is the wave's LDS staging area, kStageFloats
//                     floats (0 for estimators that do not stage)
//   Epi               values the epilogue needs besides the states (kept
//                     apart from Chunk: the raw inputs are dead once the
//                     steps are built, only these stay live until the store)
//   steps<CARRY>(...)  build the chunk's steps, in memory order, and its Epi
//                     (CARRY: kernels built for the carry arguments; without
//                     it every carry branch is compiled out)
//   store<VEC,FULL>   write outputs from the states after each element (x)
//                     and before it (before: x_{t+1} for reverse estimators)
//   edge_value        the output written to carry_out for element j
//   reads_before      whether the output of element j reads the state before
//                     it (x_{t+1} for reverse estimators) even though its
//                     step has a == 0 -- the tile's entering state is then
//                     needed although nothing else depends on it
//
// Flags (terminated, truncated, dones) are float (set iff != 0.0f) or uint8_t
// (set iff != 0): every estimator takes the flag element type F as a template
// parameter, and the loads turn either into 0/1 floats in registers.
//
// Shared conventions: row-major [N, T]; a flag is set iff != 0; for reverse
// estimators step t cuts the chain if terminated, truncated or t = T-1, and
// the successor value seen from step t is 0 (terminated, which wins), the
// per-step bootstrap value (truncated), the per-row bootstrap value (t = T-1)
// or V_{t+1}.
//
// Carry (streaming one rollout through several calls; the chunked fallback
// of the rl-triton README, Kernels table, last column): every Params has
// carry_in [N] (NULL: each row is a whole rollout) and carry_out [N] (NULL:
// not written).  carry_in[n] is the output just past the chunk -- t = T for
// reverse estimators, t = -1 for forward ones -- and the chunk's edge step
// (t = T-1, resp. t = 0) continues into it unless terminated, truncated or
// done there.  The carry is a known value, so the edge step (a, b) applied
// to it is folded into the cut step (0, b + a*carry): the scan keeps its
// row-edge cuts and nothing else changes.  carry_out[n] is the output at
// the opposite edge (t = 0 reverse, t = T-1 forward).
//
// Sources are cited per estimator: the rl-triton README,
// section "Kernels" (one row per estimator) and section "Performance"
// (truncation/bootstrap inputs), and the estimators' published definitions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "scan_core.hpp"

namespace rlscan {

struct Geometry {
    int64_t N, T, NT;       // rows, row length, N*T
    int64_t num_tiles;      // tiles of tile_span consecutive elements
    int64_t grid;           // workgroups launched
    int64_t tile_span;      // elements of memory per tile: the tile's capacity, or
                            // (packed mapping) the whole rows it holds, a multiple
                            // of 4 that can fall short of the capacity
    int64_t xcd_run;        // packed, one tile per workgroup: runs of this many
                            // consecutive tiles per XCD (xcd_tile); 0: tile = blockIdx
    double inv_T;           // 1.0 / T, for the row/time split of an index
};

// Position of one lane's chunk: 4 consecutive elements starting at g0.
struct ChunkPos {
    int64_t g0;
    int64_t n0, t0;  // row and time of element g0
    int valid;       // elements of the chunk below N*T (0..4)
};

__device__ __forceinline__ ChunkPos chunk_pos(int64_t g0, const Geometry& geo) {
    ChunkPos q;
    q.g0 = g0;
    const int64_t rem = geo.NT - g0;
    q.valid = rem <= 0 ? 0 : (rem >= kChunk ? kChunk : static_cast<int>(rem));
    // g0 < 2^49, so the float64 quotient is within one of the true quotient.
    int64_t n = static_cast<int64_t>(static_cast<double>(g0) * geo.inv_T);
    int64_t t = g0 - n * geo.T;
    if (t < 0) {
        --n;
        t += geo.T;
    } else if (t >= geo.T) {
        ++n;
        t -= geo.T;
    }
    q.n0 = n;
    q.t0 = t;
    return q;
}

__device__ __forceinline__ void next_position(int64_t& n, int64_t& t, int64_t T) {
    if (++t == T) {
        t = 0;
        ++n;
    }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
// A float in LDS (address space 3): loads through it are ds_read.
typedef __attribute__((address_space(3))) float lds_float;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));

// Loads of a 4-element chunk.  Elements at or past N*T read as 0 (their
// steps are replaced by the identity before the scan).  FULL: the whole tile
// lies below N*T, so no element needs a bounds check.
//
// Every input is read once and every output written once, so the 16-byte
// accesses carry the non-temporal hint (`nt`): the lines are streamed
// through the caches instead of displacing others.  On MI355X this made
// long-row calls 2-6 % faster and a 2^25-element packed call 13 % faster.
template <bool VEC, bool FULL>
__device__ __forceinline__ void load4(const float* __restrict__ p, const ChunkPos& q, float v[4]) {
    if (VEC && (FULL || q.valid == kChunk)) {
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + q.g0));
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
        return;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) v[j] = (FULL || j < q.valid) ? p[q.g0 + j] : 0.0f;
}

template <bool VEC, bool FULL>
__device__ __forceinline__ void load4(const int32_t* __restrict__ p, const ChunkPos& q, int32_t v[4]) {
    if (VEC && (FULL || q.valid == kChunk)) {
        const i32x4 w = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p + q.g0));
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
        return;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) v[j] = (FULL || j < q.valid) ? p[q.g0 + j] : 0;
}

// One-byte flags: a chunk's four flags are one 4-byte word (a wave reads
// 256 contiguous bytes per instruction), unpacked to 0/1 floats.
template <bool VEC, bool FULL>
__device__ __forceinline__ void load4(const uint8_t* __restrict__ p, const ChunkPos& q, float v[4]) {
    if (VEC && (FULL || q.valid == kChunk)) {
        const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + q.g0));
#pragma unroll
        for (int j = 0; j < kChunk; ++j) v[j] = ((w >> (8 * j)) & 0xffu) != 0u ? 1.0f : 0.0f;
        return;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
        v[j] = ((FULL || j < q.valid) && p[q.g0 + j] != 0) ? 1.0f : 0.0f;
}

template <bool VEC, bool FULL>
__device__ __forceinline__ void store4(float* __restrict__ p, const ChunkPos& q, const float v[4]) {
    if (VEC && (FULL || q.valid == kChunk)) {
        f32x4 w;
        w.x = v[0]; w.y = v[1]; w.z = v[2]; w.w = v[3];
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p + q.g0));
        return;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
        if (FULL || j < q.valid) p[q.g0 + j] = v[j];
}

template <bool VEC, bool FULL>
__device__ __forceinline__ void store4(int64_t* __restrict__ p, const ChunkPos& q, const int64_t v[4]) {
    if (VEC && (FULL || q.valid == kChunk)) {
        i64x2 w0, w1;
        w0.x = v[0]; w0.y = v[1]; w1.x = v[2]; w1.y = v[3];
        __builtin_nontemporal_store(w0, reinterpret_cast<i64x2*>(p + q.g0));
        __builtin_nontemporal_store(w1, reinterpret_cast<i64x2*>(p + q.g0) + 1);
        return;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
        if (FULL || j < q.valid) p[q.g0 + j] = v[j];
}

// One element past the chunk (the halo).  Past the end of the data the
// index is clamped to the last element; the value is then never used, since
// the chunk's last element ends its row.
template <class T>
__device__ __forceinline__ T load_halo(const T* __restrict__ p, const ChunkPos& q, int64_t NT) {
    const int64_t i = q.g0 + kChunk;
    return p[i < NT ? i : NT - 1];
}

// The value just above a reverse estimator's chunk (V_{t+1} of its top
// element) is the first value of the chunk above it, which the previous
// lane holds: chunks run downwards from lane 0.  Only lane 0 reads it from
// memory, at load time (halo_load); the others take it from that lane once
// every round's loads are in flight (halo_exchange, called from `steps`: an
// exchange at load time would wait for the round's data before the next
// round's loads are issued).  One load per wave instead of one per lane.
__device__ __forceinline__ float halo_load(const float* __restrict__ p, const ChunkPos& q,
                                           int64_t NT) {
    return (threadIdx.x & (kWave - 1)) == 0 ? load_halo(p, q, NT) : 0.0f;
}
__device__ __forceinline__ float halo_exchange(float first, float lane0_value) {
    return lane_before(first, threadIdx.x & (kWave - 1), lane0_value);
}

struct NoEpi {};

// Shared episode logic of the reverse estimators: the flags of one chunk and
// the bootstrap value of the row its first element lies in.
struct EpisodeChunk {
    float r[4], term[4], trunc[4], bv[4];
    float boot;   // V at t = T of the chunk's first row
    float carry;  // carry_in of the chunk's first row
};

template <bool VEC, bool FULL, bool TRUNC, bool CARRY, class F>
__device__ __forceinline__ void load_episode(const float* rewards, const F* terminated,
                                             const F* truncated,
                                             const float* bootstrap_values,
                                             const float* bootstrap_value,
                                             const float* carry_in, const Geometry& geo,
                                             const ChunkPos& q, EpisodeChunk& c) {
    // loaded with the chunk so that the row-end case costs no dependent load,
    // and only by lanes whose chunk holds the end of its first row (the
    // others issue no request)
    const int64_t nr = q.n0 < geo.N ? q.n0 : geo.N - 1;
    const bool first_row_ends = q.t0 >= geo.T - kChunk;
    c.boot = (bootstrap_value != nullptr && first_row_ends) ? bootstrap_value[nr] : 0.0f;
    c.carry = (CARRY && carry_in != nullptr && first_row_ends) ? carry_in[nr] : 0.0f;
    load4<VEC, FULL>(rewards, q, c.r);
    load4<VEC, FULL>(terminated, q, c.term);
    if constexpr (TRUNC) {
        load4<VEC, FULL>(truncated, q, c.trunc);
        load4<VEC, FULL>(bootstrap_values, q, c.bv);
    } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) c.trunc[j] = c.bv[j] = 0.0f;
    }
}

// Successor value for a chain cut (terminated > truncated > row end), and
// whether the step is a cut.  `v_next` is V_{t+1}, used when it is not a cut.
// A chunk holds at most one row end unless T < 4; only then can a row end
// belong to a later row than the chunk's first element.  `continues`: a
// carry_in was given, so a row end is not a cut by itself (its successor
// value is still V at t = T).
__device__ __forceinline__ float successor_value(const EpisodeChunk& c, int j, bool row_end,
                                                 bool in_range, const float* bootstrap_value,
                                                 int64_t n, int64_t n0, float v_next,
                                                 bool continues, bool& cut) {
    const bool term = c.term[j] != 0.0f;
    const bool trunc = c.trunc[j] != 0.0f;
    cut = term || trunc || (row_end && !continues);
    float v = v_next;
    if (row_end) v = c.boot;
    if (row_end && in_range && n != n0 && bootstrap_value != nullptr) v = bootstrap_value[n];
    if (trunc) v = c.bv[j];
    if (term) v = 0.0f;
    return v;
}

// carry_in of row n, for an element of a chunk whose first row is n0 (the
// first row's value is preloaded with the chunk).
__device__ __forceinline__ float row_carry(const EpisodeChunk& c, const float* carry_in,
                                           int64_t n, int64_t n0) {
    return n == n0 ? c.carry : carry_in[n];
}

// The edge step (a, b) applied to the known carry, as a cut step.
__device__ __forceinline__ void fold_carry(StepF& e, float carry) {
    e.b = fmaf(e.a, carry, e.b);
    e.a = 0.0f;
}
__device__ __forceinline__ void fold_carry(StepW& e, double carry) {
    e.b = fma(e.a, carry, e.b);
    e.a = 0.0;
}

__device__ __forceinline__ float fma_of(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double fma_of(double a, double b, double c) { return fma(a, b, c); }
__device__ __forceinline__ float fmin_of(float a, float b) { return fminf(a, b); }
__device__ __forceinline__ double fmin_of(double a, double b) { return fmin(a, b); }

// ------------------------------------------------------------------ GAE
// README, Kernels table, compute_gae row (backward scan of TD errors with
// weight gamma*lambda); Schulman et al. 2016.
//   a_t = cut ? 0 : gamma*lambda,   b_t = r_t + gamma*Vhat_{t+1} - V_t
template <class F>
struct GaeParams {
    const float *rewards, *values, *bootstrap_value;
    const F *terminated, *truncated;
    const float *bootstrap_values, *carry_in;
    float *out, *carry_out;
    float gamma, gamma_lambda;
};

template <bool kTrunc, class F = float>
struct Gae {
    using S = StepF;
    using V = float;
    static constexpr bool kReverse = true;
    using Params = GaeParams<F>;
    using Epi = NoEpi;
    static constexpr int kStageFloats = 0;
    static constexpr int kOutStageFloats = 0;
    struct Chunk {
        EpisodeChunk ep;
        float v[4];
        float v_halo;
    };
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load_episode<VEC, FULL, kTrunc, CARRY>(p.rewards, p.terminated, p.truncated,
                                        p.bootstrap_values, p.bootstrap_value, p.carry_in, geo,
                                        q, c.ep);
        load4<VEC, FULL>(p.values, q, c.v);
        c.v_halo = halo_load(p.values, q, geo.NT);
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi&) {
        int64_t n = q.n0, t = q.t0;
        const bool continues = CARRY && p.carry_in != nullptr;
        const float v_halo = halo_exchange(c.v[0], c.v_halo);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            bool cut;
            const bool row_end = t == geo.T - 1;
            const float v_next = j < kChunk - 1 ? c.v[j + 1] : v_halo;
            const float vh = successor_value(c.ep, j, row_end, j < q.valid,
                                             p.bootstrap_value, n, q.n0, v_next, continues, cut);
            e[j].a = cut ? 0.0f : p.gamma_lambda;
            e[j].b = fmaf(p.gamma, vh, c.ep.r[j]) - c.v[j];
            if (row_end && continues && !cut && j < q.valid)
                fold_carry(e[j], row_carry(c.ep, p.carry_in, n, q.n0));  // A_T
            next_position(n, t, geo.T);
        }
    }
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float*) {
        store4<VEC, FULL>(p.out, q, x);
    }
};

// ------------------------------------------------------------ TD(lambda)
// README, Kernels table, compute_lambda_returns row; lambda-return.
//   a_t = cut ? 0 : gamma*lambda
//   b_t = cut ? r_t + gamma*Vhat_{t+1} : r_t + gamma*(1-lambda)*V_{t+1}
template <class F>
struct LambdaReturnsParams {
    const float *rewards, *values, *bootstrap_value;
    const F *terminated, *truncated;
    const float *bootstrap_values, *carry_in;
    float *out, *carry_out;
    float gamma, gamma_lambda, gamma_one_minus_lambda;
};

template <bool kTrunc, class F = float>
struct LambdaReturns {
    using S = StepF;
    using V = float;
    static constexpr bool kReverse = true;
    using Params = LambdaReturnsParams<F>;
    using Epi = NoEpi;
    static constexpr int kStageFloats = 0;
    static constexpr int kOutStageFloats = 0;
    using Chunk = typename Gae<kTrunc, F>::Chunk;
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load_episode<VEC, FULL, kTrunc, CARRY>(p.rewards, p.terminated, p.truncated,
                                        p.bootstrap_values, p.bootstrap_value, p.carry_in, geo,
                                        q, c.ep);
        load4<VEC, FULL>(p.values, q, c.v);
        c.v_halo = halo_load(p.values, q, geo.NT);
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi&) {
        int64_t n = q.n0, t = q.t0;
        const bool continues = CARRY && p.carry_in != nullptr;
        const float v_halo = halo_exchange(c.v[0], c.v_halo);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            bool cut;
            const bool row_end = t == geo.T - 1;
            const float v_next = j < kChunk - 1 ? c.v[j + 1] : v_halo;
            // vh is V_{t+1} on a step that is not a cut (V at t = T at a
            // continued row end)
            const float vh = successor_value(c.ep, j, row_end, j < q.valid,
                                             p.bootstrap_value, n, q.n0, v_next, continues, cut);
            e[j].a = cut ? 0.0f : p.gamma_lambda;
            e[j].b = cut ? fmaf(p.gamma, vh, c.ep.r[j])
                         : fmaf(p.gamma_one_minus_lambda, vh, c.ep.r[j]);
            if (row_end && continues && !cut && j < q.valid)
                fold_carry(e[j], row_carry(c.ep, p.carry_in, n, q.n0));  // G_T
            next_position(n, t, geo.T);
        }
    }
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float*) {
        store4<VEC, FULL>(p.out, q, x);
    }
};

// ------------------------------------------------------ discounted returns
// README, Kernels table, compute_discounted_returns row (reward-to-go).
//   a_t = cut ? 0 : gamma,   b_t = cut ? r_t + gamma*Vhat_{t+1} : r_t
template <class F>
struct DiscountedParams {
    const float *rewards, *bootstrap_value;
    const F *terminated, *truncated;
    const float *bootstrap_values, *carry_in;
    float *out, *carry_out;
    float gamma;
};

template <bool kTrunc, class F = float>
struct Discounted {
    using S = StepF;
    using V = float;
    static constexpr bool kReverse = true;
    using Params = DiscountedParams<F>;
    using Epi = NoEpi;
    static constexpr int kStageFloats = 0;
    static constexpr int kOutStageFloats = 0;
    struct Chunk {
        EpisodeChunk ep;
    };
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load_episode<VEC, FULL, kTrunc, CARRY>(p.rewards, p.terminated, p.truncated,
                                        p.bootstrap_values, p.bootstrap_value, p.carry_in, geo,
                                        q, c.ep);
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi&) {
        int64_t n = q.n0, t = q.t0;
        const bool continues = CARRY && p.carry_in != nullptr;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            bool cut;
            const bool row_end = t == geo.T - 1;
            const float vh = successor_value(c.ep, j, row_end, j < q.valid,
                                             p.bootstrap_value, n, q.n0, 0.0f, continues, cut);
            e[j].a = cut ? 0.0f : p.gamma;
            e[j].b = cut ? fmaf(p.gamma, vh, c.ep.r[j]) : c.ep.r[j];
            if (row_end && continues && !cut && j < q.valid)
                fold_carry(e[j], row_carry(c.ep, p.carry_in, n, q.n0));  // G_T
            next_position(n, t, geo.T);
        }
    }
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float*) {
        store4<VEC, FULL>(p.out, q, x);
    }
};

// ------------------------------------------------------------------ V-trace
// README, Kernels table, compute_vtrace row (importance-weighted targets and
// advantages); Espeholt et al. 2018, with that paper's optional factor
// lambda on the trace coefficients and a truncation level rho_bar_pg of its
// own for the policy-gradient weight (lambda = 1, rho_bar_pg = rho_bar is
// the plain form).  With ratio_t = exp(log_rho_t), rho_t = min(rho_bar,
// ratio_t), c_t = lambda*min(c_bar, ratio_t), rho'_t = min(rho_bar_pg,
// ratio_t) and td_t = r_t + gamma*Vhat_{t+1} - V_t, the scan computes
// u_t = vs_t - V_t:
//   a_t = cut ? 0 : gamma*c_t,   b_t = delta_t = rho_t*td_t
// and the epilogue forms vs_t = V_t + u_t and
//   pg_t = rho'_t*td_t + (cut ? 0 : gamma*rho'_t*u_{t+1})
// which equals rho'_t*(r_t + gamma*(cut ? Vhat_{t+1} : vs_{t+1}) - V_t).
// kWide: the float64 form (StepW) for calls whose trace coefficients can
// exceed 1 (gamma*lambda*c_bar > 1): the ratio, rho, c, the TD error, the
// scan and the epilogue are float64, and only vs and pg are rounded.
template <class F>
struct VtraceParams {
    const float *rewards, *values, *bootstrap_value, *log_rhos;
    const F *terminated, *truncated;
    const float *bootstrap_values, *carry_in;  // carry_in: vs at t = T
    float *vs, *pg, *carry_out;               // carry_out: vs at t = 0
    float gamma, lambda, rho_bar, c_bar, rho_bar_pg;
};

template <bool kTrunc, class F = float, bool kWide = false>
struct Vtrace {
    using S = typename std::conditional<kWide, StepW, StepF>::type;
    using V = typename std::conditional<kWide, double, float>::type;
    static constexpr bool kReverse = true;
    using Params = VtraceParams<F>;
    struct Chunk {
        EpisodeChunk ep;
        float v[4];
        float lr[4];
        float v_halo;
    };
    struct Epi {
        float v[4];
        V pg_base[4];    // rho'_t * td_t
        V gamma_rho[4];  // gamma * rho'_t, 0 at a cut
    };
    static constexpr int kStageFloats = 0;
    static constexpr int kOutStageFloats = 0;
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load_episode<VEC, FULL, kTrunc, CARRY>(p.rewards, p.terminated, p.truncated,
                                        p.bootstrap_values, p.bootstrap_value, p.carry_in, geo,
                                        q, c.ep);
        load4<VEC, FULL>(p.values, q, c.v);
        load4<VEC, FULL>(p.log_rhos, q, c.lr);
        c.v_halo = halo_load(p.values, q, geo.NT);
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi& epi) {
        int64_t n = q.n0, t = q.t0;
        const bool continues = CARRY && p.carry_in != nullptr;
        const float v_halo = halo_exchange(c.v[0], c.v_halo);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            bool cut;
            const bool row_end = t == geo.T - 1;
            const float v_next = j < kChunk - 1 ? c.v[j + 1] : v_halo;
            const float vh = successor_value(c.ep, j, row_end, j < q.valid,
                                             p.bootstrap_value, n, q.n0, v_next, continues, cut);
            V ratio;
            if constexpr (kWide)
                ratio = exp(static_cast<double>(c.lr[j]));
            else
                ratio = expf(c.lr[j]);
            const V gamma = p.gamma;
            const V rho = fmin_of(static_cast<V>(p.rho_bar), ratio);
            const V cc = static_cast<V>(p.lambda) * fmin_of(static_cast<V>(p.c_bar), ratio);
            const V rho_pg = fmin_of(static_cast<V>(p.rho_bar_pg), ratio);
            const V td = fma_of(gamma, static_cast<V>(vh), static_cast<V>(c.ep.r[j])) -
                         static_cast<V>(c.v[j]);
            epi.v[j] = c.v[j];
            epi.pg_base[j] = rho_pg * td;
            epi.gamma_rho[j] = cut ? V(0) : gamma * rho_pg;
            e[j].a = cut ? V(0) : gamma * cc;
            e[j].b = rho * td;
            if (row_end && continues && !cut && j < q.valid) {
                // u at t = T is vs_T - V_T; the state before this element is
                // not in the scan, so pg takes it here
                const V u_T = static_cast<V>(row_carry(c.ep, p.carry_in, n, q.n0)) -
                              static_cast<V>(vh);
                fold_carry(e[j], u_T);
                epi.pg_base[j] = fma_of(epi.gamma_rho[j], u_T, epi.pg_base[j]);
                epi.gamma_rho[j] = V(0);
            }
            next_position(n, t, geo.T);
        }
    }
    // carry_out of V-trace is vs, like its carry_in
    __device__ __forceinline__ static V edge_value(const Epi& c, const V x[4], int j) {
        return static_cast<V>(c.v[j]) + x[j];
    }
    // pg_t reads u_{t+1} unless t is a cut, also where c_t = 0 makes a_t = 0
    // (lambda = 0, or lambda * c underflowing)
    __device__ __forceinline__ static bool reads_before(const Epi& c, int j) {
        return c.gamma_rho[j] != V(0);
    }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi& c,
                                                 const V x[4], const V before[4], lds_float*) {
        float vs[4], pg[4];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            vs[j] = static_cast<float>(static_cast<V>(c.v[j]) + x[j]);
            pg[j] = static_cast<float>(fma_of(c.gamma_rho[j], before[j], c.pg_base[j]));
        }
        store4<VEC, FULL>(p.vs, q, vs);
        store4<VEC, FULL>(p.pg, q, pg);
    }
};

// ------------------------------------------------------------------ Retrace
// README, Kernels table, compute_retrace row (off-policy return with
// truncated importance ratios) and section "Performance" (both flags
// required; continuation value inside next_q_values_all); Munos et al. 2016.
//   EQ_t = sum_a pi'[t,a] Q'[t,a],  c'_t = lambda*min(1, pi'[t,a_{t+1}] / mu_{t+1})
//   a_t = cut ? 0 : gamma*c'_t
//   b_t = cut ? r_t + (terminated ? 0 : gamma*EQ_t)
//             : r_t + gamma*(EQ_t - c'_t*Q'[t,a_{t+1}])
// kA > 0: A known at compile time, the chunk's 4*A action values are read
// with 16-byte loads into registers; kA == 0: any A, read element-wise.
// kStaged: full tiles stage the action values through LDS (below); without
// it they are read straight into registers, which needs no LDS -- the form
// grouped launches use, where the LDS of one workgroup limits every call.
template <int kA, class F = float, bool kStaged = true>
struct Retrace {
    using S = StepF;
    using V = float;
    static constexpr bool kReverse = true;
    using Epi = NoEpi;
    // With A known and at most 8, full tiles stage the wave's 256 x A action
    // values of each tensor through LDS: every load instruction then reads
    // 1 KiB of contiguous memory (a lane's own 4 x A values would be a
    // 16-byte piece every 16 x A bytes, which the L2 fetched ~14% over).
    static constexpr int kStageFloats =
        (kStaged && kA >= 1 && kA <= 8) ? 2 * kWave * kChunk * kA : 0;
    static constexpr int kOutStageFloats = 0;
    struct Params {
        const float *rewards, *next_q, *next_pi;
        const int32_t* actions;
        const float* behaviour_probs;
        const F *terminated, *truncated;
        float* out;
        int64_t A;
        float gamma, lambda;
        // carry: G at t = T, and a_T, mu(a_T | x_T) of the chunk that follows
        const float* carry_in;
        const int32_t* next_actions;
        const float* next_mu;
        float* carry_out;
    };
    static constexpr int kRegA = kA > 0 ? kA : 1;
    struct Chunk {
        EpisodeChunk ep;  // bv unused
        int32_t act[4];
        float mu[4];
        int32_t act_halo;
        float mu_halo;
        float q[4 * kRegA], pi[4 * kRegA];
        const lds_float* lds;  // this lane's staged Q' values (pi' follow at
                               // +kWave*kChunk*kA) when `staged`
        bool staged;           // (LDS address 0 is valid: no null sentinel)
    };
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float* stage) {
        load4<VEC, FULL>(p.rewards, q, c.ep.r);
        load4<VEC, FULL>(p.terminated, q, c.ep.term);
        load4<VEC, FULL>(p.truncated, q, c.ep.trunc);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) c.ep.bv[j] = 0.0f;
        c.ep.boot = 0.0f;
        c.ep.carry = 0.0f;
        load4<VEC, FULL>(p.actions, q, c.act);
        load4<VEC, FULL>(p.behaviour_probs, q, c.mu);
        // a_{t+1} and mu_{t+1} of the chunk's top element: element 0 of the
        // next chunk up, held by the previous lane; lane 0 reads memory here,
        // the exchange follows in `steps` (after the action-value loads are
        // issued)
        const int lane = threadIdx.x & (kWave - 1);
        c.act_halo = 0;
        c.mu_halo = 1.0f;
        if (lane == 0) {
            c.act_halo = load_halo(p.actions, q, geo.NT);
            c.mu_halo = load_halo(p.behaviour_probs, q, geo.NT);
        }
        c.lds = stage;
        c.staged = false;
        if constexpr (kA > 0 && VEC && FULL && kStageFloats > 0) {
            // the wave's chunks are contiguous; lane 63 holds the lowest one
            constexpr int kSpan = kWave * kChunk * kA;  // floats per tensor
            const int64_t span = q.g0 - static_cast<int64_t>(kChunk) * (kWave - 1 - lane);
            const float* gq = p.next_q + span * kA;
            const float* gp = p.next_pi + span * kA;
#pragma unroll
            for (int i = 0; i < kA; ++i) {  // cache policy 2: non-temporal (nt)
                __builtin_amdgcn_global_load_lds(gq + 4 * (kWave * i + lane), stage + kWave * 4 * i,
                                                 16, 0, 2);
                __builtin_amdgcn_global_load_lds(gp + 4 * (kWave * i + lane),
                                                 stage + kSpan + kWave * 4 * i, 16, 0, 2);
            }
            c.lds = stage + (kWave - 1 - lane) * kChunk * kA;
            c.staged = true;
        } else if constexpr (kA > 0) {
            const int64_t base = q.g0 * kA;
            if (VEC && (FULL || q.valid == kChunk)) {
                // 4*kA floats = kA 16-byte vectors per tensor, 16-byte aligned
                const f32x4* qv = reinterpret_cast<const f32x4*>(p.next_q + base);
                const f32x4* pv = reinterpret_cast<const f32x4*>(p.next_pi + base);
#pragma unroll
                for (int i = 0; i < kA; ++i) {
                    const f32x4 a = qv[i], b = pv[i];
                    c.q[4 * i + 0] = a.x; c.q[4 * i + 1] = a.y;
                    c.q[4 * i + 2] = a.z; c.q[4 * i + 3] = a.w;
                    c.pi[4 * i + 0] = b.x; c.pi[4 * i + 1] = b.y;
                    c.pi[4 * i + 2] = b.z; c.pi[4 * i + 3] = b.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4 * kA; ++i) {
                    const bool ok = FULL || i / kA < q.valid;
                    c.q[i] = ok ? p.next_q[base + i] : 0.0f;
                    c.pi[i] = ok ? p.next_pi[base + i] : 0.0f;
                }
            }
        }
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi&) {
        // action values: registers, or the LDS staging area (16-byte reads)
        float qv[4 * kRegA], pv[4 * kRegA];
        if constexpr (kA > 0) {
            if (c.staged) {
                // The direct-to-LDS loads count in vmcnt, and the compiler does
                // not order these reads after all of them (it was seen issuing
                // reads of the last-loaded block before the wait): wait here,
                // with a memory clobber so no LDS read moves above the wait.
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                constexpr int kSpan = kWave * kChunk * kA;
                typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
                lds_f32x4* lq = reinterpret_cast<lds_f32x4*>(c.lds);
                lds_f32x4* lp = reinterpret_cast<lds_f32x4*>(c.lds + kSpan);
#pragma unroll
                for (int i = 0; i < kA; ++i) {
                    const f32x4 a = lq[i], b = lp[i];
                    qv[4 * i + 0] = a.x; qv[4 * i + 1] = a.y;
                    qv[4 * i + 2] = a.z; qv[4 * i + 3] = a.w;
                    pv[4 * i + 0] = b.x; pv[4 * i + 1] = b.y;
                    pv[4 * i + 2] = b.z; pv[4 * i + 3] = b.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4 * kA; ++i) {
                    qv[i] = c.q[i];
                    pv[i] = c.pi[i];
                }
            }
        }
        const bool continues = CARRY && p.carry_in != nullptr;
        const int lane = threadIdx.x & (kWave - 1);
        const int32_t act_halo = static_cast<int32_t>(lane_before_u32(
            static_cast<uint32_t>(c.act[0]), lane, static_cast<uint32_t>(c.act_halo)));
        const float mu_halo = lane_before(c.mu[0], lane, c.mu_halo);
        int64_t n = q.n0, t = q.t0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const bool term = c.ep.term[j] != 0.0f;
            const bool row_end = t == geo.T - 1;
            const bool cut = term || c.ep.trunc[j] != 0.0f || (row_end && !continues);
            const bool edge = row_end && continues && !cut && j < q.valid;
            int32_t a_next = j < kChunk - 1 ? c.act[j + 1] : act_halo;
            float mu_next = j < kChunk - 1 ? c.mu[j + 1] : mu_halo;
            if (edge) {  // the next step lies in the chunk that follows
                a_next = p.next_actions[n];
                mu_next = p.next_mu[n];
            }
            float eq = 0.0f, q_sel = 0.0f, pi_sel = 0.0f;
            if constexpr (kA > 0) {
                a_next = a_next < 0 ? 0 : (a_next >= kA ? kA - 1 : a_next);
#pragma unroll
                for (int a = 0; a < kA; ++a) {
                    const float qa = qv[j * kA + a], pa = pv[j * kA + a];
                    eq = fmaf(pa, qa, eq);
                    q_sel = a == a_next ? qa : q_sel;
                    pi_sel = a == a_next ? pa : pi_sel;
                }
            } else {
                if (j < q.valid) {
                    const int64_t A = p.A;
                    const int64_t base = (q.g0 + j) * A;
                    for (int64_t a = 0; a < A; ++a)
                        eq = fmaf(p.next_pi[base + a], p.next_q[base + a], eq);
                    const int64_t as = a_next < 0 ? 0 : (a_next >= A ? A - 1 : a_next);
                    q_sel = p.next_q[base + as];
                    pi_sel = p.next_pi[base + as];
                }
            }
            const float cprime = p.lambda * fminf(1.0f, pi_sel / mu_next);
            e[j].a = cut ? 0.0f : p.gamma * cprime;
            e[j].b = cut ? (term ? c.ep.r[j] : fmaf(p.gamma, eq, c.ep.r[j]))
                         : fmaf(p.gamma, fmaf(-cprime, q_sel, eq), c.ep.r[j]);
            if (edge) fold_carry(e[j], p.carry_in[n]);  // G_T
            next_position(n, t, geo.T);
        }
    }
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float*) {
        store4<VEC, FULL>(p.out, q, x);
    }
};

// Row of the first row start (t = 0) at or after a forward chunk's first
// element, clamped to a valid row (its carry is then simply unused).
__device__ __forceinline__ int64_t first_start_row(const ChunkPos& q, const Geometry& geo) {
    const int64_t n = q.t0 == 0 ? q.n0 : q.n0 + 1;
    return n < geo.N ? n : geo.N - 1;
}

// ------------------------------------------------------- eligibility traces
// README, Kernels table, compute_eligibility_traces row: forward traces, the
// done flag at step t dropping the previous trace.
//   a_t = (d_t or t = 0) ? 0 : gamma*lambda,   b_t = x_t
// With gamma*lambda = 1 this is also the episodic prefix sum of float
// values (README, Kernels table, compute_episodic_prefix_sum row).
template <class F = float>
struct Eligibility {
    using S = StepF;
    using V = float;
    static constexpr bool kReverse = false;
    using Epi = NoEpi;
    static constexpr int kStageFloats = 0;
    static constexpr int kOutStageFloats = 0;
    struct Params {
        const float* x;
        const F* dones;
        float* out;
        float gamma_lambda;
        const float* carry_in;  // e at t = -1
        float* carry_out;       // e at t = T-1
    };
    struct Chunk {
        float x[4], d[4];
        float carry;  // carry_in of the first row that starts in the chunk
    };
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load4<VEC, FULL>(p.x, q, c.x);
        load4<VEC, FULL>(p.dones, q, c.d);
        c.carry = (CARRY && p.carry_in != nullptr) ? p.carry_in[first_start_row(q, geo)] : 0.0f;
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo, const ChunkPos& q,
                                 const Chunk& c, S e[4], Epi&) {
        const bool continues = CARRY && p.carry_in != nullptr;
        const int64_t n_first = first_start_row(q, geo);
        int64_t n = q.n0, t = q.t0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const float a_live = c.d[j] != 0.0f ? 0.0f : p.gamma_lambda;
            e[j].a = t == 0 ? 0.0f : a_live;
            e[j].b = c.x[j];
            if (t == 0 && continues && j < q.valid)  // e_{-1} from the previous chunk
                e[j].b = fmaf(a_live, n == n_first ? c.carry : p.carry_in[n], c.x[j]);
            next_position(n, t, geo.T);
        }
    }
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float*) {
        store4<VEC, FULL>(p.out, q, x);
    }
};

// ------------------------------------------------------- episodic prefix sum
// README, Kernels table, compute_episodic_prefix_sum row: cumulative sum
// restarted by the done mask; exact int64 accumulation of int32 inputs.
//   a_t = (d_t or t = 0) ? 0 : 1,   b_t = x_t
template <class F = float>
struct PrefixSum {
    using S = StepI;
    using V = int64_t;
    static constexpr bool kReverse = false;
    using Epi = NoEpi;
    static constexpr int kStageFloats = 0;
    // 32 output bytes per lane: a wave's 2 KiB of results pass through LDS
    static constexpr int kOutStageFloats = kWave * kChunk * 2;
    struct Params {
        const int32_t* x;
        const F* dones;
        int64_t* out;
        const int64_t* carry_in;  // y at t = -1
        int64_t* carry_out;       // y at t = T-1
    };
    struct Chunk {
        int32_t x[4];
        float d[4];
        int64_t carry;  // carry_in of the first row that starts in the chunk
    };
    template <bool VEC, bool FULL, bool CARRY>
    __device__ __forceinline__ static void load(const Params& p, const Geometry& geo,
                                                const ChunkPos& q, Chunk& c, lds_float*) {
        load4<VEC, FULL>(p.x, q, c.x);
        load4<VEC, FULL>(p.dones, q, c.d);
        c.carry = (CARRY && p.carry_in != nullptr) ? p.carry_in[first_start_row(q, geo)] : 0;
    }
    template <bool CARRY>
    __device__ __forceinline__ static void steps(const Params& p, const Geometry& geo,
                                                 const ChunkPos& q, const Chunk& c, S e[4], Epi&) {
        const bool continues = CARRY && p.carry_in != nullptr;
        const int64_t n_first = first_start_row(q, geo);
        int64_t n = q.n0, t = q.t0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const bool done = c.d[j] != 0.0f;
            e[j].a = (done || t == 0) ? 0u : 1u;
            e[j].b = static_cast<int64_t>(c.x[j]);
            if (t == 0 && continues && !done && j < q.valid)  // y_{-1} from the previous chunk
                e[j].b += n == n_first ? c.carry : p.carry_in[n];
            next_position(n, t, geo.T);
        }
    }
    // A lane's four int64 results are 32 contiguous bytes.  Stored directly,
    // each of its two 16-byte store instructions would cover only every
    // other 16 bytes of the wave's span -- half of every cache line -- and
    // streamed (non-temporal) partial lines reach HBM as separate writes
    // (measured: 1.19x the output bytes).  So a full wave first transposes
    // its 2 KiB through LDS; each store instruction then writes one
    // contiguous KiB: lane i stores bytes [16i, 16i+16) of each half.
    __device__ __forceinline__ static V edge_value(const Epi&, const V x[4], int j) {
        return x[j];
    }
    __device__ __forceinline__ static bool reads_before(const Epi&, int) { return false; }
    template <bool VEC, bool FULL>
    __device__ __forceinline__ static void store(const Params& p, const ChunkPos& q, const Epi&,
                                                 const V x[4], const V[4], lds_float* ostage) {
        static_assert(!kReverse, "the transposed store assumes lane-ascending chunks");
        if constexpr (VEC && FULL) {
            typedef __attribute__((address_space(3))) i64x2 lds_i64x2;
            const int lane = threadIdx.x & (kWave - 1);
            lds_i64x2* s = reinterpret_cast<lds_i64x2*>(ostage);
            i64x2 w0, w1;
            w0.x = x[0]; w0.y = x[1]; w1.x = x[2]; w1.y = x[3];
            s[2 * lane] = w0;
            s[2 * lane + 1] = w1;
            __builtin_amdgcn_wave_barrier();
            const i64x2 r0 = s[lane];
            const i64x2 r1 = s[kWave + lane];
            __builtin_amdgcn_wave_barrier();
            i64x2* g = reinterpret_cast<i64x2*>(p.out + (q.g0 - static_cast<int64_t>(kChunk) * lane));
            __builtin_nontemporal_store(r0, g + lane);
            __builtin_nontemporal_store(r1, g + kWave + lane);
        } else {
            store4<VEC, FULL>(p.out, q, x);
        }
    }
};

}  // namespace rlscan
