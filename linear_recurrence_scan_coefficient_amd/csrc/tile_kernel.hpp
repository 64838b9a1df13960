// tile_kernel.hpp -- the scan kernel template of librlscan (gfx950 only)
// and its launchers; every estimator translation unit instantiates it.
//
// One kernel template serves all seven estimators.  The N*T elements are
// taken as one flattened row-major sequence and cut into tiles of
// 256*W*R consecutive elements (R "rounds"), one workgroup of W wave64s per
// tile.  Row boundaries need no special handling: the step at a row's end
// (reverse estimators) or start (forward ones) has a == 0, which makes the
// plain scan a segmented one.  Within a tile:
//   1. every lane loads R chunks of 4 consecutive elements (16-byte loads;
//      a wave's 64 chunks are 1 KiB of contiguous memory per input);
//   2. builds the chunk's steps (a_t, b_t) in registers (estimators.hpp);
//   3. composes its 4 steps serially, then a wave64 DPP scan combines the 64
//      lane aggregates of each round (scan_core.hpp);
//   4. round totals compose within the wave, wave totals go through LDS;
//   5. the state entering the tile is 0 when the tile holds whole rows
//      (packed mapping), else comes from the decoupled look-back
//      (lookback.hpp);
//   6. each lane replays its 4 steps from its entering state and stores.
// Reverse-time estimators run the same forward scan in "scan order": lane
// chunks are laid out from the tile's high end downwards, so a wave still
// reads contiguous memory with every load instruction.
//
// Sources: "rl-triton: High-Performance Triton GPU Kernels for Reinforcement
// Learning Credit Assignment" (arXiv 2608.17641), abstract -- seven
// estimators as one first-order linear recurrence, one associative operator,
// coefficients built on chip by fused per-estimator kernels; rl-triton
// README, section "Kernels" -- the seven kernels and, in its last column,
// that long sequences need a path beyond one fused block.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "estimators.hpp"
#include "lookback.hpp"
#include "rlscan.h"
#include "scan_core.hpp"

namespace rlscan {

// ------------------------------------------------------------------ kernel
// Phases of one tile, shared by the two kernels below.

// Elements per tile.
template <int R, int W>
constexpr int64_t tile_elems() {
    return static_cast<int64_t>(kWave) * W * kChunk * R;
}

// The packed mapping at a tile capacity of `cap` elements: every tile holds
// whole rows, `span` elements of them, a multiple of 4 (so that no 4-element
// chunk straddles two tiles); `tiles` tiles in all.  One tile holds all rows
// when they fit.  False if no tile can hold a row that way.
inline bool packed_layout(int64_t N, int64_t T, int64_t cap, int64_t& span, int64_t& tiles) {
    if (N * T <= cap) {
        span = cap;
        tiles = 1;
        return true;
    }
    int64_t rows = cap / T;
    while (rows > 0 && (rows * T) % kChunk != 0) --rows;
    if (rows == 0) return false;
    span = rows * T;
    tiles = (N + rows - 1) / rows;
    return true;
}

// Memory position of lane `lane`'s chunk in round r of wave `wave`, and
// whether the chunk lies in the tile's span.  A tile spans tile_span
// elements from mem_tile * tile_span; its chunks run from the span's high
// end downwards for reverse estimators.  When the span falls short of the
// tile's capacity (whole rows that do not fill it), the chunks past it hold
// no elements: they are placed at the span's first element, so that every
// value an estimator preloads for a chunk (bootstrap value, halo, carry)
// stays in bounds, and take the identity step.
// kFixed: the tile spans its whole capacity -- FULL tiles (tile_is_full) and
// every tile of the look-back mapping -- so positions use the compile-time
// tile size.  With a runtime span the compiler kept more of the addresses
// live across the scan: the prefix sum's four-round look-back kernel went
// from 94 to 119 VGPRs and lost a wave per SIMD.
template <class E, int R, int W, bool kFixed>
__device__ __forceinline__ int64_t chunk_base(const Geometry& geo, uint64_t tile, int wave, int r,
                                              int lane, bool& inside) {
    const int64_t mem_tile = E::kReverse ? geo.num_tiles - 1 - static_cast<int64_t>(tile)
                                         : static_cast<int64_t>(tile);
    const int c = (wave * R + r) * kWave + lane;  // chunk index in scan order
    if constexpr (kFixed) {
        constexpr int64_t kTile = tile_elems<R, W>();
        inside = true;
        const int64_t off = E::kReverse ? kTile - static_cast<int64_t>(kChunk) * (c + 1)
                                        : static_cast<int64_t>(kChunk) * c;
        return mem_tile * kTile + off;
    } else {
        const int64_t off = E::kReverse ? geo.tile_span - static_cast<int64_t>(kChunk) * (c + 1)
                                        : static_cast<int64_t>(kChunk) * c;
        inside = off >= 0 && off < geo.tile_span;
        return mem_tile * geo.tile_span + (inside ? off : 0);
    }
}

// Lane `lane`'s chunk in round r of wave `wave`: elements that lie in the
// tile's span and below N*T are valid.
template <class E, int R, int W, bool kFixed>
__device__ __forceinline__ ChunkPos chunk_at(const Geometry& geo, uint64_t tile, int wave, int r,
                                             int lane) {
    bool inside;
    ChunkPos q = chunk_pos(chunk_base<E, R, W, kFixed>(geo, tile, wave, r, lane, inside), geo);
    if (!kFixed && !inside) q.valid = 0;
    return q;
}

// Whether every element of the tile lies in its span and below N*T
// (SPAN: the span may fall short of the tile's capacity).
template <class E, int R, int W, bool SPAN>
__device__ __forceinline__ bool tile_is_full(const Geometry& geo, uint64_t tile) {
    constexpr int64_t kTile = tile_elems<R, W>();
    const int64_t mem_tile = E::kReverse ? geo.num_tiles - 1 - static_cast<int64_t>(tile)
                                         : static_cast<int64_t>(tile);
    return (!SPAN || geo.tile_span == kTile) && (mem_tile + 1) * kTile <= geo.NT;
}

// The dispatcher hands workgroups to the XCDs round-robin: workgroup b runs
// on XCD b % kXcds (each with its own L2).  For launches whose tiles are
// independent (packed, one tile per workgroup) the order below gives each
// XCD runs of `run` consecutive tiles instead of every kXcds-th tile: the
// tiles are cut into groups of kXcds*run, and in each group XCD x takes the
// x-th run.  A cache line shared by two neighbouring tiles (whole rows
// whose span is not a multiple of 128 bytes) is then mostly fetched and
// written back through one L2.  A group cut short by the end of the grid
// keeps tile = b, so the order is a permutation of [0, tiles).
constexpr uint64_t kXcds = 8;

__device__ __forceinline__ uint64_t xcd_tile(uint64_t b, uint64_t tiles, uint64_t run) {
    const uint64_t group = kXcds * run;
    if (b >= tiles / group * group) return b;
    const uint64_t x = b % kXcds, i = b / kXcds;
    return (i / run) * group + x * run + i % run;
}

// 1. loads, all rounds first so every load of the tile is in flight
// (kFixed: the tile spans its whole capacity, see chunk_base)
template <class E, int R, int W, bool VEC, bool FULL, bool CARRY, bool kFixed>
__device__ __forceinline__ void load_tile(const typename E::Params& p, const Geometry& geo,
                                          uint64_t tile, typename E::Chunk (&ch)[R],
                                          ChunkPos (&pos)[R], lds_float* stage) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        pos[r] = chunk_at<E, R, W, kFixed>(geo, tile, wave, r, lane);
        E::template load<VEC, FULL, CARRY>(p, geo, pos[r], ch[r],
                                    stage + (wave * R + r) * E::kStageFloats);
    }
}

// 2. steps in scan order; elements past N*T become the identity
template <class E, int R, bool FULL, bool CARRY>
__device__ __forceinline__ void build_steps(const typename E::Params& p, const Geometry& geo,
                                            const typename E::Chunk (&ch)[R],
                                            const ChunkPos (&pos)[R],
                                            typename E::S (&e)[R][kChunk],
                                            typename E::Epi (&epi)[R]) {
    using S = typename E::S;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        S em[kChunk];
        E::template steps<CARRY>(p, geo, pos[r], ch[r], em, epi[r]);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const S s = (FULL || j < pos[r].valid) ? em[j] : identity_step(S{});
            e[r][E::kReverse ? kChunk - 1 - j : j] = s;
        }
    }
}

// 3. lane aggregates, wave scans and the wave's total
template <int R, class S, class A>
__device__ __forceinline__ A scan_wave(const S (&e)[R][kChunk], A (&incl)[R]) {
    A wtot = identity_step(A{});
#pragma unroll
    for (int r = 0; r < R; ++r) {
        A agg = promote(e[r][0]);
#pragma unroll
        for (int k = 1; k < kChunk; ++k) agg = compose(promote(e[r][k]), agg);
        incl[r] = wave_inclusive_scan(agg);
        wtot = compose(read_lane(incl[r], kWave - 1), wtot);
    }
    return wtot;
}

// 5. state entering the tile, written to *sm_carry by wave 0 (call after the
// wave totals are in sm_wave and the workgroup has synchronised).
// `first_free` (lane 0 of wave 0): the tile's first step in scan order has
// a == 0 and its output does not read the state before it, so no output of
// the tile depends on the entering state and the look-back is skipped.
template <class E, int W, bool LOOKBACK>
__device__ __forceinline__ void tile_carry(const LookbackArgs& lb, uint64_t tile,
                                           const typename AggOf<typename E::S>::type* sm_wave,
                                           bool first_free, typename E::V* sm_carry) {
    using A = typename AggOf<typename E::S>::type;
    using V = typename E::V;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if constexpr (LOOKBACK) {
        if (wave == 0) {
            A agg = identity_step(A{});
#pragma unroll
            for (int w = 0; w < W; ++w) agg = compose(sm_wave[w], agg);
            TileStatus* st = status_of<A>(lb.status, static_cast<int64_t>(tile));
            const bool known = tile == 0 || cuts_chain(agg);
            if (lane == 0) {
                if (known)
                    publish_inclusive(st, apply(agg, V(0)), lb.tag);
                else
                    publish_aggregate(st, agg, lb.tag);
            }
            const bool first_cuts = __ballot(lane == 0 && first_free) != 0;
            V carry = V(0);
            if (tile > 0 && !first_cuts) carry = look_back<A, V>(lb, tile, lane);
            if (lane == 0) {
                if (!known) publish_inclusive(st, apply(agg, carry), lb.tag);
                *sm_carry = carry;
            }
        }
    } else {
        if (threadIdx.x == 0) *sm_carry = V(0);
    }
}

// 6. replay each lane's steps from its entering state and store
template <class E, int R, int W, bool VEC, bool FULL, bool CARRY, bool kFixed, class A>
__device__ __forceinline__ void replay_store(const typename E::Params& p, const Geometry& geo,
                                             uint64_t tile,
                                             const typename E::S (&e)[R][kChunk],
                                             const typename E::Epi (&epi)[R],
                                             const A (&incl)[R], A wpre,
                                             typename E::V carry, lds_float* ostage) {
    using V = typename E::V;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    V state = apply(wpre, carry);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const V after_lane = apply(incl[r], state);
        V x = lane_before(after_lane, lane, state);
        state = read_lane(after_lane, kWave - 1);
        V out[kChunk], before[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const int j = E::kReverse ? kChunk - 1 - k : k;
            before[j] = x;
            x = apply(e[r][k], x);
            out[j] = x;
        }
        ChunkPos q;
        bool inside;
        q.g0 = chunk_base<E, R, W, kFixed>(geo, tile, wave, r, lane, inside);
        const int64_t rem = geo.NT - q.g0;
        // (the compile-time kFixed test keeps the compiler from carrying
        // `inside` where it is always true: 8 more VGPRs in the prefix sum's
        // four-round look-back kernel otherwise)
        const bool outside = !kFixed && !inside;
        q.valid = (outside || rem <= 0) ? 0 : (rem >= kChunk ? kChunk : static_cast<int>(rem));
        E::template store<VEC, FULL>(p, q, epi[r], out, before,
                                     ostage + wave * E::kOutStageFloats);
        if (CARRY && p.carry_out != nullptr) {
            // the output at the row edge the next call continues from:
            // t = 0 (reverse estimators) or t = T-1 (forward ones)
            const ChunkPos qp = chunk_pos(q.g0, geo);
            int64_t n = qp.n0, t = qp.t0;
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (j < q.valid && t == (E::kReverse ? 0 : geo.T - 1))
                    p.carry_out[n] = E::edge_value(epi[r], out, j);
                next_position(n, t, geo.T);
            }
        }
    }
}

// SPAN: the tile's span may fall short of its capacity (a packed mapping of
// whole rows that do not fill the tile); kernels built without it compute
// chunk positions from the compile-time tile size throughout.
template <class E, int R, int W, bool LOOKBACK, bool VEC, bool FULL, bool CARRY, bool SPAN>
__device__ __forceinline__ void scan_tile(const typename E::Params& p, const Geometry& geo,
                                          const LookbackArgs& lb, uint64_t tile,
                                          typename AggOf<typename E::S>::type* sm_wave,
                                          typename E::V* sm_carry, lds_float* stage,
                                          lds_float* ostage) {
    using S = typename E::S;
    using A = typename AggOf<S>::type;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    constexpr bool kFixed = FULL || !SPAN;
    typename E::Chunk ch[R];
    ChunkPos pos[R];
    load_tile<E, R, W, VEC, FULL, CARRY, kFixed>(p, geo, tile, ch, pos, stage);
    S e[R][kChunk];
    typename E::Epi epi[R];
    build_steps<E, R, FULL, CARRY>(p, geo, ch, pos, e, epi);
    A incl[R];
    const A wtot = scan_wave<R>(e, incl);
    if (lane == 0) sm_wave[wave] = wtot;
    __syncthreads();
    A wpre = identity_step(A{});
#pragma unroll
    for (int w = 0; w < W; ++w)
        if (w < wave) wpre = compose(sm_wave[w], wpre);
    // lane 0 of wave 0 holds the tile's first step in scan order: element
    // kChunk-1 of its first chunk for reverse estimators, element 0 otherwise
    const bool first_free =
        cuts_chain(e[0][0]) && !E::reads_before(epi[0], E::kReverse ? kChunk - 1 : 0);
    tile_carry<E, W, LOOKBACK>(lb, tile, sm_wave, first_free, sm_carry);
    __syncthreads();
    replay_store<E, R, W, VEC, FULL, CARRY, kFixed>(p, geo, tile, e, epi, incl, wpre, *sm_carry,
                                                     ostage);
}

// One tile per workgroup (or, grid-capped, a loop over tiles).  SPAN (packed
// only): tiles of whole rows that may fall short of the tile's capacity.
template <class E, int R, int W, bool LOOKBACK, bool VEC, bool CARRY, bool SPAN>
__global__ __launch_bounds__(kWave * W) void scan_kernel(const typename E::Params p,
                                                        const Geometry geo,
                                                        const LookbackArgs lb) {
    static_assert(!(SPAN && LOOKBACK), "look-back tiles span their whole capacity");
    using A = typename AggOf<typename E::S>::type;
    using V = typename E::V;
    __shared__ A sm_wave[W];
    __shared__ V sm_carry;
    __shared__ uint64_t sm_tile;
    // staging area of the estimators that stage loads through LDS
    constexpr int kStage = E::kStageFloats > 0 ? W * R * E::kStageFloats : 1;
    __shared__ __attribute__((aligned(16))) float sm_stage[kStage];
    lds_float* stage = (lds_float*)sm_stage;
    // per-wave output staging of the estimators that transpose their stores
    constexpr int kOutStage = E::kOutStageFloats > 0 ? W * E::kOutStageFloats : 1;
    __shared__ __attribute__((aligned(16))) float sm_out[kOutStage];
    lds_float* ostage = (lds_float*)sm_out;
    const bool one_tile_per_group = geo.grid >= geo.num_tiles;
    uint64_t tile = blockIdx.x;
    if (!LOOKBACK && one_tile_per_group && geo.xcd_run > 0)
        tile = xcd_tile(blockIdx.x, static_cast<uint64_t>(geo.num_tiles),
                        static_cast<uint64_t>(geo.xcd_run));
    for (;;) {
        if constexpr (LOOKBACK) {
            if (lb.use_tickets) {
                if (threadIdx.x == 0) sm_tile = take_ticket(lb);
                __syncthreads();
                tile = sm_tile;
            }
        }
        if (tile >= static_cast<uint64_t>(geo.num_tiles)) break;
        // only the tile holding the end of the data needs bounds checks
        if (tile_is_full<E, R, W, SPAN>(geo, tile))
            scan_tile<E, R, W, LOOKBACK, VEC, true, CARRY, SPAN>(p, geo, lb, tile, sm_wave,
                                                                 &sm_carry, stage, ostage);
        else
            scan_tile<E, R, W, LOOKBACK, VEC, false, CARRY, SPAN>(p, geo, lb, tile, sm_wave,
                                                                  &sm_carry, stage, ostage);
        if (one_tile_per_group) break;
        if (!LOOKBACK || !lb.use_tickets) tile += gridDim.x;
        __syncthreads();  // LDS is reused by the next tile
    }
}


}  // namespace rlscan
