// rlscan.hip -- scan kernels and the C ABI of librlscan (gfx950 only).
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
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <utility>

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

// Memory position of lane `lane`'s chunk in round r of wave `wave`.
template <class E, int R, int W>
__device__ __forceinline__ int64_t chunk_base(const Geometry& geo, uint64_t tile, int wave, int r,
                                              int lane) {
    constexpr int64_t kTile = tile_elems<R, W>();
    const int64_t mem_tile = E::kReverse ? geo.num_tiles - 1 - static_cast<int64_t>(tile)
                                         : static_cast<int64_t>(tile);
    const int c = (wave * R + r) * kWave + lane;  // chunk index in scan order
    const int64_t off = E::kReverse ? kTile - static_cast<int64_t>(kChunk) * (c + 1)
                                    : static_cast<int64_t>(kChunk) * c;
    return mem_tile * kTile + off;
}

// Whether every element of the tile lies below N*T.
template <class E, int R, int W>
__device__ __forceinline__ bool tile_is_full(const Geometry& geo, uint64_t tile) {
    constexpr int64_t kTile = tile_elems<R, W>();
    const int64_t mem_tile = E::kReverse ? geo.num_tiles - 1 - static_cast<int64_t>(tile)
                                         : static_cast<int64_t>(tile);
    return (mem_tile + 1) * kTile <= geo.NT;
}

// 1. loads, all rounds first so every load of the tile is in flight
template <class E, int R, int W, bool VEC, bool FULL, bool CARRY>
__device__ __forceinline__ void load_tile(const typename E::Params& p, const Geometry& geo,
                                          uint64_t tile, typename E::Chunk (&ch)[R],
                                          ChunkPos (&pos)[R], lds_float* stage) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        pos[r] = chunk_pos(chunk_base<E, R, W>(geo, tile, wave, r, lane), geo);
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
// wave totals are in sm_wave and the workgroup has synchronised)
template <class E, int W, bool LOOKBACK>
__device__ __forceinline__ void tile_carry(const LookbackArgs& lb, uint64_t tile,
                                           const typename AggOf<typename E::S>::type* sm_wave,
                                           typename E::S first_step,
                                           typename E::V* sm_carry) {
    using A = typename AggOf<typename E::S>::type;
    using V = typename E::V;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if constexpr (LOOKBACK) {
        if (wave == 0) {
            A agg = identity_step(A{});
#pragma unroll
            for (int w = 0; w < W; ++w) agg = compose(sm_wave[w], agg);
            TileStatus* st = lb.status + tile;
            const bool known = tile == 0 || cuts_chain(agg);
            if (lane == 0) {
                if (known)
                    publish_inclusive(st, apply(agg, V(0)), lb.tag);
                else
                    publish_aggregate(st, agg, lb.tag);
            }
            // lane 0 of wave 0 holds the tile's first step in scan order
            const bool first_cuts = __ballot(lane == 0 && cuts_chain(first_step)) != 0;
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
template <class E, int R, int W, bool VEC, bool FULL, bool CARRY, class A>
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
        q.g0 = chunk_base<E, R, W>(geo, tile, wave, r, lane);
        const int64_t rem = geo.NT - q.g0;
        q.valid = rem <= 0 ? 0 : (rem >= kChunk ? kChunk : static_cast<int>(rem));
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

template <class E, int R, int W, bool LOOKBACK, bool VEC, bool FULL, bool CARRY>
__device__ __forceinline__ void scan_tile(const typename E::Params& p, const Geometry& geo,
                                          const LookbackArgs& lb, uint64_t tile,
                                          typename AggOf<typename E::S>::type* sm_wave,
                                          typename E::V* sm_carry, lds_float* stage,
                                          lds_float* ostage) {
    using S = typename E::S;
    using A = typename AggOf<S>::type;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    typename E::Chunk ch[R];
    ChunkPos pos[R];
    load_tile<E, R, W, VEC, FULL, CARRY>(p, geo, tile, ch, pos, stage);
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
    tile_carry<E, W, LOOKBACK>(lb, tile, sm_wave, e[0][0], sm_carry);
    __syncthreads();
    replay_store<E, R, W, VEC, FULL, CARRY>(p, geo, tile, e, epi, incl, wpre, *sm_carry,
                                             ostage);
}

// One tile per workgroup (or, grid-capped, a loop over tiles).
template <class E, int R, int W, bool LOOKBACK, bool VEC, bool CARRY>
__global__ __launch_bounds__(kWave * W) void scan_kernel(const typename E::Params p,
                                                        const Geometry geo,
                                                        const LookbackArgs lb) {
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
        if (tile_is_full<E, R, W>(geo, tile))
            scan_tile<E, R, W, LOOKBACK, VEC, true, CARRY>(p, geo, lb, tile, sm_wave, &sm_carry,
                                                           stage, ostage);
        else
            scan_tile<E, R, W, LOOKBACK, VEC, false, CARRY>(p, geo, lb, tile, sm_wave, &sm_carry,
                                                            stage, ostage);
        if (one_tile_per_group) break;
        if (!LOOKBACK || !lb.use_tickets) tile += gridDim.x;
        __syncthreads();  // LDS is reused by the next tile
    }
}

// An empty kernel: the launch floor that a scan launch of the same grid
// cannot go below.
constexpr int kFloorThreads = 256;
__global__ __launch_bounds__(kFloorThreads) void empty_kernel() {}

// A plain streaming copy: the bandwidth a kernel that reads and writes the
// same bytes, in the same 16-byte non-temporal accesses, can reach.  Each
// thread moves kCopyUnroll 16-byte words, a workgroup a contiguous span.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const f32x4* __restrict__ src,
                                                            f32x4* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
    f32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

// ------------------------------------------------------------------ host
namespace {

constexpr int64_t kMaxElements = int64_t(1) << 48;
constexpr int64_t kMaxGrid = (int64_t(1) << 23) - 1;  // grid * 512 threads < 2^32

struct LaunchOverride {
    std::atomic<int> mapping{RLSCAN_MAP_AUTO};
    std::atomic<int> rounds{0};
    std::atomic<int> waves{0};
    std::atomic<int64_t> grid_cap{0};
    std::atomic<int> flags{0};  // RLSCAN_FLAG_* bits
};
LaunchOverride g_override;

struct Scratch {
    std::mutex m;
    TileStatus* status = nullptr;
    unsigned long long* counter = nullptr;
    int64_t capacity = 0;       // tiles
    uint64_t next_ticket = 0;   // counter value at the start of the next call
    uint64_t epoch = 0;         // tag of the last call (32-bit, 0 = none)
    bool broken = false;        // a launch failed: counter position unknown
};

std::mutex g_scratch_mutex;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<Scratch>> g_scratch;

Scratch* scratch_for(int device, hipStream_t stream) {
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    auto& slot = g_scratch[{device, reinterpret_cast<uintptr_t>(stream)}];
    if (!slot) slot.reset(new Scratch());
    return slot.get();
}

// Called with sc->m held.  Makes room for `tiles` status entries.
int ensure_capacity(Scratch* sc, hipStream_t stream, int64_t tiles) {
    if (sc->capacity >= tiles && !sc->broken) return RLSCAN_OK;
    int64_t cap = 1024;
    while (cap < tiles) cap *= 2;
    // earlier work on this stream may still read the old buffers
    if (sc->status != nullptr && hipStreamSynchronize(stream) != hipSuccess) return RLSCAN_ERR_HIP;
    if (sc->status != nullptr) (void)hipFree(sc->status);
    if (sc->counter != nullptr) (void)hipFree(sc->counter);
    sc->status = nullptr;
    sc->counter = nullptr;
    sc->capacity = 0;
    void* st = nullptr;
    void* ctr = nullptr;
    if (hipMalloc(&st, sizeof(TileStatus) * cap) != hipSuccess) return RLSCAN_ERR_ALLOC;
    if (hipMalloc(&ctr, 256) != hipSuccess) {
        (void)hipFree(st);
        return RLSCAN_ERR_ALLOC;
    }
    // ordered before the first kernel that uses the buffers (same stream)
    if (hipMemsetAsync(st, 0, sizeof(TileStatus) * cap, stream) != hipSuccess ||
        hipMemsetAsync(ctr, 0, 256, stream) != hipSuccess) {
        (void)hipFree(st);
        (void)hipFree(ctr);
        return RLSCAN_ERR_HIP;
    }
    sc->status = static_cast<TileStatus*>(st);
    sc->counter = static_cast<unsigned long long*>(ctr);
    sc->capacity = cap;
    sc->next_ticket = 0;
    sc->epoch = 0;
    sc->broken = false;
    return RLSCAN_OK;
}

struct Plan {
    int mapping;
    int rounds;
    int waves;
    int64_t tile_elems, tiles, grid;
};

int auto_rounds(int est, int64_t NT) {
    if (est == RLSCAN_EST_RETRACE) return 1;
    if (NT <= (int64_t(1) << 20)) return 1;
    if (NT <= (int64_t(1) << 22)) return 2;
    return 4;
}

// Eight waves per workgroup double the tile, which halves the look-back
// hops per element but also the workgroups that fit on a CU.  That pays for
// the estimators whose four-round kernels need few registers (discounted
// returns, eligibility traces, prefix sum: at most ~96 VGPRs, five waves per
// SIMD); GAE, TD(lambda) and V-trace hold more per lane and run four waves.
int auto_waves(int est, int rounds) {
    if (rounds != 4) return 4;
    return (est == RLSCAN_EST_DISCOUNTED || est == RLSCAN_EST_ELIGIBILITY ||
            est == RLSCAN_EST_PREFIX_SUM) ? 8 : 4;
}

// `vec`: every pointer is 16-byte aligned.  Multi-round and eight-wave
// kernels exist only for the vectorised path, Retrace always runs one round
// of four waves, and calls with carry arguments (`carry`) four waves.
Plan make_plan(int est, int64_t N, int64_t T, bool vec, bool carry = false) {
    const int64_t NT = N * T;
    Plan pl;
    const int ro = g_override.rounds.load();
    pl.rounds = ro > 0 ? ro : auto_rounds(est, NT);
    if (!vec || est == RLSCAN_EST_RETRACE) pl.rounds = 1;
    const int wo = g_override.waves.load();
    pl.waves = wo > 0 ? wo : auto_waves(est, pl.rounds);
    if (!vec || carry || est == RLSCAN_EST_RETRACE) pl.waves = 4;
    pl.tile_elems = int64_t(kWave) * pl.waves * kChunk * pl.rounds;
    pl.tiles = (NT + pl.tile_elems - 1) / pl.tile_elems;
    const bool packed_ok = pl.tiles <= 1 || pl.tile_elems % T == 0;
    const int mo = g_override.mapping.load();
    pl.mapping = (packed_ok && mo != RLSCAN_MAP_LOOKBACK) ? RLSCAN_MAP_PACKED : RLSCAN_MAP_LOOKBACK;
    const int64_t cap = g_override.grid_cap.load();
    int64_t grid = pl.tiles;
    if (cap > 0 && grid > cap) grid = cap;
    if (grid > kMaxGrid) grid = kMaxGrid;
    pl.grid = grid;
    return pl;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool unit_interval(float x) { return x >= 0.0f && x <= 1.0f; }  // false for NaN
bool positive_clip(float x) { return x > 0.0f; }                 // +inf allowed, NaN not

int check_shape(int64_t N, int64_t T, int64_t A = 1) {
    if (N < 0 || T < 0 || A < 1) return RLSCAN_ERR_SHAPE;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (N > kMaxElements / T) return RLSCAN_ERR_SHAPE;
    if (N * T > kMaxElements / A) return RLSCAN_ERR_SHAPE;
    return RLSCAN_OK;
}

// Outputs must not equal an input or each other; NULL (an optional output
// not asked for) is skipped.
int check_alias(std::initializer_list<const void*> outs, std::initializer_list<const void*> ins) {
    for (const void* o : outs) {
        if (o == nullptr) continue;
        for (const void* i : ins)
            if (i != nullptr && i == o) return RLSCAN_ERR_ALIAS;
        int same = 0;
        for (const void* o2 : outs) same += (o2 == o);
        if (same > 1) return RLSCAN_ERR_ALIAS;
    }
    return RLSCAN_OK;
}

template <class E, int R, int W, bool VEC, bool CARRY>
hipError_t launch_r(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                    const Plan& pl, hipStream_t stream) {
    const bool lookback = pl.mapping == RLSCAN_MAP_LOOKBACK;
    const dim3 grid(static_cast<unsigned>(geo.grid)), block(kWave * W);
    if (lookback)
        hipLaunchKernelGGL((scan_kernel<E, R, W, true, VEC, CARRY>), grid, block, 0, stream, p,
                           geo, lb);
    else
        hipLaunchKernelGGL((scan_kernel<E, R, W, false, VEC, CARRY>), grid, block, 0, stream, p,
                           geo, lb);
    return hipGetLastError();
}

template <class E, int W, bool CARRY>
hipError_t launch_w(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                    const Plan& pl, hipStream_t stream) {
    switch (pl.rounds) {
        case 1: return launch_r<E, 1, W, true, CARRY>(p, geo, lb, pl, stream);
        case 2: return launch_r<E, 2, W, true, CARRY>(p, geo, lb, pl, stream);
        default: return launch_r<E, 4, W, true, CARRY>(p, geo, lb, pl, stream);
    }
}

// Kernels built for the carry arguments exist with four waves only (the
// plan forces it); all others come with four or eight.
template <class E>
hipError_t launch_kernel(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                         const Plan& pl, bool vec, bool carry, hipStream_t stream) {
    if (carry) {
        if (!vec) return launch_r<E, 1, 4, false, true>(p, geo, lb, pl, stream);
        return launch_w<E, 4, true>(p, geo, lb, pl, stream);
    }
    if (!vec) return launch_r<E, 1, 4, false, false>(p, geo, lb, pl, stream);
    return pl.waves == 8 ? launch_w<E, 8, false>(p, geo, lb, pl, stream)
                         : launch_w<E, 4, false>(p, geo, lb, pl, stream);
}

// Retrace keeps 2*4*A action values per round in LDS or registers: one
// round of four waves only.
template <class E>
hipError_t launch_kernel_r1(const typename E::Params& p, const Geometry& geo,
                            const LookbackArgs& lb, const Plan& pl, bool vec, bool carry,
                            hipStream_t stream) {
    if (carry)
        return vec ? launch_r<E, 1, 4, true, true>(p, geo, lb, pl, stream)
                   : launch_r<E, 1, 4, false, true>(p, geo, lb, pl, stream);
    return vec ? launch_r<E, 1, 4, true, false>(p, geo, lb, pl, stream)
               : launch_r<E, 1, 4, false, false>(p, geo, lb, pl, stream);
}

// Plans, takes the look-back scratch if needed, and launches through `fn`.
template <class Fn>
int run(int est, int64_t N, int64_t T, bool vec, bool carry, hipStream_t stream, Fn&& fn) {
    const Plan pl = make_plan(est, N, T, vec, carry);
    if (pl.rounds != 1 && pl.rounds != 2 && pl.rounds != 4) return RLSCAN_ERR_PARAM;
    if (pl.waves != 4 && pl.waves != 8) return RLSCAN_ERR_PARAM;
    Geometry geo;
    geo.N = N;
    geo.T = T;
    geo.NT = N * T;
    geo.num_tiles = pl.tiles;
    geo.grid = pl.grid;
    geo.inv_T = 1.0 / static_cast<double>(T);
    LookbackArgs lb{};
    if (pl.mapping == RLSCAN_MAP_PACKED) {
        return fn(geo, lb, pl) == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
    }
    // a captured look-back launch would replay with a stale ticket base
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) return RLSCAN_ERR_HIP;
    if (capture != hipStreamCaptureStatusNone) return RLSCAN_ERR_CAPTURE;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return RLSCAN_ERR_HIP;
    Scratch* sc = scratch_for(device, stream);
    std::lock_guard<std::mutex> g(sc->m);
    const int rc = ensure_capacity(sc, stream, pl.tiles);
    if (rc != RLSCAN_OK) return rc;
    // tile = blockIdx needs every tile to have its own workgroup
    const bool tickets = pl.grid < pl.tiles || (g_override.flags.load() & RLSCAN_FLAG_TICKETS);
    lb.use_tickets = tickets ? 1u : 0u;
    lb.status = sc->status;
    lb.ticket_counter = sc->counter;
    lb.timeouts = reinterpret_cast<unsigned int*>(sc->counter + 1);
    lb.ticket_base = sc->next_ticket;
    if (sc->epoch == 0xffffffffull) {
        // the 32-bit call tags are about to repeat: clear the status words
        if (hipMemsetAsync(sc->status, 0, sizeof(TileStatus) * sc->capacity, stream) != hipSuccess)
            return RLSCAN_ERR_HIP;
        sc->epoch = 0;
    }
    lb.tag = static_cast<uint32_t>(++sc->epoch);
    if (fn(geo, lb, pl) != hipSuccess) {
        sc->broken = true;
        return RLSCAN_ERR_HIP;
    }
    // every workgroup takes one ticket per tile it runs plus, when looping,
    // one final ticket that finds no tile
    if (tickets)
        sc->next_ticket += static_cast<uint64_t>(pl.tiles) +
                           (pl.grid >= pl.tiles ? 0u : static_cast<uint64_t>(pl.grid));
    return RLSCAN_OK;
}

bool all_aligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return false;
    return true;
}

}  // namespace
}  // namespace rlscan

using namespace rlscan;

// ------------------------------------------------------------------ C ABI
extern "C" {

int rlscan_gae_carry(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* advantages,
                     float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                     hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !terminated || !advantages) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({advantages, carry_out}, {rewards, values, bootstrap_value, terminated,
                                               truncated, bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const GaeParams p{rewards,  values,     bootstrap_value, terminated, truncated,
                      bootstrap_values, carry_in, advantages, carry_out, gamma,
                      gamma * lambda};
    const bool vec = all_aligned({rewards, values, terminated, truncated, bootstrap_values,
                                  advantages});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_GAE, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated ? launch_kernel<Gae<true>>(p, g, lb, pl, vec, carry, stream)
                                    : launch_kernel<Gae<false>>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_gae(const float* rewards, const float* values, const float* bootstrap_value,
               const float* terminated, const float* truncated, const float* bootstrap_values,
               float* advantages, int64_t N, int64_t T, float gamma, float lambda,
               hipStream_t stream) {
    return rlscan_gae_carry(rewards, values, bootstrap_value, terminated, truncated,
                            bootstrap_values, nullptr, advantages, nullptr, N, T, gamma, lambda,
                            stream);
}

int rlscan_lambda_returns_carry(const float* rewards, const float* values,
                                const float* bootstrap_value, const float* terminated,
                                const float* truncated, const float* bootstrap_values,
                                const float* carry_in, float* returns, float* carry_out,
                                int64_t N, int64_t T, float gamma, float lambda,
                                hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !terminated || !returns) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({returns, carry_out}, {rewards, values, bootstrap_value, terminated,
                                            truncated, bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const LambdaReturnsParams p{rewards,   values,   bootstrap_value, terminated,
                                truncated, bootstrap_values, carry_in, returns,
                                carry_out, gamma,    gamma * lambda,
                                gamma * (1.0f - lambda)};
    const bool vec = all_aligned({rewards, values, terminated, truncated, bootstrap_values,
                                  returns});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_LAMBDA_RETURNS, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated
                              ? launch_kernel<LambdaReturns<true>>(p, g, lb, pl, vec, carry, stream)
                              : launch_kernel<LambdaReturns<false>>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_lambda_returns(const float* rewards, const float* values, const float* bootstrap_value,
                          const float* terminated, const float* truncated,
                          const float* bootstrap_values, float* returns, int64_t N, int64_t T,
                          float gamma, float lambda, hipStream_t stream) {
    return rlscan_lambda_returns_carry(rewards, values, bootstrap_value, terminated, truncated,
                                       bootstrap_values, nullptr, returns, nullptr, N, T, gamma,
                                       lambda, stream);
}

int rlscan_discounted_returns_carry(const float* rewards, const float* bootstrap_value,
                                    const float* terminated, const float* truncated,
                                    const float* bootstrap_values, const float* carry_in,
                                    float* returns, float* carry_out, int64_t N, int64_t T,
                                    float gamma, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !terminated || !returns) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({returns, carry_out}, {rewards, bootstrap_value, terminated, truncated,
                                            bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const DiscountedParams p{rewards, bootstrap_value, terminated, truncated, bootstrap_values,
                             carry_in, returns, carry_out, gamma};
    const bool vec = all_aligned({rewards, terminated, truncated, bootstrap_values, returns});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_DISCOUNTED, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated
                              ? launch_kernel<Discounted<true>>(p, g, lb, pl, vec, carry, stream)
                              : launch_kernel<Discounted<false>>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_discounted_returns(const float* rewards, const float* bootstrap_value,
                              const float* terminated, const float* truncated,
                              const float* bootstrap_values, float* returns, int64_t N,
                              int64_t T, float gamma, hipStream_t stream) {
    return rlscan_discounted_returns_carry(rewards, bootstrap_value, terminated, truncated,
                                           bootstrap_values, nullptr, returns, nullptr, N, T,
                                           gamma, stream);
}

int rlscan_vtrace_carry(const float* rewards, const float* values, const float* bootstrap_value,
                        const float* log_rhos, const float* terminated, const float* truncated,
                        const float* bootstrap_values, const float* carry_in, float* vs,
                        float* pg_advantages, float* carry_out, int64_t N, int64_t T,
                        float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !positive_clip(rho_bar) || !positive_clip(c_bar))
        return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !log_rhos || !terminated || !vs || !pg_advantages)
        return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({vs, pg_advantages, carry_out},
                     {rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                      bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const VtraceParams p{rewards,   values,        bootstrap_value, log_rhos,
                         terminated, truncated,    bootstrap_values, carry_in,
                         vs,        pg_advantages, carry_out,        gamma,
                         rho_bar,   c_bar};
    const bool vec = all_aligned({rewards, values, log_rhos, terminated, truncated,
                                  bootstrap_values, vs, pg_advantages});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_VTRACE, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated ? launch_kernel<Vtrace<true>>(p, g, lb, pl, vec, carry, stream)
                                    : launch_kernel<Vtrace<false>>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_vtrace(const float* rewards, const float* values, const float* bootstrap_value,
                  const float* log_rhos, const float* terminated, const float* truncated,
                  const float* bootstrap_values, float* vs, float* pg_advantages, int64_t N,
                  int64_t T, float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    return rlscan_vtrace_carry(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                               bootstrap_values, nullptr, vs, pg_advantages, nullptr, N, T,
                               gamma, rho_bar, c_bar, stream);
}

int rlscan_retrace_carry(const float* rewards, const float* next_q_values_all,
                         const float* next_target_probs, const int32_t* actions,
                         const float* behaviour_probs, const float* terminated,
                         const float* truncated, const float* carry_in,
                         const int32_t* next_actions, const float* next_behaviour_probs,
                         float* targets, float* carry_out, int64_t N, int64_t T, int64_t A,
                         float gamma, float lambda, hipStream_t stream) {
    int rc = check_shape(N, T, A);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !next_q_values_all || !next_target_probs || !actions || !behaviour_probs ||
        !terminated || !truncated || !targets)
        return RLSCAN_ERR_NULL;
    if (carry_in && (!next_actions || !next_behaviour_probs)) return RLSCAN_ERR_NULL;
    rc = check_alias({targets, carry_out},
                     {rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                      terminated, truncated, carry_in, next_actions, next_behaviour_probs});
    if (rc != RLSCAN_OK) return rc;
    const bool vec = all_aligned({rewards, next_q_values_all, next_target_probs, actions,
                                  behaviour_probs, terminated, truncated, targets});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    auto go = [&](auto tag) {
        using E = decltype(tag);
        typename E::Params p{rewards,  next_q_values_all, next_target_probs, actions,
                             behaviour_probs, terminated, truncated, targets,
                             A,        gamma,             lambda,            carry_in,
                             next_actions, next_behaviour_probs, carry_out};
        return run(RLSCAN_EST_RETRACE, N, T, vec, carry, stream,
                   [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                       return launch_kernel_r1<E>(p, g, lb, pl, vec, carry, stream);
                   });
    };
    switch (vec ? A : 0) {
        case 4: return go(Retrace<4>{});
        case 6: return go(Retrace<6>{});
        case 8: return go(Retrace<8>{});
        case 18: return go(Retrace<18>{});
        default: return go(Retrace<0>{});
    }
}

int rlscan_retrace(const float* rewards, const float* next_q_values_all,
                   const float* next_target_probs, const int32_t* actions,
                   const float* behaviour_probs, const float* terminated, const float* truncated,
                   float* targets, int64_t N, int64_t T, int64_t A, float gamma, float lambda,
                   hipStream_t stream) {
    return rlscan_retrace_carry(rewards, next_q_values_all, next_target_probs, actions,
                                behaviour_probs, terminated, truncated, nullptr, nullptr, nullptr,
                                targets, nullptr, N, T, A, gamma, lambda, stream);
}

int rlscan_eligibility_traces_carry(const float* x, const float* dones, const float* carry_in,
                                    float* traces, float* carry_out, int64_t N, int64_t T,
                                    float gamma, float lambda, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!x || !dones || !traces) return RLSCAN_ERR_NULL;
    rc = check_alias({traces, carry_out}, {x, dones, carry_in});
    if (rc != RLSCAN_OK) return rc;
    Eligibility::Params p{x, dones, traces, gamma * lambda, carry_in, carry_out};
    const bool vec = all_aligned({x, dones, traces});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_ELIGIBILITY, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return launch_kernel<Eligibility>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_eligibility_traces(const float* x, const float* dones, float* traces, int64_t N,
                              int64_t T, float gamma, float lambda, hipStream_t stream) {
    return rlscan_eligibility_traces_carry(x, dones, nullptr, traces, nullptr, N, T, gamma,
                                           lambda, stream);
}

int rlscan_episodic_prefix_sum_carry(const int32_t* x, const float* dones,
                                     const int64_t* carry_in, int64_t* out, int64_t* carry_out,
                                     int64_t N, int64_t T, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!x || !dones || !out) return RLSCAN_ERR_NULL;
    rc = check_alias({out, carry_out}, {x, dones, carry_in});
    if (rc != RLSCAN_OK) return rc;
    PrefixSum::Params p{x, dones, out, carry_in, carry_out};
    const bool vec = all_aligned({x, dones, out});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_PREFIX_SUM, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return launch_kernel<PrefixSum>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_episodic_prefix_sum(const int32_t* x, const float* dones, int64_t* out, int64_t N,
                               int64_t T, hipStream_t stream) {
    return rlscan_episodic_prefix_sum_carry(x, dones, nullptr, out, nullptr, N, T, stream);
}

const char* rlscan_status_string(int status) {
    switch (status) {
        case RLSCAN_OK: return "ok";
        case RLSCAN_ERR_NULL: return "a required pointer is NULL";
        case RLSCAN_ERR_SHAPE: return "invalid shape (negative size, A < 1, or more than 2^48 elements)";
        case RLSCAN_ERR_PARAM: return "parameter out of range";
        case RLSCAN_ERR_ALIAS: return "an output aliases an input or the other output";
        case RLSCAN_ERR_HIP: return "HIP runtime call or kernel launch failed";
        case RLSCAN_ERR_ALLOC: return "could not allocate the look-back scratch";
        case RLSCAN_ERR_CAPTURE:
            return "this shape needs the look-back mapping, which cannot be captured into a graph";
        default: return "unknown rlscan status";
    }
}

const char* rlscan_version(void) { return "rlscan 0.1.0 gfx950"; }

int rlscan_release_scratch(void) {
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    int rc = RLSCAN_OK;
    for (auto& kv : g_scratch) {
        Scratch* sc = kv.second.get();
        std::lock_guard<std::mutex> gs(sc->m);
        if (sc->status == nullptr && sc->counter == nullptr) continue;
        if (hipSetDevice(kv.first.first) != hipSuccess) {
            rc = RLSCAN_ERR_HIP;
            continue;
        }
        if (sc->status) (void)hipFree(sc->status);
        if (sc->counter) (void)hipFree(sc->counter);
        sc->status = nullptr;
        sc->counter = nullptr;
        sc->capacity = 0;
        sc->next_ticket = 0;
        sc->epoch = 0;
    }
    g_scratch.clear();
    if (have_prev) (void)hipSetDevice(prev);
    return rc;
}

int rlscan_plan(int estimator, int64_t N, int64_t T, int64_t A, rlscan_plan_info* info) {
    if (info == nullptr) return RLSCAN_ERR_NULL;
    if (estimator < RLSCAN_EST_GAE || estimator > RLSCAN_EST_PREFIX_SUM) return RLSCAN_ERR_PARAM;
    const int rc = check_shape(N, T, A);
    if (rc != RLSCAN_OK) return rc;
    std::memset(info, 0, sizeof(*info));
    info->threads = kWave * 4;
    if (N == 0 || T == 0) return RLSCAN_OK;
    const Plan pl = make_plan(estimator, N, T, true);
    info->threads = kWave * pl.waves;
    info->mapping = pl.mapping;
    info->rounds = pl.rounds;
    info->tile_elems = pl.tile_elems;
    info->tiles = pl.tiles;
    info->grid = pl.grid;
    return RLSCAN_OK;
}

int rlscan_launch_floor(int64_t grid, hipStream_t stream) {
    if (grid < 1 || grid > kMaxGrid) return RLSCAN_ERR_SHAPE;
    hipLaunchKernelGGL(empty_kernel, dim3(static_cast<unsigned>(grid)), dim3(kFloorThreads), 0,
                       stream);
    return hipGetLastError() == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
}

int rlscan_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
    if (bytes < 0 || (bytes & 15) != 0) return RLSCAN_ERR_SHAPE;
    if (bytes == 0) return RLSCAN_OK;
    if (dst == nullptr || src == nullptr) return RLSCAN_ERR_NULL;
    if (!aligned16(dst) || !aligned16(src)) return RLSCAN_ERR_PARAM;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (d < s + static_cast<uintptr_t>(bytes) && s < d + static_cast<uintptr_t>(bytes))
        return RLSCAN_ERR_ALIAS;
    const int64_t n = bytes / 16;
    const int64_t per_group = int64_t(kCopyThreads) * kCopyUnroll;
    const int64_t grid = (n + per_group - 1) / per_group;
    if (grid > kMaxGrid) return RLSCAN_ERR_SHAPE;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), 0,
                       stream, static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
}

int rlscan_lookback_timeouts(uint64_t* count) {
    if (count == nullptr) return RLSCAN_ERR_NULL;
    *count = 0;
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    int rc = RLSCAN_OK;
    for (auto& kv : g_scratch) {
        Scratch* sc = kv.second.get();
        std::lock_guard<std::mutex> gs(sc->m);
        if (sc->counter == nullptr) continue;
        unsigned int n = 0;
        if (hipSetDevice(kv.first.first) != hipSuccess ||
            hipStreamSynchronize(reinterpret_cast<hipStream_t>(kv.first.second)) != hipSuccess ||
            hipMemcpy(&n, sc->counter + 1, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) {
            rc = RLSCAN_ERR_HIP;
            continue;
        }
        *count += n;
    }
    if (have_prev) (void)hipSetDevice(prev);
    return rc;
}

int rlscan_set_launch_override(int mapping, int rounds, int waves, int64_t grid_cap, int flags) {
    if (mapping < RLSCAN_MAP_AUTO || mapping > RLSCAN_MAP_LOOKBACK) return RLSCAN_ERR_PARAM;
    if (rounds != 0 && rounds != 1 && rounds != 2 && rounds != 4) return RLSCAN_ERR_PARAM;
    if (waves != 0 && waves != 4 && waves != 8) return RLSCAN_ERR_PARAM;
    if (grid_cap < 0 || (flags & ~RLSCAN_FLAG_TICKETS) != 0) return RLSCAN_ERR_PARAM;
    g_override.mapping.store(mapping);
    g_override.rounds.store(rounds);
    g_override.waves.store(waves);
    g_override.grid_cap.store(grid_cap);
    g_override.flags.store(flags);
    return RLSCAN_OK;
}

}  // extern "C"
