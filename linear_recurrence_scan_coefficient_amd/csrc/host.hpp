// host.hpp -- host side of librlscan shared by its translation units: the
// launch planner, the look-back scratch, argument checks, and the launch
// path every estimator entry point takes (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "estimators.hpp"
#include "group.hpp"
#include "lookback.hpp"
#include "rlscan.h"
#include "tile_kernel.hpp"

namespace rlscan {


constexpr int64_t kMaxElements = int64_t(1) << 48;
constexpr int64_t kMaxGrid = (int64_t(1) << 23) - 1;  // grid * 512 threads < 2^32

struct LaunchOverride {
    std::atomic<int> mapping{RLSCAN_MAP_AUTO};
    std::atomic<int> rounds{0};
    std::atomic<int> waves{0};
    std::atomic<int64_t> grid_cap{0};
    std::atomic<int> flags{0};  // RLSCAN_FLAG_* bits
    std::atomic<int64_t> xcd_run{-1};  // -1: the library's choice
};
extern LaunchOverride g_override;

// Run length of the XCD tile order (xcd_tile) of packed launches with
// `tiles` tiles whose span is `span` elements, and of grouped launches
// (0: tile = blockIdx).
int64_t xcd_run(int64_t tiles, int64_t span);
int64_t group_xcd_run();

struct Scratch {
    std::mutex m;
    TileStatus* status = nullptr;
    unsigned long long* counter = nullptr;  // [0]: tickets; low half of [1]: timeouts
    int64_t capacity = 0;       // tiles
    uint64_t next_ticket = 0;   // counter value at the start of the next call
    uint64_t epoch = 0;         // tag of the last call (below 2^31, 0 = none)
    bool broken = false;        // a launch failed: counter position unknown
    bool fixed = false;         // a static device array: never allocated, grown or freed
};

// Look-back scratch of (device, stream); created on first use and kept until
// the process ends (rlscan_release_scratch frees its device buffers only, so
// a pointer returned here stays valid).  nullptr if the host is out of memory.
Scratch* scratch_for(int device, hipStream_t stream);

// Where a call takes its look-back scratch from.  The default (nullptr)
// allocates per (device, stream) with scratch_for; a source with `get` set
// hands out a fixed array of at most `max_tiles` tiles per device, and the
// call then allocates nothing: it is refused with RLSCAN_ERR_SCRATCH, before
// any HIP call, when its plan needs more tiles.
struct ScratchSource {
    Scratch* (*get)(int device);
    int64_t max_tiles;
};

// Enqueues a kernel that zeroes `words` 64-bit words at `p` (the status
// words and counters are cleared this way, never by a memset node).
hipError_t clear_words(uint64_t* p, int64_t words, hipStream_t stream);

// The call tag of look-back calls captured into a graph (fixed scratch
// only); eager calls take the tags below it.
constexpr uint32_t kCaptureTag = kLastTag;

// rlscan_gae_carry with its look-back scratch taken from `src`.
int gae_with_scratch(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* advantages,
                     float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                     hipStream_t stream, const ScratchSource* src);

// Timeouts recorded in the fixed scratch arrays of the no-allocation entry
// point (waits for each device that has one).
int static_scratch_timeouts(uint64_t* count);

// Order of the look-back launches of one device across streams.  A look-back
// workgroup waits on lower tiles of its own launch; one launch always makes
// progress because each XCD dispatches its workgroups in index order.  Two
// look-back launches running at once on different streams could each hold
// slots that the other's undispatched tiles need, so a look-back launch on a
// stream other than the previous one's first waits for that launch.  While
// one stream does all the look-back launches of a device nothing is recorded
// (an event per launch costs ~3 us of GPU time between back-to-back long
// calls); from the first launch on another stream on, an event is recorded
// after every look-back launch.  Packed launches are not ordered.
struct LaunchOrder {
    std::mutex m;
    hipEvent_t last = nullptr;          // recorded after the latest launch
    hipStream_t last_stream = nullptr;
    bool any = false;                   // a look-back launch has happened
    bool multi = false;                 // launches came from several streams
};
LaunchOrder* launch_order(int device);
// Called with sc->m held.  Makes room for `tiles` status entries.
int ensure_capacity(Scratch* sc, hipStream_t stream, int64_t tiles);

// Planning id of V-trace's float64 form (not a public estimator id): at most
// two rounds per tile (four spill its float64 registers), two status
// entries per look-back tile.
constexpr int kEstVtraceWide = RLSCAN_EST_PREFIX_SUM + 1;

struct Plan {
    int mapping;
    int rounds;
    int waves;
    int64_t tile_elems;  // capacity of a tile
    int64_t tile_span;   // elements of memory per tile (packed: its whole rows)
    int64_t tiles, grid;
};

// `vec`: every pointer is 16-byte aligned; `carry`: a carry argument is given.
Plan make_plan(int est, int64_t N, int64_t T, bool vec, bool carry = false);

// V-trace launches in the float64 form (est_vtrace_wide.hip: a translation
// unit of their own, compiled in parallel with the float32 form's).
template <class F>
hipError_t launch_vtrace_wide(const VtraceParams<F>& p, const Geometry& geo,
                              const LookbackArgs& lb, const Plan& pl, bool vec, bool carry,
                              bool trunc, hipStream_t stream);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool unit_interval(float x) { return x >= 0.0f && x <= 1.0f; }  // false for NaN
inline bool positive_clip(float x) { return x > 0.0f; }                 // +inf allowed, NaN not

inline int check_shape(int64_t N, int64_t T, int64_t A = 1) {
    if (N < 0 || T < 0 || A < 1) return RLSCAN_ERR_SHAPE;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (N > kMaxElements / T) return RLSCAN_ERR_SHAPE;
    if (N * T > kMaxElements / A) return RLSCAN_ERR_SHAPE;
    return RLSCAN_OK;
}

// Outputs must not equal an input or each other; NULL (an optional output
// not asked for) is skipped.
inline int check_alias(std::initializer_list<const void*> outs, std::initializer_list<const void*> ins) {
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

inline bool all_aligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return false;
    return true;
}

// A flag tensor's 4-element chunks are 16 bytes (float) or 4 bytes
// (uint8_t): what the vector path needs of its base address.
template <class F>
inline bool flags_aligned(const F* p) {
    return (reinterpret_cast<uintptr_t>(p) % (sizeof(F) * 4)) == 0;  // NULL is aligned
}

// Three builds per shape: look-back; packed with tiles that span their
// whole capacity; packed with tiles of whole rows that fall short of it.
template <class E, int R, int W, bool VEC, bool CARRY>
hipError_t launch_r(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                    const Plan& pl, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(geo.grid)), block(kWave * W);
    if (pl.mapping == RLSCAN_MAP_LOOKBACK)
        hipLaunchKernelGGL((scan_kernel<E, R, W, true, VEC, CARRY, false>), grid, block, 0, stream,
                           p, geo, lb);
    else if (pl.tile_span != pl.tile_elems)
        hipLaunchKernelGGL((scan_kernel<E, R, W, false, VEC, CARRY, true>), grid, block, 0, stream,
                           p, geo, lb);
    else
        hipLaunchKernelGGL((scan_kernel<E, R, W, false, VEC, CARRY, false>), grid, block, 0,
                           stream, p, geo, lb);
    return hipGetLastError();
}

// Most rounds per tile an estimator's kernels are built for (the planner
// never asks for more).
template <class E> struct MaxRounds { static constexpr int value = 4; };
template <bool kTrunc, class F> struct MaxRounds<Vtrace<kTrunc, F, true>> {
    static constexpr int value = 2;
};

template <class E, int W, bool CARRY>
hipError_t launch_w(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                    const Plan& pl, hipStream_t stream) {
    switch (pl.rounds) {
        case 1: return launch_r<E, 1, W, true, CARRY>(p, geo, lb, pl, stream);
        case 2: return launch_r<E, 2, W, true, CARRY>(p, geo, lb, pl, stream);
        default:
            if constexpr (MaxRounds<E>::value >= 4)
                return launch_r<E, 4, W, true, CARRY>(p, geo, lb, pl, stream);
            else
                return hipErrorInvalidValue;
    }
}

// Kernels built for the carry arguments exist with four or eight waves (the
// plan sees to it); all others with 1 or 2 waves (one round), 4 or 8.
template <class E>
hipError_t launch_kernel(const typename E::Params& p, const Geometry& geo, const LookbackArgs& lb,
                         const Plan& pl, bool vec, bool carry, hipStream_t stream) {
    if (t_group != nullptr) {  // collected for a grouped launch instead
        t_group->add<E>(p, geo, pl.mapping, vec, carry);
        return hipSuccess;
    }
    if (carry) {
        if (!vec) return launch_r<E, 1, 4, false, true>(p, geo, lb, pl, stream);
        return pl.waves == 8 ? launch_w<E, 8, true>(p, geo, lb, pl, stream)
                             : launch_w<E, 4, true>(p, geo, lb, pl, stream);
    }
    if (!vec) return launch_r<E, 1, 4, false, false>(p, geo, lb, pl, stream);
    switch (pl.waves) {
        case 1: return launch_r<E, 1, 1, true, false>(p, geo, lb, pl, stream);
        case 2: return launch_r<E, 1, 2, true, false>(p, geo, lb, pl, stream);
        case 8: return launch_w<E, 8, false>(p, geo, lb, pl, stream);
        default: return launch_w<E, 4, false>(p, geo, lb, pl, stream);
    }
}

// Retrace keeps 2*4*A action values per round in LDS or registers: one
// round of at most four waves.
template <class E>
hipError_t launch_kernel_r1(const typename E::Params& p, const Geometry& geo,
                            const LookbackArgs& lb, const Plan& pl, bool vec, bool carry,
                            hipStream_t stream) {
    if (t_group != nullptr) {
        t_group->add<E>(p, geo, pl.mapping, vec, carry);
        return hipSuccess;
    }
    if (carry)
        return vec ? launch_r<E, 1, 4, true, true>(p, geo, lb, pl, stream)
                   : launch_r<E, 1, 4, false, true>(p, geo, lb, pl, stream);
    if (!vec) return launch_r<E, 1, 4, false, false>(p, geo, lb, pl, stream);
    switch (pl.waves) {
        case 1: return launch_r<E, 1, 1, true, false>(p, geo, lb, pl, stream);
        case 2: return launch_r<E, 1, 2, true, false>(p, geo, lb, pl, stream);
        default: return launch_r<E, 1, 4, true, false>(p, geo, lb, pl, stream);
    }
}

// Plans, takes the look-back scratch if needed, and launches through `fn`.
// `src`: where the scratch comes from (nullptr: allocated per stream).
template <class Fn>
int run(int est, int64_t N, int64_t T, bool vec, bool carry, hipStream_t stream, Fn&& fn,
        const ScratchSource* src = nullptr) {
    const Plan pl = make_plan(est, N, T, vec, carry);
    // status entries per tile: two for float64 steps (StatusEntries)
    const int entries = est == kEstVtraceWide ? StatusEntries<StepW>::value : 1;
    if (pl.rounds != 1 && pl.rounds != 2 && pl.rounds != 4) return RLSCAN_ERR_PARAM;
    if (pl.waves != 1 && pl.waves != 2 && pl.waves != 4 && pl.waves != 8)
        return RLSCAN_ERR_PARAM;
    if (src != nullptr && t_group == nullptr && pl.mapping == RLSCAN_MAP_LOOKBACK &&
        pl.tiles > src->max_tiles / entries)
        return RLSCAN_ERR_SCRATCH;
    Geometry geo;
    geo.N = N;
    geo.T = T;
    geo.NT = N * T;
    geo.num_tiles = pl.tiles;
    geo.grid = pl.grid;
    geo.tile_span = pl.tile_span;
    geo.xcd_run = pl.mapping == RLSCAN_MAP_PACKED ? xcd_run(pl.tiles, pl.tile_span) : 0;
    geo.inv_T = 1.0 / static_cast<double>(T);
    LookbackArgs lb{};
    if (t_group != nullptr) {  // collecting for a grouped launch: no side effects
        if (pl.mapping == RLSCAN_MAP_PACKED)
            (void)fn(geo, lb, pl);  // records the call; launches nothing
        else
            t_group->reject = true;
        return RLSCAN_OK;
    }
    if (pl.mapping == RLSCAN_MAP_PACKED) {
        return fn(geo, lb, pl) == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
    }
    // tile = blockIdx needs every tile to have its own workgroup
    const bool tickets = pl.grid < pl.tiles || (g_override.flags.load() & RLSCAN_FLAG_TICKETS);
    // Under graph capture a replay would reuse the call's tag (reading the
    // last replay's status words as its own), its ticket base, and a
    // scratch buffer that later calls may move.  Only the fixed array,
    // whose address never changes, serves captured look-back calls, with
    // one tile per workgroup: each records a clear of its status words
    // before the scan and takes the tag reserved for captured calls.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) return RLSCAN_ERR_HIP;
    const bool captured = capture != hipStreamCaptureStatusNone;
    if (captured && (src == nullptr || tickets)) return RLSCAN_ERR_CAPTURE;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return RLSCAN_ERR_HIP;
    Scratch* sc = src != nullptr ? src->get(device) : scratch_for(device, stream);
    if (sc == nullptr) return src != nullptr ? RLSCAN_ERR_HIP : RLSCAN_ERR_ALLOC;
    std::lock_guard<std::mutex> g(sc->m);
    const int rc = ensure_capacity(sc, stream, pl.tiles * entries);
    if (rc != RLSCAN_OK) return rc;
    lb.use_tickets = tickets ? 1u : 0u;
    lb.status = sc->status;
    lb.ticket_counter = sc->counter;
    lb.timeouts = reinterpret_cast<unsigned int*>(sc->counter + 1);
    lb.ticket_base = sc->next_ticket;
    if (captured) {
        // cleared words carry tag 0, which no call uses
        if (clear_words(reinterpret_cast<uint64_t*>(sc->status),
                        static_cast<int64_t>(sizeof(TileStatus) / 8) * pl.tiles * entries,
                        stream) != hipSuccess)
            return RLSCAN_ERR_HIP;
        lb.tag = kCaptureTag;
    } else {
        if (sc->epoch >= kCaptureTag - 1) {
            // the eager call tags (below kCaptureTag; at most kLastTag in
            // all, as a one-word integer value's top bit marks its form)
            // are about to repeat: clear the status words
            if (clear_words(reinterpret_cast<uint64_t*>(sc->status),
                            static_cast<int64_t>(sizeof(TileStatus) / 8) * sc->capacity,
                            stream) != hipSuccess)
                return RLSCAN_ERR_HIP;
            sc->epoch = 0;
        }
        lb.tag = static_cast<uint32_t>(++sc->epoch);
    }
    const bool give_up = (g_override.flags.load() & RLSCAN_FLAG_LOOKBACK_GIVE_UP) != 0;
    lb.read_tag = give_up ? kNeverTag : lb.tag;
    lb.max_polls = give_up ? 8u : kMaxPolls;
    if (sc->fixed) {
        // the fixed array's calls are not ordered across streams (ordering
        // them would need an event, i.e. an allocation): the caller keeps
        // them from overlapping with other look-back launches of the device
        if (fn(geo, lb, pl) != hipSuccess) {
            sc->broken = true;
            return RLSCAN_ERR_HIP;
        }
        if (tickets)
            sc->next_ticket += static_cast<uint64_t>(pl.tiles) +
                               (pl.grid >= pl.tiles ? 0u : static_cast<uint64_t>(pl.grid));
        return RLSCAN_OK;
    }
    LaunchOrder* order = launch_order(device);
    if (order == nullptr) return RLSCAN_ERR_HIP;
    std::lock_guard<std::mutex> go(order->m);
    if (order->any && order->last_stream != stream) {
        if (!order->multi) {
            // first switch: the event covers everything enqueued so far on
            // the previous stream, its latest look-back launch included
            if (hipEventRecord(order->last, order->last_stream) != hipSuccess)
                return RLSCAN_ERR_HIP;
            order->multi = true;
        }
        if (hipStreamWaitEvent(stream, order->last, 0) != hipSuccess) return RLSCAN_ERR_HIP;
    }
    if (fn(geo, lb, pl) != hipSuccess) {
        sc->broken = true;
        return RLSCAN_ERR_HIP;
    }
    if (order->multi && hipEventRecord(order->last, stream) != hipSuccess)
        return RLSCAN_ERR_HIP;
    order->last_stream = stream;
    order->any = true;
    // every workgroup takes one ticket per tile it runs plus, when looping,
    // one final ticket that finds no tile
    if (tickets)
        sc->next_ticket += static_cast<uint64_t>(pl.tiles) +
                           (pl.grid >= pl.tiles ? 0u : static_cast<uint64_t>(pl.grid));
    return RLSCAN_OK;
}

}  // namespace rlscan
