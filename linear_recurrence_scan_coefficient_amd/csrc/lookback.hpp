// lookback.hpp -- single-pass decoupled look-back between the workgroups that
// share one long row (Merrill & Garland, "Single-pass Parallel Prefix Scan
// with Decoupled Look-back", 2016), for the (a, b) recurrence steps.
//
// Protocol, per call:
//  * Each workgroup takes a ticket from a 64-bit counter that is never reset;
//    the host passes `ticket_base`, the counter value at the start of the
//    call (it knows how many tickets every earlier call on this scratch
//    took), so tile = ticket - ticket_base.  Tickets, not blockIdx, order the
//    tiles, so a workgroup only ever waits on tiles already claimed by
//    running workgroups: forward progress needs no assumption about the
//    dispatch order.
//  * Tile s publishes its aggregate step (flag AGG) as soon as its local scan
//    is done -- or, when it already knows its outgoing state (it is tile 0,
//    or its aggregate cuts the chain, a == 0), that state directly (flag
//    INCL).  After the look-back it publishes INCL.
//  * Flags carry the call's epoch (flag = epoch << 2 | kind), so entries left
//    by earlier calls read as "not ready" and no clearing pass is needed.
//  * The look-back walks s-1, s-2, ... composing aggregates until it meets an
//    INCL entry or the composed step cuts the chain.
//
// Values and flags live in separate 64-bit words.  Each value word is written
// once per call before its flag is released (agent-scope release store), and
// read only after the flag is acquired (agent-scope acquire load), so readers
// on other XCDs never see a torn or stale value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_core.hpp"

namespace rlscan {

struct TileStatus {
    uint64_t flag;   // epoch << 2 | kind
    uint64_t agg_a;  // aggregate step, a part  } written before flag = AGG
    uint64_t agg_b;  // aggregate step, b part  }
    uint64_t incl;   // outgoing state (written before flag = INCL)
};

constexpr uint64_t kFlagAgg = 1;
constexpr uint64_t kFlagIncl = 2;

struct LookbackArgs {
    TileStatus* status;       // >= number of tiles entries
    unsigned long long* ticket_counter;
    unsigned int* timeouts;   // count of look-back waits that gave up
    uint64_t ticket_base;
    uint64_t epoch;           // >= 1, distinct for every call on this scratch
};

// Upper bound on the polls of one predecessor's status (each poll sleeps
// about 64 cycles plus a memory round trip: several seconds in all).  A wait
// that long means the protocol is broken; the workgroup then records the
// failure, writes a poisoned result and finishes, so the kernel always ends.
constexpr uint32_t kMaxPolls = 1u << 22;

__device__ __forceinline__ float poisoned(float) { return __builtin_nanf(""); }
__device__ __forceinline__ int64_t poisoned(int64_t) { return INT64_MIN; }

// Packing of aggregate steps and states into 64-bit words.
struct PackedStep {
    uint64_t a, b;
};
__device__ __forceinline__ PackedStep pack_step(StepD s) {
    return {static_cast<uint64_t>(__double_as_longlong(s.a)), __float_as_uint(s.b)};
}
__device__ __forceinline__ StepD unpack_step(PackedStep u, StepD) {
    return {__longlong_as_double(static_cast<long long>(u.a)),
            __uint_as_float(static_cast<uint32_t>(u.b))};
}
// An integer aggregate that is published as AGG never cuts the chain (a cut
// aggregate is published as INCL), so its a is 1 and only b is stored.
__device__ __forceinline__ PackedStep pack_step(StepI s) {
    return {1u, static_cast<uint64_t>(s.b)};
}
__device__ __forceinline__ StepI unpack_step(PackedStep u, StepI) {
    return {1u, static_cast<int64_t>(u.b)};
}
__device__ __forceinline__ uint64_t pack_state(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float unpack_state(uint64_t u, float) {
    return __uint_as_float(static_cast<uint32_t>(u));
}
__device__ __forceinline__ uint64_t pack_state(int64_t x) { return static_cast<uint64_t>(x); }
__device__ __forceinline__ int64_t unpack_state(uint64_t u, int64_t) {
    return static_cast<int64_t>(u);
}

__device__ __forceinline__ void publish_aggregate(TileStatus* st, PackedStep value,
                                                  uint64_t epoch) {
    __hip_atomic_store(&st->agg_a, value.a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&st->agg_b, value.b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&st->flag, (epoch << 2) | kFlagAgg, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_inclusive(TileStatus* st, uint64_t state, uint64_t epoch) {
    __hip_atomic_store(&st->incl, state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&st->flag, (epoch << 2) | kFlagIncl, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t take_ticket(const LookbackArgs& lb) {
    const unsigned long long t = __hip_atomic_fetch_add(lb.ticket_counter, 1ull, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
    return static_cast<uint64_t>(t) - lb.ticket_base;
}

// State entering tile `tile` (tile >= 1), by walking back over tiles
// tile-1, tile-2, ...  Called by one thread.  Terminates: tile 0 always
// publishes INCL, and every earlier tile has been claimed by a running
// workgroup that publishes without waiting on later tiles; the poll bound
// above ends the wait even if that invariant were ever broken.
template <class S, class V>
__device__ V look_back(const LookbackArgs& lb, uint64_t tile) {
    S acc = identity_step(S{});
    uint64_t p = tile - 1;
    for (;;) {
        TileStatus* st = lb.status + p;
        uint64_t f;
        for (uint32_t polls = 0;; ++polls) {
            f = __hip_atomic_load(&st->flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if ((f >> 2) == lb.epoch) break;
            if (polls >= kMaxPolls) {
                __hip_atomic_fetch_add(lb.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return poisoned(V{});
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if ((f & 3u) == kFlagIncl) {
            const uint64_t u = __hip_atomic_load(&st->incl, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            return apply(acc, unpack_state(u, V{}));
        }
        PackedStep u;
        u.a = __hip_atomic_load(&st->agg_a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        u.b = __hip_atomic_load(&st->agg_b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        acc = compose(acc, unpack_step(u, S{}));
        if (cuts_chain(acc)) return acc.b;
        --p;  // p >= 1 here: tile 0 publishes INCL only
    }
}

}  // namespace rlscan
