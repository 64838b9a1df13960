// lookback.hpp -- single-pass decoupled look-back between the workgroups that
// share one long row (after Merrill & Garland, "Single-pass Parallel Prefix
// Scan with Decoupled Look-back", 2016), for the (a, b) recurrence steps.
//
// Protocol, per call:
//  * Tile order.  By default tile = blockIdx.x with one tile per workgroup:
//    the dispatcher hands workgroups to the XCDs round-robin and, within an
//    XCD, in increasing index order, so every tile a workgroup waits on
//    belongs to a workgroup that has been or will be dispatched without
//    needing the waiter's slot.  When workgroups loop over tiles (grid
//    capped) the order comes from tickets instead: each tile is claimed from
//    a 64-bit counter that is never reset (the host passes `ticket_base`,
//    the counter value at the start of the call), so a workgroup only waits
//    on tiles claimed by running workgroups.  Tickets cost one atomic on a
//    single address per tile -- about 12 ns each on MI355X, serialised
//    across the XCDs -- which is why they are not the default.
//  * Tile s publishes its aggregate step (AGG) as soon as its local scan is
//    done -- or, when it already knows its outgoing state (it is tile 0, or
//    its aggregate cuts the chain, a == 0), that state (INCL).  After the
//    look-back it publishes INCL.
//  * Every status word is self-validating: 64 bits = 32-bit call tag (the
//    call's epoch) | 32-bit payload.  A word whose tag is not the current
//    epoch is "not ready", so entries left by earlier calls need no clearing
//    pass, and each word is read and written with one relaxed agent-scope
//    atomic: no release/acquire fences, hence no L2 write-back or invalidate
//    on any XCD.  A payload wider than 32 bits spans two words, each
//    validated by its own tag; each word is written once per call.
//  * Integer states take two words only when they need them: a value that
//    fits in 32 bits (signed) is published as one word whose tag has its top
//    bit set (call tags stay below 2^31), so the common case costs a poll
//    two status reads instead of four.
//  * The look-back is wave-parallel: wave 0 reads the status of 64
//    predecessors at once, waits until every one of them up to the nearest
//    terminal entry (INCL, or an aggregate that cuts the chain) is ready,
//    folds them with one wave scan, and moves the window back by 64 tiles
//    if no terminal entry was in it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_core.hpp"

namespace rlscan {

struct TileStatus {
    uint64_t w[4];  // float: agg a, agg b, incl x, -; int: agg b lo/hi, incl x lo/hi
};

// Status entries per tile: one, or two for float64 steps, whose aggregate
// (a, b) and inclusive value take six 32-bit payloads: entry 0 holds a lo/hi
// and b lo/hi, entry 1 the inclusive value lo/hi.
template <class A> struct StatusEntries { static constexpr int value = 1; };
template <> struct StatusEntries<StepW> { static constexpr int value = 2; };

template <class A>
__host__ __device__ __forceinline__ TileStatus* status_of(TileStatus* base, int64_t tile) {
    return base + StatusEntries<A>::value * tile;
}

struct LookbackArgs {
    TileStatus* status;       // >= number of tiles entries
    unsigned long long* ticket_counter;
    unsigned int* timeouts;   // count of look-back waits that gave up
    uint64_t ticket_base;
    uint32_t tag;             // the call's epoch: nonzero, at most
                              // kLastTag, distinct for every call since the
                              // status buffer was cleared
    uint32_t use_tickets;     // 1: tiles from tickets; 0: tile = blockIdx.x
    uint32_t read_tag;        // tag the look-back accepts: `tag`, or kNeverTag
                              // to make every wait give up (tests)
    uint32_t max_polls;       // polls of one window before a wait gives up
};

// Call tags run from 1 to kLastTag; kNeverTag is never written, in either
// form (a float or two-word integer word carries the tag, a one-word integer
// the tag with its top bit set), so a look-back reading with it never sees a
// ready predecessor.
constexpr uint32_t kLastTag = 0x7ffffffeu;
constexpr uint32_t kNeverTag = 0x7fffffffu;

// Upper bound on the polls of one look-back window (each poll sleeps about
// 64 cycles plus a memory round trip: several seconds in all).  A wait that
// long means the protocol is broken; the workgroup then records the failure,
// writes a poisoned result and finishes, so the kernel always ends.  (Tests
// force this path with a few polls and kNeverTag.)
constexpr uint32_t kMaxPolls = 1u << 22;

// Predecessors read by a look-back poll before it widens to the whole window.
constexpr int kNarrow = 4;

__device__ __forceinline__ float poisoned(float) { return __builtin_nanf(""); }
__device__ __forceinline__ double poisoned(double) { return __builtin_nan(""); }
__device__ __forceinline__ int64_t poisoned(int64_t) { return INT64_MIN; }

__host__ __device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t payload) {
    return (static_cast<uint64_t>(tag) << 32) | payload;
}
__host__ __device__ __forceinline__ void store_word(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__host__ __device__ __forceinline__ uint64_t load_word(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__host__ __device__ __forceinline__ bool has_tag(uint64_t w, uint32_t tag) {
    return static_cast<uint32_t>(w >> 32) == tag;
}

// Tag bit of an integer word that holds a whole value (sign-extended from its
// 32-bit payload).
constexpr uint32_t kShortForm = 0x80000000u;

__host__ __device__ __forceinline__ bool fits_short(int64_t v) {
    return v == static_cast<int64_t>(static_cast<int32_t>(v));
}
__host__ __device__ __forceinline__ int64_t short_value(uint64_t w) {
    return static_cast<int64_t>(static_cast<int32_t>(static_cast<uint32_t>(w)));
}
__host__ __device__ __forceinline__ int64_t long_value(uint64_t lo, uint64_t hi) {
    return static_cast<int64_t>(((hi & 0xffffffffull) << 32) | (lo & 0xffffffffull));
}

// ---------------------------------------------------------------- publish
// The float aggregate's a is published rounded once to float32: a single
// rounding, unlike the many that motivated the float64 a in StepD.
__host__ __device__ __forceinline__ void publish_aggregate(TileStatus* st, StepD s, uint32_t tag) {
    store_word(&st->w[0], tagged(tag, __builtin_bit_cast(uint32_t, static_cast<float>(s.a))));
    store_word(&st->w[1], tagged(tag, __builtin_bit_cast(uint32_t, s.b)));
}
__host__ __device__ __forceinline__ void publish_inclusive(TileStatus* st, float x, uint32_t tag) {
    store_word(&st->w[2], tagged(tag, __builtin_bit_cast(uint32_t, x)));
}
// Integer value v into words w[k] (and w[k+1] if it needs 64 bits).
__host__ __device__ __forceinline__ void publish_int(uint64_t* w, int64_t v, uint32_t tag) {
    const uint64_t u = static_cast<uint64_t>(v);
    if (fits_short(v)) {
        store_word(w, tagged(tag | kShortForm, static_cast<uint32_t>(u)));
    } else {
        store_word(w, tagged(tag, static_cast<uint32_t>(u)));
        store_word(w + 1, tagged(tag, static_cast<uint32_t>(u >> 32)));
    }
}
// An integer aggregate published as AGG never cuts the chain (a cut aggregate
// is published as INCL), so its a is 1 and only b is stored.
__host__ __device__ __forceinline__ void publish_aggregate(TileStatus* st, StepI s, uint32_t tag) {
    publish_int(&st->w[0], s.b, tag);
}
__host__ __device__ __forceinline__ void publish_inclusive(TileStatus* st, int64_t x, uint32_t tag) {
    publish_int(&st->w[2], x, tag);
}

// Float64 values: each 32-bit half is a word of its own, validated by its
// own tag (each is written once per call, so two current halves are the
// value).
__host__ __device__ __forceinline__ void publish_f64(uint64_t* w, double v, uint32_t tag) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    store_word(w, tagged(tag, static_cast<uint32_t>(u)));
    store_word(w + 1, tagged(tag, static_cast<uint32_t>(u >> 32)));
}
__host__ __device__ __forceinline__ double f64_value(uint64_t lo, uint64_t hi) {
    return __builtin_bit_cast(double, static_cast<uint64_t>(long_value(lo, hi)));
}
__host__ __device__ __forceinline__ void publish_aggregate(TileStatus* st, StepW s, uint32_t tag) {
    publish_f64(&st[0].w[0], s.a, tag);
    publish_f64(&st[0].w[2], s.b, tag);
}
__host__ __device__ __forceinline__ void publish_inclusive(TileStatus* st, double x, uint32_t tag) {
    publish_f64(&st[1].w[0], x, tag);
}

// ---------------------------------------------------------------- read
// Returns 0 (not ready), 1 (aggregate) or 2 (inclusive state, given as the
// step (0, x)), and the step in `s`.
__host__ __device__ __forceinline__ int read_status(TileStatus* st, uint32_t tag, StepD& s) {
    const uint64_t x = load_word(&st->w[2]);
    const uint64_t a = load_word(&st->w[0]);
    const uint64_t b = load_word(&st->w[1]);
    if (has_tag(x, tag)) {
        s = {0.0, __builtin_bit_cast(float, static_cast<uint32_t>(x))};
        return 2;
    }
    if (has_tag(a, tag) && has_tag(b, tag)) {
        s = {static_cast<double>(__builtin_bit_cast(float, static_cast<uint32_t>(a))),
             __builtin_bit_cast(float, static_cast<uint32_t>(b))};
        return 1;
    }
    return 0;
}
// The high word of a two-word value is read only once its low word is seen
// (one dependent read, the inclusive value's if its low word is there).
__host__ __device__ __forceinline__ int read_status(TileStatus* st, uint32_t tag, StepI& s) {
    const uint64_t x = load_word(&st->w[2]);
    const uint64_t b = load_word(&st->w[0]);
    if (has_tag(x, tag | kShortForm)) {
        s = {0u, short_value(x)};
        return 2;
    }
    const bool x_long = has_tag(x, tag);
    if (!x_long && has_tag(b, tag | kShortForm)) {
        s = {1u, short_value(b)};
        return 1;
    }
    if (x_long || has_tag(b, tag)) {
        const uint64_t hi = load_word(&st->w[x_long ? 3 : 1]);
        if (has_tag(hi, tag)) {
            s = {x_long ? 0u : 1u, long_value(x_long ? x : b, hi)};
            return x_long ? 2 : 1;
        }
    }
    return 0;
}

__host__ __device__ __forceinline__ int read_status(TileStatus* st, uint32_t tag, StepW& s) {
    const uint64_t xl = load_word(&st[1].w[0]);
    const uint64_t xh = load_word(&st[1].w[1]);
    if (has_tag(xl, tag) && has_tag(xh, tag)) {
        s = {0.0, f64_value(xl, xh)};
        return 2;
    }
    const uint64_t al = load_word(&st[0].w[0]);
    const uint64_t ah = load_word(&st[0].w[1]);
    const uint64_t bl = load_word(&st[0].w[2]);
    const uint64_t bh = load_word(&st[0].w[3]);
    if (has_tag(al, tag) && has_tag(ah, tag) && has_tag(bl, tag) && has_tag(bh, tag)) {
        s = {f64_value(al, ah), f64_value(bl, bh)};
        return 1;
    }
    return 0;
}

// One poll of a look-back window, decided from two lane masks of the window
// (lane 63 the nearest predecessor): `term_mask` marks the entries that end
// the walk (an inclusive value, or an aggregate that cuts the chain),
// `ready_mask` the entries read with the call's tag (lanes before tile 0
// count as ready).  The walk needs every entry from the nearest terminal one
// up to lane 63, or the whole window if none is terminal; a narrow poll
// (width < 64) that finds its lanes ready and none terminal widens.
struct PollStep {
    int stop;    // nearest terminal lane, -1 if none
    bool done;   // every entry the walk needs is ready
    bool widen;  // read the whole window next
};
__host__ __device__ __forceinline__ PollStep poll_step(uint64_t term_mask, uint64_t ready_mask,
                                                       int width) {
    PollStep r;
    r.stop = term_mask ? 63 - __builtin_clzll(term_mask) : -1;
    const uint64_t need = r.stop >= 0 ? (~0ull << r.stop) : ~0ull;
    r.done = (ready_mask & need) == need;
    const uint64_t narrow = ~0ull << (kWave - kNarrow);
    r.widen = !r.done && r.stop < 0 && width < kWave && (ready_mask & narrow) == narrow;
    return r;
}

__device__ __forceinline__ uint64_t take_ticket(const LookbackArgs& lb) {
    const unsigned long long t = __hip_atomic_fetch_add(lb.ticket_counter, 1ull, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
    return static_cast<uint64_t>(t) - lb.ticket_base;
}

// State entering tile `tile` (tile >= 1).  Called by all 64 lanes of one
// wave; every lane returns the same value.  Terminates: tile 0 always
// publishes INCL, and every earlier tile has been claimed by a running
// workgroup that publishes its aggregate without waiting on later tiles; the
// poll bound ends the wait even if that invariant were ever broken.
template <class A, class V>
__device__ V look_back(const LookbackArgs& lb, uint64_t tile, int lane) {
    A acc = identity_step(A{});  // steps between the window and `tile`
    int64_t top = static_cast<int64_t>(tile) - 1;  // nearest tile not yet folded
    for (;;) {
        // lane 63 reads the nearest predecessor, lane 0 the farthest; lanes
        // before tile 0 keep the identity and count as ready
        const int64_t q = top - (kWave - 1 - lane);
        A s = identity_step(A{});
        int stop = -1;
        // Polls read the kNarrow nearest predecessors first (most walks end
        // there: about half the tiles of a long row hold a chain cut) and
        // the whole window only once those are ready and hold no terminal
        // entry -- the status reads are uncached round trips that compete
        // with the streaming loads.
        int width = kNarrow;
        for (uint32_t polls = 0;; ++polls) {
            const bool in_window = kWave - 1 - lane < width;
            int kind = q < 0 ? 3 : 0;
            if (q >= 0 && in_window) kind = read_status(status_of<A>(lb.status, q), lb.read_tag, s);
            const bool terminal = kind == 2 || (kind == 1 && cuts_chain(s));
            const PollStep step = poll_step(__ballot(terminal), __ballot(kind != 0), width);
            stop = step.stop;
            if (step.done) break;
            if (step.widen) {
                width = kWave;  // no terminal entry near: read the whole window now
                continue;
            }
            if (polls >= lb.max_polls) {
                if (lane == 0)
                    __hip_atomic_fetch_add(lb.timeouts, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                return poisoned(V{});
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // entries beyond the nearest terminal one are not needed (and may not
        // be ready)
        if (lane < stop) s = identity_step(A{});
        const A total = read_lane(wave_inclusive_scan(s), kWave - 1);
        acc = compose(acc, total);
        if (stop >= 0) return acc.b;  // the terminal entry made acc.a zero
        top -= kWave;
    }
}

}  // namespace rlscan
