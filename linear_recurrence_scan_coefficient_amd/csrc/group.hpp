// group.hpp -- several independent estimator calls in one kernel launch.
//
// A call of 4096 x 128 elements moves 6-38 MB: about the HBM bandwidth x
// latency product, so its time is mostly the launch, the ramp-up of its
// workgroups and its tail, and a step of seven such calls on one stream
// pays them seven times.  A grouped launch runs the tiles of every call in
// one grid, each tile exactly as the call's own packed kernel would run it
// (one round, whole rows per tile, entering state 0), so the ramps and tails
// overlap.
//
// Layout of the grid.  By default each call's tiles form one contiguous
// stretch of workgroups, call after call, in the order given.  The order
// matters: on the seven 4096 x 128 production calls (two waves, inputs
// rotating over 2 GB of buffers) the order GAE, V-trace, Retrace, TD(lambda),
// discounted, traces, prefix sum takes 18.4 us and the reverse order 21.5 us,
// where Retrace's tiles (72 B per element, 4.5x the bytes of a GAE tile)
// form the kernel's tail.  RLSCAN_FLAG_GROUP_INTERLEAVED deals the
// workgroups to the calls' tiles in turn instead: with the calls sorted by
// tile count, the grid is cut into segments; segment s runs the calls that
// still have tiles after the s shortest ones are done, one tile of each in
// turn, the turn order rotating by one call every row (workgroups go to the
// XCDs round-robin, so a fixed turn order of 8 calls would put each call on
// one XCD).  Every stretch of the grid then holds the same mix of heavy and
// light tiles and the time no longer depends on the order: 20.0 us in
// either order.  Runs of 4 to 256 consecutive tiles per turn were no faster.
//
// Calls join a group when their own plan is packed, every pointer takes the
// vector path, no carry is given, and a tile at the group's wave count still
// holds at least one whole row (packed_layout).  Estimator instantiations that can be grouped are
// listed in GroupKinds; the kernel dispatches on the call's index in it.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <type_traits>
#include <vector>

#include "estimators.hpp"
#include "tile_kernel.hpp"

namespace rlscan {

template <class... Es>
struct KindList {
    static constexpr int size = sizeof...(Es);
};

// Instantiations a grouped launch can run (Retrace: the action counts whose
// values are read with 16-byte loads, in the form without LDS staging).
using GroupKinds =
    KindList<Gae<false, float>, Gae<true, float>, Gae<false, uint8_t>, Gae<true, uint8_t>,
             LambdaReturns<false, float>, LambdaReturns<true, float>,
             LambdaReturns<false, uint8_t>, LambdaReturns<true, uint8_t>,
             Discounted<false, float>, Discounted<true, float>, Discounted<false, uint8_t>,
             Discounted<true, uint8_t>, Vtrace<false, float>, Vtrace<true, float>,
             Vtrace<false, uint8_t>, Vtrace<true, uint8_t>, Retrace<4, float, false>,
             Retrace<6, float, false>, Retrace<8, float, false>, Retrace<4, uint8_t, false>,
             Retrace<6, uint8_t, false>, Retrace<8, uint8_t, false>, Eligibility<float>,
             Eligibility<uint8_t>, PrefixSum<float>, PrefixSum<uint8_t>,
             Vtrace<false, float, true>, Vtrace<true, float, true>, Vtrace<false, uint8_t, true>,
             Vtrace<true, uint8_t, true>>;

// The form an estimator call takes inside a group (same Params layout).
template <class E>
struct GroupForm {
    using type = E;
};
template <int kA, class F>
struct GroupForm<Retrace<kA, F, true>> {
    using type = Retrace<kA, F, false>;
};

// Kinds that hold many values per lane in registers (Retrace with 8 actions:
// 64 action values per lane; V-trace's float64 form) run in a second build
// of the kernel, so that groups without them keep the register count, and
// occupancy, of the rest.
template <class E>
struct GroupWide : std::false_type {};
template <class F>
struct GroupWide<Retrace<8, F, false>> : std::true_type {};
template <bool kTrunc, class F>
struct GroupWide<Vtrace<kTrunc, F, true>> : std::true_type {};

template <class E, class L>
struct KindOf;
template <class E>
struct KindOf<E, KindList<>> {
    static constexpr int value = -1;
};
template <class E, class H, class... Ts>
struct KindOf<E, KindList<H, Ts...>> {
    static constexpr int rest = KindOf<E, KindList<Ts...>>::value;
    static constexpr int value = std::is_same<E, H>::value ? 0 : (rest < 0 ? -1 : rest + 1);
};

constexpr int kGroupMax = 8;             // calls per grouped launch
constexpr size_t kGroupParamBytes = 128;  // largest Params of a grouped kind

struct GroupEntry {  // dword-sized fields only (read in place as dwords)
    int32_t kind;  // index in GroupKinds
    int32_t pad;
    Geometry geo;  // the call's geometry at the group's tile size
    alignas(16) unsigned char params[kGroupParamBytes];  // the call's E::Params
};

struct GroupArgs {
    int32_t count;
    int32_t interleaved;                 // 1: the segment schedule, 0: contiguous
    int64_t first_block[kGroupMax + 1];  // contiguous: call i's first workgroup;
                                         // first_block[count] = grid
    // interleaved: segment s holds workgroups [seg_first[s], seg_first[s+1])
    // and runs calls order[s..count-1], tiles seg_tile0[s] onwards
    int32_t seg_first[kGroupMax + 1];
    int32_t seg_tile0[kGroupMax];
    int32_t order[kGroupMax];  // call indices by ascending tile count
    int32_t xcd_run;           // > 0: workgroups take grid slots in XCD runs (xcd_tile)
    GroupEntry e[kGroupMax];
};

static_assert(sizeof(GroupArgs) <= 4096, "the kernel argument block holds at most 4 KiB");

constexpr size_t align16(size_t n) { return (n + 15) & ~size_t(15); }

// LDS of one workgroup of W waves running a tile of E: the wave totals, the
// entering state, and the estimator's staging areas (one round).
template <class E>
constexpr size_t group_lds_offset_carry(int W) {
    return align16(W * sizeof(typename AggOf<typename E::S>::type));
}
template <class E>
constexpr size_t group_lds_offset_stage(int W) {
    return group_lds_offset_carry<E>(W) + 16;
}
template <class E>
constexpr size_t group_lds_offset_ostage(int W) {
    return group_lds_offset_stage<E>(W) + sizeof(float) * W * E::kStageFloats;
}
template <class E>
constexpr size_t group_lds_bytes(int W) {
    return group_lds_offset_ostage<E>(W) + sizeof(float) * W * E::kOutStageFloats;
}

// ------------------------------------------------------------------ device
// The kernel's argument block, read in place: indexing the by-value argument
// with the (workgroup-uniform) call index would copy all of it to scratch.
typedef __attribute__((address_space(4))) const uint32_t kernarg_u32;

template <class T>
__device__ __forceinline__ T kernarg_copy(kernarg_u32* src) {
    static_assert(sizeof(T) % 4 == 0, "copied as dwords");
    uint32_t words[sizeof(T) / 4];
#pragma unroll
    for (size_t k = 0; k < sizeof(T) / 4; ++k) words[k] = src[k];
    T v;
    __builtin_memcpy(&v, words, sizeof(T));
    return v;
}

template <class E, int W>
__device__ __forceinline__ void group_tile(kernarg_u32* entry, uint64_t tile, char* lds) {
    using A = typename AggOf<typename E::S>::type;
    using V = typename E::V;
    static_assert(sizeof(typename E::Params) <= kGroupParamBytes, "Params too large");
    const typename E::Params p =
        kernarg_copy<typename E::Params>(entry + offsetof(GroupEntry, params) / 4);
    const Geometry geo = kernarg_copy<Geometry>(entry + offsetof(GroupEntry, geo) / 4);
    A* sm_wave = reinterpret_cast<A*>(lds);
    V* sm_carry = reinterpret_cast<V*>(lds + group_lds_offset_carry<E>(W));
    lds_float* stage = (lds_float*)(lds + group_lds_offset_stage<E>(W));
    lds_float* ostage = (lds_float*)(lds + group_lds_offset_ostage<E>(W));
    const LookbackArgs lb{};
    if (tile_is_full<E, 1, W, true>(geo, tile))
        scan_tile<E, 1, W, false, true, true, false, true>(p, geo, lb, tile, sm_wave, sm_carry,
                                                           stage, ostage);
    else
        scan_tile<E, 1, W, false, true, false, false, true>(p, geo, lb, tile, sm_wave, sm_carry,
                                                            stage, ostage);
}

template <class E, int W, bool kWide>
__device__ __forceinline__ void group_tile_if(kernarg_u32* entry, uint64_t tile, char* lds) {
    if constexpr (kWide || !GroupWide<E>::value) group_tile<E, W>(entry, tile, lds);
}

template <int W, bool kWide, class... Es>
__device__ __forceinline__ void group_dispatch(int kind, kernarg_u32* entry, uint64_t tile,
                                               char* lds, KindList<Es...>) {
    int k = 0;
    ((kind == k++ ? group_tile_if<Es, W, kWide>(entry, tile, lds) : void()), ...);
}

// One workgroup per tile of every call in the group; the dynamic LDS size is
// the largest any call of the group needs.  `args` is the kernel's only
// argument, so it starts the argument block.  kWide: the build that also
// runs the GroupWide kinds.
template <int W, bool kWide>
__global__ __launch_bounds__(kWave * W) void group_kernel(const GroupArgs args) {
    extern __shared__ __attribute__((aligned(16))) char group_lds[];
    kernarg_u32* base = (kernarg_u32*)__builtin_amdgcn_kernarg_segment_ptr();
    const int64_t b =
        args.xcd_run > 0
            ? static_cast<int64_t>(xcd_tile(blockIdx.x,
                                            static_cast<uint64_t>(args.first_block[kGroupMax]),
                                            static_cast<uint64_t>(args.xcd_run)))
            : static_cast<int64_t>(blockIdx.x);
    int i = 0;
    uint64_t tile = 0;
    if (args.interleaved) {
        // the segment: the last one starting at or before b (an empty
        // segment shares its start with the next, which then wins)
        int s = 0;
#pragma unroll
        for (int k = 1; k < kGroupMax; ++k)
            if (k < args.count && b >= args.seg_first[k]) s = k;
        const uint32_t r = static_cast<uint32_t>(b) - base[offsetof(GroupArgs, seg_first) / 4 + s];
        const uint32_t m = static_cast<uint32_t>(args.count - s);  // calls in the segment
        const uint32_t row = r / m, col = r - row * m;
        const uint32_t j = static_cast<uint32_t>(s) + (col + row) % m;
        i = static_cast<int>(base[offsetof(GroupArgs, order) / 4 + j]);
        tile = base[offsetof(GroupArgs, seg_tile0) / 4 + s] + static_cast<uint64_t>(row);
    } else {
#pragma unroll
        for (int k = 1; k < kGroupMax; ++k)
            if (k < args.count && b >= args.first_block[k]) i = k;
        const int64_t first = kernarg_copy<int64_t>(base + (offsetof(GroupArgs, first_block) +
                                                            sizeof(int64_t) * i) / 4);
        tile = static_cast<uint64_t>(b - first);
    }
    kernarg_u32* entry = base + (offsetof(GroupArgs, e) + sizeof(GroupEntry) * i) / 4;
    const int kind = static_cast<int>(entry[offsetof(GroupEntry, kind) / 4]);
    group_dispatch<W, kWide>(kind, entry, tile, group_lds, GroupKinds{});
}

// ------------------------------------------------------------------ host
// Collects the calls of one rlscan_group instead of launching them: while a
// collector is installed for the calling thread, the estimator entry points
// check their arguments and plan as usual, then hand their launch here.
struct GroupCollector {
    int waves = 1;        // W of the grouped launches
    bool reject = false;  // a call cannot be grouped
    size_t lds = 0;       // largest LDS need of a collected call
    std::vector<GroupEntry> entries;
    std::vector<bool> wide;  // per entry: a GroupWide kind

    template <class E>
    void add(const typename E::Params& p, const Geometry& geo, int mapping, bool vec, bool carry) {
        using G = typename GroupForm<E>::type;
        constexpr int kind = KindOf<G, GroupKinds>::value;
        static_assert(sizeof(typename G::Params) == sizeof(typename E::Params), "same layout");
        const int64_t tile = int64_t(kWave) * waves * kChunk;
        if constexpr (kind < 0) {
            reject = true;
        } else {
            int64_t span = 0, tiles = 0;
            if (!vec || carry || mapping != RLSCAN_MAP_PACKED ||
                !packed_layout(geo.N, geo.T, tile, span, tiles)) {
                reject = true;
                return;
            }
            GroupEntry e{};
            e.kind = kind;
            e.geo = geo;
            e.geo.num_tiles = tiles;
            e.geo.grid = tiles;
            e.geo.tile_span = span;
            std::memcpy(e.params, &p, sizeof(p));
            const size_t need = group_lds_bytes<G>(waves);
            lds = need > lds ? need : lds;
            entries.push_back(e);
            wide.push_back(GroupWide<G>::value);
        }
    }
};

// Installed by rlscan_group for the duration of its collection pass.
extern thread_local GroupCollector* t_group;

hipError_t launch_group(const GroupArgs& args, int waves, bool wide, size_t lds,
                        hipStream_t stream);

}  // namespace rlscan
