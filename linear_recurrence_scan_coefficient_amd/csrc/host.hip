// host.hip -- librlscan's launch planner, look-back scratch and the entry
// points that are not estimators (status text, version, planning, launch
// override, diagnostics), plus the two diagnostic kernels (gfx950 only).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "host.hpp"

namespace rlscan {

thread_local GroupCollector* t_group = nullptr;

LaunchOverride g_override;

namespace {
std::mutex g_scratch_mutex;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<Scratch>> g_scratch;
std::mutex g_order_mutex;
std::map<int, std::unique_ptr<LaunchOrder>> g_order;
}  // namespace

// Created with its event on first use (the event records no timing).
// nullptr if the host is out of memory or the event cannot be created: no
// exception leaves the library.
LaunchOrder* launch_order(int device) {
    std::lock_guard<std::mutex> g(g_order_mutex);
    try {
        auto& slot = g_order[device];
        if (!slot) {
            std::unique_ptr<LaunchOrder> o(new LaunchOrder());
            if (hipEventCreateWithFlags(&o->last, hipEventDisableTiming) != hipSuccess)
                return nullptr;
            slot = std::move(o);
        }
        return slot.get();
    } catch (...) {
        return nullptr;
    }
}

// nullptr if the host is out of memory.
Scratch* scratch_for(int device, hipStream_t stream) {
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    try {
        auto& slot = g_scratch[{device, reinterpret_cast<uintptr_t>(stream)}];
        if (!slot) slot.reset(new Scratch());
        return slot.get();
    } catch (...) {
        return nullptr;
    }
}

// A grid-stride loop of plain vector stores.
__global__ __launch_bounds__(256) void clear_kernel(uint64_t* p, int64_t words) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
         i += stride)
        p[i] = 0;
}

hipError_t clear_words(uint64_t* p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    int64_t grid = (words + 255) / 256;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p,
                       words);
    return hipGetLastError();
}

int ensure_capacity(Scratch* sc, hipStream_t stream, int64_t tiles) {
    if (sc->fixed) {
        if (tiles > sc->capacity) return RLSCAN_ERR_SCRATCH;
        if (!sc->broken) return RLSCAN_OK;
        // a failed launch left the ticket counter at an unknown value: start
        // the array afresh (status words and counters)
        const int64_t words = static_cast<int64_t>(sizeof(TileStatus) / 8) * sc->capacity;
        if (clear_words(reinterpret_cast<uint64_t*>(sc->status), words, stream) != hipSuccess ||
            clear_words(reinterpret_cast<uint64_t*>(sc->counter), 256 / 8, stream) != hipSuccess)
            return RLSCAN_ERR_HIP;
        sc->next_ticket = 0;
        sc->epoch = 0;
        sc->broken = false;
        return RLSCAN_OK;
    }
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
    if (clear_words(static_cast<uint64_t*>(st), static_cast<int64_t>(sizeof(TileStatus) / 8) * cap,
                    stream) != hipSuccess ||
        clear_words(static_cast<uint64_t*>(ctr), 256 / 8, stream) != hipSuccess) {
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

// Rounds per tile: one up to 2^20 elements (the production shapes: more,
// smaller workgroups in flight), two below 2^22, four from there (measured
// at 8 x 2^19: four rounds 8-30 % faster than two).  Retrace keeps its
// action values per round in registers: always one.
int auto_rounds(int est, int64_t NT) {
    if (est == RLSCAN_EST_RETRACE) return 1;
    if (NT <= (int64_t(1) << 20)) return 1;
    if (NT < (int64_t(1) << 22) || est == kEstVtraceWide) return 2;
    return 4;
}

// Waves per workgroup (the tile is 256*W*R elements).
//  - Four rounds (long inputs): four waves.  Eight double the tile, which
//    halves the look-back waits per element but also the workgroups that fit
//    on a CU; with the narrow first poll of the look-back the waits are
//    cheap, and four waves measured as fast or faster for every estimator
//    (8 x 2^20: discounted 32.9 -> 31.4 us, eligibility 20.9 -> 20.0, prefix
//    28.0 -> 27.6; GAE 47.5 -> 36.6).
//  - One round (at most 2^20 elements, bound by launch and one memory round
//    trip): the smallest tile that still holds whole rows -- more, smaller
//    workgroups in flight.  Measured at 4096 x 128: one wave beat four by
//    2-8 %, two waves by as much for GAE and V-trace.  Where no tile of up
//    to eight waves holds whole rows (the look-back mapping), eight waves:
//    half the tiles, so half the look-back waits.  Measured on GAE, V-trace
//    and discounted returns against four waves: 64 x 8192 and 16 x 32768
//    5-7 % faster, 8 x 131072 12-18 % faster (Retrace stays at four).
//  - Two rounds: eight waves.  Measured against four: 32 x 65536 (look-back)
//    10-18 % faster; 4096 x 512 and 16384 x 128 (packed) up to 12 % for GAE
//    and V-trace, the same within 4 % for the others.
//    V-trace's float64 form takes four: at two rounds of eight waves it
//    needs 178 VGPRs (one workgroup per CU), at four waves 162 (three);
//    measured with c_bar = 2: 8 x 2^20 75.6 -> 58.2 us, 32 x 65536
//    21.1 -> 19.8 us.
//    Where T divides no such tile, the smallest tile whose whole rows fill
//    at least 7/8 of it (100-step rows: 500 of 512 elements), else the
//    best-filled one if its rows fill at least 3/4.  Retrace and the prefix
//    sum take the smallest tile filled to 3/4: measured at 2^19 elements,
//    one wave beat two for Retrace at T = 96, 100 and 200 (9.20 / 9.56 /
//    9.56 us against 9.91 / 10.15 / 9.84) and for the prefix sum at T = 96
//    and 100 (3.64 / 3.92 against 3.84 / 4.06); for the others the two were
//    within a few per cent, either way between runs.
int auto_waves(int est, int rounds, int64_t N, int64_t T) {
    if (rounds == 4) return 4;
    if (rounds == 1) {
        const int first =
            (est == RLSCAN_EST_GAE || est == RLSCAN_EST_VTRACE || est == kEstVtraceWide) ? 2 : 1;
        const int last = est == RLSCAN_EST_RETRACE ? 4 : 8;
        for (int w = first; w <= last; w *= 2)
            if ((int64_t(kWave) * w * kChunk) % T == 0) return w;
        const int64_t enough =  // fill (in 1/1024 of the tile) taken at once
            (est == RLSCAN_EST_RETRACE || est == RLSCAN_EST_PREFIX_SUM) ? 768 : 896;
        int best = 0;
        int64_t best_fill = 0;
        for (int w = first; w <= last; w *= 2) {
            const int64_t cap = int64_t(kWave) * w * kChunk;
            int64_t span = 0, tiles = 0;
            if (!packed_layout(N, T, cap, span, tiles)) continue;
            const int64_t fill = span * 1024 / cap;
            if (fill >= enough) return w;
            if (fill > best_fill) best = w, best_fill = fill;
        }
        if (best_fill >= 768) return best;
        return last;
    }
    return est == kEstVtraceWide ? 4 : 8;  // two rounds
}

Plan make_plan(int est, int64_t N, int64_t T, bool vec, bool carry) {
    const int64_t NT = N * T;
    Plan pl;
    const int ro = g_override.rounds.load();
    pl.rounds = ro > 0 ? ro : auto_rounds(est, NT);
    if (!vec || est == RLSCAN_EST_RETRACE) pl.rounds = 1;
    if (est == kEstVtraceWide && pl.rounds > 2) pl.rounds = 2;
    const int wo = g_override.waves.load();
    pl.waves = wo > 0 ? wo : auto_waves(est, pl.rounds, N, T);
    // kernels exist for 1 and 2 waves with one round only, for 8 waves not
    // for Retrace, for the unaligned path with 4 waves only and for the
    // carry path with 4 or 8
    if (pl.waves < 4 && pl.rounds != 1) pl.waves = 4;
    if (pl.waves == 8 && est == RLSCAN_EST_RETRACE) pl.waves = 4;
    if (!vec || (carry && pl.waves != 8)) pl.waves = 4;
    pl.tile_elems = int64_t(kWave) * pl.waves * kChunk * pl.rounds;
    // Packed when every tile can hold whole rows and (unless forced) they
    // fill at least 3/4 of it: the lanes past the rows idle, but no tile
    // waits on another.
    int64_t span = 0, tiles = 0;
    const bool can_pack = packed_layout(N, T, pl.tile_elems, span, tiles);
    const bool filled = can_pack && (tiles == 1 || 4 * span >= 3 * pl.tile_elems);
    const int mo = g_override.mapping.load();
    const bool packed = mo == RLSCAN_MAP_PACKED ? can_pack : (mo == RLSCAN_MAP_AUTO && filled);
    pl.mapping = packed ? RLSCAN_MAP_PACKED : RLSCAN_MAP_LOOKBACK;
    pl.tile_span = packed ? span : pl.tile_elems;
    pl.tiles = packed ? tiles : (NT + pl.tile_elems - 1) / pl.tile_elems;
    const int64_t cap = g_override.grid_cap.load();
    int64_t grid = pl.tiles;
    if (cap > 0 && grid > cap) grid = cap;
    if (grid > kMaxGrid) grid = kMaxGrid;
    pl.grid = grid;
    return pl;
}

// The library's choice of XCD runs (xcd_tile): runs of 16 tiles when a
// tile's span is not a multiple of 128 bytes (32 elements), so that most
// lines shared by neighbouring tiles stay in one L2; else tile = blockIdx.
// Measured on MI355X (cold inputs): runs of 16 made such calls 1-5 % faster
// (4200 x 125: prefix sum 4.34 -> 4.14 us; 4096 x 100: Retrace 8.78 -> 8.43
// us), one contiguous run per XCD 5-9 % on another box; on aligned calls
// (4096 x 128) runs cost up to 5 %, and one contiguous run per XCD made the
// 2^20 x 32 calls 13 % and the grouped production step 50 % slower.
int64_t xcd_run(int64_t tiles, int64_t span) {
    const int64_t o = g_override.xcd_run.load();
    if (o >= 0) return o;
    return (span % 32 != 0 && tiles > 1) ? 16 : 0;
}

int64_t group_xcd_run() {
    const int64_t o = g_override.xcd_run.load();
    return o >= 0 ? o : 0;
}

// An empty kernel: the launch floor that a scan launch of the same grid and
// workgroup size cannot go below.
__global__ __launch_bounds__(1024) void empty_kernel() {}

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

// A streaming kernel with a read:write mix: each thread reads `reads`
// 16-byte words of `src` (at most kMixMaxReads) and then writes `writes`
// words of `dst` (at most kMixMaxWrites), every written word the sum of the
// thread's read words -- all reads are used before any write, as in a scan
// kernel.  Workgroup b reads the contiguous words [b*256*reads, ...) and
// writes [b*256*writes, ...); accesses are 16-byte and non-temporal.
constexpr int kMixThreads = 256;
constexpr int kMixMaxReads = 16;
constexpr int kMixMaxWrites = 4;
__global__ __launch_bounds__(kMixThreads) void mix_kernel(const f32x4* __restrict__ src,
                                                          int64_t nr, f32x4* __restrict__ dst,
                                                          int64_t nw, int reads, int writes) {
    const int64_t rb = static_cast<int64_t>(blockIdx.x) * kMixThreads * reads + threadIdx.x;
    f32x4 v[kMixMaxReads];
#pragma unroll
    for (int u = 0; u < kMixMaxReads; ++u) {
        const int64_t i = rb + static_cast<int64_t>(u) * kMixThreads;
        v[u] = 0.0f;
        if (u < reads && i < nr) v[u] = __builtin_nontemporal_load(src + i);
    }
    f32x4 acc = v[0];
#pragma unroll
    for (int u = 1; u < kMixMaxReads; ++u) acc += v[u];
    const int64_t wb = static_cast<int64_t>(blockIdx.x) * kMixThreads * writes + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kMixMaxWrites; ++u) {
        const int64_t i = wb + static_cast<int64_t>(u) * kMixThreads;
        if (u < writes && i < nw) __builtin_nontemporal_store(acc, dst + i);
    }
}

// The same reference in a scan's access pattern: `ain` input arrays and
// `aout` output arrays of n_in and n_out 16-byte words.  Indices are laid
// out as the scan lays out its chunks: lane l of wave w in workgroup b takes
// indices b*256*words + (w*words + u)*64 + l (u < words), so each wave
// covers `words` consecutive KiB of every array.  It reads that word of
// every input array and writes their sum to that word of every output
// array.  Indices past an array's end read as zero / are not written.
constexpr int kMixMaxWords = 4;
template <int WORDS>
__global__ __launch_bounds__(kMixThreads) void mix_arrays_kernel(
    const f32x4* __restrict__ src, int64_t n_in, f32x4* __restrict__ dst, int64_t n_out, int ain,
    int aout) {
    constexpr int kArrays = kMixMaxReads / WORDS;  // most input arrays at this width
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kMixThreads * WORDS +
                         static_cast<int64_t>(wave) * WORDS * kWave + lane;
    f32x4 v[kArrays][WORDS];
#pragma unroll
    for (int a = 0; a < kArrays; ++a)
#pragma unroll
        for (int u = 0; u < WORDS; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kWave;
            v[a][u] = 0.0f;
            if (a < ain && i < n_in) v[a][u] = __builtin_nontemporal_load(src + a * n_in + i);
        }
#pragma unroll
    for (int u = 0; u < WORDS; ++u) {
        f32x4 acc = v[0][u];
#pragma unroll
        for (int a = 1; a < kArrays; ++a) acc += v[a][u];
        const int64_t i = base + static_cast<int64_t>(u) * kWave;
#pragma unroll
        for (int o = 0; o < kMixMaxWrites; ++o)
            if (o < aout && i < n_out) __builtin_nontemporal_store(acc, dst + o * n_out + i);
    }
}

}  // namespace rlscan

using namespace rlscan;

extern "C" {

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
        case RLSCAN_ERR_SCRATCH:
            return "the call needs more look-back tiles than the fixed scratch array holds";
        default: return "unknown rlscan status";
    }
}

const char* rlscan_version(void) { return "rlscan 0.1.0 gfx950"; }

// The Scratch objects themselves stay (a call on another thread may hold a
// pointer to one): only their device buffers are freed, under each object's
// own lock, and the next call that needs one allocates it afresh.
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
        sc->broken = false;
    }
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
    info->tile_span = pl.tile_span;
    info->tiles = pl.tiles;
    info->grid = pl.grid;
    return RLSCAN_OK;
}

int rlscan_launch_floor(int64_t grid, int32_t threads, hipStream_t stream) {
    if (grid < 1 || grid > kMaxGrid) return RLSCAN_ERR_SHAPE;
    if (threads < kWave || threads > 1024 || threads % kWave != 0) return RLSCAN_ERR_SHAPE;
    hipLaunchKernelGGL(empty_kernel, dim3(static_cast<unsigned>(grid)),
                       dim3(static_cast<unsigned>(threads)), 0, stream);
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

// Waits for each device that holds look-back scratch (not for the streams
// the scratch was keyed by: the caller may have destroyed them since).
int rlscan_stream_mix(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                      int32_t reads, int32_t writes, hipStream_t stream) {
    if (read_bytes < 0 || write_bytes < 0 || (read_bytes & 15) != 0 || (write_bytes & 15) != 0)
        return RLSCAN_ERR_SHAPE;
    if (reads < 1 || reads > kMixMaxReads || writes < 1 || writes > kMixMaxWrites)
        return RLSCAN_ERR_PARAM;
    if (read_bytes == 0 && write_bytes == 0) return RLSCAN_OK;
    if ((read_bytes > 0 && src == nullptr) || (write_bytes > 0 && dst == nullptr))
        return RLSCAN_ERR_NULL;
    if ((src != nullptr && !aligned16(src)) || (dst != nullptr && !aligned16(dst)))
        return RLSCAN_ERR_PARAM;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (read_bytes > 0 && write_bytes > 0 && d < s + static_cast<uintptr_t>(read_bytes) &&
        s < d + static_cast<uintptr_t>(write_bytes))
        return RLSCAN_ERR_ALIAS;
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    const int64_t gr = (nr + int64_t(kMixThreads) * reads - 1) / (int64_t(kMixThreads) * reads);
    const int64_t gw = (nw + int64_t(kMixThreads) * writes - 1) / (int64_t(kMixThreads) * writes);
    const int64_t grid = gr > gw ? gr : gw;
    if (grid > kMaxGrid) return RLSCAN_ERR_SHAPE;
    hipLaunchKernelGGL(mix_kernel, dim3(static_cast<unsigned>(grid)), dim3(kMixThreads), 0,
                       stream, static_cast<const f32x4*>(src), nr, static_cast<f32x4*>(dst), nw,
                       reads, writes);
    return hipGetLastError() == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
}

int rlscan_stream_mix_arrays(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                             int32_t arrays_in, int32_t arrays_out, int32_t words,
                             int32_t workgroups_per_cu, hipStream_t stream) {
    if (read_bytes < 0 || write_bytes < 0) return RLSCAN_ERR_SHAPE;
    if (arrays_in < 1 || arrays_in > kMixMaxReads || arrays_out < 1 ||
        arrays_out > kMixMaxWrites || words < 1 || words > kMixMaxWords ||
        arrays_in * words > kMixMaxReads || workgroups_per_cu < 0 || workgroups_per_cu == 1 ||
        workgroups_per_cu > 8)
        return RLSCAN_ERR_PARAM;
    if (read_bytes % (16 * int64_t(arrays_in)) != 0 || write_bytes % (16 * int64_t(arrays_out)) != 0)
        return RLSCAN_ERR_SHAPE;
    if (read_bytes == 0 && write_bytes == 0) return RLSCAN_OK;
    if ((read_bytes > 0 && src == nullptr) || (write_bytes > 0 && dst == nullptr))
        return RLSCAN_ERR_NULL;
    if ((src != nullptr && !aligned16(src)) || (dst != nullptr && !aligned16(dst)))
        return RLSCAN_ERR_PARAM;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (read_bytes > 0 && write_bytes > 0 && d < s + static_cast<uintptr_t>(read_bytes) &&
        s < d + static_cast<uintptr_t>(write_bytes))
        return RLSCAN_ERR_ALIAS;
    const int64_t n_in = read_bytes / 16 / arrays_in, n_out = write_bytes / 16 / arrays_out;
    const int64_t n = n_in > n_out ? n_in : n_out;
    const int64_t per_group = int64_t(kMixThreads) * words;
    const int64_t grid = (n + per_group - 1) / per_group;
    if (grid > kMaxGrid) return RLSCAN_ERR_SHAPE;
    // the residency cap: an unused share of the CU's LDS per workgroup, just
    // over 1/(cap+1) of it, so that at most `cap` fit
    size_t lds = 0;
    if (workgroups_per_cu > 0) {
        int dev = 0, per_cu = 0, per_block = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess)
            return RLSCAN_ERR_HIP;
        lds = static_cast<size_t>(per_cu) / (workgroups_per_cu + 1) + 1024;
        if (lds > static_cast<size_t>(per_block) ||
            lds * workgroups_per_cu > static_cast<size_t>(per_cu))
            return RLSCAN_ERR_PARAM;
    }
    const dim3 g(static_cast<unsigned>(grid)), b(kMixThreads);
    const f32x4* in = static_cast<const f32x4*>(src);
    f32x4* out = static_cast<f32x4*>(dst);
    switch (words) {
        case 1:
            hipLaunchKernelGGL(mix_arrays_kernel<1>, g, b, lds, stream, in, n_in, out, n_out,
                               arrays_in, arrays_out);
            break;
        case 2:
            hipLaunchKernelGGL(mix_arrays_kernel<2>, g, b, lds, stream, in, n_in, out, n_out,
                               arrays_in, arrays_out);
            break;
        case 3:
            hipLaunchKernelGGL(mix_arrays_kernel<3>, g, b, lds, stream, in, n_in, out, n_out,
                               arrays_in, arrays_out);
            break;
        default:
            hipLaunchKernelGGL(mix_arrays_kernel<4>, g, b, lds, stream, in, n_in, out, n_out,
                               arrays_in, arrays_out);
            break;
    }
    return hipGetLastError() == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP;
}

int rlscan_set_xcd_run(int64_t run) {
    if (run < -1 || run > (int64_t(1) << 20)) return RLSCAN_ERR_PARAM;
    g_override.xcd_run.store(run);
    return RLSCAN_OK;
}

int rlscan_lookback_timeouts(uint64_t* count) {
    if (count == nullptr) return RLSCAN_ERR_NULL;
    *count = 0;
    int rc = RLSCAN_OK;
    {
        std::lock_guard<std::mutex> g(g_scratch_mutex);
        int prev = 0;
        const bool have_prev = hipGetDevice(&prev) == hipSuccess;
        int synced = -1;
        for (auto& kv : g_scratch) {  // ordered by device
            Scratch* sc = kv.second.get();
            std::lock_guard<std::mutex> gs(sc->m);
            if (sc->counter == nullptr) continue;
            unsigned int n = 0;
            const int dev = kv.first.first;
            if (hipSetDevice(dev) != hipSuccess ||
                (synced != dev && hipDeviceSynchronize() != hipSuccess) ||
                hipMemcpy(&n, sc->counter + 1, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) {
                rc = RLSCAN_ERR_HIP;
                continue;
            }
            synced = dev;
            *count += n;
        }
        if (have_prev) (void)hipSetDevice(prev);
    }
    uint64_t fixed = 0;
    const int rs = static_scratch_timeouts(&fixed);
    *count += fixed;
    return rc != RLSCAN_OK ? rc : rs;
}

int rlscan_set_launch_override(int mapping, int rounds, int waves, int64_t grid_cap, int flags) {
    if (mapping < RLSCAN_MAP_AUTO || mapping > RLSCAN_MAP_LOOKBACK) return RLSCAN_ERR_PARAM;
    if (rounds != 0 && rounds != 1 && rounds != 2 && rounds != 4) return RLSCAN_ERR_PARAM;
    if (waves != 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8)
        return RLSCAN_ERR_PARAM;
    if (grid_cap < 0 || (flags & ~(RLSCAN_FLAG_TICKETS | RLSCAN_FLAG_GROUP_INTERLEAVED |
                                    RLSCAN_FLAG_LOOKBACK_GIVE_UP)) != 0)
        return RLSCAN_ERR_PARAM;
    g_override.mapping.store(mapping);
    g_override.rounds.store(rounds);
    g_override.waves.store(waves);
    g_override.grid_cap.store(grid_cap);
    g_override.flags.store(flags);
    return RLSCAN_OK;
}

}  // extern "C"
