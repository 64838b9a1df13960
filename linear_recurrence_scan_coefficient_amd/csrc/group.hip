// group.hip -- rlscan_group: several independent estimator calls in one
// kernel launch (group.hpp).  Each call goes through its own entry point
// with a collector installed, so it is checked and planned exactly as when
// called alone; the collected tiles are then launched together.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "host.hpp"

using namespace rlscan;

namespace rlscan {

template <int W, bool kWide>
static hipError_t launch_group_w(const GroupArgs& args, size_t lds, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.first_block[args.count])), block(kWave * W);
    hipLaunchKernelGGL((group_kernel<W, kWide>), grid, block, static_cast<unsigned>(lds), stream,
                       args);
    return hipGetLastError();
}

hipError_t launch_group(const GroupArgs& args, int waves, bool wide, size_t lds,
                        hipStream_t stream) {
    switch (waves) {
        case 1: return wide ? launch_group_w<1, true>(args, lds, stream)
                            : launch_group_w<1, false>(args, lds, stream);
        case 2: return wide ? launch_group_w<2, true>(args, lds, stream)
                            : launch_group_w<2, false>(args, lds, stream);
        default: return wide ? launch_group_w<4, true>(args, lds, stream)
                             : launch_group_w<4, false>(args, lds, stream);
    }
}

}  // namespace rlscan

namespace {

static_assert(sizeof(rlscan_call) == 136 && offsetof(rlscan_call, in) == 56 &&
                  offsetof(rlscan_call, out) == 120,
              "rlscan_call layout");

// Waves per workgroup of the grouped launches: the override if one is set,
// else the smallest count (at least kGroupWavesMin) whose tile holds whole
// rows of every call filling at least 3/4 of it, else the smallest whose
// tile holds a whole row of every call; 0 if none does.  Measured on the
// seven 4096 x 128 production calls: two waves 16.5 us per group, one wave
// 17.1 us.
constexpr int kGroupWavesMin = 2;

int group_waves(const rlscan_call* calls, int32_t count) {
    const int wo = g_override.waves.load();
    const bool forced = wo == 1 || wo == 2 || wo == 4;
    const int first = forced ? wo : kGroupWavesMin;
    for (int pass = 0; pass < 2; ++pass) {
        for (int w = first; w <= 4; w *= 2) {
            const int64_t tile = int64_t(kWave) * w * kChunk;
            bool ok = true;
            for (int32_t i = 0; i < count && ok; ++i) {
                const int64_t N = calls[i].N, T = calls[i].T;
                if (N <= 0 || T <= 0 || N > kMaxElements / T) continue;  // rejected later
                int64_t span = 0, tiles = 0;
                ok = packed_layout(N, T, tile, span, tiles) &&
                     (pass == 1 || tiles == 1 || 4 * span >= 3 * tile);
            }
            if (ok) return w;
            if (forced) break;
        }
    }
    return 0;
}

int collect(const rlscan_call& c, hipStream_t stream) {
    const bool byte = (c.flags & RLSCAN_CALL_BYTE_FLAGS) != 0;
    auto f = [&](int i) { return static_cast<const float*>(c.in[i]); };
    auto u = [&](int i) { return static_cast<const uint8_t*>(c.in[i]); };
    float* o0 = static_cast<float*>(c.out[0]);
    float* o1 = static_cast<float*>(c.out[1]);
    switch (c.estimator) {
        case RLSCAN_EST_GAE:
            return byte ? rlscan_gae_u8(f(0), f(1), f(2), u(3), u(4), f(5), nullptr, o0, nullptr,
                                        c.N, c.T, c.gamma, c.lambda, stream)
                        : rlscan_gae_carry(f(0), f(1), f(2), f(3), f(4), f(5), nullptr, o0,
                                           nullptr, c.N, c.T, c.gamma, c.lambda, stream);
        case RLSCAN_EST_LAMBDA_RETURNS:
            return byte ? rlscan_lambda_returns_u8(f(0), f(1), f(2), u(3), u(4), f(5), nullptr, o0,
                                                   nullptr, c.N, c.T, c.gamma, c.lambda, stream)
                        : rlscan_lambda_returns_carry(f(0), f(1), f(2), f(3), f(4), f(5), nullptr,
                                                      o0, nullptr, c.N, c.T, c.gamma, c.lambda,
                                                      stream);
        case RLSCAN_EST_DISCOUNTED:
            return byte ? rlscan_discounted_returns_u8(f(0), f(1), u(2), u(3), f(4), nullptr, o0,
                                                       nullptr, c.N, c.T, c.gamma, stream)
                        : rlscan_discounted_returns_carry(f(0), f(1), f(2), f(3), f(4), nullptr,
                                                          o0, nullptr, c.N, c.T, c.gamma, stream);
        case RLSCAN_EST_VTRACE:
            return byte ? rlscan_vtrace_u8(f(0), f(1), f(2), f(3), u(4), u(5), f(6), nullptr, o0,
                                           o1, nullptr, c.N, c.T, c.gamma, c.lambda, c.rho_bar,
                                           c.c_bar, c.rho_bar_pg, stream)
                        : rlscan_vtrace_ex(f(0), f(1), f(2), f(3), f(4), f(5), f(6), nullptr, o0,
                                           o1, nullptr, c.N, c.T, c.gamma, c.lambda, c.rho_bar,
                                           c.c_bar, c.rho_bar_pg, stream);
        case RLSCAN_EST_RETRACE: {
            const int32_t* acts = static_cast<const int32_t*>(c.in[3]);
            return byte ? rlscan_retrace_u8(f(0), f(1), f(2), acts, f(4), u(5), u(6), nullptr,
                                            nullptr, nullptr, o0, nullptr, c.N, c.T, c.A, c.gamma,
                                            c.lambda, stream)
                        : rlscan_retrace_carry(f(0), f(1), f(2), acts, f(4), f(5), f(6), nullptr,
                                               nullptr, nullptr, o0, nullptr, c.N, c.T, c.A,
                                               c.gamma, c.lambda, stream);
        }
        case RLSCAN_EST_ELIGIBILITY:
            return byte ? rlscan_eligibility_traces_u8(f(0), u(1), nullptr, o0, nullptr, c.N, c.T,
                                                       c.gamma, c.lambda, stream)
                        : rlscan_eligibility_traces_carry(f(0), f(1), nullptr, o0, nullptr, c.N,
                                                          c.T, c.gamma, c.lambda, stream);
        case RLSCAN_EST_PREFIX_SUM: {
            const int32_t* x = static_cast<const int32_t*>(c.in[0]);
            int64_t* out = static_cast<int64_t*>(c.out[0]);
            return byte ? rlscan_episodic_prefix_sum_u8(x, u(1), nullptr, out, nullptr, c.N, c.T,
                                                        stream)
                        : rlscan_episodic_prefix_sum_carry(x, f(1), nullptr, out, nullptr, c.N,
                                                           c.T, stream);
        }
        default:
            return RLSCAN_ERR_PARAM;
    }
}

// No call may write a buffer another call reads or writes (exact pointer
// equality, as the single calls check their own outputs).
bool independent(const rlscan_call* calls, int32_t count) {
    for (int32_t i = 0; i < count; ++i)
        for (const void* o : calls[i].out) {
            if (o == nullptr) continue;
            for (int32_t j = 0; j < count; ++j) {
                if (j == i) continue;
                for (const void* x : calls[j].in)
                    if (x == o) return false;
                for (const void* x : calls[j].out)
                    if (x == o) return false;
            }
        }
    return true;
}

struct CollectorScope {
    explicit CollectorScope(GroupCollector* c) { t_group = c; }
    ~CollectorScope() { t_group = nullptr; }
};

int group(const rlscan_call* calls, int32_t count, hipStream_t stream) {
    if (count < 0) return RLSCAN_ERR_SHAPE;
    if (count == 0) return RLSCAN_OK;
    if (calls == nullptr) return RLSCAN_ERR_NULL;
    if (!independent(calls, count)) return RLSCAN_ERR_ALIAS;
    GroupCollector col;
    col.waves = group_waves(calls, count);
    if (col.waves == 0) return RLSCAN_ERR_PARAM;
    {
        CollectorScope scope(&col);
        for (int32_t i = 0; i < count; ++i) {
            const int rc = collect(calls[i], stream);
            if (rc != RLSCAN_OK) return rc;
            if (col.reject) return RLSCAN_ERR_PARAM;
        }
    }
    // batches of at most kGroupMax calls and kMaxGrid workgroups
    const size_t n = col.entries.size();
    for (const GroupEntry& e : col.entries)
        if (e.geo.num_tiles > kMaxGrid) return RLSCAN_ERR_SHAPE;
    size_t start = 0;
    while (start < n) {
        GroupArgs a{};
        int64_t blocks = 0;
        int32_t k = 0;
        bool wide = false;
        while (start + k < n && k < kGroupMax &&
               blocks + col.entries[start + k].geo.num_tiles <= kMaxGrid) {
            a.first_block[k] = blocks;
            a.e[k] = col.entries[start + k];
            blocks += col.entries[start + k].geo.num_tiles;
            wide = wide || col.wide[start + k];
            ++k;
        }
        a.count = k;
        for (int32_t j = k; j <= kGroupMax; ++j) a.first_block[j] = blocks;
        a.interleaved = (g_override.flags.load() & RLSCAN_FLAG_GROUP_INTERLEAVED) ? 1 : 0;
        a.xcd_run = static_cast<int32_t>(group_xcd_run());
        // interleaved schedule: calls by ascending tile count; segment s runs
        // the calls order[s..k-1] for the tiles the shorter ones do not have
        for (int32_t j = 0; j < k; ++j) a.order[j] = j;
        for (int32_t j = 1; j < k; ++j)  // insertion sort: stable, k <= 8
            for (int32_t q = j; q > 0 && a.e[a.order[q]].geo.num_tiles <
                                             a.e[a.order[q - 1]].geo.num_tiles; --q) {
                const int32_t t = a.order[q];
                a.order[q] = a.order[q - 1];
                a.order[q - 1] = t;
            }
        int64_t seg_block = 0, done_tiles = 0;
        for (int32_t sg = 0; sg < k; ++sg) {
            const int64_t tiles = a.e[a.order[sg]].geo.num_tiles;
            a.seg_first[sg] = static_cast<int32_t>(seg_block);
            a.seg_tile0[sg] = static_cast<int32_t>(done_tiles);
            seg_block += (tiles - done_tiles) * (k - sg);  // sums to `blocks`
            done_tiles = tiles;
        }
        for (int32_t sg = k; sg <= kGroupMax; ++sg) a.seg_first[sg] = static_cast<int32_t>(blocks);
        if (launch_group(a, col.waves, wide, col.lds, stream) != hipSuccess)
            return RLSCAN_ERR_HIP;
        start += k;
    }
    return RLSCAN_OK;
}

}  // namespace

extern "C" {

// The collector's table lives on the host heap: an allocation failure is
// returned as RLSCAN_ERR_ALLOC, never thrown across the C interface.
int rlscan_group(const rlscan_call* calls, int32_t count, hipStream_t stream) {
    try {
        return group(calls, count, stream);
    } catch (...) {
        t_group = nullptr;
        return RLSCAN_ERR_ALLOC;
    }
}

}  // extern "C"
