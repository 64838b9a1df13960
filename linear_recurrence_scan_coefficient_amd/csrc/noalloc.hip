// noalloc.hip -- rlscan_gae_noalloc: rlscan_gae_carry for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The only device memory the GAE kernels use beyond the caller's inputs and
// outputs is the look-back scratch of calls whose rows span several tiles:
// 32 bytes of status words per tile plus a ticket and a timeout counter.
// Here it is one file-scope device array, `scratch`, of fixed size: each GPU
// the library runs on holds its own copy from module load until the process
// ends.  Its address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever passed to kernels; the
// array's name in host code is a host-side stand-in, not a device address.
//
// Contents persist between calls.  The status words carry the tag of the
// call that wrote them, so a later call never reads an earlier call's words
// as its own; the tags repeat only after 2^31 - 2 look-back calls, and then
// the words are cleared by a kernel first (as after a failed launch, which
// leaves the ticket counter at an unknown value).  Calls that overlap on one
// GPU share the array and race: run them on one stream, and keep them from
// overlapping with the library's other look-back launches on that GPU.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "host.hpp"

using namespace rlscan;

namespace {

// 65536 tiles: rows of up to 2^28 elements (4096-element tiles).
constexpr int64_t kFixedTiles = 65536;
constexpr size_t kCounterBytes = 256;
constexpr size_t kScratchBytes = kCounterBytes + sizeof(TileStatus) * kFixedTiles;  // 2 MiB + 256 B

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceArray {
    std::mutex m;
    bool ready = false;
    Scratch sc;  // sc.fixed: the counters and status words live in `scratch`
};
DeviceArray g_arrays[kMaxDevices];

// The device's copy of the array, its address looked up on first use.
Scratch* fixed_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    DeviceArray& d = g_arrays[device];
    std::lock_guard<std::mutex> g(d.m);
    if (!d.ready) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        unsigned char* base = static_cast<unsigned char*>(ptr);
        d.sc.counter = reinterpret_cast<unsigned long long*>(base);
        d.sc.status = reinterpret_cast<TileStatus*>(base + kCounterBytes);
        d.sc.capacity = kFixedTiles;
        d.sc.fixed = true;
        d.ready = true;  // zero at module load: tags start at 1, tickets at 0
    }
    return &d.sc;
}

const ScratchSource kFixed{fixed_scratch, kFixedTiles};

}  // namespace

namespace rlscan {

int static_scratch_timeouts(uint64_t* count) {
    *count = 0;
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    int rc = RLSCAN_OK;
    for (int dev = 0; dev < kMaxDevices; ++dev) {
        DeviceArray& d = g_arrays[dev];
        std::lock_guard<std::mutex> g(d.m);
        if (!d.ready) continue;
        std::lock_guard<std::mutex> gs(d.sc.m);
        unsigned int n = 0;
        if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(&n, d.sc.counter + 1, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) {
            rc = RLSCAN_ERR_HIP;
            continue;
        }
        *count += n;
    }
    if (have_prev) (void)hipSetDevice(prev);
    return rc;
}

}  // namespace rlscan

extern "C" {

int rlscan_gae_noalloc(const float* rewards, const float* values, const float* bootstrap_value,
                       const float* terminated, const float* truncated,
                       const float* bootstrap_values, const float* carry_in, float* advantages,
                       float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                       hipStream_t stream) {
    return gae_with_scratch(rewards, values, bootstrap_value, terminated, truncated,
                            bootstrap_values, carry_in, advantages, carry_out, N, T, gamma, lambda,
                            stream, &kFixed);
}

}  // extern "C"
