// est_episodic_prefix_sum.hip -- C entry points of the episodic prefix sum (rlscan_episodic_prefix_sum, rlscan_episodic_prefix_sum_carry, rlscan_episodic_prefix_sum_u8):
// argument checks, then the scan kernel instantiated for its estimator
// (estimators.hpp) through the shared launch path (host.hpp).  The flag
// element type F is float for the plain entry points and uint8_t for the
// `_u8` ones; both run the same arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "host.hpp"

using namespace rlscan;

namespace {

template <class F>
int prefix_sum(const int32_t* x, const F* dones, const int64_t* carry_in, int64_t* out,
               int64_t* carry_out, int64_t N, int64_t T, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!x || !dones || !out) return RLSCAN_ERR_NULL;
    rc = check_alias({out, carry_out}, {x, dones, carry_in});
    if (rc != RLSCAN_OK) return rc;
    typename PrefixSum<F>::Params p{x, dones, out, carry_in, carry_out};
    const bool vec = all_aligned({x, out}) && flags_aligned(dones);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_PREFIX_SUM, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return launch_kernel<PrefixSum<F>>(p, g, lb, pl, vec, carry, stream);
               });
}

}  // namespace

extern "C" {

int rlscan_episodic_prefix_sum_carry(const int32_t* x, const float* dones,
                                     const int64_t* carry_in, int64_t* out, int64_t* carry_out,
                                     int64_t N, int64_t T, hipStream_t stream) {
    return prefix_sum(x, dones, carry_in, out, carry_out, N, T, stream);
}

int rlscan_episodic_prefix_sum_u8(const int32_t* x, const uint8_t* dones,
                                  const int64_t* carry_in, int64_t* out, int64_t* carry_out,
                                  int64_t N, int64_t T, hipStream_t stream) {
    return prefix_sum(x, dones, carry_in, out, carry_out, N, T, stream);
}

int rlscan_episodic_prefix_sum(const int32_t* x, const float* dones, int64_t* out, int64_t N,
                               int64_t T, hipStream_t stream) {
    return prefix_sum(x, dones, nullptr, out, nullptr, N, T, stream);
}

}  // extern "C"
