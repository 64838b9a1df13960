// est_discounted_returns.hip -- C entry points of discounted returns (rlscan_discounted_returns, rlscan_discounted_returns_carry, rlscan_discounted_returns_u8):
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
int discounted_returns(const float* rewards, const float* bootstrap_value, const F* terminated,
                       const F* truncated, const float* bootstrap_values, const float* carry_in,
                       float* returns, float* carry_out, int64_t N, int64_t T, float gamma,
                       hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !terminated || !returns) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({returns, carry_out}, {rewards, bootstrap_value, terminated, truncated,
                                            bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const DiscountedParams<F> p{rewards,  bootstrap_value, terminated, truncated,
                                bootstrap_values, carry_in, returns, carry_out, gamma};
    const bool vec = all_aligned({rewards, bootstrap_values, returns}) &&
                     flags_aligned(terminated) && flags_aligned(truncated);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_DISCOUNTED, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated ? launch_kernel<Discounted<true, F>>(p, g, lb, pl, vec, carry,
                                                                         stream)
                                    : launch_kernel<Discounted<false, F>>(p, g, lb, pl, vec,
                                                                          carry, stream);
               });
}

}  // namespace

extern "C" {

int rlscan_discounted_returns_carry(const float* rewards, const float* bootstrap_value,
                                    const float* terminated, const float* truncated,
                                    const float* bootstrap_values, const float* carry_in,
                                    float* returns, float* carry_out, int64_t N, int64_t T,
                                    float gamma, hipStream_t stream) {
    return discounted_returns(rewards, bootstrap_value, terminated, truncated, bootstrap_values,
                              carry_in, returns, carry_out, N, T, gamma, stream);
}

int rlscan_discounted_returns_u8(const float* rewards, const float* bootstrap_value,
                                 const uint8_t* terminated, const uint8_t* truncated,
                                 const float* bootstrap_values, const float* carry_in,
                                 float* returns, float* carry_out, int64_t N, int64_t T,
                                 float gamma, hipStream_t stream) {
    return discounted_returns(rewards, bootstrap_value, terminated, truncated, bootstrap_values,
                              carry_in, returns, carry_out, N, T, gamma, stream);
}

int rlscan_discounted_returns(const float* rewards, const float* bootstrap_value,
                              const float* terminated, const float* truncated,
                              const float* bootstrap_values, float* returns, int64_t N,
                              int64_t T, float gamma, hipStream_t stream) {
    return discounted_returns(rewards, bootstrap_value, terminated, truncated, bootstrap_values,
                              nullptr, returns, nullptr, N, T, gamma, stream);
}

}  // extern "C"
