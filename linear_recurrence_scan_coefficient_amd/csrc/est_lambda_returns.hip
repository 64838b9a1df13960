// est_lambda_returns.hip -- C entry points of TD(lambda) returns (rlscan_lambda_returns, rlscan_lambda_returns_carry, rlscan_lambda_returns_u8):
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
int lambda_returns(const float* rewards, const float* values, const float* bootstrap_value,
                   const F* terminated, const F* truncated, const float* bootstrap_values,
                   const float* carry_in, float* returns, float* carry_out, int64_t N,
                   int64_t T, float gamma, float lambda, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !terminated || !returns) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({returns, carry_out}, {rewards, values, bootstrap_value, terminated,
                                            truncated, bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const LambdaReturnsParams<F> p{rewards,   values,   bootstrap_value, terminated,
                                   truncated, bootstrap_values, carry_in, returns,
                                   carry_out, gamma,    gamma * lambda,
                                   gamma * (1.0f - lambda)};
    const bool vec = all_aligned({rewards, values, bootstrap_values, returns}) &&
                     flags_aligned(terminated) && flags_aligned(truncated);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_LAMBDA_RETURNS, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated ? launch_kernel<LambdaReturns<true, F>>(p, g, lb, pl, vec,
                                                                            carry, stream)
                                    : launch_kernel<LambdaReturns<false, F>>(p, g, lb, pl, vec,
                                                                             carry, stream);
               });
}

}  // namespace

extern "C" {

int rlscan_lambda_returns_carry(const float* rewards, const float* values,
                                const float* bootstrap_value, const float* terminated,
                                const float* truncated, const float* bootstrap_values,
                                const float* carry_in, float* returns, float* carry_out,
                                int64_t N, int64_t T, float gamma, float lambda,
                                hipStream_t stream) {
    return lambda_returns(rewards, values, bootstrap_value, terminated, truncated,
                          bootstrap_values, carry_in, returns, carry_out, N, T, gamma, lambda,
                          stream);
}

int rlscan_lambda_returns_u8(const float* rewards, const float* values,
                             const float* bootstrap_value, const uint8_t* terminated,
                             const uint8_t* truncated, const float* bootstrap_values,
                             const float* carry_in, float* returns, float* carry_out, int64_t N,
                             int64_t T, float gamma, float lambda, hipStream_t stream) {
    return lambda_returns(rewards, values, bootstrap_value, terminated, truncated,
                          bootstrap_values, carry_in, returns, carry_out, N, T, gamma, lambda,
                          stream);
}

int rlscan_lambda_returns(const float* rewards, const float* values, const float* bootstrap_value,
                          const float* terminated, const float* truncated,
                          const float* bootstrap_values, float* returns, int64_t N, int64_t T,
                          float gamma, float lambda, hipStream_t stream) {
    return lambda_returns(rewards, values, bootstrap_value, terminated, truncated,
                          bootstrap_values, nullptr, returns, nullptr, N, T, gamma, lambda,
                          stream);
}

}  // extern "C"
