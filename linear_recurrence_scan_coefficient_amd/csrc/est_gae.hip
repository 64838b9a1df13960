// est_gae.hip -- C entry points of GAE (rlscan_gae, rlscan_gae_carry, rlscan_gae_u8):
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
int gae(const float* rewards, const float* values, const float* bootstrap_value,
        const F* terminated, const F* truncated, const float* bootstrap_values,
        const float* carry_in, float* advantages, float* carry_out, int64_t N, int64_t T,
        float gamma, float lambda, hipStream_t stream, const ScratchSource* src = nullptr) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !terminated || !advantages) return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({advantages, carry_out}, {rewards, values, bootstrap_value, terminated,
                                               truncated, bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const GaeParams<F> p{rewards,  values,     bootstrap_value, terminated, truncated,
                         bootstrap_values, carry_in, advantages, carry_out, gamma,
                         gamma * lambda};
    const bool vec = all_aligned({rewards, values, bootstrap_values, advantages}) &&
                     flags_aligned(terminated) && flags_aligned(truncated);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_GAE, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated
                              ? launch_kernel<Gae<true, F>>(p, g, lb, pl, vec, carry, stream)
                              : launch_kernel<Gae<false, F>>(p, g, lb, pl, vec, carry, stream);
               },
               src);
}

}  // namespace

namespace rlscan {

int gae_with_scratch(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* advantages,
                     float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                     hipStream_t stream, const ScratchSource* src) {
    return gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
               carry_in, advantages, carry_out, N, T, gamma, lambda, stream, src);
}

}  // namespace rlscan

extern "C" {

int rlscan_gae_carry(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* advantages,
                     float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                     hipStream_t stream) {
    return gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
               carry_in, advantages, carry_out, N, T, gamma, lambda, stream);
}

int rlscan_gae_u8(const float* rewards, const float* values, const float* bootstrap_value,
                  const uint8_t* terminated, const uint8_t* truncated,
                  const float* bootstrap_values, const float* carry_in, float* advantages,
                  float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                  hipStream_t stream) {
    return gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
               carry_in, advantages, carry_out, N, T, gamma, lambda, stream);
}

int rlscan_gae(const float* rewards, const float* values, const float* bootstrap_value,
               const float* terminated, const float* truncated, const float* bootstrap_values,
               float* advantages, int64_t N, int64_t T, float gamma, float lambda,
               hipStream_t stream) {
    return gae(rewards, values, bootstrap_value, terminated, truncated, bootstrap_values,
               nullptr, advantages, nullptr, N, T, gamma, lambda, stream);
}

}  // extern "C"
