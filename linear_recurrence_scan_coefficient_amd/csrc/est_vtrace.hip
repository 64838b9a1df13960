// est_vtrace.hip -- C entry points of V-trace (rlscan_vtrace, rlscan_vtrace_carry):
// argument checks, then the scan kernel instantiated for its estimator
// (estimators.hpp) through the shared launch path (host.hpp).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "host.hpp"

using namespace rlscan;

extern "C" {

int rlscan_vtrace_carry(const float* rewards, const float* values, const float* bootstrap_value,
                        const float* log_rhos, const float* terminated, const float* truncated,
                        const float* bootstrap_values, const float* carry_in, float* vs,
                        float* pg_advantages, float* carry_out, int64_t N, int64_t T,
                        float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !positive_clip(rho_bar) || !positive_clip(c_bar))
        return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !log_rhos || !terminated || !vs || !pg_advantages)
        return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({vs, pg_advantages, carry_out},
                     {rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                      bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const VtraceParams p{rewards,   values,        bootstrap_value, log_rhos,
                         terminated, truncated,    bootstrap_values, carry_in,
                         vs,        pg_advantages, carry_out,        gamma,
                         rho_bar,   c_bar};
    const bool vec = all_aligned({rewards, values, log_rhos, terminated, truncated,
                                  bootstrap_values, vs, pg_advantages});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_VTRACE, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return truncated ? launch_kernel<Vtrace<true>>(p, g, lb, pl, vec, carry, stream)
                                    : launch_kernel<Vtrace<false>>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_vtrace(const float* rewards, const float* values, const float* bootstrap_value,
                  const float* log_rhos, const float* terminated, const float* truncated,
                  const float* bootstrap_values, float* vs, float* pg_advantages, int64_t N,
                  int64_t T, float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    return rlscan_vtrace_carry(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                               bootstrap_values, nullptr, vs, pg_advantages, nullptr, N, T,
                               gamma, rho_bar, c_bar, stream);
}

}  // extern "C"
