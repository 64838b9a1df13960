// est_vtrace.hip -- C entry points of V-trace (rlscan_vtrace, rlscan_vtrace_carry, rlscan_vtrace_ex, rlscan_vtrace_u8):
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
int vtrace(const float* rewards, const float* values, const float* bootstrap_value,
           const float* log_rhos, const F* terminated, const F* truncated,
           const float* bootstrap_values, const float* carry_in, float* vs, float* pg_advantages,
           float* carry_out, int64_t N, int64_t T, float gamma, float lambda, float rho_bar,
           float c_bar, float rho_bar_pg, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda) || !positive_clip(rho_bar) ||
        !positive_clip(c_bar) || !positive_clip(rho_bar_pg))
        return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !values || !log_rhos || !terminated || !vs || !pg_advantages)
        return RLSCAN_ERR_NULL;
    if (truncated && !bootstrap_values) return RLSCAN_ERR_NULL;
    rc = check_alias({vs, pg_advantages, carry_out},
                     {rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                      bootstrap_values, carry_in});
    if (rc != RLSCAN_OK) return rc;
    const VtraceParams<F> p{rewards,   values,        bootstrap_value, log_rhos,
                            terminated, truncated,    bootstrap_values, carry_in,
                            vs,        pg_advantages, carry_out,        gamma,
                            lambda,    rho_bar,       c_bar,            rho_bar_pg};
    const bool vec = all_aligned({rewards, values, log_rhos, bootstrap_values, vs,
                                  pg_advantages}) &&
                     flags_aligned(terminated) && flags_aligned(truncated);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    // Trace coefficients gamma*c_t can exceed 1 only if gamma*lambda*c_bar
    // does (c_bar = +inf with gamma*lambda = 0 gives NaN here: no growth).
    // Such calls run the float64 form: the trace products then grow along an
    // episode, and a float32 rounding anywhere on the way would grow with
    // them.
    const bool wide =
        static_cast<double>(gamma) * static_cast<double>(lambda) * static_cast<double>(c_bar) > 1.0;
    return run(wide ? kEstVtraceWide : RLSCAN_EST_VTRACE, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   if (wide)
                       return launch_vtrace_wide<F>(p, g, lb, pl, vec, carry, truncated != nullptr,
                                                    stream);
                   return truncated
                              ? launch_kernel<Vtrace<true, F>>(p, g, lb, pl, vec, carry, stream)
                              : launch_kernel<Vtrace<false, F>>(p, g, lb, pl, vec, carry, stream);
               });
}

}  // namespace

extern "C" {

int rlscan_vtrace_ex(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* log_rhos, const float* terminated, const float* truncated,
                     const float* bootstrap_values, const float* carry_in, float* vs,
                     float* pg_advantages, float* carry_out, int64_t N, int64_t T, float gamma,
                     float lambda, float rho_bar, float c_bar, float rho_bar_pg,
                     hipStream_t stream) {
    return vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                  bootstrap_values, carry_in, vs, pg_advantages, carry_out, N, T, gamma, lambda,
                  rho_bar, c_bar, rho_bar_pg, stream);
}

int rlscan_vtrace_u8(const float* rewards, const float* values, const float* bootstrap_value,
                     const float* log_rhos, const uint8_t* terminated, const uint8_t* truncated,
                     const float* bootstrap_values, const float* carry_in, float* vs,
                     float* pg_advantages, float* carry_out, int64_t N, int64_t T, float gamma,
                     float lambda, float rho_bar, float c_bar, float rho_bar_pg,
                     hipStream_t stream) {
    return vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                  bootstrap_values, carry_in, vs, pg_advantages, carry_out, N, T, gamma, lambda,
                  rho_bar, c_bar, rho_bar_pg, stream);
}

int rlscan_vtrace_carry(const float* rewards, const float* values, const float* bootstrap_value,
                        const float* log_rhos, const float* terminated, const float* truncated,
                        const float* bootstrap_values, const float* carry_in, float* vs,
                        float* pg_advantages, float* carry_out, int64_t N, int64_t T,
                        float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    return vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                  bootstrap_values, carry_in, vs, pg_advantages, carry_out, N, T, gamma, 1.0f,
                  rho_bar, c_bar, rho_bar, stream);
}

int rlscan_vtrace(const float* rewards, const float* values, const float* bootstrap_value,
                  const float* log_rhos, const float* terminated, const float* truncated,
                  const float* bootstrap_values, float* vs, float* pg_advantages, int64_t N,
                  int64_t T, float gamma, float rho_bar, float c_bar, hipStream_t stream) {
    return vtrace(rewards, values, bootstrap_value, log_rhos, terminated, truncated,
                  bootstrap_values, nullptr, vs, pg_advantages, nullptr, N, T, gamma, 1.0f,
                  rho_bar, c_bar, rho_bar, stream);
}

}  // extern "C"
