// est_eligibility_traces.hip -- C entry points of eligibility traces (rlscan_eligibility_traces, rlscan_eligibility_traces_carry):
// argument checks, then the scan kernel instantiated for its estimator
// (estimators.hpp) through the shared launch path (host.hpp).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "host.hpp"

using namespace rlscan;

extern "C" {

int rlscan_eligibility_traces_carry(const float* x, const float* dones, const float* carry_in,
                                    float* traces, float* carry_out, int64_t N, int64_t T,
                                    float gamma, float lambda, hipStream_t stream) {
    int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!x || !dones || !traces) return RLSCAN_ERR_NULL;
    rc = check_alias({traces, carry_out}, {x, dones, carry_in});
    if (rc != RLSCAN_OK) return rc;
    Eligibility::Params p{x, dones, traces, gamma * lambda, carry_in, carry_out};
    const bool vec = all_aligned({x, dones, traces});
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_ELIGIBILITY, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return launch_kernel<Eligibility>(p, g, lb, pl, vec, carry, stream);
               });
}

int rlscan_eligibility_traces(const float* x, const float* dones, float* traces, int64_t N,
                              int64_t T, float gamma, float lambda, hipStream_t stream) {
    return rlscan_eligibility_traces_carry(x, dones, nullptr, traces, nullptr, N, T, gamma,
                                           lambda, stream);
}

}  // extern "C"
