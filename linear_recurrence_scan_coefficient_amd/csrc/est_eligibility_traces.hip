// est_eligibility_traces.hip -- C entry points of eligibility traces and the float-valued episodic prefix sum (rlscan_eligibility_traces, rlscan_eligibility_traces_carry, rlscan_eligibility_traces_u8, rlscan_episodic_prefix_sum_f32):
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
int traces(const float* x, const F* dones, const float* carry_in, float* out, float* carry_out,
           int64_t N, int64_t T, float gamma_lambda, hipStream_t stream) {
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!x || !dones || !out) return RLSCAN_ERR_NULL;
    int rc = check_alias({out, carry_out}, {x, dones, carry_in});
    if (rc != RLSCAN_OK) return rc;
    typename Eligibility<F>::Params p{x, dones, out, gamma_lambda, carry_in, carry_out};
    const bool vec = all_aligned({x, out}) && flags_aligned(dones);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    return run(RLSCAN_EST_ELIGIBILITY, N, T, vec, carry, stream,
               [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                   return launch_kernel<Eligibility<F>>(p, g, lb, pl, vec, carry, stream);
               });
}

template <class F>
int eligibility_traces(const float* x, const F* dones, const float* carry_in, float* traces_out,
                       float* carry_out, int64_t N, int64_t T, float gamma, float lambda,
                       hipStream_t stream) {
    const int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    return traces(x, dones, carry_in, traces_out, carry_out, N, T, gamma * lambda, stream);
}

}  // namespace

extern "C" {

int rlscan_eligibility_traces_carry(const float* x, const float* dones, const float* carry_in,
                                    float* traces, float* carry_out, int64_t N, int64_t T,
                                    float gamma, float lambda, hipStream_t stream) {
    return eligibility_traces(x, dones, carry_in, traces, carry_out, N, T, gamma, lambda, stream);
}

int rlscan_eligibility_traces_u8(const float* x, const uint8_t* dones, const float* carry_in,
                                 float* traces, float* carry_out, int64_t N, int64_t T,
                                 float gamma, float lambda, hipStream_t stream) {
    return eligibility_traces(x, dones, carry_in, traces, carry_out, N, T, gamma, lambda, stream);
}

int rlscan_eligibility_traces(const float* x, const float* dones, float* traces, int64_t N,
                              int64_t T, float gamma, float lambda, hipStream_t stream) {
    return eligibility_traces(x, dones, nullptr, traces, nullptr, N, T,
                              gamma, lambda, stream);
}

// The episodic prefix sum of float values is the trace recurrence with
// gamma*lambda = 1: a_t is 0 or exactly 1.
int rlscan_episodic_prefix_sum_f32(const float* x, const float* dones, const float* carry_in,
                                   float* out, float* carry_out, int64_t N, int64_t T,
                                   hipStream_t stream) {
    const int rc = check_shape(N, T);
    if (rc != RLSCAN_OK) return rc;
    return traces(x, dones, carry_in, out, carry_out, N, T, 1.0f, stream);
}

}  // extern "C"
