// est_retrace.hip -- C entry points of Retrace(lambda) (rlscan_retrace, rlscan_retrace_carry, rlscan_retrace_u8):
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
int retrace(const float* rewards, const float* next_q_values_all, const float* next_target_probs,
            const int32_t* actions, const float* behaviour_probs, const F* terminated,
            const F* truncated, const float* carry_in, const int32_t* next_actions,
            const float* next_behaviour_probs, float* targets, float* carry_out, int64_t N,
            int64_t T, int64_t A, float gamma, float lambda, hipStream_t stream) {
    int rc = check_shape(N, T, A);
    if (rc != RLSCAN_OK) return rc;
    if (!unit_interval(gamma) || !unit_interval(lambda)) return RLSCAN_ERR_PARAM;
    if (N == 0 || T == 0) return RLSCAN_OK;
    if (!rewards || !next_q_values_all || !next_target_probs || !actions || !behaviour_probs ||
        !terminated || !truncated || !targets)
        return RLSCAN_ERR_NULL;
    if (carry_in && (!next_actions || !next_behaviour_probs)) return RLSCAN_ERR_NULL;
    rc = check_alias({targets, carry_out},
                     {rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                      terminated, truncated, carry_in, next_actions, next_behaviour_probs});
    if (rc != RLSCAN_OK) return rc;
    const bool vec = all_aligned({rewards, next_q_values_all, next_target_probs, actions,
                                  behaviour_probs, targets}) &&
                     flags_aligned(terminated) && flags_aligned(truncated);
    const bool carry = carry_in != nullptr || carry_out != nullptr;
    auto go = [&](auto tag) {
        using E = decltype(tag);
        typename E::Params p{rewards,  next_q_values_all, next_target_probs, actions,
                             behaviour_probs, terminated, truncated, targets,
                             A,        gamma,             lambda,            carry_in,
                             next_actions, next_behaviour_probs, carry_out};
        return run(RLSCAN_EST_RETRACE, N, T, vec, carry, stream,
                   [&](const Geometry& g, const LookbackArgs& lb, const Plan& pl) {
                       return launch_kernel_r1<E>(p, g, lb, pl, vec, carry, stream);
                   });
    };
    switch (vec ? A : 0) {
        case 4: return go(Retrace<4, F>{});
        case 6: return go(Retrace<6, F>{});
        case 8: return go(Retrace<8, F>{});
        case 18: return go(Retrace<18, F>{});
        default: return go(Retrace<0, F>{});
    }
}

}  // namespace

extern "C" {

int rlscan_retrace_carry(const float* rewards, const float* next_q_values_all,
                         const float* next_target_probs, const int32_t* actions,
                         const float* behaviour_probs, const float* terminated,
                         const float* truncated, const float* carry_in,
                         const int32_t* next_actions, const float* next_behaviour_probs,
                         float* targets, float* carry_out, int64_t N, int64_t T, int64_t A,
                         float gamma, float lambda, hipStream_t stream) {
    return retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                   terminated, truncated, carry_in, next_actions, next_behaviour_probs, targets,
                   carry_out, N, T, A, gamma, lambda, stream);
}

int rlscan_retrace_u8(const float* rewards, const float* next_q_values_all,
                      const float* next_target_probs, const int32_t* actions,
                      const float* behaviour_probs, const uint8_t* terminated,
                      const uint8_t* truncated, const float* carry_in,
                      const int32_t* next_actions, const float* next_behaviour_probs,
                      float* targets, float* carry_out, int64_t N, int64_t T, int64_t A,
                      float gamma, float lambda, hipStream_t stream) {
    return retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                   terminated, truncated, carry_in, next_actions, next_behaviour_probs, targets,
                   carry_out, N, T, A, gamma, lambda, stream);
}

int rlscan_retrace(const float* rewards, const float* next_q_values_all,
                   const float* next_target_probs, const int32_t* actions,
                   const float* behaviour_probs, const float* terminated, const float* truncated,
                   float* targets, int64_t N, int64_t T, int64_t A, float gamma, float lambda,
                   hipStream_t stream) {
    return retrace(rewards, next_q_values_all, next_target_probs, actions, behaviour_probs,
                   terminated, truncated, nullptr, nullptr, nullptr, targets, nullptr, N, T, A,
                   gamma, lambda, stream);
}

}  // extern "C"
