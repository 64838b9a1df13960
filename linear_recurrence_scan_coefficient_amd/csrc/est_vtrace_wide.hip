// est_vtrace_wide.hip -- V-trace's float64 form: the kernels that the V-trace
// entry points (est_vtrace.hip) launch when gamma*lambda*c_bar > 1, so that a
// trace coefficient gamma*c_t can exceed 1 (README, Kernels table,
// compute_vtrace row; Espeholt et al. 2018, whose trace clip c_bar may be
// set above 1).  The recurrence then expands along an episode and amplifies
// every rounding made before it, so the coefficients, the scan state and the
// epilogue are float64 here and only vs and pg are rounded to float32.  A
// translation unit of its own so that it compiles in parallel with the
// float32 form.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "host.hpp"

namespace rlscan {

template <class F>
hipError_t launch_vtrace_wide(const VtraceParams<F>& p, const Geometry& geo,
                              const LookbackArgs& lb, const Plan& pl, bool vec, bool carry,
                              bool trunc, hipStream_t stream) {
    return trunc ? launch_kernel<Vtrace<true, F, true>>(p, geo, lb, pl, vec, carry, stream)
                 : launch_kernel<Vtrace<false, F, true>>(p, geo, lb, pl, vec, carry, stream);
}

template hipError_t launch_vtrace_wide<float>(const VtraceParams<float>&, const Geometry&,
                                              const LookbackArgs&, const Plan&, bool, bool, bool,
                                              hipStream_t);
template hipError_t launch_vtrace_wide<uint8_t>(const VtraceParams<uint8_t>&, const Geometry&,
                                                const LookbackArgs&, const Plan&, bool, bool,
                                                bool, hipStream_t);

}  // namespace rlscan
