// Backward kernels of one pipeline chunk of the gated delta rule.
#include "gdn_kernels.hpp"

namespace sfgdn {

template <typename T, int D>
hipError_t launch_bwd(const BwdArgs&, hipStream_t, Profiler*) {
  return hipErrorNotSupported;
}

template hipError_t launch_bwd<bf16, 128>(const BwdArgs&, hipStream_t, Profiler*);
template hipError_t launch_bwd<bf16, 64>(const BwdArgs&, hipStream_t, Profiler*);
template hipError_t launch_bwd<float, 64>(const BwdArgs&, hipStream_t, Profiler*);

}  // namespace sfgdn
