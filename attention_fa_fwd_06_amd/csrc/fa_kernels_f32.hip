// Kernel instantiations for f32 inputs (fp32 accumulation).
#include "fa_kernels.hpp"

namespace fa {
hipError_t launch_fwd_f32(int dmax, const FwdArgs& a, hipStream_t s) { return launch_fwd_t<float>(dmax, a, s); }
hipError_t launch_pre_f32(const PreArgs& a, hipStream_t s) { return launch_pre_t<float>(a, s); }
hipError_t launch_dkv_f32(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dkv_t<float>(dmax, a, s); }
hipError_t launch_dq_f32(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dq_t<float>(dmax, a, s); }
}  // namespace fa
