// Kernel instantiations for bf16 inputs (fp32 accumulation).
#include "fa_kernels.hpp"

namespace fa {
hipError_t launch_fwd_bf16(int dmax, const FwdArgs& a, hipStream_t s) { return launch_fwd_t<__bf16>(dmax, a, s); }
hipError_t launch_pre_bf16(const PreArgs& a, hipStream_t s) { return launch_pre_t<__bf16>(a, s); }
hipError_t launch_dkv_bf16(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dkv_t<__bf16>(dmax, a, s); }
hipError_t launch_dq_bf16(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dq_t<__bf16>(dmax, a, s); }
}  // namespace fa
