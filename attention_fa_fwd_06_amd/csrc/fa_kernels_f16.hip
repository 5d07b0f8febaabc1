// Kernel instantiations for f16 inputs (fp32 accumulation).
#include "fa_kernels.hpp"

namespace fa {
hipError_t launch_fwd_f16(int dmax, const FwdArgs& a, hipStream_t s) { return launch_fwd_t<_Float16>(dmax, a, s); }
hipError_t launch_pre_f16(const PreArgs& a, hipStream_t s) { return launch_pre_t<_Float16>(a, s); }
hipError_t launch_dkv_f16(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dkv_t<_Float16>(dmax, a, s); }
hipError_t launch_dq_f16(int dmax, const BwdArgs& a, hipStream_t s) { return launch_dq_t<_Float16>(dmax, a, s); }
}  // namespace fa
