// Kernel instantiations for float inputs (fp32 MFMA, fp32 accumulation).
#include "fa_kernels.hpp"

namespace fa {
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) { return launch_fwd_t<float>(dmax_bucket(a.D > a.Dv ? a.D : a.Dv), a, s); }
hipError_t launch_pre_f32(const PreArgs& a, hipStream_t s) { return launch_pre_t<float>(a, s); }
hipError_t launch_dkv_f32(const BwdArgs& a, hipStream_t s) { return launch_dkv_t<float>(dmax_bucket(a.D > a.Dv ? a.D : a.Dv), a, s); }
hipError_t launch_dq_f32(const BwdArgs& a, hipStream_t s) { return launch_dq_t<float>(dmax_bucket(a.D > a.Dv ? a.D : a.Dv), a, s); }
}  // namespace fa
