// Kernel instantiations for f16 inputs (fp32 accumulation): the gfx950
// LDS-DMA path for the attention kernels, the streaming pre-pass.
#include "fa_dispatch16.hpp"

namespace fa {
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s) { return lds::launch_fwd16<_Float16>(a, s); }
hipError_t launch_pre_f16(const PreArgs& a, hipStream_t s) { return launch_pre_t<_Float16>(a, s); }
hipError_t launch_dkv_f16(const BwdArgs& a, hipStream_t s) { return lds::launch_dkv16<_Float16>(a, s); }
hipError_t launch_dq_f16(const BwdArgs& a, hipStream_t s) { return lds::launch_dq16<_Float16>(a, s); }
}  // namespace fa
