// Kernel instantiations for bf16 inputs (fp32 accumulation): the gfx950
// LDS-DMA path for the attention kernels, the streaming pre-pass.
#include "fa_dispatch16.hpp"

namespace fa {
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) { return lds::launch_fwd16<__bf16>(a, s); }
hipError_t launch_pre_bf16(const PreArgs& a, hipStream_t s) { return launch_pre_t<__bf16>(a, s); }
hipError_t launch_dkv_bf16(const BwdArgs& a, hipStream_t s) { return lds::launch_dkv16<__bf16>(a, s); }
hipError_t launch_dq_bf16(const BwdArgs& a, hipStream_t s) { return lds::launch_dq16<__bf16>(a, s); }
}  // namespace fa
