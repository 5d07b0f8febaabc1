// Kernel choice for 16-bit inputs: the short-query kernels for query lengths
// up to kShortLq with both head dims <= 128 (forward and dQ in their
// few-key-block configuration when Lkv is at most 32 * kShortFewBlocks),
// otherwise the tiled kernels of the head-dim bucket max(D, Dv).
#pragma once

#include "fa_kernels_short.hpp"
#include "fa_kernels_dkvq.hpp"
#include "fa_kernels_dq3.hpp"

namespace fa {
namespace lds {

template <class T> hipError_t launch_fwd16(const FwdArgs& a, hipStream_t s) {
    const int dm = dmax16(a.D > a.Dv ? a.D : a.Dv);
    if (use_short(a.Lq, a.D, a.Dv)) {
        if ((a.Lkv + 31) / 32 <= kShortFewBlocks)
            return dm <= 64 ? launch_fwd_short<T, 64, FA2_SHORT_FEW>(a, s) : launch_fwd_short<T, 128, FA2_SHORT_FEW>(a, s);
        return dm <= 64 ? launch_fwd_short<T, 64, FA2_SHORT_FWD_64>(a, s)
                        : launch_fwd_short<T, 128, FA2_SHORT_FWD_128>(a, s);
    }
    switch (dm) {
        case 32: return launch_fwd2<T, 32, FA2_FWD_32>(a, s);
        case 64: return launch_fwd2<T, 64, FA2_FWD_64>(a, s);
        case 96: return launch_fwd2<T, 96, FA2_FWD_96>(a, s);
        case 128: return launch_fwd2<T, 128, FA2_FWD_128>(a, s);
        case 256: return launch_fwd2<T, 256, FA2_FWD_256>(a, s);
        default: return launch_fwd2<T, 512, FA2_FWD_512>(a, s);
    }
}
template <class T> hipError_t launch_dq16(const BwdArgs& a, hipStream_t s) {
    const int dm = dmax16(a.D > a.Dv ? a.D : a.Dv);
    if (use_short(a.Lq, a.D, a.Dv)) {
        if ((a.Lkv + 31) / 32 <= kShortFewBlocks)
            return dm <= 64 ? launch_dq_short<T, 64, FA2_SHORT_FEW>(a, s) : launch_dq_short<T, 128, FA2_SHORT_FEW>(a, s);
        return dm <= 64 ? launch_dq_short<T, 64, FA2_SHORT_DQ_64>(a, s)
                        : launch_dq_short<T, 128, FA2_SHORT_DQ_128>(a, s);
    }
    switch (dm) {
        case 32: return launch_dq2<T, 32, FA2_DQ_32>(a, s);
        case 64: return launch_dq2<T, 64, FA2_DQ_64>(a, s);
        case 96: return launch_dq2<T, 96, FA2_DQ_96>(a, s);
        case 128: return launch_dq2<T, 128, FA2_DQ_128>(a, s);
        case 256: return launch_dq_tri<T, 256>(a, s);
        default: return launch_dq2<T, 512, FA2_DQ_512>(a, s);
    }
}
template <class T> hipError_t launch_dkv16(const BwdArgs& a, hipStream_t s) {
    const int dm = dmax16(a.D > a.Dv ? a.D : a.Dv);
    if (use_short(a.Lq, a.D, a.Dv))
        return dm <= 64 ? launch_dkv_short<T, 64, FA2_SHORT_DKV_64>(a, s)
                        : launch_dkv_short<T, 128, FA2_SHORT_DKV_128>(a, s);
    switch (dm) {
        case 32: return launch_dkv_pipe<T, 32, FA2_DKVS_32>(a, s);
        case 64: return launch_dkv_pipe<T, 64, FA2_DKVS_64>(a, s);
        case 96: return launch_dkv_pipe<T, 96, FA2_DKVS_96>(a, s);
        case 128: return launch_dkv_pipe<T, 128, FA2_DKVS_128>(a, s);
        case 256: return launch_dkv_quad<T, 256, 32>(a, s);
        default: return launch_dkv2<T, 512, FA2_DKV_512>(a, s);
    }
}

}  // namespace lds
}  // namespace fa
