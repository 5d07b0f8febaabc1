// Kernel argument blocks and per-dtype launcher declarations shared by the
// C-ABI front end (fa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Forward: O = softmax(scale * Q K^T + mask) V and the natural-log LSE per row.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Lq, Lkv, D;  // D: query/key head dim
    float c;      // scale * log2(e): scores are handled in the exp2 domain
    int causal;
    int window;
    // additive mask (masked entry points only; nullptr otherwise): element
    // (b, h, i, j) at mask[b * msb + h * msh + i * Lkv + j]
    const float* mask;
    long long msb, msh;
    int mvec;     // rows of four keys may be read with one load (16 bytes float, 4 bytes boolean)
    int Dv;       // value head dim (v, o): D unless the extended call sets another
    // boolean mask (extended entry points only; nullptr otherwise, and never
    // together with `mask`): same indexing, nonzero = the pair may attend
    const unsigned char* bmask;
};

// Backward pre-pass: delta = rowsum(dO * O) over rows of length D.
struct PreArgs {
    const void* o;
    const void* dO;
    float* delta;
    long long rows;
    int D;
};

// dK/dV and dQ kernels.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dO;
    const float* lse;
    const float* delta;
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, Lq, Lkv, D;
    float c;      // scale * log2(e)
    float scale;  // applied once to dQ and dK in the epilogue
    int causal;
    int window;
    const float* mask;  // as in FwdArgs
    long long msb, msh;
    int mvec;
    int Dv;       // value head dim (v, dO, dV)
    const unsigned char* bmask;  // as in FwdArgs
};

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_pre_f32(const PreArgs& a, hipStream_t s);
hipError_t launch_pre_f16(const PreArgs& a, hipStream_t s);
hipError_t launch_pre_bf16(const PreArgs& a, hipStream_t s);
hipError_t launch_dkv_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_dkv_f16(const BwdArgs& a, hipStream_t s);
hipError_t launch_dkv_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_dq_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_dq_f16(const BwdArgs& a, hipStream_t s);
hipError_t launch_dq_bf16(const BwdArgs& a, hipStream_t s);

}  // namespace fa
