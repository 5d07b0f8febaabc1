// C-ABI front end: argument checks, head-dim bucket selection, launch.
//
// Every check runs before any HIP call, so a bad argument returns a status
// code without touching the device (ggmlR R/ag_flash_attn.R checks its
// arguments and raises an error instead of letting the backend abort; the MLX
// VJP dispatch throws rather than running an unsupported path).
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_types.hpp"

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;
constexpr int kMaxLen = 1 << 24;
// One head's rows (L x D elements) must stay below 2^29 elements: the kernels
// address a head through 32-bit byte offsets and mark out-of-range reads
// with offsets at 2^31 and above.
constexpr long long kMaxHeadElems = 1LL << 29;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status_t check_dtype(fa_dtype_t dt) {
    return (dt == FA_F32 || dt == FA_F16 || dt == FA_BF16) ? FA_OK : FA_ERR_DTYPE;
}

fa_status_t check_headdim(int D) { return (D < 32 || D > 512 || D % 8 != 0) ? FA_ERR_HEADDIM : FA_OK; }

fa_status_t check_attn(int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale, int window) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lkv < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (Lq >= kMaxLen || Lkv >= kMaxLen) return FA_ERR_SHAPE;
    fa_status_t st = check_headdim(D);
    if (st != FA_OK) return st;
    if ((long long)B * Hq * Lq * D > kMaxElems || (long long)B * Hkv * Lkv * D > kMaxElems) return FA_ERR_SHAPE;
    if ((long long)Lq * D > kMaxHeadElems || (long long)Lkv * D > kMaxHeadElems) return FA_ERR_SHAPE;
    if (window < 0 || !std::isfinite(scale)) return FA_ERR_ARG;
    return FA_OK;
}

// The value head dim of the extended calls: the same rules as D, and the same
// size limits for the tensors that carry it (v, o, dO, dV).
fa_status_t check_dv(int B, int Hq, int Hkv, int Lq, int Lkv, int Dv) {
    fa_status_t st = check_headdim(Dv);
    if (st != FA_OK) return st;
    if ((long long)B * Hq * Lq * Dv > kMaxElems || (long long)B * Hkv * Lkv * Dv > kMaxElems) return FA_ERR_SHAPE;
    if ((long long)Lq * Dv > kMaxHeadElems || (long long)Lkv * Dv > kMaxHeadElems) return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status_t from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// Mask tensor of the masked entry points: non-NULL, 4-byte aligned, strides
// in [0, 2^40] elements (far from any overflow of the 64-bit offsets).
constexpr long long kMaxMaskStride = 1LL << 40;
fa_status_t check_mask(const float* mask, long long msb, long long msh) {
    if (!mask) return FA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(mask) & 3u) != 0) return FA_ERR_ALIGN;
    if (msb < 0 || msh < 0 || msb > kMaxMaskStride || msh > kMaxMaskStride) return FA_ERR_ARG;
    return FA_OK;
}
// 16-byte loads of four consecutive keys are possible when every row of every
// (batch, head) slice starts 16-byte aligned.
int mask_vec4(const float* mask, long long msb, long long msh, int Lkv) {
    return aligned16(mask) && msb % 4 == 0 && msh % 4 == 0 && Lkv % 4 == 0;
}
// Boolean mask of the extended calls: one byte per pair, any alignment, the
// same stride range. Four consecutive keys are one 4-byte load when every row
// starts 4-byte aligned.
fa_status_t check_bool_mask(long long msb, long long msh) {
    if (msb < 0 || msh < 0 || msb > kMaxMaskStride || msh > kMaxMaskStride) return FA_ERR_ARG;
    return FA_OK;
}
int bool_mask_vec4(const unsigned char* m, long long msb, long long msh, int Lkv) {
    return (reinterpret_cast<uintptr_t>(m) & 3u) == 0 && msb % 4 == 0 && msh % 4 == 0 && Lkv % 4 == 0;
}
int vec4(const float* mask, const unsigned char* bmask, long long msb, long long msh, int Lkv) {
    return mask ? mask_vec4(mask, msb, msh, Lkv) : bmask ? bool_mask_vec4(bmask, msb, msh, Lkv) : 0;
}

// A window of Lq or more keys never masks anything (i - j <= Lq - 1 for every
// pair), so it is the same as no window; folding it to 0 also keeps the
// kernels' tile-range arithmetic far from int overflow.
int effective_window(int window, int Lq) { return window >= Lq ? 0 : window; }

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "bad shape: sizes must be >= 1, Hq a multiple of Hkv, within the size limits";
        case FA_ERR_HEADDIM: return "head dim must be a multiple of 8 in [32, 512]";
        case FA_ERR_DTYPE: return "unsupported dtype (FA_F32, FA_F16 or FA_BF16)";
        case FA_ERR_ALIGN: return "every pointer must be 16-byte aligned";
        case FA_ERR_ARG: return "window must be >= 0, scale finite, mask strides in [0, 2^40] and at most one mask";
        case FA_ERR_LAUNCH: return "HIP kernel launch failed";
    }
    return "unknown status";
}

static fa_status_t fwd_impl(const void* q, const void* k, const void* v, const float* mask, long long msb,
                            long long msh, const unsigned char* bmask, void* o, float* lse, int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                            int Dv, float scale, int causal, int window, fa_dtype_t dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    fa_status_t st = check_dtype(dtype);
    if (st != FA_OK) return st;
    st = check_attn(B, Hq, Hkv, Lq, Lkv, D, scale, window);
    if (st != FA_OK) return st;
    st = check_dv(B, Hq, Hkv, Lq, Lkv, Dv);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;

    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Lq, Lkv, D,
                  (float)((double)scale * 1.4426950408889634), causal ? 1 : 0, effective_window(window, Lq),
                  mask, msb, msh, vec4(mask, bmask, msb, msh, Lkv), Dv, bmask};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case FA_F32: return from_hip(fa::launch_fwd_f32(a, s));
        case FA_F16: return from_hip(fa::launch_fwd_f16(a, s));
        case FA_BF16: return from_hip(fa::launch_fwd_bf16(a, s));
    }
    return FA_ERR_DTYPE;
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                   int Lq, int Lkv, int D, float scale, int causal, int window, fa_dtype_t dtype, void* stream) {
    return fwd_impl(q, k, v, nullptr, 0, 0, nullptr, o, lse, B, Hq, Hkv, Lq, Lkv, D, D, scale, causal, window, dtype, stream);
}

fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, const float* mask, long long mask_stride_b,
                          long long mask_stride_h, void* o, float* lse, int B, int Hq, int Hkv, int Lq, int Lkv,
                          int D, float scale, int causal, int window, fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_mask(mask, mask_stride_b, mask_stride_h);
    if (st != FA_OK) return st;
    return fwd_impl(q, k, v, mask, mask_stride_b, mask_stride_h, nullptr, o, lse, B, Hq, Hkv, Lq, Lkv, D, D, scale, causal,
                    window, dtype, stream);
}

fa_status_t fa_bwd_preprocess(const void* o, const void* dO, float* delta, int B, int Hq, int Lq, int D,
                              fa_dtype_t dtype, void* stream) {
    if (!o || !dO || !delta) return FA_ERR_NULL;
    fa_status_t st = check_dtype(dtype);
    if (st != FA_OK) return st;
    if (B < 1 || Hq < 1 || Lq < 1 || Lq >= kMaxLen) return FA_ERR_SHAPE;
    st = check_headdim(D);
    if (st != FA_OK) return st;
    if ((long long)B * Hq * Lq * D > kMaxElems || (long long)Lq * D > kMaxHeadElems) return FA_ERR_SHAPE;
    if (!aligned16(o) || !aligned16(dO) || !aligned16(delta)) return FA_ERR_ALIGN;

    fa::PreArgs a{o, dO, delta, (long long)B * Hq * Lq, D};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case FA_F32: return from_hip(fa::launch_pre_f32(a, s));
        case FA_F16: return from_hip(fa::launch_pre_f16(a, s));
        case FA_BF16: return from_hip(fa::launch_pre_bf16(a, s));
    }
    return FA_ERR_DTYPE;
}

static fa_status_t bwd_common(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                              const float* delta, int B, int Hq, int Hkv, int Lq, int Lkv, int D, int Dv,
                              float scale, int window, fa_dtype_t dtype) {
    if (!q || !k || !v || !dO || !lse || !delta) return FA_ERR_NULL;
    fa_status_t st = check_dtype(dtype);
    if (st != FA_OK) return st;
    st = check_attn(B, Hq, Hkv, Lq, Lkv, D, scale, window);
    if (st != FA_OK) return st;
    st = check_dv(B, Hq, Hkv, Lq, Lkv, Dv);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(delta))
        return FA_ERR_ALIGN;
    return FA_OK;
}

static fa_status_t dkv_impl(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                            const float* delta, const float* mask, long long msb, long long msh,
                            const unsigned char* bmask, void* dk, void* dv,
                            int B, int Hq, int Hkv, int Lq, int Lkv, int D, int Dv, float scale, int causal,
                            int window, fa_dtype_t dtype, void* stream) {
    if (!dk || !dv) return FA_ERR_NULL;
    fa_status_t st = bwd_common(q, k, v, dO, lse, delta, B, Hq, Hkv, Lq, Lkv, D, Dv, scale, window, dtype);
    if (st != FA_OK) return st;
    if (!aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;

    fa::BwdArgs a{q, k, v, dO, lse, delta, nullptr, dk, dv, B, Hq, Hkv, Lq, Lkv, D,
                  (float)((double)scale * 1.4426950408889634), scale, causal ? 1 : 0,
                  effective_window(window, Lq), mask, msb, msh, vec4(mask, bmask, msb, msh, Lkv), Dv, bmask};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case FA_F32: return from_hip(fa::launch_dkv_f32(a, s));
        case FA_F16: return from_hip(fa::launch_dkv_f16(a, s));
        case FA_BF16: return from_hip(fa::launch_dkv_bf16(a, s));
    }
    return FA_ERR_DTYPE;
}

fa_status_t fa_bwd_dkv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                       const float* delta, void* dk, void* dv, int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                       float scale, int causal, int window, fa_dtype_t dtype, void* stream) {
    return dkv_impl(q, k, v, dO, lse, delta, nullptr, 0, 0, nullptr, dk, dv, B, Hq, Hkv, Lq, Lkv, D, D, scale, causal, window,
                    dtype, stream);
}

fa_status_t fa_bwd_dkv_masked(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                              const float* delta, const float* mask, long long mask_stride_b,
                              long long mask_stride_h, void* dk, void* dv, int B, int Hq, int Hkv, int Lq, int Lkv,
                              int D, float scale, int causal, int window, fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_mask(mask, mask_stride_b, mask_stride_h);
    if (st != FA_OK) return st;
    return dkv_impl(q, k, v, dO, lse, delta, mask, mask_stride_b, mask_stride_h, nullptr, dk, dv, B, Hq, Hkv, Lq, Lkv, D, D,
                    scale, causal, window, dtype, stream);
}

static fa_status_t dq_impl(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                           const float* delta, const float* mask, long long msb, long long msh,
                           const unsigned char* bmask, void* dq, int B,
                           int Hq, int Hkv, int Lq, int Lkv, int D, int Dv, float scale, int causal, int window,
                           fa_dtype_t dtype, void* stream) {
    if (!dq) return FA_ERR_NULL;
    fa_status_t st = bwd_common(q, k, v, dO, lse, delta, B, Hq, Hkv, Lq, Lkv, D, Dv, scale, window, dtype);
    if (st != FA_OK) return st;
    if (!aligned16(dq)) return FA_ERR_ALIGN;

    fa::BwdArgs a{q, k, v, dO, lse, delta, dq, nullptr, nullptr, B, Hq, Hkv, Lq, Lkv, D,
                  (float)((double)scale * 1.4426950408889634), scale, causal ? 1 : 0,
                  effective_window(window, Lq), mask, msb, msh, vec4(mask, bmask, msb, msh, Lkv), Dv, bmask};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case FA_F32: return from_hip(fa::launch_dq_f32(a, s));
        case FA_F16: return from_hip(fa::launch_dq_f16(a, s));
        case FA_BF16: return from_hip(fa::launch_dq_bf16(a, s));
    }
    return FA_ERR_DTYPE;
}

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                      const float* delta, void* dq, int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                      int causal, int window, fa_dtype_t dtype, void* stream) {
    return dq_impl(q, k, v, dO, lse, delta, nullptr, 0, 0, nullptr, dq, B, Hq, Hkv, Lq, Lkv, D, D, scale, causal, window, dtype,
                   stream);
}

fa_status_t fa_bwd_dq_masked(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                             const float* delta, const float* mask, long long mask_stride_b, long long mask_stride_h,
                             void* dq, int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale, int causal,
                             int window, fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_mask(mask, mask_stride_b, mask_stride_h);
    if (st != FA_OK) return st;
    return dq_impl(q, k, v, dO, lse, delta, mask, mask_stride_b, mask_stride_h, nullptr, dq, B, Hq, Hkv, Lq, Lkv, D, D, scale,
                   causal, window, dtype, stream);
}

// The descriptor's layout is part of the ABI (the Python binding mirrors it).
static_assert(sizeof(fa_attn_desc_t) == 72 && offsetof(fa_attn_desc_t, mask) == 40 &&
                  offsetof(fa_attn_desc_t, bool_mask) == 64,
              "fa_attn_desc_t layout");

// Extended calls: one descriptor carries the sizes (with a value head dim),
// the mask flags and the optional mask (additive or boolean, not both).
static fa_status_t check_desc(const fa_attn_desc_t* d) {
    if (!d) return FA_ERR_NULL;
    if (d->mask && d->bool_mask) return FA_ERR_ARG;
    if (d->mask) return check_mask(d->mask, d->mask_stride_b, d->mask_stride_h);
    if (d->bool_mask) return check_bool_mask(d->mask_stride_b, d->mask_stride_h);
    return FA_OK;
}

fa_status_t fa_fwd_ex(const fa_attn_desc_t* d, const void* q, const void* k, const void* v, void* o, float* lse,
                      fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_desc(d);
    if (st != FA_OK) return st;
    return fwd_impl(q, k, v, d->mask, d->mask_stride_b, d->mask_stride_h, d->bool_mask, o, lse, d->B, d->Hq, d->Hkv, d->Lq,
                    d->Lkv, d->D, d->Dv, d->scale, d->causal, d->window, dtype, stream);
}

fa_status_t fa_bwd_dkv_ex(const fa_attn_desc_t* d, const void* q, const void* k, const void* v, const void* dO,
                          const float* lse, const float* delta, void* dk, void* dv, fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_desc(d);
    if (st != FA_OK) return st;
    return dkv_impl(q, k, v, dO, lse, delta, d->mask, d->mask_stride_b, d->mask_stride_h, d->bool_mask, dk, dv, d->B, d->Hq,
                    d->Hkv, d->Lq, d->Lkv, d->D, d->Dv, d->scale, d->causal, d->window, dtype, stream);
}

fa_status_t fa_bwd_dq_ex(const fa_attn_desc_t* d, const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* delta, void* dq, fa_dtype_t dtype, void* stream) {
    fa_status_t st = check_desc(d);
    if (st != FA_OK) return st;
    return dq_impl(q, k, v, dO, lse, delta, d->mask, d->mask_stride_b, d->mask_stride_h, d->bool_mask, dq, d->B, d->Hq, d->Hkv,
                   d->Lq, d->Lkv, d->D, d->Dv, d->scale, d->causal, d->window, dtype, stream);
}

}  // extern "C"
