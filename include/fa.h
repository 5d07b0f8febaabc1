/*
 * fa.h — C ABI of the MI355X (gfx950) FlashAttention-2 training attention.
 *
 * Four calls make one training step of softmax attention:
 *   fa_fwd            O = softmax(scale * Q K^T + mask) V, plus the per-row LSE
 *   fa_bwd_preprocess Delta = rowsum(dO * O)
 *   fa_bwd_dkv        dK, dV (each workgroup owns a block of K/V rows; no atomics)
 *   fa_bwd_dq         dQ
 * and masked variants of the forward and both backward calls that take an
 * additive mask tensor (fa_fwd_masked, fa_bwd_dkv_masked, fa_bwd_dq_masked),
 * and extended variants whose value head dim may differ from the query/key
 * head dim (fa_fwd_ex, fa_bwd_dkv_ex, fa_bwd_dq_ex).
 *
 * Sources: mlx-bun flash-attention.ts (flashForward and flashBackward host
 * functions and the forward, D pre-pass, dK/dV and dQ shaders); the MLX pull
 * request "[Metal] Add Flash Attention VJP for training" (implementation notes:
 * LSE cached by the forward, two-kernel atomics-free backward with K-row
 * ownership); ggmlR R/ag_flash_attn.R (ag_flash_attention: argument checks that
 * raise errors instead of aborting, default scale 1/sqrt(d_head)).
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout: row-major, head_dim fastest, contiguous.
 *   q, o, dO, dQ : [B, Hq,  Lq,  D]
 *   k, v, dK, dV : [B, Hkv, Lkv, D]
 *   lse, delta   : [B, Hq,  Lq]  always float32
 * q, k, v, o, dO, dQ, dK and dV share one element type (fa_dtype_t); all
 * accumulation is float32.
 * GQA/MQA: Hq must be a multiple of Hkv; query head h reads kv head h / (Hq/Hkv),
 * so consecutive query heads share a kv head.
 * Mask: query row i may attend key j iff
 *   (!causal || j <= i) && (window == 0 || j > i || i - j < window).
 * Causal is aligned top-left (row i sees keys 0..i) also when Lq != Lkv. A
 * window keeps the query's own key and the window-1 keys before it; without
 * causal it trims only the past. window == 0 disables it.
 * scale multiplies Q K^T before masking and before the LSE; the usual value is
 * 1/sqrt(D).
 * lse is the NATURAL-log logsumexp of the scaled, masked scores of each row.
 * A row with no allowed key gets O = 0, lse = -inf and no gradient.
 *
 * Ownership and execution
 * -----------------------
 * Every pointer is a DEVICE pointer owned by the caller; the library allocates,
 * frees and synchronises nothing and keeps no state. All work is enqueued on
 * `stream` (a hipStream_t; NULL = the null stream) and the call returns right
 * after the launch. Outputs must not alias inputs. Required order on one
 * stream: fa_fwd -> fa_bwd_preprocess -> {fa_bwd_dkv, fa_bwd_dq} (the last two
 * are independent of each other). Results are deterministic: the same inputs
 * give bit-identical outputs.
 *
 * Errors
 * ------
 * Arguments are checked before anything is launched; a bad argument returns a
 * negative fa_status_t and touches no memory. The library never aborts.
 * FA_ERR_LAUNCH reports a failure of the HIP launch itself.
 *
 * Limits: 1 <= B, Hq, Hkv, Lq, Lkv; Hq % Hkv == 0; 32 <= D <= 512 and
 * D % 8 == 0; window >= 0; scale finite; every pointer 16-byte aligned;
 * B*Hq*Lq*D and B*Hkv*Lkv*D below 2^31; Lq*D and Lkv*D at most 2^29;
 * Lq, Lkv below 2^24.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_F32 = 0,
    FA_F16 = 1,
    FA_BF16 = 2
} fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,    /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,   /* a size is < 1, too large, or Hq % Hkv != 0 */
    FA_ERR_HEADDIM = -3, /* D outside [32, 512] or not a multiple of 8 */
    FA_ERR_DTYPE = -4,   /* dtype is not one of fa_dtype_t */
    FA_ERR_ALIGN = -5,   /* a pointer is not 16-byte aligned */
    FA_ERR_ARG = -6,     /* negative window, non-finite scale, or a mask stride outside [0, 2^40] */
    FA_ERR_LAUNCH = -7   /* the HIP kernel launch failed */
} fa_status_t;

/*
 * Forward (mlx-bun flash-attention.ts, flashForward and the forward shader).
 * Reads q, k, v; writes o [B,Hq,Lq,D] (dtype) and lse [B,Hq,Lq] (float32).
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                   float scale, int causal, int window, fa_dtype_t dtype, void* stream);

/*
 * Backward pre-pass (mlx-bun flash-attention.ts, D pre-pass shader):
 * delta[b,h,i] = sum_d dO[b,h,i,d] * o[b,h,i,d] in float32, from the stored o.
 * Reads o and dO [B,Hq,Lq,D]; writes delta [B,Hq,Lq] (float32).
 */
fa_status_t fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                              int B, int Hq, int Lq, int D, fa_dtype_t dtype, void* stream);

/*
 * dK and dV (mlx-bun flash-attention.ts, dK/dV shader; MLX VJP pull request,
 * K-row ownership). Each workgroup owns a block of K/V rows of one kv head and
 * loops over every query tile of every query head in its group, so dK and dV
 * are written once, without atomics:
 *   P  = exp(scale * Q K^T - lse)   (0 where masked)
 *   dS = P * (dO V^T - delta)
 *   dV = sum_h P^T dO,   dK = scale * sum_h dS^T Q.
 * Reads q, k, v, dO, lse, delta; writes dk, dv [B,Hkv,Lkv,D] (dtype).
 */
fa_status_t fa_bwd_dkv(const void* q, const void* k, const void* v, const void* dO,
                       const float* lse, const float* delta, void* dk, void* dv,
                       int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                       float scale, int causal, int window, fa_dtype_t dtype, void* stream);

/*
 * dQ (mlx-bun flash-attention.ts, dQ shader; MLX VJP pull request, dQ kernel
 * with an outer loop over KV blocks): dQ = scale * dS K with dS as above.
 * Reads q, k, v, dO, lse, delta; writes dq [B,Hq,Lq,D] (dtype).
 */
fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                      const float* lse, const float* delta, void* dq,
                      int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                      float scale, int causal, int window, fa_dtype_t dtype, void* stream);

/*
 * Masked variants (ggmlR R/ag_flash_attn.R, ag_flash_attention: an optional
 * numeric mask per (query, key), 0 to attend and -Inf to block, used for the
 * forward and for the gradient alike).
 *
 * mask is a DEVICE pointer to float32 values; the value for batch b, query
 * head h, query row i and key j is
 *     mask[b * mask_stride_b + h * mask_stride_h + i * Lkv + j]
 * with the strides in elements and 0 broadcasting over that dimension: one
 * [Lq, Lkv] mask for every head has both strides 0, a [B, 1, Lq, Lkv] mask
 * has mask_stride_b = Lq*Lkv and mask_stride_h = 0, a [B, Hq, Lq, Lkv] mask
 * Hq*Lq*Lkv and Lq*Lkv. Rows are query-major (i is the slow index), the
 * memory order of ggml's [n_kv, n_q] mask.
 * The value is added to the scaled score before the softmax:
 *     s_ij = scale * q_i . k_j + mask_ij,
 * so 0 leaves a score alone and -inf removes the pair; the causal flag and
 * the window apply on top, and lse is the natural-log logsumexp of these
 * s_ij. Values must be finite or -inf (NaN and +inf are not checked and give
 * undefined results). The three calls of one step must get the same mask;
 * fa_bwd_preprocess needs none. A row whose keys are all removed gets O = 0,
 * lse = -inf and no gradient. The mask carries no gradient.
 * Extra checks: mask non-NULL (FA_ERR_NULL) and 4-byte aligned (FA_ERR_ALIGN);
 * both strides in [0, 2^40] (FA_ERR_ARG). The mask is read with 16-byte loads
 * when it is 16-byte aligned and Lkv and both strides are multiples of 4, with
 * 4-byte loads otherwise. Everything else is as for the unmasked calls.
 */
fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, const float* mask,
                          long long mask_stride_b, long long mask_stride_h, void* o, float* lse,
                          int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                          float scale, int causal, int window, fa_dtype_t dtype, void* stream);

fa_status_t fa_bwd_dkv_masked(const void* q, const void* k, const void* v, const void* dO,
                              const float* lse, const float* delta, const float* mask,
                              long long mask_stride_b, long long mask_stride_h, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                              float scale, int causal, int window, fa_dtype_t dtype, void* stream);

fa_status_t fa_bwd_dq_masked(const void* q, const void* k, const void* v, const void* dO,
                             const float* lse, const float* delta, const float* mask,
                             long long mask_stride_b, long long mask_stride_h, void* dq,
                             int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                             float scale, int causal, int window, fa_dtype_t dtype, void* stream);

/*
 * Extended calls: everything the calls above do, described by one struct, plus
 * a value head dim Dv that may differ from the query/key head dim D (the pages'
 * Dv != Dk case).
 *   q, dq       : [B, Hq,  Lq,  D]      k, dk : [B, Hkv, Lkv, D]
 *   o, dO       : [B, Hq,  Lq,  Dv]     v, dv : [B, Hkv, Lkv, Dv]
 *   lse, delta  : [B, Hq,  Lq]
 * fa_bwd_preprocess is called with its D set to Dv. Dv follows the rules of
 * D (a multiple of 8 in [32, 512], the same size
 * limits for the tensors that carry it); both head dims are served by the
 * tile shape of the larger one (the columns past each tensor's own head dim
 * are zero in the tiles and never stored). mask == NULL means no mask (the
 * strides are then ignored); otherwise it is read exactly as by the masked
 * calls. desc == NULL returns FA_ERR_NULL.
 *
 * bool_mask (ggmlR R/ag_flash_attn.R, .ag_flash_mask: a logical mask is the
 * friendlier spelling, TRUE where attention is allowed, and stands for 0 where
 * TRUE and -Inf where FALSE): one byte per (query, key) pair, indexed with the
 * same strides (in bytes, since an element is one byte) and broadcasting as the
 * additive mask; a nonzero byte lets the pair attend, a zero byte removes it.
 * It behaves exactly as the additive mask holding 0 and -inf in those places,
 * at a quarter of its size. Any alignment is accepted (four keys are read with
 * one 4-byte load when the pointer is 4-byte aligned and Lkv and both strides
 * are multiples of 4). mask and bool_mask may not both be set (FA_ERR_ARG);
 * the strides must lie in [0, 2^40] (FA_ERR_ARG).
 */
typedef struct {
    int B, Hq, Hkv, Lq, Lkv;
    int D;                      /* query/key head dim */
    int Dv;                     /* value head dim (v, o, dO, dv) */
    float scale;
    int causal;
    int window;
    const float* mask;          /* optional additive mask (device pointer) */
    long long mask_stride_b;    /* element strides of the mask, 0 broadcasts */
    long long mask_stride_h;
    const unsigned char* bool_mask; /* optional boolean mask (device pointer) */
} fa_attn_desc_t;

fa_status_t fa_fwd_ex(const fa_attn_desc_t* desc, const void* q, const void* k, const void* v,
                      void* o, float* lse, fa_dtype_t dtype, void* stream);

fa_status_t fa_bwd_dkv_ex(const fa_attn_desc_t* desc, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const float* delta, void* dk, void* dv,
                          fa_dtype_t dtype, void* stream);

fa_status_t fa_bwd_dq_ex(const fa_attn_desc_t* desc, const void* q, const void* k, const void* v,
                         const void* dO, const float* lse, const float* delta, void* dq,
                         fa_dtype_t dtype, void* stream);

/* Static, never-NULL description of a status code. */
const char* fa_status_string(fa_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
