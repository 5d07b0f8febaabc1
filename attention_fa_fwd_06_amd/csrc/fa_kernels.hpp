// gfx950 (CDNA4) kernels of FlashAttention-2 training attention.
//
// Method (mlx-bun flash-attention.ts: forward, D pre-pass, dK/dV and dQ
// shaders; MLX pull request "[Metal] Add Flash Attention VJP for training":
// log2-domain softmax, atomics-free dK/dV by K-row ownership):
//   forward : per query tile, stream the allowed KV tiles; S = scale Q K^T;
//             online softmax with a running max m and sum l; O = P V / l;
//             LSE = m + log l (natural log).
//   backward: Delta = rowsum(dO O); P = exp(S - LSE); dP = dO V^T;
//             dS = P (dP - Delta); dV = P^T dO; dK = scale dS^T Q;
//             dQ = scale dS K.
//
// MI355X mapping. Every product runs on v_mfma_f32_32x32x16_{bf16,f16}
// (v_mfma_f32_32x32x2_f32 for float inputs) with fp32 accumulators. The
// 32x32 accumulator of lane l holds column n = l%32 and rows
// 8*(r/4) + 4*(l/32) + r%4 (r = 0..15). The kernels are arranged so that
// the accumulator of one product feeds the next product's B operand with no
// data movement: a product C[m][n] = sum_k A[m][k] B[k][n] takes B with n on
// lanes and k in registers, which is exactly the accumulator's shape with m
// read as k. The key (or row) order that this implies inside each group of 16
// is matched on the A side by storing the transposed operand in LDS with
// bits 2 and 3 of the row index swapped (tr_pos below). So
//   forward : S^T = K Q^T   (keys x rows)  -> O^T += V^T P^T
//   dQ      : S^T, dP^T = V dO^T           -> dQ^T += K^T dS^T
//   dK/dV   : S = Q K^T, dP = dO V^T       -> dV^T += dO^T P, dK^T += Q^T dS
// In the forward and dQ kernels each lane owns one query row, so the row max,
// the rescale and LSE/Delta lookups are per-lane values plus one exchange
// with lane l^32.
//
// Head dims above 128 split d across DW waves that share the same rows: each
// computes a partial score product over its d slice, the partials are summed
// in LDS in a fixed order (bit-identical in every wave), and each wave then
// accumulates only its d slice of the output.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_types.hpp"

namespace fa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLdsBudget = 160 * 1024;
constexpr float kRescaleLog2 = 8.f;  // forward: move the reference max only past 2^8 growth

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (which __syncthreads()
// would drain), so loads for later tiles stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Position of row j of a tile inside the transposed (row-contiguous) LDS copy:
// bits 2 and 3 swapped, so that lane half h reads its 8 accumulator-ordered
// rows {4h..4h+3, 8+4h..8+4h+3} of each 16-group as one contiguous run.
__device__ __forceinline__ int tr_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// ---------------------------------------------------------------------------
// MFMA on one 16-byte chunk per lane of each operand (natural layout: the
// contraction index runs along the chunk). 16-bit types: one 32x32x16 MFMA.
// float: four 32x32x2 MFMAs, one element each.
// ---------------------------------------------------------------------------
template <class T> struct Mma;

template <> struct Mma<__bf16> {
    static __device__ __forceinline__ void nat(f32x16& acc, u32x4 a, u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};
template <> struct Mma<_Float16> {
    static __device__ __forceinline__ void nat(f32x16& acc, u32x4 a, u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    // The chunk is reinterpreted as a whole float vector before indexing: a
    // bit cast of a single vector element subscript compiles to element 0.
    static __device__ __forceinline__ void nat(f32x16& acc, u32x4 a, u32x4 b) {
        const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[i], acc, 0, 0, 0);
    }
};

// Operand built from 8 accumulator values of one 16-group (accumulator
// indices 8*(g%2) .. 8*(g%2)+7 of block g/2), converted to the input type.
template <class T> struct PF {
    u32x4 v;
};
template <> struct PF<float> {
    f32x4 lo, hi;
};

template <class T> __device__ __forceinline__ PF<T> make_pf(const f32x16& x, int half);

template <> __device__ __forceinline__ PF<__bf16> make_pf<__bf16>(const f32x16& x, int half) {
    bf16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = (__bf16)x[8 * half + i];
    return PF<__bf16>{__builtin_bit_cast(u32x4, t)};
}
template <> __device__ __forceinline__ PF<_Float16> make_pf<_Float16>(const f32x16& x, int half) {
    f16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = (_Float16)x[8 * half + i];
    return PF<_Float16>{__builtin_bit_cast(u32x4, t)};
}
template <> __device__ __forceinline__ PF<float> make_pf<float>(const f32x16& x, int half) {
    PF<float> p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p.lo[i] = x[8 * half + i];
        p.hi[i] = x[8 * half + 4 + i];
    }
    return p;
}

// acc += A_tr * pf where A_tr comes from the transposed LDS copy: p points at
// position 16g + 8h of the lane's row.
template <class T> struct MmaTr {
    static __device__ __forceinline__ void run(f32x16& acc, const char* p, const PF<T>& pf) {
        Mma<T>::nat(acc, ld16(p), pf.v);
    }
};
template <> struct MmaTr<float> {
    static __device__ __forceinline__ void run(f32x16& acc, const char* p, const PF<float>& pf) {
        const f32x4 a0 = __builtin_bit_cast(f32x4, ld16(p)), a1 = __builtin_bit_cast(f32x4, ld16(p + 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[i], pf.lo[i], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[i], pf.hi[i], acc, 0, 0, 0);
    }
};

// float only: acc += X^T * pf with X read element by element from its natural
// (row-major) LDS copy, for tiles whose transposed copy does not fit. p points
// at row 16g + 4h of X and at the lane's column; pitch is the row pitch. The
// rows taken follow the accumulator rows that make_pf packs into lo and hi.
__device__ __forceinline__ void mma_rows_f32(f32x16& acc, const char* p, int pitch, const PF<float>& pf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(*reinterpret_cast<const float*>(p + i * pitch), pf.lo[i], acc, 0,
                                                   0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(*reinterpret_cast<const float*>(p + (8 + i) * pitch), pf.hi[i],
                                                   acc, 0, 0, 0);
}

// Four fp32 values -> four elements of T, stored at p (8 or 16 bytes).
template <class T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
    bf16x4 t = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    st8(p, __builtin_bit_cast(u32x2, t));
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
    f16x4 t = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    st8(p, __builtin_bit_cast(u32x2, t));
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
    st16(p, __builtin_bit_cast(u32x4, f32x4{a, b, c, d}));
}

// ---------------------------------------------------------------------------
// Cooperative tile loaders: global -> registers -> LDS. Rows past `L` and
// 16-byte chunks past D are zero-filled.
// ---------------------------------------------------------------------------

// Natural layout, R rows x NDC chunks; consecutive threads take consecutive
// chunks of a row (coalesced reads, conflict-free 16-byte LDS writes).
template <class T, int R, int NDC, int NT> struct NatTile {
    static constexpr int E = 16 / sizeof(T);
    static constexpr int N = (R * NDC + NT - 1) / NT;
    u32x4 v[N];
    __device__ __forceinline__ void load(const T* base, int row0, int L, int D, int tid) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = tid + n * NT;
            const int r = idx / NDC, c = idx % NDC;
            u32x4 x = zero4();
            if ((R * NDC % NT == 0 || idx < R * NDC) && row0 + r < L && c * E < D)
                x = ld16(base + (size_t)(row0 + r) * D + c * E);
            v[n] = x;
        }
    }
    __device__ __forceinline__ void store(char* lds, int stride, int tid) const {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = tid + n * NT;
            const int r = idx / NDC, c = idx % NDC;
            if (R * NDC % NT == 0 || idx < R * NDC) st16(lds + r * stride + c * 16, v[n]);
        }
    }
};

// Groups of 4 consecutive rows x one chunk. Feeds both the natural copy and
// the transposed copy ([d][tr_pos(row)], rows contiguous) from one read.
template <class T, int R, int NDC, int NT> struct QuadTile {
    static constexpr int E = 16 / sizeof(T);
    static constexpr int G = R / 4;
    static constexpr int N = (G * NDC + NT - 1) / NT;
    u32x4 v[N][4];
    __device__ __forceinline__ void load(const T* base, int row0, int L, int D, int tid) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = tid + n * NT;
            const int t = idx % G, c = idx / G;
            const bool in = (G * NDC % NT == 0 || idx < G * NDC) && c * E < D;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = row0 + 4 * t + rr;
                u32x4 x = zero4();
                if (in && row < L) x = ld16(base + (size_t)row * D + c * E);
                v[n][rr] = x;
            }
        }
    }
    __device__ __forceinline__ void store_nat(char* lds, int stride, int tid) const {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = tid + n * NT;
            const int t = idx % G, c = idx / G;
            if (G * NDC % NT == 0 || idx < G * NDC) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) st16(lds + (4 * t + rr) * stride + c * 16, v[n][rr]);
            }
        }
    }
    __device__ __forceinline__ void store_tr(char* lds, int tstride, int tid) const {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = tid + n * NT;
            const int t = idx % G, c = idx / G;
            if (!(G * NDC % NT == 0 || idx < G * NDC)) continue;
            char* dst = lds + tr_pos(4 * t) * (int)sizeof(T);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    u32x2 o;
                    if (e & 1) {
                        o[0] = (v[n][0][w] >> 16) | (v[n][1][w] & 0xffff0000u);
                        o[1] = (v[n][2][w] >> 16) | (v[n][3][w] & 0xffff0000u);
                    } else {
                        o[0] = (v[n][0][w] & 0xffffu) | (v[n][1][w] << 16);
                        o[1] = (v[n][2][w] & 0xffffu) | (v[n][3][w] << 16);
                    }
                    st8(dst + (c * 8 + e) * tstride, o);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u32x4 o = {v[n][0][e], v[n][1][e], v[n][2][e], v[n][3][e]};
                    st16(dst + (c * 4 + e) * tstride, o);
                }
            }
        }
    }
};

// Sum a per-wave partial accumulator over the DW waves that share it. The
// layout [slot][4][64] of float4 keeps both the writes and the reads
// conflict-free. Every wave sums in the same order, so all get the same bits.
template <int DW, int NB>
__device__ __forceinline__ void reduce_partials(f32x16 (&x)[NB], float* red, int slot0, int dw, int lane) {
    f32x4* r4 = reinterpret_cast<f32x4*>(red);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r4[(((slot0 + dw) * NB + b) * 4 + q) * 64 + lane] =
                f32x4{x[b][4 * q], x[b][4 * q + 1], x[b][4 * q + 2], x[b][4 * q + 3]};
    lds_barrier();
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 s = r4[(((slot0 + 0) * NB + b) * 4 + q) * 64 + lane];
#pragma unroll
            for (int d = 1; d < DW; ++d) s += r4[(((slot0 + d) * NB + b) * 4 + q) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[b][4 * q + i] = s[i];
        }
}

__device__ __forceinline__ bool mask_ok(int i, int j, int causal, int window) {
    return !(causal && j > i) && !(window && i >= j && i - j >= window);
}

// ---------------------------------------------------------------------------
// Mask of the masked entry points (ggmlR R/ag_flash_attn.R, ag_flash_attention
// `mask`, and .ag_flash_mask). Additive float32 form: 0 attends, -inf blocks,
// a finite value is added to the scaled score. Boolean form (a byte per pair):
// nonzero where attention is allowed, read as 0, and zero read as -inf — the
// rule by which the pages turn a logical mask into the additive one. Values
// come back multiplied by log2(e), ready to be added to c * S in the exp2
// domain; positions past Lq or Lkv read as 0 (the flags mask them anyway).
// ---------------------------------------------------------------------------
struct MaskRow {
    const float* f;          // additive mask of one (batch, head), or
    const unsigned char* u;  // boolean mask of one (batch, head)
};
template <class A> __device__ __forceinline__ MaskRow mask_slice(const A& a, int b, int h) {
    const long long off = b * a.msb + h * a.msh;
    return a.bmask ? MaskRow{nullptr, a.bmask + off} : MaskRow{a.mask + off, nullptr};
}
__device__ __forceinline__ float bool_l2(unsigned v) { return v ? 0.f : -INFINITY; }
__device__ __forceinline__ float mask_l2(MaskRow mb, int i, int j, int Lq, int Lkv) {
    if (!(i < Lq && j < Lkv)) return 0.f;
    const size_t idx = (size_t)i * Lkv + j;
    return mb.u ? bool_l2(mb.u[idx]) : mb.f[idx] * kLog2e;
}
// keys j0 .. j0+3 of row i; one load (16 bytes float, 4 bytes boolean) when the
// caller guarantees the alignment (vec) and the four keys exist
__device__ __forceinline__ f32x4 mask4_l2(MaskRow mb, int i, int j0, int Lq, int Lkv, int vec) {
    f32x4 r;
    const size_t idx = (size_t)i * Lkv + j0;
    if (mb.u) {
        if (vec && i < Lq && j0 + 3 < Lkv) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(mb.u + idx);
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = bool_l2((w >> (8 * e)) & 0xffu);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = (i < Lq && j0 + e < Lkv) ? bool_l2(mb.u[idx + e]) : 0.f;
        }
        return r;
    }
    if (vec && i < Lq && j0 + 3 < Lkv) {
        r = *reinterpret_cast<const f32x4*>(mb.f + idx);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (i < Lq && j0 + e < Lkv) ? mb.f[idx + e] : 0.f;
    }
    return r * kLog2e;
}
// LSE in the exp2 domain for the masked backward: a row with no allowed key
// (lse = -inf) becomes +inf, so that c*S + mask - lse is -inf (p = 0) for
// every entry of that row instead of NaN for entries the mask also blocks.
__device__ __forceinline__ float lse_l2_masked(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ===========================================================================
// Forward
// ===========================================================================
template <class T, int DMAX, int BKV, int RW, int DW> struct FwdCfg {
    static constexpr int NT = 64 * RW * DW;
    static constexpr int BQ = 32 * RW;
    static constexpr int E = 16 / sizeof(T);
    static constexpr int DS = DMAX / DW;
    static constexpr int NDC = DMAX / E;
    static constexpr int SCH = DS / E;
    static constexpr int NKG = SCH / 2;
    static constexpr int NDB = DS / 32;
    static constexpr int NKB = BKV / 32;
    static constexpr int NPG = BKV / 16;
    static constexpr int KSTR = DMAX * (int)sizeof(T) + 16;
    static constexpr int VSTR = BKV * (int)sizeof(T) + 16;
    static constexpr int KBYTES = BKV * KSTR;
    static constexpr int VBYTES = DMAX * VSTR;
    static constexpr int RED = DW > 1 ? RW * DW * NKB * 16 * 64 * 4 : 0;
    static constexpr bool DB = 2 * (KBYTES + VBYTES) + RED <= kLdsBudget / 2 ||
                               (DMAX <= 256 && 2 * (KBYTES + VBYTES) + RED <= kLdsBudget);
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int LDS = (DB ? 2 : 1) * STAGE + RED;
    static_assert(LDS <= kLdsBudget, "forward tile does not fit in LDS");
    static_assert(DS % 32 == 0 && BKV % 32 == 0, "tile shape");
};

template <class T, int DMAX, int BKV, int RW, int DW, int OCC, bool MASK>
__global__ __launch_bounds__(64 * RW * DW, OCC) void fa_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<T, DMAX, BKV, RW, DW>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, ln = lane & 31;
    const int rw = w / DW, dw = w % DW;

    const int nqt = (a.Lq + C::BQ - 1) / C::BQ;
    const int BH = a.B * a.Hq;
    int qt = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    if (a.causal) qt = nqt - 1 - qt;  // heaviest query tiles first
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int g = hq / (a.Hq / a.Hkv);
    const int i0 = qt * C::BQ;
    const int row = i0 + 32 * rw + ln;

    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)(b * a.Hq + hq) * a.Lq * a.D;
    const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Lkv * a.D;
    const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Lkv * a.Dv;

    // Q fragments of this wave's 32 rows and d slice (B operand of S^T = K Q^T).
    u32x4 qf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        qf[gi] = (row < a.Lq && c * C::E < a.D) ? ld16(qp + (size_t)row * a.D + c * C::E) : zero4();
    }

    // A negative scale is folded into Q: negating bf16/f16/f32 values is exact,
    // and it keeps the scaling factor c >= 0 for the row max below.
    float c = a.c;
    if (c < 0.f) {
        c = -c;
        const uint32_t sign = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
        for (int gi = 0; gi < C::NKG; ++gi) qf[gi] ^= sign;
    }

    f32x16 o[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) o[i] = zero16();
    float m_ref = -INFINITY, l_run = 0.f;

    // KV tiles that hold at least one allowed key for some row of this tile.
    const int i_last = min(i0 + C::BQ, a.Lq) - 1;
    const int j_lo = a.window ? max(0, i0 - a.window + 1) : 0;
    const int j_hi = a.causal ? min(i_last, a.Lkv - 1) : a.Lkv - 1;
    const int t_lo = j_lo / BKV;
    const int n_t = j_hi >= j_lo ? j_hi / BKV - t_lo + 1 : 0;

    char* kb0 = smem;
    char* vb0 = smem + C::KBYTES;
    float* red = reinterpret_cast<float*>(smem + (C::DB ? 2 : 1) * C::STAGE);

    NatTile<T, BKV, C::NDC, C::NT> kt;
    QuadTile<T, BKV, C::NDC, C::NT> vt;

    auto compute = [&](int it, const char* kl, const char* vl) {
        const int t0 = (t_lo + it) * BKV;
        f32x16 s[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            s[kb] = zero16();
            const char* ka = kl + (32 * kb + ln) * C::KSTR + (dw * C::SCH + h) * 16;
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) Mma<T>::nat(s[kb], ld16(ka + gi * 32), qf[gi]);
        }
        if constexpr (DW > 1) reduce_partials<DW, C::NKB>(s, red, rw * DW, dw, lane);
        if constexpr (MASK) {
            // masked entry points: c S + log2(e) mask, from here on in the exp2 domain
            const MaskRow mb = mask_slice(a, b, hq);
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4 m4 = mask4_l2(mb, row, t0 + 32 * kb + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[kb][4 * qd + i] = fmaf(s[kb][4 * qd + i], c, m4[i]);
                }
        }
        const float cs = MASK ? 1.f : c;  // factor that takes the scores below to the exp2 domain

        const bool need = (t0 + BKV > a.Lkv) || (a.causal && t0 + BKV - 1 > i0) ||
                          (a.window && i_last - t0 >= a.window);
        // Row max of the raw scores (cs >= 0 here, so it commutes with the scaling).
        float mx = -INFINITY;
        if (need) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = t0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (!(j < a.Lkv && mask_ok(row, j, a.causal, a.window))) s[kb][r] = -INFINITY;
                    mx = fmaxf(mx, s[kb][r]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_tile = mx == -INFINITY ? -INFINITY : mx * cs;
        // The reference max moves only when a row's max grows by more than
        // 2^kRescaleLog2: probabilities stay below 2^kRescaleLog2 and O is
        // rescaled rarely. O, l and the LSE all use the same reference, so
        // the result is the same up to rounding. A tile whose scores are all
        // masked leaves the reference at -inf (no update, no NaN).
        const bool upd = m_tile > m_ref + kRescaleLog2;
        // Skipping the rescale for a whole wave pays off only where the branch
        // does not force the accumulators through extra registers (OCC >= 2).
        if (OCC < 2 || __ballot(upd)) {
            const float m_new = upd ? m_tile : m_ref;
            // 0 on a row's first update (O and l are still 0); 1 for rows that keep
            // their reference, including rows still at -inf (no -inf - -inf).
            const float alpha = upd ? fast_exp2(m_ref - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
            m_ref = m_new;
        }
        const float moff = m_ref == -INFINITY ? 0.f : m_ref;
        float ls = 0.f;
        if (need) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sv = s[kb][r];
                    s[kb][r] = sv == -INFINITY ? 0.f : fast_exp2(fmaf(sv, cs, -moff));
                    ls += s[kb][r];
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = fast_exp2(fmaf(s[kb][r], cs, -moff));
                    ls += s[kb][r];
                }
        }
        l_run += ls;

        PF<T> pf[C::NPG];
#pragma unroll
        for (int gg = 0; gg < C::NPG; ++gg) pf[gg] = make_pf<T>(s[gg >> 1], gg & 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const char* va = vl + (dw * C::DS + 32 * db + ln) * C::VSTR + 8 * h * (int)sizeof(T);
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) MmaTr<T>::run(o[db], va + 16 * gg * (int)sizeof(T), pf[gg]);
        }
    };

    if constexpr (C::DB) {
        if (n_t > 0) {
            kt.load(kp, t_lo * BKV, a.Lkv, a.D, tid);
            vt.load(vp, t_lo * BKV, a.Lkv, a.Dv, tid);
            kt.store(kb0, C::KSTR, tid);
            vt.store_tr(vb0, C::VSTR, tid);
            __syncthreads();
        }
        for (int it = 0; it < n_t; ++it) {
            const int cur = it & 1;
            const bool next = it + 1 < n_t;
            if (next) {
                kt.load(kp, (t_lo + it + 1) * BKV, a.Lkv, a.D, tid);
                vt.load(vp, (t_lo + it + 1) * BKV, a.Lkv, a.Dv, tid);
            }
            compute(it, kb0 + cur * C::STAGE, vb0 + cur * C::STAGE);
            if (next) {
                kt.store(kb0 + (cur ^ 1) * C::STAGE, C::KSTR, tid);
                vt.store_tr(vb0 + (cur ^ 1) * C::STAGE, C::VSTR, tid);
            }
            __syncthreads();
        }
    } else {
        for (int it = 0; it < n_t; ++it) {
            __syncthreads();
            kt.load(kp, (t_lo + it) * BKV, a.Lkv, a.D, tid);
            vt.load(vp, (t_lo + it) * BKV, a.Lkv, a.Dv, tid);
            kt.store(kb0, C::KSTR, tid);
            vt.store_tr(vb0, C::VSTR, tid);
            __syncthreads();
            compute(it, kb0, vb0);
        }
    }

    const float l = l_run + __shfl_xor(l_run, 32);
    if (row < a.Lq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        T* op = reinterpret_cast<T*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Lq + row) * a.Dv;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < a.Dv)
                    store4<T>(op + d, o[db][4 * qd] * inv, o[db][4 * qd + 1] * inv, o[db][4 * qd + 2] * inv,
                              o[db][4 * qd + 3] * inv);
            }
        if (h == 0 && dw == 0)
            a.lse[(size_t)(b * a.Hq + hq) * a.Lq + row] = l > 0.f ? (m_ref + fast_log2(l)) * kLn2 : -INFINITY;
    }
}

// ===========================================================================
// Backward pre-pass: delta = rowsum(dO * O). Streaming, HBM-bound: LPR lanes
// per row read consecutive 16-byte chunks and reduce with a butterfly.
// ===========================================================================
template <class T> __device__ __forceinline__ float dot_chunk(u32x4 a, u32x4 b) {
    float s = 0.f;
    if constexpr (sizeof(T) == 2) {
        typedef T tx8 __attribute__((ext_vector_type(8)));
        tx8 x = __builtin_bit_cast(tx8, a), y = __builtin_bit_cast(tx8, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) s += (float)x[i] * (float)y[i];
    } else {
        f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) s += x[i] * y[i];
    }
    return s;
}

template <class T>
__global__ __launch_bounds__(256) void fa_pre_kernel(PreArgs a, int lpr) {
    constexpr int E = 16 / sizeof(T);
    const int nch = a.D / E;
    const int sub = threadIdx.x % lpr;
    const long long row = (long long)blockIdx.x * (256 / lpr) + threadIdx.x / lpr;
    float s = 0.f;
    if (row < a.rows) {
        const T* op = reinterpret_cast<const T*>(a.o) + row * a.D;
        const T* dp = reinterpret_cast<const T*>(a.dO) + row * a.D;
        for (int c = sub; c < nch; c += lpr) s += dot_chunk<T>(ld16(op + c * E), ld16(dp + c * E));
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (row < a.rows && sub == 0) a.delta[row] = s;
}

// ===========================================================================
// dQ: each lane owns one query row; loop over the allowed KV tiles.
// ===========================================================================
template <class T, int DMAX, int BKV, int RW, int DW> struct DqCfg {
    static constexpr int NT = 64 * RW * DW;
    static constexpr int BQ = 32 * RW;
    static constexpr int E = 16 / sizeof(T);
    static constexpr int DS = DMAX / DW;
    static constexpr int NDC = DMAX / E;
    static constexpr int SCH = DS / E;
    static constexpr int NKG = SCH / 2;
    static constexpr int NDB = DS / 32;
    static constexpr int NKB = BKV / 32;
    static constexpr int NPG = BKV / 16;
    static constexpr int KSTR = DMAX * (int)sizeof(T) + 16;
    static constexpr int TSTR = BKV * (int)sizeof(T) + 16;
    static constexpr int KBYTES = BKV * KSTR;
    static constexpr int TBYTES = DMAX * TSTR;
    // Head dim 512 (float): no transposed K copy (the dQ product reads K
    // element by element from the natural copy), and the S and dP partial
    // sums take turns in one buffer, one extra barrier apart.
    static constexpr bool TR = DMAX <= 256;
    static_assert(TR || sizeof(T) == 4, "the natural-copy dQ product is float only");
    static constexpr int STAGE = 2 * KBYTES + (TR ? TBYTES : 0);  // K, V natural (+ K transposed)
    static constexpr int RED1 = DW > 1 ? RW * DW * NKB * 16 * 64 * 4 : 0;
    static constexpr bool SEQ = !TR;
    static constexpr int RED = (SEQ ? 1 : 2) * RED1;
    static constexpr bool DB = 2 * STAGE + RED <= kLdsBudget / 2 || (DMAX <= 128 && 2 * STAGE + RED <= kLdsBudget);
    static constexpr int LDS = (DB ? 2 : 1) * STAGE + RED;
    static_assert(LDS <= kLdsBudget, "dQ tile does not fit in LDS");
};

template <class T, int DMAX, int BKV, int RW, int DW, int OCC, bool MASK>
__global__ __launch_bounds__(64 * RW * DW, OCC) void fa_dq_kernel(BwdArgs a) {
    using C = DqCfg<T, DMAX, BKV, RW, DW>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, ln = lane & 31;
    const int rw = w / DW, dw = w % DW;

    const int nqt = (a.Lq + C::BQ - 1) / C::BQ;
    const int BH = a.B * a.Hq;
    int qt = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    if (a.causal) qt = nqt - 1 - qt;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int g = hq / (a.Hq / a.Hkv);
    const int i0 = qt * C::BQ;
    const int row = i0 + 32 * rw + ln;

    const size_t qoff = (size_t)(b * a.Hq + hq) * a.Lq * a.D;
    const T* qp = reinterpret_cast<const T*>(a.q) + qoff;
    const T* dop = reinterpret_cast<const T*>(a.dO) + (size_t)(b * a.Hq + hq) * a.Lq * a.Dv;
    const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Lkv * a.D;
    const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Lkv * a.Dv;

    u32x4 qf[C::NKG], df[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        qf[gi] = (row < a.Lq && c * C::E < a.D) ? ld16(qp + (size_t)row * a.D + c * C::E) : zero4();
        df[gi] = (row < a.Lq && c * C::E < a.Dv) ? ld16(dop + (size_t)row * a.Dv + c * C::E) : zero4();
    }
    const size_t lrow = (size_t)(b * a.Hq + hq) * a.Lq + row;
    const float lse2 = row < a.Lq ? (MASK ? lse_l2_masked(a.lse[lrow]) : a.lse[lrow] * kLog2e) : 0.f;
    const float dl = row < a.Lq ? a.delta[lrow] : 0.f;
    const MaskRow mb = MASK ? mask_slice(a, b, hq) : MaskRow{nullptr, nullptr};

    f32x16 acc[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) acc[i] = zero16();

    const int i_last = min(i0 + C::BQ, a.Lq) - 1;
    const int j_lo = a.window ? max(0, i0 - a.window + 1) : 0;
    const int j_hi = a.causal ? min(i_last, a.Lkv - 1) : a.Lkv - 1;
    const int t_lo = j_lo / BKV;
    const int n_t = j_hi >= j_lo ? j_hi / BKV - t_lo + 1 : 0;

    float* red = reinterpret_cast<float*>(smem + (C::DB ? 2 : 1) * C::STAGE);
    QuadTile<T, BKV, C::NDC, C::NT> kt;
    NatTile<T, BKV, C::NDC, C::NT> vt;

    auto compute = [&](int it, const char* st) {
        const char* kl = st;
        const char* vl = st + C::KBYTES;
        const char* ktl = st + 2 * C::KBYTES;
        const int t0 = (t_lo + it) * BKV;
        f32x16 s[C::NKB], dp[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            s[kb] = zero16();
            dp[kb] = zero16();
            const int off = (32 * kb + ln) * C::KSTR + (dw * C::SCH + h) * 16;
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) {
                Mma<T>::nat(s[kb], ld16(kl + off + gi * 32), qf[gi]);
                Mma<T>::nat(dp[kb], ld16(vl + off + gi * 32), df[gi]);
            }
        }
        if constexpr (DW > 1) {
            reduce_partials<DW, C::NKB>(s, red, rw * DW, dw, lane);
            if constexpr (C::SEQ) __syncthreads();  // every wave has read the S sums
            reduce_partials<DW, C::NKB>(dp, red + (C::SEQ ? 0 : RW * DW * C::NKB * 16 * 64), rw * DW, dw, lane);
        }
        const bool need = (t0 + BKV > a.Lkv) || (a.causal && t0 + BKV - 1 > i0) ||
                          (a.window && i_last - t0 >= a.window);
        f32x4 m4[C::NKB][4];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
                m4[kb][qd] = MASK ? mask4_l2(mb, row, t0 + 32 * kb + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(MASK ? fmaf(s[kb][r], a.c, m4[kb][r >> 2][r & 3] - lse2) : s[kb][r] * a.c - lse2);
                if (need) {
                    const int j = t0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (!(j < a.Lkv && mask_ok(row, j, a.causal, a.window))) p = 0.f;
                }
                s[kb][r] = p * (dp[kb][r] - dl);  // dS^T
            }
        PF<T> pf[C::NPG];
#pragma unroll
        for (int gg = 0; gg < C::NPG; ++gg) pf[gg] = make_pf<T>(s[gg >> 1], gg & 1);
        if constexpr (C::TR) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const char* ka = ktl + (dw * C::DS + 32 * db + ln) * C::TSTR + 8 * h * (int)sizeof(T);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) MmaTr<T>::run(acc[db], ka + 16 * gg * (int)sizeof(T), pf[gg]);
            }
        } else {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const char* ka = kl + 4 * h * C::KSTR + (dw * C::DS + 32 * db + ln) * (int)sizeof(T);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) mma_rows_f32(acc[db], ka + 16 * gg * C::KSTR, C::KSTR, pf[gg]);
            }
        }
    };

    auto stage_store = [&](char* st) {
        kt.store_nat(st, C::KSTR, tid);
        vt.store(st + C::KBYTES, C::KSTR, tid);
        if constexpr (C::TR) kt.store_tr(st + 2 * C::KBYTES, C::TSTR, tid);
    };

    if constexpr (C::DB) {
        if (n_t > 0) {
            kt.load(kp, t_lo * BKV, a.Lkv, a.D, tid);
            vt.load(vp, t_lo * BKV, a.Lkv, a.Dv, tid);
            stage_store(smem);
            __syncthreads();
        }
        for (int it = 0; it < n_t; ++it) {
            const int cur = it & 1;
            const bool next = it + 1 < n_t;
            if (next) {
                kt.load(kp, (t_lo + it + 1) * BKV, a.Lkv, a.D, tid);
                vt.load(vp, (t_lo + it + 1) * BKV, a.Lkv, a.Dv, tid);
            }
            compute(it, smem + cur * C::STAGE);
            if (next) stage_store(smem + (cur ^ 1) * C::STAGE);
            __syncthreads();
        }
    } else {
        for (int it = 0; it < n_t; ++it) {
            __syncthreads();
            kt.load(kp, (t_lo + it) * BKV, a.Lkv, a.D, tid);
            vt.load(vp, (t_lo + it) * BKV, a.Lkv, a.Dv, tid);
            stage_store(smem);
            __syncthreads();
            compute(it, smem);
        }
    }

    if (row < a.Lq) {
        T* op = reinterpret_cast<T*>(a.dq) + qoff + (size_t)row * a.D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < a.D)
                    store4<T>(op + d, acc[db][4 * qd] * sc, acc[db][4 * qd + 1] * sc, acc[db][4 * qd + 2] * sc,
                              acc[db][4 * qd + 3] * sc);
            }
    }
}

// ===========================================================================
// dK/dV: the workgroup owns BKV = 32*KW keys of one kv head; each lane owns
// one key. It walks every query tile of every query head of the group that
// can see those keys, so dK and dV are written exactly once, without atomics.
// ===========================================================================
template <class T, int DMAX, int BQ, int KW, int DW> struct DkvCfg {
    static constexpr int NT = 64 * KW * DW;
    static constexpr int BKV = 32 * KW;
    static constexpr int E = 16 / sizeof(T);
    static constexpr int DS = DMAX / DW;
    static constexpr int NDC = DMAX / E;
    static constexpr int SCH = DS / E;
    static constexpr int NKG = SCH / 2;
    static constexpr int NDB = DS / 32;
    static constexpr int NRB = BQ / 32;  // 32-row blocks of S
    static constexpr int NPG = BQ / 16;
    static constexpr int QSTR = DMAX * (int)sizeof(T) + 16;
    static constexpr int TSTR = BQ * (int)sizeof(T) + 16;
    static constexpr int QBYTES = BQ * QSTR;
    static constexpr int TBYTES = DMAX * TSTR;
    // Head dim 512 (float): no transposed Q/dO copies (the dV and dK products
    // read them element by element from the natural copies), and the S and
    // dP partial sums take turns in one buffer, one extra barrier apart.
    static constexpr bool TR = DMAX <= 256;
    static_assert(TR || sizeof(T) == 4, "the natural-copy dK/dV products are float only");
    static constexpr int TOFF = 2 * QBYTES + (TR ? 2 * TBYTES : 0);  // lse2 and delta of the tile's rows
    static constexpr int STAGE = TOFF + 2 * BQ * 4;                   // Q, dO (+ Q^T, dO^T), lse2, delta
    static constexpr int RED1 = DW > 1 ? KW * DW * NRB * 16 * 64 * 4 : 0;
    static constexpr bool SEQ = !TR;
    static constexpr int RED = (SEQ ? 1 : 2) * RED1;
    static constexpr bool DB = 2 * STAGE + RED <= kLdsBudget;
    // When even one stage plus the partial-sum buffer overflows LDS, the
    // partial sums reuse the natural Q/dO copies, which are no longer read
    // once the partial score products are done (one extra barrier).
    static constexpr bool ALIAS = TR && !DB && STAGE + RED > kLdsBudget;
    static_assert(!ALIAS || RED <= 2 * QBYTES, "partial sums must fit over the Q/dO copies");
    static constexpr int LDS = ALIAS ? STAGE : (DB ? 2 : 1) * STAGE + RED;
    static_assert(LDS <= kLdsBudget, "dK/dV tile does not fit in LDS");
};

template <class T, int DMAX, int BQ, int KW, int DW, int OCC, bool MASK>
__global__ __launch_bounds__(64 * KW * DW, OCC) void fa_dkv_kernel(BwdArgs a) {
    using C = DkvCfg<T, DMAX, BQ, KW, DW>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, ln = lane & 31;
    const int kw = w / DW, dw = w % DW;

    const int BG = a.B * a.Hkv;
    const int kt_idx = blockIdx.x / BG;  // small key blocks (most work under causal) first
    const int bg = blockIdx.x % BG;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int reps = a.Hq / a.Hkv;
    const int j0 = kt_idx * C::BKV;
    const int key = j0 + 32 * kw + ln;

    const size_t kvoff = (size_t)(b * a.Hkv + g) * a.Lkv * a.D, kvoff_v = (size_t)(b * a.Hkv + g) * a.Lkv * a.Dv;
    const T* kp = reinterpret_cast<const T*>(a.k) + kvoff;
    const T* vp = reinterpret_cast<const T*>(a.v) + kvoff_v;

    // K and V fragments of this lane's key and this wave's d slice
    // (B operands of S = Q K^T and dP = dO V^T).
    u32x4 kf[C::NKG], vf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        kf[gi] = (key < a.Lkv && c * C::E < a.D) ? ld16(kp + (size_t)key * a.D + c * C::E) : zero4();
        vf[gi] = (key < a.Lkv && c * C::E < a.Dv) ? ld16(vp + (size_t)key * a.Dv + c * C::E) : zero4();
    }

    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }

    // Query rows that can attend some key of this block.
    const int j_last = min(j0 + C::BKV, a.Lkv) - 1;
    const int i_lo = a.causal ? j0 : 0;
    const int i_hi = a.window ? min(a.Lq - 1, j_last + a.window - 1) : a.Lq - 1;
    const int qt_lo = i_lo / BQ;
    const int nqt = i_hi >= i_lo ? i_hi / BQ - qt_lo + 1 : 0;
    const int n_it = nqt * reps;

    float* red = reinterpret_cast<float*>(C::ALIAS ? smem : smem + (C::DB ? 2 : 1) * C::STAGE);
    QuadTile<T, BQ, C::NDC, C::NT> qtile, dtile;
    float lse_r = 0.f, dl_r = 0.f;

    auto load = [&](int it) {
        const int hq = g * reps + it / nqt;
        const int q0 = (qt_lo + it % nqt) * BQ;
        const size_t qrow0 = (size_t)(b * a.Hq + hq) * a.Lq;
        qtile.load(reinterpret_cast<const T*>(a.q) + qrow0 * a.D, q0, a.Lq, a.D, tid);
        dtile.load(reinterpret_cast<const T*>(a.dO) + qrow0 * a.Dv, q0, a.Lq, a.Dv, tid);
        if (tid < BQ) {
            const int r = q0 + tid;
            const size_t li = (size_t)(b * a.Hq + hq) * a.Lq + r;
            lse_r = r < a.Lq ? a.lse[li] * kLog2e : 0.f;
            dl_r = r < a.Lq ? a.delta[li] : 0.f;
        }
    };
    auto store = [&](char* st) {
        qtile.store_nat(st, C::QSTR, tid);
        dtile.store_nat(st + C::QBYTES, C::QSTR, tid);
        if constexpr (C::TR) {
            qtile.store_tr(st + 2 * C::QBYTES, C::TSTR, tid);
            dtile.store_tr(st + 2 * C::QBYTES + C::TBYTES, C::TSTR, tid);
        }
        float* lf = reinterpret_cast<float*>(st + C::TOFF);
        if (tid < BQ) {
            lf[tid] = lse_r;
            lf[BQ + tid] = dl_r;
        }
    };
    auto compute = [&](int it, const char* st) {
        const char* ql = st;
        const char* dol = st + C::QBYTES;
        const char* qtl = st + 2 * C::QBYTES;
        const char* dotl = st + 2 * C::QBYTES + C::TBYTES;
        const float* lf = reinterpret_cast<const float*>(st + C::TOFF);
        const int q0 = (qt_lo + it % nqt) * BQ;

        f32x16 s[C::NRB], dp[C::NRB];
#pragma unroll
        for (int rb = 0; rb < C::NRB; ++rb) {
            s[rb] = zero16();
            dp[rb] = zero16();
            const int off = (32 * rb + ln) * C::QSTR + (dw * C::SCH + h) * 16;
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) {
                Mma<T>::nat(s[rb], ld16(ql + off + gi * 32), kf[gi]);
                Mma<T>::nat(dp[rb], ld16(dol + off + gi * 32), vf[gi]);
            }
        }
        if constexpr (DW > 1) {
            if constexpr (C::ALIAS) __syncthreads();  // every wave is done with the natural copies
            reduce_partials<DW, C::NRB>(s, red, kw * DW, dw, lane);
            if constexpr (C::SEQ) __syncthreads();  // every wave has read the S sums
            reduce_partials<DW, C::NRB>(dp, red + (C::SEQ ? 0 : KW * DW * C::NRB * 16 * 64), kw * DW, dw, lane);
        }
        const bool need = (q0 + BQ > a.Lq) || (a.causal && j0 + C::BKV - 1 > q0) ||
                          (a.window && min(q0 + BQ, a.Lq) - 1 - j0 >= a.window);
#pragma unroll
        for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int rl = 32 * rb + 8 * qd + 4 * h;  // first of 4 rows held by this lane
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lf + rl);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(lf + BQ + rl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * qd + i;
                    float p;
                    if constexpr (MASK) {
                        const MaskRow mb = mask_slice(a, b, g * reps + it / nqt);
                        const float l2 = l4[i] == -INFINITY ? INFINITY : l4[i];
                        p = fast_exp2(fmaf(s[rb][r], a.c, mask_l2(mb, q0 + rl + i, key, a.Lq, a.Lkv) - l2));
                    } else {
                        p = fast_exp2(s[rb][r] * a.c - l4[i]);
                    }
                    if (need) {
                        const int irow = q0 + rl + i;
                        if (!(irow < a.Lq && mask_ok(irow, key, a.causal, a.window))) p = 0.f;
                    }
                    s[rb][r] = p;
                    dp[rb][r] = p * (dp[rb][r] - d4[i]);  // dS
                }
            }
        PF<T> pf[C::NPG], sf[C::NPG];
#pragma unroll
        for (int gg = 0; gg < C::NPG; ++gg) {
            pf[gg] = make_pf<T>(s[gg >> 1], gg & 1);
            sf[gg] = make_pf<T>(dp[gg >> 1], gg & 1);
        }
        if constexpr (C::TR) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const int off = (dw * C::DS + 32 * db + ln) * C::TSTR + 8 * h * (int)sizeof(T);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) {
                    MmaTr<T>::run(dv[db], dotl + off + 16 * gg * (int)sizeof(T), pf[gg]);
                    MmaTr<T>::run(dk[db], qtl + off + 16 * gg * (int)sizeof(T), sf[gg]);
                }
            }
        } else {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const int off = 4 * h * C::QSTR + (dw * C::DS + 32 * db + ln) * (int)sizeof(T);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) {
                    mma_rows_f32(dv[db], dol + off + 16 * gg * C::QSTR, C::QSTR, pf[gg]);
                    mma_rows_f32(dk[db], ql + off + 16 * gg * C::QSTR, C::QSTR, sf[gg]);
                }
            }
        }
    };

    if constexpr (C::DB) {
        if (n_it > 0) {
            load(0);
            store(smem);
            __syncthreads();
        }
        for (int it = 0; it < n_it; ++it) {
            const int cur = it & 1;
            const bool next = it + 1 < n_it;
            if (next) load(it + 1);
            compute(it, smem + cur * C::STAGE);
            if (next) store(smem + (cur ^ 1) * C::STAGE);
            __syncthreads();
        }
    } else {
        for (int it = 0; it < n_it; ++it) {
            __syncthreads();
            load(it);
            store(smem);
            __syncthreads();
            compute(it, smem);
        }
    }

    if (key < a.Lkv) {
        T* kop = reinterpret_cast<T*>(a.dk) + kvoff + (size_t)key * a.D;
        T* vop = reinterpret_cast<T*>(a.dv) + kvoff_v + (size_t)key * a.Dv;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < a.D)
                    store4<T>(kop + d, dk[db][4 * qd] * sc, dk[db][4 * qd + 1] * sc, dk[db][4 * qd + 2] * sc,
                              dk[db][4 * qd + 3] * sc);
                if (d < a.Dv)
                    store4<T>(vop + d, dv[db][4 * qd], dv[db][4 * qd + 1], dv[db][4 * qd + 2], dv[db][4 * qd + 3]);
            }
    }
}

// ===========================================================================
// Launchers: tile configuration per (type, head-dim bucket).
// ===========================================================================
template <class K> inline hipError_t set_lds(K kernel, int bytes) {
    if (bytes > 64 * 1024)
        return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return hipSuccess;
}

template <class T, int DMAX, int BKV, int RW, int DW, int OCC>
hipError_t launch_fwd_cfg(const FwdArgs& a, hipStream_t s) {
    using C = FwdCfg<T, DMAX, BKV, RW, DW>;
    auto kern = (a.mask || a.bmask) ? fa_fwd_kernel<T, DMAX, BKV, RW, DW, OCC, true> : fa_fwd_kernel<T, DMAX, BKV, RW, DW, OCC, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long nqt = (a.Lq + C::BQ - 1) / C::BQ;
    const long long grid = nqt * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}

template <class T, int DMAX, int BKV, int RW, int DW, int OCC>
hipError_t launch_dq_cfg(const BwdArgs& a, hipStream_t s) {
    using C = DqCfg<T, DMAX, BKV, RW, DW>;
    auto kern = (a.mask || a.bmask) ? fa_dq_kernel<T, DMAX, BKV, RW, DW, OCC, true> : fa_dq_kernel<T, DMAX, BKV, RW, DW, OCC, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long nqt = (a.Lq + C::BQ - 1) / C::BQ;
    const long long grid = nqt * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}

template <class T, int DMAX, int BQ, int KW, int DW, int OCC>
hipError_t launch_dkv_cfg(const BwdArgs& a, hipStream_t s) {
    using C = DkvCfg<T, DMAX, BQ, KW, DW>;
    auto kern = (a.mask || a.bmask) ? fa_dkv_kernel<T, DMAX, BQ, KW, DW, OCC, true> : fa_dkv_kernel<T, DMAX, BQ, KW, DW, OCC, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long nkt = (a.Lkv + C::BKV - 1) / C::BKV;
    const long long grid = nkt * a.B * a.Hkv;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}

template <class T> hipError_t launch_pre_t(const PreArgs& a, hipStream_t s) {
    constexpr int E = 16 / sizeof(T);
    const int nch = a.D / E;
    int lpr = 1;
    while (lpr < nch && lpr < 64) lpr <<= 1;
    const int rows_per_block = 256 / lpr;
    const long long grid = (a.rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(fa_pre_kernel<T>, dim3((unsigned)grid), dim3(256), 0, s, a, lpr);
    return hipGetLastError();
}

// Head-dim buckets of this path: a runtime D is served by the smallest bucket
// >= D, with the columns past D zero-filled on load and never stored.
inline int dmax_bucket(int D) {
    if (D <= 32) return 32;
    if (D <= 64) return 64;
    if (D <= 96) return 96;
    if (D <= 128) return 128;
    if (D <= 256) return 256;
    return 512;
}

// float tables (the 16-bit types run the LDS-DMA kernels of fa_kernels_lds.hpp):
// <KV or Q tile, waves along rows or keys, waves along d, minimum waves per
// SIMD>. float operands take twice the registers of 16-bit ones, so forward
// tiles at head dim 96/128 take 32 keys and most tables run one wave per
// SIMD; 256 splits d in two slices of 128 and 512 in four (one 32-row or
// 32-key block per workgroup, the backward kernels without transposed copies).
template <class T> hipError_t launch_fwd_t(int dmax, const FwdArgs& a, hipStream_t s) {
    static_assert(sizeof(T) == 4, "float tables");
    switch (dmax) {
        case 32: return launch_fwd_cfg<T, 32, 64, 4, 1, 1>(a, s);
        case 64: return launch_fwd_cfg<T, 64, 64, 4, 1, 1>(a, s);
        case 96: return launch_fwd_cfg<T, 96, 32, 4, 1, 1>(a, s);
        case 128: return launch_fwd_cfg<T, 128, 32, 4, 1, 1>(a, s);
        case 256: return launch_fwd_cfg<T, 256, 32, 2, 2, 1>(a, s);
        case 512: return launch_fwd_cfg<T, 512, 32, 1, 4, 1>(a, s);
    }
    return hipErrorInvalidValue;
}
template <class T> hipError_t launch_dq_t(int dmax, const BwdArgs& a, hipStream_t s) {
    static_assert(sizeof(T) == 4, "float tables");
    switch (dmax) {
        case 32: return launch_dq_cfg<T, 32, 32, 4, 1, 1>(a, s);
        case 64: return launch_dq_cfg<T, 64, 32, 4, 1, 1>(a, s);
        case 96: return launch_dq_cfg<T, 96, 32, 4, 1, 1>(a, s);
        case 128: return launch_dq_cfg<T, 128, 64, 4, 1, 1>(a, s);
        case 256: return launch_dq_cfg<T, 256, 32, 2, 2, 1>(a, s);
        case 512: return launch_dq_cfg<T, 512, 32, 1, 4, 1>(a, s);
    }
    return hipErrorInvalidValue;
}
template <class T> hipError_t launch_dkv_t(int dmax, const BwdArgs& a, hipStream_t s) {
    static_assert(sizeof(T) == 4, "float tables");
    switch (dmax) {
        case 32: return launch_dkv_cfg<T, 32, 64, 4, 1, 1>(a, s);
        case 64: return launch_dkv_cfg<T, 64, 64, 4, 1, 1>(a, s);
        case 96: return launch_dkv_cfg<T, 96, 64, 4, 1, 1>(a, s);
        case 128: return launch_dkv_cfg<T, 128, 64, 4, 1, 1>(a, s);
        case 256: return launch_dkv_cfg<T, 256, 32, 1, 2, 1>(a, s);
        case 512: return launch_dkv_cfg<T, 512, 32, 1, 4, 1>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
