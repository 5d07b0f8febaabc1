// Short-query kernels for 16-bit inputs: query length Lq <= kShortLq and both
// head dims <= 128.
//
// The MLX training-attention pull request ("[Metal] Add Flash Attention VJP
// for training", implementation notes) keeps a separate vector kernel for
// query lengths up to 8, with float32 accumulators and a reduction through
// threadgroup memory, because the tiled kernels spend a whole tile on a
// handful of rows there. The same situation on gfx950 (a 32-row MFMA tile per
// query head, one workgroup per (head, query tile), so a decode-like shape
// leaves most lanes idle, reads every K/V tile once per query head and has
// few workgroups walking long key ranges) is handled by three kernels:
//   * Row packing. The rows of all query heads of one GQA group form one
//     contiguous block of reps*Lq rows in q, o, dO, dQ, lse and delta. The
//     kernels tile that block (packed row p is query head g*reps + p/Lq at
//     position p%Lq), so one tile holds rows of several heads and a K/V tile
//     read serves all of them.
//   * Forward and dQ split the keys inside the workgroup: the KW waves share
//     one row tile and take interleaved 32-key blocks. Each wave streams its
//     own blocks through a private LDS ring (no barrier inside the loop) and
//     keeps its own running max, row sum and accumulators; the partial
//     results are merged through LDS once, at the end. When the (batch, kv
//     head) groups are too few to fill the chip, the host makes the row
//     tiles smaller than 32 rows, so that more workgroups stream the same
//     K/V (the tiles of a group sit on one XCD and share its L2).
//   * dK/dV: each wave owns 32 keys (their K/V fragments stay in registers)
//     and the workgroup walks the packed row tiles, a single tile for
//     reps*Lq <= 32, so the group's query heads cost one pass, not reps.
// The arithmetic per element is that of the tiled kernels (exp2 domain,
// masks, LSE as the natural logarithm, scale applied to dQ and dK at the end).
#pragma once

#include "fa_kernels_lds.hpp"

namespace fa {
namespace lds {

constexpr int kShortLq = 16;
// Forward and dQ shrink the row tile below 32 rows until the grid holds this
// many workgroups (or a tile holds a single row).
#ifndef FA2_SHORT_MIN_GRID
#define FA2_SHORT_MIN_GRID 256
#endif
constexpr int kShortMinGrid = FA2_SHORT_MIN_GRID;

// Query positions [imin, imax] held by the packed rows p0..p1 of a group
// whose heads have Lq rows each (every position when the rows span heads).
__device__ __forceinline__ void packed_span(int p0, int p1, int Lq, int& imin, int& imax) {
    if (p0 / Lq == p1 / Lq) {
        imin = p0 % Lq;
        imax = p1 % Lq;
    } else {
        imin = 0;
        imax = Lq - 1;
    }
}

// Wait until this wave's LDS DMA for the current block has landed, with
// `ahead` later blocks (LPT instructions each) allowed to stay in flight.
template <int LPT, int K> __device__ __forceinline__ void wait_blocks(int ahead) {
    if constexpr (K == 0) {
        wait_vm<0>();
    } else {
        if (ahead >= K) wait_vm<K * LPT>();
        else wait_blocks<LPT, K - 1>(ahead);
    }
}

// Partial accumulators of the KW waves through LDS: [wave][block][4][64]
// float4, one 16-byte slot per lane (conflict-free writes and reads). Every
// wave adds the partials in the same order.
template <int NDB>
__device__ __forceinline__ void put_partials(const f32x16 (&x)[NDB], f32x4* buf, int w, int lane) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            buf[((w * NDB + db) * 4 + q) * 64 + lane] = f32x4{x[db][4 * q], x[db][4 * q + 1], x[db][4 * q + 2],
                                                              x[db][4 * q + 3]};
}
template <int NDB>
__device__ __forceinline__ f32x4 merged(const f32x4* buf, int db, int q, int lane, int kwm) {
    f32x4 s = buf[(db * 4 + q) * 64 + lane];
    for (int u = 1; u < kwm; ++u) s += buf[((u * NDB + db) * 4 + q) * 64 + lane];
    return s;
}

// Launch parameters of the forward and dQ kernels (chosen by the host):
// rows per tile; bytes between the rings of consecutive waves; number of
// waves that can own a key block (only their partial results are merged).
// With at most KW key blocks in all, each wave has at most one block and its
// ring shrinks to one stage, so a short key range needs little LDS.
struct ShortLaunch {
    int rt, stride, kwm;
};

// Forward and dQ: KW waves, each with an NS-stage ring of (K block, V block)
// of 32 keys; after the loop the rings hold the merge buffers instead. LDS is
// the most a launch can use (see ShortLaunch).
template <int DMAX, int KW, int NS> struct ShortCfg {
    static constexpr int ROWB = DMAX * 2, TILEB = 32 * ROWB, STAGEB = 2 * TILEB;
    static constexpr int NKG = DMAX / 16, NDB = DMAX / 32;
    static constexpr int RING = KW * NS * STAGEB;
    static constexpr int ML = (2 * KW * 32 * 4 + 1023) / 1024 * 1024;  // max and sum per row and wave
    static constexpr int MERGE = ML + KW * NDB * 4096;                   // then the accumulators
    static constexpr int LDS = RING > MERGE ? RING : MERGE;
    static_assert(LDS <= kLdsBudget, "short-query rings do not fit in LDS");
    static_assert(NS >= 1 && (DMAX == 64 || DMAX == 128) && KW >= 1 && KW <= 16, "configuration");
    static constexpr int LPT = 2 * DmaPlan<32, DMAX, 1>::NIW;  // DMA instructions per key block
    static_assert((NS - 1) * LPT < 64, "vmcnt range");
};

// Packed-row tile of a forward or dQ workgroup.
struct ShortRows {
    int b, g, reps, P, p0, p1, p, imin, imax;
    bool valid;
    int pc;       // the lane's row, or the tile's first row for lanes without one
    size_t R0;    // first row of the group in q / o / dO / dQ / lse / delta
    __device__ __forceinline__ void init(int Bn, int Hq, int Hkv, int Lq, int RT, int ln) {
        reps = Hq / Hkv;
        P = reps * Lq;
        const int ntile = (P + RT - 1) / RT;
        const int L = xcd_remap(blockIdx.x, ntile * Bn * Hkv);
        const int grp = L / ntile;
        b = grp / Hkv;
        g = grp % Hkv;
        p0 = (L % ntile) * RT;
        p1 = min(p0 + RT, P) - 1;
        p = p0 + ln;
        valid = ln < RT && p <= p1;
        pc = valid ? p : p0;
        packed_span(p0, p1, Lq, imin, imax);
        R0 = (size_t)(b * Hq + g * reps) * Lq;
    }
};

// ===========================================================================
// Forward
// ===========================================================================
template <class T, int DMAX, int KW, int NS, bool MASK>
__global__ __launch_bounds__(64 * KW, 1) void fa_fwd_short_kernel(FwdArgs a, ShortLaunch sl) {
    using C = ShortCfg<DMAX, KW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    ShortRows R;
    R.init(a.B, a.Hq, a.Hkv, a.Lq, sl.rt, ln);
    const int i = R.pc % a.Lq, hq = R.g * R.reps + R.pc / a.Lq;
    const int D = a.D, Dv = a.Dv;

    const rsrc_t rq = make_rsrc(reinterpret_cast<const T*>(a.q) + R.R0 * D, (uint32_t)R.P * (uint32_t)D * 2u);
    const dsc_t rk = make_dsc(reinterpret_cast<const T*>(a.k) + (size_t)(R.b * a.Hkv + R.g) * a.Lkv * D,
                                (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const dsc_t rv = make_dsc(reinterpret_cast<const T*>(a.v) + (size_t)(R.b * a.Hkv + R.g) * a.Lkv * Dv,
                                (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    // Q fragments of the lane's row (B operand of S^T = K Q^T); lanes without
    // a row and the head-dim tail read zero.
    u32x4 qf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = 2 * gi + h;
        qf[gi] = buf_ld16(rq, (R.valid && c * 8 < D) ? (uint32_t)((R.p * D + c * 8) * 2) : kOob);
    }
    float c = a.c;
    if (c < 0.f) {  // fold a negative scale into Q (exact), so that c >= 0 below
        c = -c;
#pragma unroll
        for (int gi = 0; gi < C::NKG; ++gi) qf[gi] ^= 0x80008000u;
    }

    f32x16 o[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] = zero16();
    float m_ref = -INFINITY, l_run = 0.f;

    // key blocks that some row of the tile may see; wave w takes blo + w + KW t
    const int j_lo = a.window ? max(0, R.imin - a.window + 1) : 0;
    const int j_hi = a.causal ? min(R.imax, a.Lkv - 1) : a.Lkv - 1;
    const int blo = j_lo >> 5;
    const int nb = j_hi >= j_lo ? (j_hi >> 5) - blo + 1 : 0;
    const int n_w = nb > w ? (nb - w + KW - 1) / KW : 0;
    // allowed entries: position - key in [dlo, dhi)
    const int dlo = a.causal ? 0 : INT_MIN;
    const int dhi = a.window ? a.window : INT_MAX;

    char* const ring = smem + w * sl.stride;
    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<32, DMAX, 1> dma;
    dma.init(lane, 0, D);
    auto issue = [&](int t, auto slot) {
        char* st = ring + decltype(slot)::value * C::STAGEB;
        const int r0 = (blo + w + KW * t) * 32;
        dma.issue(rk, lds_of(st, smem), r0, D, 0);
        if (Dv == D) dma.issue(rv, lds_of(st + C::TILEB, smem), r0, D, 0);
        else DmaPlan<32, DMAX, 1>::issue_pitch(rv, lds_of(st + C::TILEB, smem), r0, Dv, 0, lane);
    };
    unroll_slots<0, NS - 1>(0, n_w, issue);

    auto step = [&](int t, auto slot) {
        constexpr int SL = decltype(slot)::value;  // stage of block t
        // The slot of block t-1 is free (its reads fed MFMAs that have
        // issued): refill it first, then wait for block t.
        asm volatile("" ::: "memory");
        if (t + NS - 1 < n_w) issue(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
        wait_blocks<C::LPT, NS - 1>(n_w - 1 - t);
        asm volatile("" ::: "memory");

        const char* kl = ring + SL * C::STAGEB;
        const char* vl = kl + C::TILEB;
        const int j0 = (blo + w + KW * t) * 32;
        // two accumulators over the even and odd head-dim fragments, so that
        // consecutive MFMAs do not wait on each other's result
        f32x16 s = zero16(), s1 = zero16();
        {
            u32x4 kfr[C::NKG];
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) kfr[gi] = ld16(kl + to.natural(0, gi, 0));
            sched_fence();
#pragma unroll
            for (int gi = 0; gi < C::NKG; gi += 2) {
                Mma<T>::nat(s, kfr[gi], qf[gi]);
                Mma<T>::nat(s1, kfr[gi + 1], qf[gi + 1]);
            }
        }
        s += s1;
        if constexpr (MASK) {
            // masked entry points: c S + log2(e) mask, from here on in the exp2 domain
            const MaskRow mb = mask_slice(a, R.b, hq);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const f32x4 m4 = mask4_l2(mb, i, j0 + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * qd + e] = fmaf(s[4 * qd + e], c, m4[e]);
            }
        }
        const float cs = MASK ? 1.f : c;

        // V^T fragments, in flight during the softmax
        u32x4 vt[C::NDB][2];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg)
                vt[db][gg] = rd_tr(vl + to.transposed(gg, db, 0, 0), vl + to.transposed(gg, db, 0, 1));

        const bool need = (j0 + 32 > a.Lkv) || (a.causal && j0 + 31 > R.imin) || (a.window && R.imax - j0 >= a.window);
        float mx = -INFINITY;
        if (need) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + 8 * (r >> 2) + 4 * h + (r & 3), dd = i - j;
                const bool ok = (j < a.Lkv) & (dd >= dlo) & (dd < dhi);
                s[r] = ok ? s[r] : -INFINITY;
                mx = fmaxf(mx, s[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_tile = mx == -INFINITY ? -INFINITY : mx * cs;
        const bool upd = m_tile > m_ref + kRescaleLog2;
        if (__ballot(upd)) {
            const float m_new = upd ? m_tile : m_ref;
            const float alpha = upd ? fast_exp2(m_ref - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
            m_ref = m_new;
        }
        const float moff = m_ref == -INFINITY ? 0.f : m_ref;
        if (need) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = s[r] == -INFINITY ? 0.f : fast_exp2(fmaf(s[r], cs, -moff));
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], cs, -moff));
        }

        // O^T += V^T P^T; the row sum adds the probabilities as rounded for the MFMA
        const PF<T> pf0 = make_pf<T>(s, 0), pf1 = make_pf<T>(s, 1);
        float ls0 = add_pair<T>(pf0.v[0], 0.f), ls1 = add_pair<T>(pf0.v[1], 0.f);
        ls0 = add_pair<T>(pf0.v[2], ls0);
        ls1 = add_pair<T>(pf0.v[3], ls1);
        ls0 = add_pair<T>(pf1.v[0], ls0);
        ls1 = add_pair<T>(pf1.v[1], ls1);
        ls0 = add_pair<T>(pf1.v[2], ls0);
        ls1 = add_pair<T>(pf1.v[3], ls1);
        l_run += ls0 + ls1;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            Mma<T>::nat(o[db], vt[db][0], pf0.v);
            Mma<T>::nat(o[db], vt[db][1], pf1.v);
        }
    };
    for (int t = 0; t < n_w; t += NS) unroll_slots<0, NS>(t, n_w, step);

    // Merge: M = max over waves of the reference max; each wave's partial O
    // and row sum are scaled by exp2(m_w - M) and added.
    const float l = l_run + __shfl_xor(l_run, 32);
    lds_barrier();  // every wave is done with its ring and has no DMA in flight
    float* ml = reinterpret_cast<float*>(smem);  // [KW] maxima, then [KW] sums, 32 rows each
    f32x4* part = reinterpret_cast<f32x4*>(smem + C::ML);
    if (h == 0) {
        ml[w * 32 + ln] = m_ref;
        ml[(KW + w) * 32 + ln] = l;
    }
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < KW; ++u) M = fmaxf(M, ml[u * 32 + ln]);
    float lt = 0.f;
#pragma unroll
    for (int u = 0; u < KW; ++u) {
        const float mu = ml[u * 32 + ln];
        lt += (mu == -INFINITY ? 0.f : fast_exp2(mu - M)) * ml[(KW + u) * 32 + ln];
    }
    const float f_own = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - M);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] *= f_own;
    if (w < sl.kwm) put_partials<C::NDB>(o, part, w, lane);
    lds_barrier();
    if (R.valid) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        T* op = reinterpret_cast<T*>(a.o) + (R.R0 + R.p) * Dv;
        for (int db = w; db < C::NDB; db += KW)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * db + 8 * q + 4 * h;
                if (d < Dv) {
                    const f32x4 x = merged<C::NDB>(part, db, q, lane, sl.kwm);
                    store4<T>(op + d, x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
                }
            }
        if (w == 0 && h == 0) a.lse[R.R0 + R.p] = lt > 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
    }
}

// ===========================================================================
// dQ: dQ^T = scale * K^T dS^T summed over the waves' key blocks
// ===========================================================================
template <class T, int DMAX, int KW, int NS, bool MASK, bool VP>
__global__ __launch_bounds__(64 * KW, 1) void fa_dq_short_kernel(BwdArgs a, ShortLaunch sl) {
    using C = ShortCfg<DMAX, KW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    ShortRows R;
    R.init(a.B, a.Hq, a.Hkv, a.Lq, sl.rt, ln);
    const int i = R.pc % a.Lq, hq = R.g * R.reps + R.pc / a.Lq;
    const int D = a.D, Dv = VP ? a.Dv : a.D;

    const rsrc_t rq = make_rsrc(reinterpret_cast<const T*>(a.q) + R.R0 * D, (uint32_t)R.P * (uint32_t)D * 2u);
    const rsrc_t rdo = make_rsrc(reinterpret_cast<const T*>(a.dO) + R.R0 * Dv, (uint32_t)R.P * (uint32_t)Dv * 2u);
    const dsc_t rk = make_dsc(reinterpret_cast<const T*>(a.k) + (size_t)(R.b * a.Hkv + R.g) * a.Lkv * D,
                                (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const dsc_t rv = make_dsc(reinterpret_cast<const T*>(a.v) + (size_t)(R.b * a.Hkv + R.g) * a.Lkv * Dv,
                                (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    u32x4 qf[C::NKG], df[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = 2 * gi + h;
        qf[gi] = buf_ld16(rq, (R.valid && c * 8 < D) ? (uint32_t)((R.p * D + c * 8) * 2) : kOob);
        df[gi] = buf_ld16(rdo, (R.valid && c * 8 < Dv) ? (uint32_t)((R.p * Dv + c * 8) * 2) : kOob);
    }
    const size_t lrow = R.R0 + R.p;
    const float lse2 = R.valid ? (MASK ? lse_l2_masked(a.lse[lrow]) : a.lse[lrow] * kLog2e) : 0.f;
    const float dl = R.valid ? a.delta[lrow] : 0.f;
    const MaskRow mb = MASK ? mask_slice(a, R.b, hq) : MaskRow{nullptr, nullptr};

    f32x16 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = zero16();

    const int j_lo = a.window ? max(0, R.imin - a.window + 1) : 0;
    const int j_hi = a.causal ? min(R.imax, a.Lkv - 1) : a.Lkv - 1;
    const int blo = j_lo >> 5;
    const int nb = j_hi >= j_lo ? (j_hi >> 5) - blo + 1 : 0;
    const int n_w = nb > w ? (nb - w + KW - 1) / KW : 0;
    const int dlo = a.causal ? 0 : INT_MIN;
    const int dhi = a.window ? a.window : INT_MAX;

    char* const ring = smem + w * sl.stride;
    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<32, DMAX, 1> dma;
    dma.init(lane, 0, D);
    auto issue = [&](int t, auto slot) {
        char* st = ring + decltype(slot)::value * C::STAGEB;
        const int r0 = (blo + w + KW * t) * 32;
        dma.issue(rk, lds_of(st, smem), r0, D, 0);
        if constexpr (VP) DmaPlan<32, DMAX, 1>::issue_pitch(rv, lds_of(st + C::TILEB, smem), r0, Dv, 0, lane);
        else dma.issue(rv, lds_of(st + C::TILEB, smem), r0, D, 0);
    };
    unroll_slots<0, NS - 1>(0, n_w, issue);

    auto step = [&](int t, auto slot) {
        constexpr int SL = decltype(slot)::value;
        asm volatile("" ::: "memory");
        if (t + NS - 1 < n_w) issue(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
        wait_blocks<C::LPT, NS - 1>(n_w - 1 - t);
        asm volatile("" ::: "memory");

        const char* kl = ring + SL * C::STAGEB;
        const char* vl = kl + C::TILEB;
        const int j0 = (blo + w + KW * t) * 32;
        // S^T = K Q^T and dP^T = V dO^T, in two halves of the head dim
        f32x16 s = zero16(), dp = zero16();
        {
            constexpr int H = C::NKG / 2;
#pragma unroll
            for (int g0 = 0; g0 < C::NKG; g0 += H) {
                u32x4 kfr[H], vfr[H];
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    const int off = to.natural(0, g0 + e, 0);
                    kfr[e] = ld16(kl + off);
                    vfr[e] = ld16(vl + off);
                }
                sched_fence();
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    Mma<T>::nat(s, kfr[e], qf[g0 + e]);
                    Mma<T>::nat(dp, vfr[e], df[g0 + e]);
                }
            }
        }
        // K^T fragments of the dQ product, in flight during the elementwise part
        u32x4 kt[C::NDB][2];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg)
                kt[db][gg] = rd_tr(kl + to.transposed(gg, db, 0, 0), kl + to.transposed(gg, db, 0, 1));

        const bool need = (j0 + 32 > a.Lkv) || (a.causal && j0 + 31 > R.imin) || (a.window && R.imax - j0 >= a.window);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            f32x4 m4;
            if constexpr (MASK) m4 = mask4_l2(mb, i, j0 + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * qd + e;
                float pv = fast_exp2(fmaf(s[r], a.c, MASK ? m4[e] - lse2 : -lse2));
                if (need) {
                    const int j = j0 + 8 * qd + 4 * h + e, dd = i - j;
                    pv = ((j < a.Lkv) & (dd >= dlo) & (dd < dhi)) ? pv : 0.f;
                }
                s[r] = pv * (dp[r] - dl);  // dS^T
            }
        }
        const PF<T> sf0 = make_pf<T>(s, 0), sf1 = make_pf<T>(s, 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            Mma<T>::nat(acc[db], kt[db][0], sf0.v);
            Mma<T>::nat(acc[db], kt[db][1], sf1.v);
        }
    };
    for (int t = 0; t < n_w; t += NS) unroll_slots<0, NS>(t, n_w, step);

    lds_barrier();  // every wave is done with its ring and has no DMA in flight
    f32x4* part = reinterpret_cast<f32x4*>(smem + C::ML);
    if (w < sl.kwm) put_partials<C::NDB>(acc, part, w, lane);
    lds_barrier();
    if (R.valid) {
        T* op = reinterpret_cast<T*>(a.dq) + (R.R0 + R.p) * D;
        const float sc = a.scale;
        for (int db = w; db < C::NDB; db += KW)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * db + 8 * q + 4 * h;
                if (d < D) {
                    const f32x4 x = merged<C::NDB>(part, db, q, lane, sl.kwm);
                    store4<T>(op + d, x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc);
                }
            }
    }
}

// ===========================================================================
// dK/dV: the workgroup owns 32*KW keys of one kv head, one per lane of each
// wave, and walks the packed row tiles of the group (32 rows each) through an
// NS-stage LDS ring of (Q tile, dO tile, lse, delta).
// ===========================================================================
template <int DMAX, int KW, int NS> struct ShortDkvCfg {
    static constexpr int ROWB = DMAX * 2, TILEB = 32 * ROWB;
    static constexpr int STAGEB = 2 * TILEB + 1024;  // Q, dO, then lse and delta of the 32 rows
    static constexpr int NKG = DMAX / 16, NDB = DMAX / 32;
    static constexpr int LDS = NS * STAGEB;
    static constexpr int LPT = 2 * DmaPlan<32, DMAX, KW>::NIW;
    static_assert(LDS <= kLdsBudget && NS >= 2 && (DMAX == 64 || DMAX == 128) && KW >= 2, "configuration");
    static_assert((NS - 2) * (LPT + 2) < 64, "vmcnt range");
};

template <class T, int DMAX, int KW, int NS, int OCC, bool MASK>
__global__ __launch_bounds__(64 * KW, OCC) void fa_dkv_short_kernel(BwdArgs a) {
    using C = ShortDkvCfg<DMAX, KW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;

    // key blocks of one (batch, kv head) group are consecutive in the logical
    // order, so they share an XCD and read the group's Q/dO through one L2
    const int BKV = 32 * KW;
    const int nkb = (a.Lkv + BKV - 1) / BKV;
    const int L = xcd_remap(blockIdx.x, nkb * a.B * a.Hkv);
    const int grp = L / nkb;
    const int b = grp / a.Hkv, g = grp % a.Hkv;
    const int reps = a.Hq / a.Hkv, P = reps * a.Lq;
    const int j0 = (L % nkb) * BKV, jw = j0 + 32 * w;  // first key of the workgroup, of this wave
    const int key = jw + ln;
    const int D = a.D, Dv = a.Dv;
    const size_t R0 = (size_t)(b * a.Hq + g * reps) * a.Lq;

    const size_t kvhead = (size_t)(b * a.Hkv + g) * a.Lkv * D, kvhead_v = (size_t)(b * a.Hkv + g) * a.Lkv * Dv;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const T*>(a.k) + kvhead, (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const T*>(a.v) + kvhead_v, (uint32_t)a.Lkv * (uint32_t)Dv * 2u);
    const dsc_t rq = make_dsc(reinterpret_cast<const T*>(a.q) + R0 * D, (uint32_t)P * (uint32_t)D * 2u);
    const dsc_t rdo = make_dsc(reinterpret_cast<const T*>(a.dO) + R0 * Dv, (uint32_t)P * (uint32_t)Dv * 2u);
    const dsc_t rl = make_dsc(a.lse + R0, (uint32_t)P * 4u);
    const dsc_t rd = make_dsc(a.delta + R0, (uint32_t)P * 4u);

    // K and V fragments of the lane's key (B operands of S = Q K^T, dP = dO V^T)
    u32x4 kf[C::NKG], vf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = 2 * gi + h;
        kf[gi] = buf_ld16(rk, c * 8 < D ? (uint32_t)((key * D + c * 8) * 2) : kOob);
        vf[gi] = buf_ld16(rv, c * 8 < Dv ? (uint32_t)((key * Dv + c * 8) * 2) : kOob);
    }
    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
        dk[db] = zero16();
        dv[db] = zero16();
    }

    // under a causal mask only keys below Lq are seen by any row
    const int n_it = (a.causal && j0 > a.Lq - 1) ? 0 : (P + 31) / 32;
    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<32, DMAX, KW> dma;
    dma.init(lane, w, D);
    constexpr int WD = 1;  // wave 0 fetches lse, wave 1 delta
    auto issue = [&](int it) {
        char* st = smem + (it % NS) * C::STAGEB;
        dma.issue(rq, lds_of(st, smem), it * 32, D, w);
        if (Dv == D) dma.issue(rdo, lds_of(st + C::TILEB, smem), it * 32, D, w);
        else DmaPlan<32, DMAX, KW>::issue_pitch(rdo, lds_of(st + C::TILEB, smem), it * 32, Dv, w, lane);
        if (w == 0 && lane < 32) dma4(rl, lds_of(st + 2 * C::TILEB, smem), (uint32_t)(it * 32 + lane) * 4u);
        if (w == WD && lane < 32) dma4(rd, lds_of(st + 2 * C::TILEB + 128, smem), (uint32_t)(it * 32 + lane) * 4u);
    };
    const int extra = (w == 0) + (w == WD);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < n_it) issue(s);

    for (int it = 0; it < n_it; ++it) {
        if (it + NS - 2 < n_it) {
            if (extra) wait_vm<(NS - 2) * (C::LPT + 1)>();
            else wait_vm<(NS - 2) * C::LPT>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();  // tile it visible to all waves; every wave is done with tile it-1
        if (it + NS - 1 < n_it) issue(it + NS - 1);

        const char* ql = smem + (it % NS) * C::STAGEB;
        const char* dol = ql + C::TILEB;
        const float* lf = reinterpret_cast<const float*>(ql + 2 * C::TILEB);
        const int p0 = it * 32, p1 = min(p0 + 31, P - 1);
        int imin, imax;
        packed_span(p0, p1, a.Lq, imin, imax);
        // nothing of this wave's keys is seen by the tile's rows
        if ((a.causal && imax < jw) || (a.window && imin - (jw + 31) >= a.window)) continue;

        f32x16 s = zero16(), dp = zero16();
        {
            constexpr int H = C::NKG / 4;
#pragma unroll
            for (int g0 = 0; g0 < C::NKG; g0 += H) {
                u32x4 qfr[H], dfr[H];
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    const int off = to.natural(0, g0 + e, 0);
                    qfr[e] = ld16(ql + off);
                    dfr[e] = ld16(dol + off);
                }
                sched_fence();
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    Mma<T>::nat(s, qfr[e], kf[g0 + e]);
                    Mma<T>::nat(dp, dfr[e], vf[g0 + e]);
                }
            }
        }
        // Rows past the group's end hold zero Q and dO; they are cleared here as
        // well, so that a large mask value cannot turn them into inf * 0.
        const bool need = (p0 + 32 > P) || (a.causal && jw + 31 > imin) || (a.window && imax - jw >= a.window);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int rl = 8 * qd + 4 * h;  // first of the 4 rows this lane holds
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lf + rl);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(lf + 32 + rl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * qd + e, prow = p0 + rl + e;
                float pv;
                if constexpr (MASK) {
                    const int pr = min(prow, P - 1);
                    const MaskRow mb = mask_slice(a, b, g * reps + pr / a.Lq);
                    pv = fast_exp2(fmaf(s[r], a.c, mask_l2(mb, pr % a.Lq, key, a.Lq, a.Lkv) - lse_l2_masked(l4[e])));
                } else {
                    pv = fast_exp2(fmaf(s[r], a.c, -l4[e] * kLog2e));
                }
                if (need && !(prow < P && mask_ok(prow % a.Lq, key, a.causal, a.window))) pv = 0.f;
                s[r] = pv;
                dp[r] = pv * (dp[r] - d4[e]);  // dS
            }
        }
        const PF<T> pf0 = make_pf<T>(s, 0), pf1 = make_pf<T>(s, 1);
        const PF<T> sf0 = make_pf<T>(dp, 0), sf1 = make_pf<T>(dp, 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            u32x4 dofr[2], qfr[2];
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int o0 = to.transposed(gg, db, 0, 0), o1 = to.transposed(gg, db, 0, 1);
                dofr[gg] = rd_tr(dol + o0, dol + o1);
                qfr[gg] = rd_tr(ql + o0, ql + o1);
            }
            sched_fence();
            Mma<T>::nat(dv[db], dofr[0], pf0.v);
            Mma<T>::nat(dv[db], dofr[1], pf1.v);
            Mma<T>::nat(dk[db], qfr[0], sf0.v);
            Mma<T>::nat(dk[db], qfr[1], sf1.v);
        }
    }

    if (key < a.Lkv) {
        T* kop = reinterpret_cast<T*>(a.dk) + kvhead + (size_t)key * D;
        T* vop = reinterpret_cast<T*>(a.dv) + kvhead_v + (size_t)key * Dv;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 32 * db + 8 * q + 4 * h;
                if (d < D)
                    store4<T>(kop + d, dk[db][4 * q] * sc, dk[db][4 * q + 1] * sc, dk[db][4 * q + 2] * sc,
                              dk[db][4 * q + 3] * sc);
                if (d < Dv)
                    store4<T>(vop + d, dv[db][4 * q], dv[db][4 * q + 1], dv[db][4 * q + 2], dv[db][4 * q + 3]);
            }
    }
}

// ===========================================================================
// Launchers
// ===========================================================================
// Rows per forward/dQ tile: 32, or fewer when the groups alone do not give
// the grid kShortMinGrid workgroups.
inline int short_rows(int P, long long groups) {
    const long long want = (kShortMinGrid + groups - 1) / groups;  // tiles per group
    const long long rt = (P + want - 1) / want;
    return rt < 1 ? 1 : rt > 32 ? 32 : (int)rt;
}

inline bool use_short(int Lq, int D, int Dv) { return Lq <= kShortLq && D <= 128 && Dv <= 128; }

// Launch parameters, LDS bytes and grid of a forward or dQ launch.
template <int DMAX, int KW, int NS>
inline ShortLaunch short_launch(int Hq, int Hkv, int Lq, int Lkv, long long groups, int& lds, long long& grid) {
    using C = ShortCfg<DMAX, KW, NS>;
    const int P = (Hq / Hkv) * Lq;
    const int nbk = (Lkv + 31) / 32;  // key blocks of the longest key range a tile can see
    ShortLaunch sl;
    sl.rt = short_rows(P, groups);
    int ring;
    if (nbk <= KW) {
        sl.stride = C::STAGEB;
        sl.kwm = nbk;
        ring = nbk * C::STAGEB;
    } else {
        sl.stride = NS * C::STAGEB;
        sl.kwm = KW;
        ring = C::RING;
    }
    const int merge = C::ML + sl.kwm * C::NDB * 4096;
    lds = ring > merge ? ring : merge;
    grid = (long long)((P + sl.rt - 1) / sl.rt) * groups;
    return sl;
}

template <class T, int DMAX, int KW, int NS>
hipError_t launch_fwd_short(const FwdArgs& a, hipStream_t s) {
    using C = ShortCfg<DMAX, KW, NS>;
    auto kern = (a.mask || a.bmask) ? fa_fwd_short_kernel<T, DMAX, KW, NS, true> : fa_fwd_short_kernel<T, DMAX, KW, NS, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    int lds;
    long long grid;
    const ShortLaunch sl = short_launch<DMAX, KW, NS>(a.Hq, a.Hkv, a.Lq, a.Lkv, (long long)a.B * a.Hkv, lds, grid);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KW), lds, s, a, sl);
    return hipGetLastError();
}
template <class T, int DMAX, int KW, int NS>
hipError_t launch_dq_short(const BwdArgs& a, hipStream_t s) {
    using C = ShortCfg<DMAX, KW, NS>;
    auto kern = a.Dv != a.D ? ((a.mask || a.bmask) ? fa_dq_short_kernel<T, DMAX, KW, NS, true, true>
                                      : fa_dq_short_kernel<T, DMAX, KW, NS, false, true>)
                            : ((a.mask || a.bmask) ? fa_dq_short_kernel<T, DMAX, KW, NS, true, false>
                                      : fa_dq_short_kernel<T, DMAX, KW, NS, false, false>);
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    int lds;
    long long grid;
    const ShortLaunch sl = short_launch<DMAX, KW, NS>(a.Hq, a.Hkv, a.Lq, a.Lkv, (long long)a.B * a.Hkv, lds, grid);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KW), lds, s, a, sl);
    return hipGetLastError();
}
template <class T, int DMAX, int KW, int NS, int OCC>
hipError_t launch_dkv_short(const BwdArgs& a, hipStream_t s) {
    using C = ShortDkvCfg<DMAX, KW, NS>;
    auto kern = (a.mask || a.bmask) ? fa_dkv_short_kernel<T, DMAX, KW, NS, OCC, true>
                       : fa_dkv_short_kernel<T, DMAX, KW, NS, OCC, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long grid = (long long)((a.Lkv + 32 * KW - 1) / (32 * KW)) * a.B * a.Hkv;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KW), C::LDS, s, a);
    return hipGetLastError();
}

// <waves splitting the keys, ring stages per wave> (forward, dQ) and
// <waves owning 32 keys each, ring stages, min waves per SIMD> (dK/dV).
// Forward and dQ run eight waves of one stage each (D = 128: two waves per
// SIMD hide each other's DMA waits) or, when the whole key range is at most
// kShortFewBlocks blocks of 32, four waves (each has at most one block, and
// smaller workgroups leave room for more of them per CU).
constexpr int kShortFewBlocks = 4;
#ifndef FA2_SHORT_FWD_64
#define FA2_SHORT_FWD_64 8, 2
#endif
#ifndef FA2_SHORT_FWD_128
#define FA2_SHORT_FWD_128 8, 1
#endif
#ifndef FA2_SHORT_DQ_64
#define FA2_SHORT_DQ_64 8, 2
#endif
#ifndef FA2_SHORT_DQ_128
#define FA2_SHORT_DQ_128 8, 1
#endif
#ifndef FA2_SHORT_FEW
#define FA2_SHORT_FEW 4, 1
#endif
#ifndef FA2_SHORT_DKV_64
#define FA2_SHORT_DKV_64 4, 2, 2
#endif
#ifndef FA2_SHORT_DKV_128
#define FA2_SHORT_DKV_128 4, 2, 2
#endif

}  // namespace lds
}  // namespace fa
