// dQ for the 256-wide head-dim bucket with four waves per 32-row block.
//
// The query-side half of the backward pass (mlx-bun flash-attention.ts, DQ
// shader: dQ += dS K over the key tiles, dS = P (dP - Delta), P = exp(S -
// LSE)), computed as in fa_dq_lds_kernel; only the division of the work
// differs.
//
// At D = 256 a wave holding the Q and dO fragments of 32 rows (128
// registers) and the dQ accumulator of those rows (128) runs alone on its
// SIMD. Here each 32-row block has two producers, and the accumulator is
// spread over consumer waves:
//   A: S^T = K Q^T and P^T = exp2(c S^T - log2(e) lse), masked, stored for C
//   C: dP^T = V dO^T and dS^T = P^T (dP^T - Delta), stored for D
//   D: dQ^T += K^T dS^T for two row blocks and a quarter of the head dim
// A keeps the Q fragments, C the dO fragments, each D wave 64 accumulator
// registers, so four waves share each SIMD (128 registers each): a workgroup
// owns four row blocks (128 rows, sixteen waves) and SIMD s runs A of row
// block s, C of s+1 and the two D waves of column quarter s, 16 + 16 + 8 + 8
// MFMAs per 32-key tile. A D wave over two row blocks uses each transposed
// K fragment for two MFMAs: with one row block and half the head dim per D
// wave every fragment was read four times per tile, and the D waves, bound
// by those LDS reads (1350-1770 cycles for 8 MFMAs per tile, by s_memtime
// stamps), set the pace: 218.4 against 211.8 us on the 8192-token windowed
// workload. (One D wave per row block, three waves per SIMD at 168
// registers, spilled.)
//
// One barrier per key tile. In iteration t (after barrier t) A computes S
// and P of tile t+1; C forms dS of t from its dP of t (computed the
// iteration before) and A's P of t, stores it and computes dP of t+1; D
// updates dQ with the dS of t-1 stored the iteration before. K goes through
// a four-slot ring (t-1 for D, t, t+1 for A, t+2 in flight), V through two
// (t+1 for C, t+2 in flight); P and dS have two buffers each. The C waves
// issue the LDS-DMA requests: 209.2 us on the 8192-token windowed workload,
// against 211.8 with the A and C waves sharing them, 214.2 by the D waves and
// 218.0 by the A waves (one box, three runs each); K by the A waves and V by
// the C waves, on another box, 217.5 against 216.2; by the first D wave of
// each SIMD (which stamps showed idle at the barrier for about 1000 cycles a
// tile), on a third, 213.9 against 207.9. The C waves issue right after the
// barrier: after their dS store the same (210.8 against 210.6), after their
// chain 214.6. Every chain requests its
// LDS fragments three MFMAs ahead (two: 220.2 against 217.5 us).
// dQ leaves through LDS (whole row pieces per store instruction): the V
// ring and the two K slots that no wave reads after the last barrier.
#pragma once

#include "fa_kernels_dkvq.hpp"

namespace fa {
namespace lds {

template <class T, int DMAX> struct DqTriCfg {
    static constexpr int RB = 4;  // 32-row blocks per workgroup
    static constexpr int NW = 4 * RB, NT = 64 * NW, BQ = 32 * RB;
    static constexpr int BKV = 32;              // keys per tile
    static constexpr int NKS = 4, NVS = 2;      // K and V ring slots
    static constexpr int NKG = DMAX / 16, NDB = DMAX / 32, NPG = BKV / 16;
    static constexpr int QD = DMAX / 4, NQB = NDB / 4;  // head-dim columns and column blocks per D wave
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BKV * ROWB;
    static constexpr int OPB = RB * NPG * 64 * 16;  // P or dS of every row block of one tile
    static constexpr int VOFF = NKS * TILEB, POFF = VOFF + NVS * TILEB, SOFF = POFF + 2 * OPB;
    static constexpr int LDS = SOFF + 2 * OPB;
    static_assert(LDS <= kLdsBudget, "dQ stages do not fit in LDS");
    static constexpr int WSB = 2 * RowStore<QD>::BYTES;  // dQ staging per D wave (two row blocks)
    static_assert(2 * RB * WSB <= (NVS + 2) * TILEB && TILEB % WSB == 0, "dQ staging does not fit");
    static_assert(DMAX == 256, "configuration");
};

// VP: the value head dim differs from D (extended calls)
template <class T, int DMAX, bool MASK, bool VP>
__global__ __launch_bounds__(1024, 4) void fa_dq_tri_kernel(BwdArgs a) {
    using C = DqTriCfg<T, DMAX>;
    using T8 = typename Vec8<T>::type;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors and roles depend on it
    const int h = lane >> 5, ln = lane & 31;
    // role 0..3 = A, C, D0, D1 (see above); waves w, w + 4, ... share SIMD w % 4
    const int role = w >> 2;
    const int rbk = ((w & 3) + role) & 3;  // row block of this wave

    // the logical order of fa_dq_lds_kernel
    const int nqt = (a.Lq + C::BQ - 1) / C::BQ;
    const int reps = a.Hq / a.Hkv;
    const int L = xcd_remap(blockIdx.x, nqt * a.B * a.Hq);
    const int r = L % reps;
    int qt = (L / reps) % nqt;
    const int grp = L / (reps * nqt);
    if (a.causal) qt = nqt - 1 - qt;
    const int b = grp / a.Hkv, g = grp % a.Hkv;
    const int hq = g * reps + r;
    const int i0 = qt * C::BQ;
    const int r0 = i0 + 32 * rbk;  // first row of this wave's block
    const int row = r0 + ln;
    const int D = a.D, Dv = VP ? a.Dv : a.D;
    const size_t qhead = (size_t)(b * a.Hq + hq) * a.Lq * D;
    const size_t lrow = (size_t)(b * a.Hq + hq) * a.Lq + row;

    const int i_last = min(i0 + C::BQ, a.Lq) - 1;
    const int j_lo = a.window ? max(0, i0 - a.window + 1) : 0;
    const int j_hi = a.causal ? min(i_last, a.Lkv - 1) : a.Lkv - 1;
    const int t_lo = j_lo / C::BKV;
    const int n_t = j_hi >= j_lo ? j_hi / C::BKV - t_lo + 1 : 0;

    constexpr int cb = 0;
    const int lofs = (rbk * C::NPG * 64 + lane) * 16;  // this lane's piece of a row block's operand
    char* const pbuf = smem + C::POFF;
    char* const sbuf = smem + C::SOFF;
    auto kslot = [&](int t) { return smem + (t % C::NKS) * C::TILEB; };
    auto vslot = [&](int t) { return smem + C::VOFF + (t % C::NVS) * C::TILEB; };
    const dsc_t rk = make_dsc(reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Lkv * D,
                              (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const dsc_t rv = make_dsc(reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Lkv * Dv,
                              (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    auto run = [&](auto rl) {
        constexpr int R = decltype(rl)::value;
        constexpr bool RA = R == 0, RC = R == 1, RD = R >= 2;
        // D: row blocks 2p, 2p + 1 and column blocks NQB q .. NQB q + NQB - 1
        const int dp = R - 2, dq4 = w & 3;
        TileOffs<C::ROWB> to;  // set up per role, so that each keeps only what it uses
        to.init(lane);
        auto issue = [&](int t) {  // C waves: K and V of tile t (offsets recomputed, no registers held)
            if constexpr (RC) {
                using P = DmaPlan<C::BKV, DMAX, C::RB>;
                const int j = (t_lo + t) * C::BKV;
                P::issue_pitch(rk, lds_of(kslot(t), smem), j, D, w & 3, lane);
                P::issue_pitch(rv, lds_of(vslot(t), smem), j, Dv, w & 3, lane);
            }
        };
        // register operand of the row: Q^T (A) or dO^T (C) fragments
        u32x4 rf[(RA || RC) ? C::NKG : 1];
        float rowv = 0.f;  // A: lse of the row in the exp2 domain; C: Delta of the row
        if constexpr (RA || RC) {
            const int Dx = RA ? D : Dv;
            const rsrc_t rs = RA ? make_rsrc(reinterpret_cast<const T*>(a.q) + qhead, (uint32_t)a.Lq * (uint32_t)D * 2u)
                                 : make_rsrc(reinterpret_cast<const T*>(a.dO) + (size_t)(b * a.Hq + hq) * a.Lq * Dv,
                                             (uint32_t)a.Lq * (uint32_t)Dv * 2u);
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) {
                const int c = cb + 2 * gi + h;
                rf[gi] = buf_ld16(rs, c * 8 < Dx ? (uint32_t)((row * Dx + c * 8) * 2) : kOob);
            }
            if (row < a.Lq) {
                if constexpr (RA) rowv = MASK ? lse_l2_masked(a.lse[lrow]) : a.lse[lrow] * kLog2e;
                else rowv = a.delta[lrow];
            }
        }
        // x = (natural fragments of the tile at `op`) x rf over the head dim
        auto chain = [&](const char* op, f32x16& x) {
            x = zero16();
            lookahead<C::NKG, 3>([&](int n) { return ld16(op + to.natural(0, n, cb)); },
                                 [&](int n, const u32x4& f) {
                                     Mma<T>::nat(x, f, rf[n < (int)(sizeof(rf) / sizeof(rf[0])) ? n : 0]);
                                 });
        };
        // A: P^T of tile t from its scores, masked, packed as MFMA operands
        auto probs = [&](int t, f32x16& x, u32x4 (&pn)[C::NPG]) {
            const int t0 = (t_lo + t) * C::BKV;
            if constexpr (MASK) {
                const MaskRow mb = mask_slice(a, b, hq);
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4 m = mask4_l2(mb, row, t0 + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[4 * qd + i] = fast_exp2(fmaf(x[4 * qd + i], a.c, m[i] - rowv));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) x[e] = fast_exp2(fmaf(x[e], a.c, -rowv));
            }
            const bool need = (t0 + C::BKV > a.Lkv) || (a.causal && t0 + C::BKV - 1 > r0) ||
                              (a.window && min(r0 + 31, a.Lq - 1) - t0 >= a.window);
            if (need) {
                // the allowed keys of this lane's row form one run [clo, chi] of the
                // tile offsets c = 8(e/4) + e%4 (key t0 + 4h + c)
                const int base = row - t0 - 4 * h;
                int chi = a.Lkv - t0 - 4 * h - 1;
                if (a.causal) chi = min(chi, base);
                const int clo = a.window ? base - a.window + 1 : INT_MIN;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int cr = 8 * (e >> 2) + (e & 3);
                    x[e] = (cr >= clo && cr <= chi) ? x[e] : 0.f;
                }
            }
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) pn[gg] = make_pf<T>(x, gg).v;
        };

        f32x16 x;  // A: scores of the next tile; C: dP of the current one
        f32x16 acc[RD ? 2 : 1][RD ? C::NQB : 1];
#pragma unroll
        for (int r2 = 0; r2 < (RD ? 2 : 1); ++r2)
#pragma unroll
            for (int i = 0; i < (RD ? C::NQB : 1); ++i) acc[r2][i] = zero16();
        // D: offsets of the transposed K fragments of its column blocks (key group 0)
        int trq[RD ? C::NQB : 1][2];
        if constexpr (RD) {
#pragma unroll
            for (int i = 0; i < C::NQB; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) trq[i][e] = to.transposed_rt(C::NQB * dq4 + i, cb, e);
        }

        if (n_t > 0) issue(0);
        if (n_t > 1) issue(1);
        wait_vm<0>();
        lds_barrier();
        if (n_t > 0) {
            if constexpr (RA) {
                u32x4 pn[C::NPG];
                chain(kslot(0), x);
                probs(0, x, pn);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) st16(pbuf + lofs + gg * 1024, pn[gg]);
            }
            if constexpr (RC) chain(vslot(0), x);
        }
#pragma unroll 1
        for (int t = 0; t <= n_t; ++t) {
            wait_vm<0>();   // this wave's share of tile t+1
            lds_barrier();  // P of t, dS of t-1 and tile t+1 visible; every wave is done with t-2
            if (t + 2 < n_t) issue(t + 2);
            if constexpr (RA) {
                if (t + 1 < n_t) {
                    u32x4 pn[C::NPG];
                    chain(kslot(t + 1), x);
                    probs(t + 1, x, pn);
                    char* pb = pbuf + ((t + 1) & 1) * C::OPB + lofs;
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) st16(pb + gg * 1024, pn[gg]);
                }
            } else if constexpr (RC) {
                if (t < n_t) {
                    u32x4 pp[C::NPG], ds[C::NPG];
                    const char* pb = pbuf + (t & 1) * C::OPB + lofs;
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) pp[gg] = ld16(pb + gg * 1024);
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) {
                        const T8 pv = __builtin_bit_cast(T8, pp[gg]);
#pragma unroll
                        for (int i = 0; i < 8; ++i) x[8 * gg + i] = (x[8 * gg + i] - rowv) * (float)pv[i];
                        ds[gg] = make_pf<T>(x, gg).v;
                    }
                    char* sb = sbuf + (t & 1) * C::OPB + lofs;
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) st16(sb + gg * 1024, ds[gg]);
                    if (t + 1 < n_t) chain(vslot(t + 1), x);
                }
            } else {
                if (t >= 1) {
                    u32x4 ds[2][C::NPG];  // dS^T of row blocks 2p and 2p + 1
                    const char* sb = sbuf + ((t - 1) & 1) * C::OPB + lane * 16;
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg)
                            ds[r2][gg] = ld16(sb + ((2 * dp + r2) * C::NPG + gg) * 1024);
                    const char* kl = kslot(t - 1);
                    // dQ^T[:, block i] of both row blocks += K^T (column block i, key group
                    // gg) x dS^T of group gg: each fragment feeds two MFMAs
                    lookahead<C::NPG * C::NQB, 3>(
                        [&](int n) {
                            const int gg = n / C::NQB, i = n % C::NQB;
                            const int go = 16 * gg * C::ROWB;
                            return rd_tr(kl + go + trq[RD ? i : 0][0], kl + go + trq[RD ? i : 0][1]);
                        },
                        [&](int n, const u32x4& f) {
                            const int gg = n / C::NQB, i = RD ? n % C::NQB : 0;
                            Mma<T>::nat(acc[0][i], f, ds[0][gg]);
                            Mma<T>::nat(acc[RD ? 1 : 0][i], f, ds[1][gg]);
                        });
                }
            }
        }

        if constexpr (RD) {
            // staging area k of this wave: the V ring, which no wave reads after
            // the last barrier, then the K slots of tiles n_t - 3 and n_t - 2 (only
            // K of tile n_t - 1 is still being read by other D waves)
            const int k = 4 * dp + dq4;
            constexpr int PER = C::TILEB / C::WSB;
            char* ws = k < C::NVS * PER ? smem + C::VOFF + k * C::WSB
                                        : kslot(n_t + 1 + (k - C::NVS * PER) / PER) + ((k - C::NVS * PER) % PER) * C::WSB;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rb0 = i0 + 32 * (2 * dp + r2);
                T* ob = reinterpret_cast<T*>(a.dq) + qhead + (size_t)rb0 * D + C::QD * dq4;
                store_rows<T, C::QD>(ws + r2 * RowStore<C::QD>::BYTES, acc[r2], a.scale, ob, (size_t)D, a.Lq - rb0,
                                     D - C::QD * dq4, lane);
            }
        }
    };
    if (role == 0) run(std::integral_constant<int, 0>{});
    else if (role == 1) run(std::integral_constant<int, 1>{});
    else if (role == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
}

template <class T, int DMAX>
hipError_t launch_dq_tri(const BwdArgs& a, hipStream_t s) {
    using C = DqTriCfg<T, DMAX>;
    auto kern = a.Dv != a.D ? ((a.mask || a.bmask) ? fa_dq_tri_kernel<T, DMAX, true, true>
                                                   : fa_dq_tri_kernel<T, DMAX, false, true>)
                            : ((a.mask || a.bmask) ? fa_dq_tri_kernel<T, DMAX, true, false>
                                                   : fa_dq_tri_kernel<T, DMAX, false, false>);
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long grid = (long long)((a.Lq + C::BQ - 1) / C::BQ) * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}

}  // namespace lds
}  // namespace fa
