// dK/dV for the 256-wide head-dim bucket with four waves per 32-key block.
//
// The key-side half of the backward pass (mlx-bun flash-attention.ts, DKV
// shader: dV += P^T dO, dK += dS^T Q, dS = P (dP - Delta), P = exp(S - LSE)),
// computed as in fa_dkv_pipe_kernel; only the division of the work differs.
//
// At D = 256 a wave holding the K (or V) fragments of 32 keys (64 registers)
// and the whole dV (or dK) accumulator of those keys (128) runs alone on its
// SIMD. Here each 32-key block has two producers and two consumers:
//   A: S = Q K^T and P = exp2(c S - log2(e) lse), stored for B and C
//   B: dV += dO^T P, from A's P
//   C: dP = dO V^T and dS = P (dP - Delta), stored for D
//   D: dK += Q^T dS, from C's dS
// A and C keep the K or V fragments and no accumulator, B and D an
// accumulator and no fragments, so two waves share each SIMD, 32 MFMAs of
// each 32-row tile on every SIMD. A workgroup owns two key blocks (eight
// waves, 64 keys). The two producers of a key block share a SIMD, and so do
// its two consumers: A's iteration is MFMAs then exponentials and C's is
// dS arithmetic then MFMAs, so each covers the other's VALU phase, while
// the consumers are MFMA streams alone. (A with B and C with D on a SIMD:
// 287.4 against 275.1 us on the 8192-token windowed workload; A with D and C
// with B, on another box: 283.4 against 277.0 us.)
//
// One barrier per element of the walk over (query tile, head). In iteration t
// (after barrier t) A computes S and P of element t+1; B updates dV with P of
// t; C forms dS of t from its dP of t (computed the iteration before) and P
// of t, stores it and computes dP of t+1; D updates dK with the dS of t-1
// stored the iteration before. Four stages: t-1 (D), t, t+1 and t+2 in
// flight; P and dS have two buffers each. The dV consumers (B) issue all the
// LDS-DMA requests right after the barrier. A wave stalls while the CU takes
// its requests; with B and D sharing them, D (the longest chain) spent about
// half of each iteration there. 8192-token windowed workload, each line one
// box: B alone 277.8 us, B and D 283.2, B and D with B's share issued after
// its products 278.8; B and D 278.4, with D's share after its products 304.1;
// B and D 275.9, the producers 306.0, C alone 292.5.
#pragma once

#include "fa_kernels_lds.hpp"

namespace fa {
namespace lds {

// f = ld(n) for n = 0 .. N-1, then use(n, f), with the loads of the next LA
// fragments requested before each use. The fence after each use keeps that
// order: left to itself the compiler requests each LDS fragment just before
// the MFMA that takes it. Both the producers' and the consumers' chains
// fenced at LA = 2: 297.8 -> 288.9 us on the 8192-token windowed workload
// (LA = 3 the same, 4 slower; only the producers' fenced 304.0, only the
// consumers' 291.8).
template <int N, int LA, class Ld, class Use>
__device__ __forceinline__ void lookahead(Ld ld, Use use) {
    u32x4 f[LA];
#pragma unroll
    for (int n = 0; n < LA && n < N; ++n) f[n] = ld(n);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const u32x4 cur = f[n % LA];
        if (n + LA < N) f[n % LA] = ld(n + LA);
        use(n, cur);
        sched_fence();
    }
}

template <class T, int DMAX, int BQ> struct DkvQuadCfg {
    static constexpr int KB = 2;  // 32-key blocks per workgroup
    static constexpr int NW = 4 * KB, NT = 64 * NW, BKV = 32 * KB;
    static constexpr int NS = 4;
    static constexpr int NKG = DMAX / 16, NDB = DMAX / 32;
    static constexpr int NRB = BQ / 32, NPG = BQ / 16;
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BQ * ROWB;
    static constexpr int ROWSB = 2 * BQ * 4;  // lse and delta of the tile's rows
    static constexpr int STAGEB = 2 * TILEB + ((ROWSB + 1023) / 1024) * 1024;
    static constexpr int OPB = KB * NPG * 64 * 16;  // P or dS of every key block of one element
    static constexpr int LDS = NS * STAGEB + 4 * OPB;
    static_assert(LDS <= kLdsBudget, "dK/dV stages do not fit in LDS");
    static_assert(DMAX % 64 == 0 && (BQ == 32 || BQ == 64), "configuration");
};

template <class T, int DMAX, int BQ, bool MASK>
__global__ __launch_bounds__(512, 2) void fa_dkv_quad_kernel(BwdArgs a, int pair) {
    using C = DkvQuadCfg<T, DMAX, BQ>;
    using T8 = typename Vec8<T>::type;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors and roles depend on it
    const int h = lane >> 5, ln = lane & 31;
    // role 0..3 = A, B, C, D (see above); waves w and w + 4 share a SIMD:
    // A and C of key block kb on SIMD 2 kb, its B and D on SIMD 2 kb + 1
    const int role = ((w & 1) ? 1 : 0) + (w >= 4 ? 2 : 0);
    const int kb = (w >> 1) & 1;
    const int cidx = w >> 1;  // B waves (w = 1, 3): index among the two that issue the DMA
    const int wl = 1, wd = 3;  // the B waves that fetch lse and delta

    const int nkt = (a.Lkv + C::BKV - 1) / C::BKV;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    int bg, kt0, kt1 = -1;
    if (pair) {
        const int np = (nkt + 1) >> 1;
        bg = L / np;
        kt0 = L - bg * np;
        if (nkt - 1 - kt0 != kt0) kt1 = nkt - 1 - kt0;
    } else {
        bg = L / nkt;
        kt0 = L - bg * nkt;
    }
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int reps = a.Hq / a.Hkv;
    const int D = a.D, Dv = a.Dv;
    const size_t kvhead = (size_t)(b * a.Hkv + g) * a.Lkv * D, kvhead_v = (size_t)(b * a.Hkv + g) * a.Lkv * Dv;
    const uint32_t qbytes = (uint32_t)a.Lq * (uint32_t)D * 2u, obytes = (uint32_t)a.Lq * (uint32_t)Dv * 2u;

    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<BQ, DMAX, 2> dma;
    dma.init(lane, role == 1 ? cidx : 0, D);
    char* const pbuf = smem + C::NS * C::STAGEB;              // P of elements with parity 0, 1
    char* const sbuf = pbuf + 2 * C::OPB;                      // dS of elements with parity 0, 1
    const int lofs = (kb * C::NPG * 64 + lane) * 16;           // this lane's piece of a key block's operand
    constexpr int cb = 0;

    auto run = [&](auto rl) {
        constexpr int R = decltype(rl)::value;
        constexpr bool RA = R == 0, RB = R == 1, RC = R == 2, RD = R == 3;
        constexpr int NAB = (RB || RD) ? C::NDB : 1;  // accumulator blocks (none used by A and C)
        const int Db = RA ? D : Dv;                     // head dim of the register operand (K or V)
        const int Do = RB ? Dv : D;                     // head dim of the output (dV or dK)
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int kt = pass ? kt1 : kt0;
            if (kt < 0) break;
            const int j0 = kt * C::BKV;
            const int key = j0 + 32 * kb + ln;

            u32x4 bf[(RA || RC) ? C::NKG : 1];
            if constexpr (RA || RC) {
                const rsrc_t rkv = RA ? make_rsrc(reinterpret_cast<const T*>(a.k) + kvhead, (uint32_t)a.Lkv * (uint32_t)D * 2u)
                                      : make_rsrc(reinterpret_cast<const T*>(a.v) + kvhead_v,
                                                  (uint32_t)a.Lkv * (uint32_t)Dv * 2u);
#pragma unroll
                for (int gi = 0; gi < C::NKG; ++gi) {
                    const int c = cb + 2 * gi + h;
                    bf[gi] = buf_ld16(rkv, c * 8 < Db ? (uint32_t)((key * Db + c * 8) * 2) : kOob);
                }
            }
            f32x16 acc[NAB];
#pragma unroll
            for (int i = 0; i < NAB; ++i) acc[i] = zero16();

            const int j_last = min(j0 + C::BKV, a.Lkv) - 1;
            const int i_lo = a.causal ? j0 : 0;
            const int i_hi = a.window ? min(a.Lq - 1, j_last + a.window - 1) : a.Lq - 1;
            const int qt_lo = i_lo / BQ, qt_hi = i_hi / BQ;
            const int nq = qt_hi - qt_lo + 1;
            const int n_it = i_hi >= i_lo ? nq * reps : 0;
            // the walk of fa_dkv_pipe_kernel: heads innermost, query tiles walked so
            // that the workgroups of one kv head share each tile in L2
            const int tdir = a.causal && !a.window && !pass ? -1 : 1;
            const int trot = a.causal && a.window && nq > 0 ? (nq - qt_lo % nq) % nq : 0;
            auto q0_of = [&](int e) {
                int u = e / reps + trot;
                if (u >= nq) u -= nq;
                return (tdir < 0 ? qt_hi - u : qt_lo + u) * BQ;
            };
            auto hq_of = [&](int e) { return g * reps + e % reps; };
            auto stage = [&](int e) { return smem + (e % C::NS) * C::STAGEB; };
            auto issue = [&](int e) {  // B waves: Q, dO, lse and delta of element e
                if constexpr (RB) {
                    const int hq = hq_of(e), qrow = q0_of(e);
                    const size_t qrow0 = (size_t)(b * a.Hq + hq) * a.Lq;
                    char* st = stage(e);
                    const dsc_t rq = make_dsc(reinterpret_cast<const T*>(a.q) + qrow0 * D, qbytes);
                    const dsc_t rdo = make_dsc(reinterpret_cast<const T*>(a.dO) + qrow0 * Dv, obytes);
                    dma.issue(rq, lds_of(st, smem), qrow, D, cidx);
                    if (Dv == D) dma.issue(rdo, lds_of(st + C::TILEB, smem), qrow, D, cidx);
                    else DmaPlan<BQ, DMAX, 2>::issue_pitch(rdo, lds_of(st + C::TILEB, smem), qrow, Dv, cidx, lane);
                    if (w == wl) {
                        const dsc_t rl = make_dsc(a.lse + qrow0, (uint32_t)a.Lq * 4u);
                        if (lane < BQ) dma4(rl, lds_of(st + 2 * C::TILEB, smem), (uint32_t)(qrow + lane) * 4u);
                    }
                    if (w == wd) {
                        const dsc_t rd = make_dsc(a.delta + qrow0, (uint32_t)a.Lq * 4u);
                        if (lane < BQ) dma4(rd, lds_of(st + 2 * C::TILEB + BQ * 4, smem), (uint32_t)(qrow + lane) * 4u);
                    }
                }
            };
            // x[rb] = sum over the head dim of the natural fragments of the tile at
            // `op` (row block rb) with bf, one fragment requested ahead
            auto chain = [&](const char* op, f32x16 (&x)[C::NRB]) {
#pragma unroll
                for (int rb = 0; rb < C::NRB; ++rb) x[rb] = zero16();
                lookahead<C::NRB * C::NKG, 2>(
                    [&](int n) { return ld16(op + to.natural(32 * (n / C::NKG), n % C::NKG, cb)); },
                    [&](int n, const u32x4& f) {
                        const int gi = n % C::NKG;
                        Mma<T>::nat(x[n / C::NKG], f, bf[gi < (int)(sizeof(bf) / sizeof(bf[0])) ? gi : 0]);
                    });
            };
            // acc[i] += (transposed fragment of row group gg, column block i of the
            // tile at `tb`) x op[gg], one fragment requested ahead
            auto update = [&](const char* tb, const u32x4 (&op)[C::NPG]) {
                lookahead<C::NPG * NAB, 2>(
                    [&](int n) {
                        const int g2 = n / NAB, d2 = n % NAB;
                        return rd_tr(tb + to.transposed(g2, d2, cb, 0), tb + to.transposed(g2, d2, cb, 1));
                    },
                    [&](int n, const u32x4& f) { Mma<T>::nat(acc[n % NAB], f, op[n / NAB]); });
            };
            auto needs_mask = [&](int q0) {
                return (q0 + BQ > a.Lq) || (a.causal && j0 + C::BKV - 1 > q0) ||
                       (a.window && min(q0 + BQ, a.Lq) - 1 - j0 >= a.window);
            };
            // A: P of element e from its scores x, packed as MFMA operands, element
            // masks applied to the packed values
            auto probs = [&](int e, f32x16 (&x)[C::NRB], u32x4 (&pn)[C::NPG]) {
                const int q0 = q0_of(e), hq = hq_of(e);
                const float* rowv = reinterpret_cast<const float*>(stage(e) + 2 * C::TILEB) + 4 * h;
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) {
                    const int rb = gg >> 1, hf = gg & 1;
                    f32x4 lg[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) lg[k] = *reinterpret_cast<const f32x4*>(rowv + 32 * rb + 8 * (2 * hf + k));
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 8 * hf + i;
                        const float l = lg[i >> 2][i & 3];
                        float ex;
                        if constexpr (MASK) {
                            const MaskRow mb = mask_slice(a, b, hq);
                            ex = mask_l2(mb, q0 + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3), key, a.Lq, a.Lkv) -
                                 lse_l2_masked(l);
                        } else {
                            ex = -l * kLog2e;
                        }
                        x[rb][r] = fast_exp2(fmaf(x[rb][r], a.c, ex));
                    }
                    pn[gg] = make_pf<T>(x[rb], hf).v;
                }
                if (needs_mask(q0)) {
                    // allowed rows of this lane's key: one run [lo, hi) of rel = row - q0 - 4h;
                    // each 32-bit word holds rows rel, rel + 1
                    const int base = q0 + 4 * h;
                    const int lo = a.causal ? key - base : INT_MIN;
                    int hi = a.Lq - base;
                    if (a.window) hi = min(hi, key + a.window - base);
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg)
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int r = 8 * (gg & 1) + 2 * k;
                            const int rel = 32 * (gg >> 1) + 8 * (r >> 2) + (r & 3);
                            const uint32_t keep = (rel >= lo && rel < hi ? 0x0000ffffu : 0u) |
                                                  (rel + 1 >= lo && rel + 1 < hi ? 0xffff0000u : 0u);
                            pn[gg][k] &= keep;
                        }
                }
            };

            f32x16 x[C::NRB];   // A: scores of the next element; C: dP of the current one
            u32x4 pn[C::NPG];   // A: P of the next element
            lds_barrier();      // the previous pass is done with every stage and buffer
            if (n_it > 0) issue(0);
            if (n_it > 1) issue(1);
            wait_vm<0>();
            lds_barrier();
            if (n_it > 0) {
                if constexpr (RA) {
                    chain(stage(0), x);
                    probs(0, x, pn);
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) st16(pbuf + lofs + gg * 1024, pn[gg]);
                }
                if constexpr (RC) chain(stage(0) + C::TILEB, x);
            }
#pragma unroll 1
            for (int t = 0; t <= n_it; ++t) {
                wait_vm<0>();   // this wave's share of element t+1
                lds_barrier();  // P of t, dS of t-1 and element t+1 visible; every wave is done with t-2
                if (t + 2 < n_it) issue(t + 2);
                const char* st = stage(t);
                if constexpr (RA) {
                    if (t + 1 < n_it) {
                        chain(stage(t + 1), x);
                        probs(t + 1, x, pn);
                        char* pb = pbuf + ((t + 1) & 1) * C::OPB + lofs;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) st16(pb + gg * 1024, pn[gg]);
                    }
                } else if constexpr (RB) {
                    if (t < n_it) {
                        u32x4 pp[C::NPG];
                        const char* pb = pbuf + (t & 1) * C::OPB + lofs;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) pp[gg] = ld16(pb + gg * 1024);
                        update(st + C::TILEB, pp);  // dV += dO^T P of element t
                    }
                } else if constexpr (RC) {
                    if (t < n_it) {
                        u32x4 pp[C::NPG], ds[C::NPG];
                        const char* pb = pbuf + (t & 1) * C::OPB + lofs;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) pp[gg] = ld16(pb + gg * 1024);
                        const float* dlv = reinterpret_cast<const float*>(st + 2 * C::TILEB) + BQ + 4 * h;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) {
                            const int rb = gg >> 1, hf = gg & 1;
                            const T8 pv = __builtin_bit_cast(T8, pp[gg]);
#pragma unroll
                            for (int k = 0; k < 2; ++k) {
                                const f32x4 dl = *reinterpret_cast<const f32x4*>(dlv + 32 * rb + 8 * (2 * hf + k));
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int r = 8 * hf + 4 * k + i;
                                    x[rb][r] = (x[rb][r] - dl[i]) * (float)pv[4 * k + i];
                                }
                            }
                            ds[gg] = make_pf<T>(x[rb], hf).v;
                        }
                        char* sb = sbuf + (t & 1) * C::OPB + lofs;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) st16(sb + gg * 1024, ds[gg]);
                        if (t + 1 < n_it) chain(stage(t + 1) + C::TILEB, x);
                    }
                } else {
                    if (t >= 1) {
                        u32x4 ds[C::NPG];
                        const char* sb = sbuf + ((t - 1) & 1) * C::OPB + lofs;
#pragma unroll
                        for (int gg = 0; gg < C::NPG; ++gg) ds[gg] = ld16(sb + gg * 1024);
                        update(stage(t - 1), ds);  // dK += Q^T dS of element t-1
                    }
                }
            }

            if ((RB || RD) && key < a.Lkv) {
                T* op = reinterpret_cast<T*>(RB ? a.dv : a.dk) + (RB ? kvhead_v : kvhead) + (size_t)key * Do;
                const float sc = RB ? 1.f : a.scale;
#pragma unroll
                for (int i = 0; i < NAB; ++i)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const int d = 32 * i + 8 * qd + 4 * h;
                        if (d < Do)
                            store4<T>(op + d, acc[i][4 * qd] * sc, acc[i][4 * qd + 1] * sc, acc[i][4 * qd + 2] * sc,
                                      acc[i][4 * qd + 3] * sc);
                    }
            }
        }
    };
    if (role == 0) run(std::integral_constant<int, 0>{});
    else if (role == 1) run(std::integral_constant<int, 1>{});
    else if (role == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
}

template <class T, int DMAX, int BQ>
hipError_t launch_dkv_quad(const BwdArgs& a, hipStream_t s) {
    using C = DkvQuadCfg<T, DMAX, BQ>;
    auto kern = (a.mask || a.bmask) ? fa_dkv_quad_kernel<T, DMAX, BQ, true> : fa_dkv_quad_kernel<T, DMAX, BQ, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long nkt = (a.Lkv + C::BKV - 1) / C::BKV;
    const long long bg = (long long)a.B * a.Hkv;
    const int pair = a.causal && !a.window && nkt >= 2 && (nkt + 1) / 2 * bg >= kPairMinGrid;
    const long long grid = pair ? (nkt + 1) / 2 * bg : nkt * bg;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a, pair);
    return hipGetLastError();
}

}  // namespace lds
}  // namespace fa
