// gfx950 kernels for 16-bit inputs built on LDS DMA and transposing LDS reads.
//
// Same method and MFMA chains as fa_kernels.hpp (forward: S^T = K Q^T ->
// O^T += V^T P^T; dQ: S^T, dP^T -> dQ^T += K^T dS^T; dK/dV: S, dP ->
// dV^T += dO^T P, dK^T += Q^T dS), with three CDNA4 features doing the data
// movement:
//   * buffer_load_dwordx4 ... lds: each streamed tile goes from HBM straight
//     into LDS (no staging registers, no LDS stores), NS stages deep. Per-head
//     buffer descriptors make rows past the sequence end read as zero; the
//     head-dim tail of a row is pointed out of range on purpose and reads as
//     zero too.
//   * ds_read_b64_tr_b16: the transposed operands (V^T, K^T, Q^T, dO^T) are
//     read from the same row-major tile: within each 16-lane group, lane j
//     receives element j%4 of the 8-byte pieces addressed by lanes j/4,
//     4+j/4, 8+j/4 and 12+j/4. Lane m of a group therefore addresses row
//     k0 + m/4, columns d0 + 4(m%4) .. +3, and receives rows k0..k0+3 of
//     column d0 + m: four consecutive k of its own column.
//   * Tiles are stored row-major with the low bits of the 16-byte chunk index
//     of row r XORed with a row-dependent swizzle (swz below), chosen for the
//     64-bank LDS: the 16 rows of a natural 16-byte fragment read and the
//     4 rows x 64 bytes of a transposing read each cover all banks once.
#pragma once

#include "fa_kernels.hpp"
#include <climits>
#include <type_traits>

namespace fa {
namespace lds {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kBufWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 descriptor word 3)
constexpr uint32_t kOob = 0x80000000u;  // an offset past every per-head extent: reads as zero

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// HBM -> LDS DMA (buffer_load ... lds) written as assembly. Issued through the
// compiler's intrinsic, every transposing LDS read (ds_read_b64_tr_b16) that
// follows a DMA gets an `s_waitcnt vmcnt(0)` in front of it, since the
// compiler cannot tell which LDS bytes the DMA writes; that wait drains the
// prefetch of the next tile in the middle of every step. The kernels order
// the DMA themselves: wait_vm + a barrier before a tile is read, a barrier
// before its slot is refilled. The descriptor lives in SGPRs (same fields as
// make_rsrc); M0 holds the wave's LDS destination and is restored afterwards.
typedef u32x4 dsc_t;
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ dsc_t make_dsc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return dsc_t{uni((uint32_t)p), uni((uint32_t)(p >> 32) & 0xffffu), uni(bytes), (uint32_t)kBufWord3};
}
// LDS byte address of p, a pointer into the dynamic LDS block `base`
__device__ __forceinline__ uint32_t lds_of(const char* p, const char* base) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)base + (uint32_t)(p - base);
}
__device__ __forceinline__ void dma16(dsc_t d, uint32_t lds_dst, uint32_t voff) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(uni(lds_dst)), "v"(voff), "s"(d)
        : "memory");
}
__device__ __forceinline__ void dma4(dsc_t d, uint32_t lds_dst, uint32_t voff) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(uni(lds_dst)), "v"(voff), "s"(d)
        : "memory");
}
// Chunk swizzle of row r for a tile of pitch ROWB bytes (LDS of 64 banks x
// 4 bytes: 256 bytes per cycle). ROWB >= 256: XOR the low 4 chunk bits with
// 4(r%4) + (r/4)%4, so 16 consecutive rows at one chunk hit 16 bank groups and
// the 4 rows x 64 bytes of a transposing read (32 lanes) cover all 64 banks.
// ROWB = 128 (two rows per 256 bytes): the same with i = r/2 over 3 bits.
template <int ROWB> __device__ __forceinline__ int swz(int r) {
    if constexpr (ROWB >= 256) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        const int i = r >> 1;
        return ((i & 1) << 2) | ((i >> 1) & 3);
    }
}

// LDS pitch of a tile row for head-dim bucket DMAX (16-bit elements): the
// swizzle needs rows of 128 bytes or a multiple of 256, so the 32 and 96
// buckets store rows of 64 and 128 elements; the padding chunks are filled
// with zeros by the DMA and never read, and every product still runs over
// DMAX columns only.
constexpr int tile_row_bytes(int DMAX) { return DMAX <= 64 ? 128 : (DMAX + 127) / 128 * 256; }

// Wait until at most N vector-memory operations of this wave are in flight
// (lgkm and export counters left unconstrained).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Transposed A fragment from two reads: `lo` at rows k0..k0+3 and `hi` at
// rows k0+8..k0+11 (k0 = 16g + 4h) of column d = d0 + lane%32.
__device__ __forceinline__ u32x4 rd_tr(const char* lo_p, const char* hi_p) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lo_p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(hi_p));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Renumber them so that XCD x receives one contiguous range of the
// logical order; the logical order groups all workgroups that share one
// (batch, kv head) together, so each L2 holds the K/V (or Q/dO) of few groups.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    return (n & 7) ? i : (i & 7) * (n >> 3) + (i >> 3);
}

// Calls f(t + S, integral_constant<S>) for S = S0 .. NS-1 while t + S < n: a
// loop over a ring of NS stages unrolled by NS, so that every stage offset is
// a compile-time constant (LDS addresses become immediate offsets).
template <int S, int NS, class F> __device__ __forceinline__ void unroll_slots(int t, int n, F& f) {
    if constexpr (S < NS) {
        if (t + S < n) {
            f(t + S, std::integral_constant<int, S>{});
            unroll_slots<S + 1, NS>(t, n, f);
        }
    }
}

// Scheduling fence: keeps a chain's LDS reads ahead of its MFMAs, so that all
// of them are in flight together and each MFMA waits only for its own
// fragment (left alone, the scheduler serialises read -> wait -> MFMA).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// K and V fragments per batch in that order (2 measured 0.2488 against 0.2508 ms
// for 4 at D = 256, the same at D = 128; 8 spills)
#ifndef FA2_DQ_FB
#define FA2_DQ_FB 2
#endif

// Issue priority around the MFMA chains of the forward and dQ kernels (two
// workgroups share a CU there): the wave in its product phase goes first, the
// other wave's softmax VALU fills the issue slots in between. In the forward
// (ASYM) the product-phase priority also depends on the parity of the wave's
// slot on its SIMD (HW_ID bits 3:0), so that of two waves in their product
// phase at once one goes first. Measured on the causal GQA workloads: forward
// 5 % faster at D = 256 with the plain priority; the asymmetric form takes the
// D = 128 forward from 0.1605 to 0.1566 ms (three same-box A/B rounds) and is
// no better for dQ.
template <bool ASYM = false> __device__ __forceinline__ void prio_mfma() {
    if constexpr (ASYM) {
        const unsigned slot = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (3 << 11));
        if (slot & 1) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
    } else {
        __builtin_amdgcn_s_setprio(1);
    }
}
__device__ __forceinline__ void prio_valu() { __builtin_amdgcn_s_setprio(0); }

// Sum of the two 16-bit values packed in `pk`, added to acc (one v_dot2 with
// ones): the forward's row sum of the probabilities as they enter the MFMA.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <class T> __device__ __forceinline__ float add_pair(uint32_t pk, float acc);
template <> __device__ __forceinline__ float add_pair<__bf16>(uint32_t pk, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), bf16x2{(__bf16)1.f, (__bf16)1.f}, acc,
                                           false);
}
template <> __device__ __forceinline__ float add_pair<_Float16>(uint32_t pk, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
}

template <class T> struct Vec8;
template <> struct Vec8<__bf16> {
    typedef bf16x8 type;
};
template <> struct Vec8<_Float16> {
    typedef f16x8 type;
};

// Per-lane byte offsets inside a row-major swizzled tile of pitch ROWB.
//   nat[j]   : row ln, logical chunk 2j + h            (natural fragment, j = g % NN)
//   tr[x][e] : row 4h + m/4 + 8e, logical chunk 4x + 2(q%2) + (m%4)/2, byte 8(m%2)
//              (transposed fragment: 32-column block with db % NX = x, half e)
// The swizzle repeats every 16 rows and touches only the low bits of the chunk
// index, so whole 16-row groups and whole swizzle spans are plain offsets.
template <int ROWB> struct TileOffs {
    static constexpr int NC = ROWB / 16;            // chunks per row
    static constexpr int SPAN = NC >= 16 ? 16 : 8;  // chunks covered by the swizzle
    static constexpr int NN = SPAN / 2;
    static constexpr int NX = SPAN / 4;
    int nat[NN];
    int tr[NX][2];
    __device__ __forceinline__ void init(int lane) {
        const int h = lane >> 5, ln = lane & 31, q = lane >> 4, m = lane & 15;
        const int sn = swz<ROWB>(ln);
#pragma unroll
        for (int j = 0; j < NN; ++j) nat[j] = ln * ROWB + (((2 * j + h) ^ sn) << 4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int row = 4 * h + (m >> 2) + 8 * e;
            const int st = swz<ROWB>(row);
#pragma unroll
            for (int x = 0; x < NX; ++x)
                tr[x][e] = row * ROWB + (((4 * x + 2 * (q & 1) + ((m & 3) >> 1)) ^ st) << 4) + 8 * (m & 1);
        }
    }
    // natural fragment: 32-row block base rb0 (multiple of 32), chunk 2g + h + cb
    // (cb a multiple of SPAN)
    __device__ __forceinline__ int natural(int rb0, int g, int cb) const {
        return rb0 * ROWB + nat[g % NN] + ((g / NN) * SPAN + cb) * 16;
    }
    // transposed fragment, half e: 16-row group gg, 32-column block db, column
    // base cb (in chunks, a multiple of SPAN)
    __device__ __forceinline__ int transposed(int gg, int db, int cb, int e) const {
        return 16 * gg * ROWB + tr[db % NX][e] + ((db / NX) * SPAN + cb) * 16;
    }
    // the same for row group 0 and a column block known only at run time
    __device__ __forceinline__ int transposed_rt(int db, int cb, int e) const {
        int v = tr[0][e];
#pragma unroll
        for (int x = 1; x < NX; ++x) v = db % NX == x ? tr[x][e] : v;
        return v + ((db / NX) * SPAN + cb) * 16;
    }
};

// LDS-DMA plan for an R x DMAX (16-bit) tile issued by NW waves: wave w owns
// instructions w, w + NW, ...; instruction i fills bytes [1024 i, 1024 i + 1024)
// of the tile with the 64 chunks whose swizzled position falls there (chunks
// past the head dim, including a padded row's, read as zero).
template <int R, int DMAX, int NW> struct DmaPlan {
    static constexpr int ROWB = tile_row_bytes(DMAX);
    static constexpr int NDC = ROWB / 16;
    static constexpr int NI = R * NDC / 64;
    static_assert(R * NDC % 64 == 0 && NI % NW == 0, "tile must split evenly into 1 KiB DMA pieces per wave");
    static constexpr int NIW = NI / NW;
    uint32_t voff[NIW];
    __device__ __forceinline__ void init(int lane, int w, int D) {
#pragma unroll
        for (int n = 0; n < NIW; ++n) {
            const int slot = 64 * (w + n * NW) + lane;
            const int r = slot / NDC, p = slot % NDC;
            const int c = p ^ swz<ROWB>(r);  // logical chunk stored at physical chunk p
            voff[n] = (c * 8 < D) ? (uint32_t)((r * D + c * 8) * 2) : kOob;
        }
    }
    // rows row0.. of the head described by `rs` (row pitch D elements) -> tile
    __device__ __forceinline__ void issue(dsc_t rs, uint32_t tile, int row0, int D, int w) const {
        const uint32_t add = (uint32_t)row0 * (uint32_t)D * 2u;
#pragma unroll
        for (int n = 0; n < NIW; ++n) dma16(rs, tile + (w + n * NW) * 1024, voff[n] + add);
    }
    // the same for a tensor whose row pitch Dx differs from the D of init():
    // the offsets are recomputed from the lane instead of kept in registers
    __device__ __forceinline__ static void issue_pitch(dsc_t rs, uint32_t tile, int row0, int Dx, int w, int lane) {
#pragma unroll
        for (int n = 0; n < NIW; ++n) {
            const int slot = 64 * (w + n * NW) + lane;
            const int r = slot / NDC, p = slot % NDC;
            const int c = p ^ swz<ROWB>(r);
            const uint32_t off = (c * 8 < Dx) ? (uint32_t)(((r + row0) * Dx + c * 8) * 2) : kOob;
            dma16(rs, tile + (w + n * NW) * 1024, off);
        }
    }
};

// max of three scores (v_max3_f32; no NaN arises from the MFMA products)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// Lane l and lane l^32 of x, as (lower half's value, upper half's value) in
// every lane: one v_permlane32_swap. (The vector elements are copied out
// before the bit casts: a bit cast of a vector element subscript reads
// element 0.)
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}
// max over lanes l and l^32 (the same bits in both lanes)
__device__ __forceinline__ float max_halves(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return fmaxf(lo, hi);
}
// sum over lanes l and l^32, added in the same order in both lanes
__device__ __forceinline__ float sum_halves(float x) {
    float lo, hi;
    halves(x, lo, hi);
    return lo + hi;
}

// ===========================================================================
// Output tiles through LDS
// ===========================================================================
// A wave's 32-row output tile is held as transposed MFMA accumulators: element
// 4qd + j of acc[db] in lane (h, n) is row n, column 32db + 8qd + 4h + j.
// Stored directly, every instruction writes 8 bytes into each of 32 rows
// (sixteen 16-byte pieces per row and instruction group); the epilogue of the
// forward spent about 4500 cycles per wave in such stores. store_rows passes
// the tile through the wave's LDS region instead (rows of COLS values,
// 16-byte chunks XOR-swizzled by row) and stores whole row pieces: RPI rows
// of COLS columns per instruction, in passes of COLS columns.
template <int DMAX> struct RowStore {
    static constexpr int COLS = DMAX >= 96 ? 128 : DMAX;  // columns per pass
    static constexpr int NCH = COLS / 8;                  // 16-byte chunks per row
    static constexpr int RPI = 64 / NCH;                  // rows per store instruction
    static constexpr int ROWB = 2 * COLS;                 // LDS bytes per row
    static constexpr int BYTES = 32 * ROWB;               // LDS bytes per wave
    static constexpr int NDB = DMAX / 32, DBP = COLS / 32, NP = (NDB + DBP - 1) / DBP;
};
template <class T> __device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d);
template <> __device__ __forceinline__ u32x2 pack4<__bf16>(float a, float b, float c, float d) {
    return __builtin_bit_cast(u32x2, bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d});
}
template <> __device__ __forceinline__ u32x2 pack4<_Float16>(float a, float b, float c, float d) {
    return __builtin_bit_cast(u32x2, f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d});
}
// Rows [0, nrows) and columns [0, ncols) of the tile, each value times `mul`
// (the lane's row factor), to base + r * pitch + col. `ws`: this wave's
// RowStore<DMAX>::BYTES of LDS, used by no other wave meanwhile.
template <class T, int DMAX>
__device__ __forceinline__ void store_rows(char* ws, const f32x16 (&acc)[DMAX / 32], float mul, T* base, size_t pitch,
                                           int nrows, int ncols, int lane) {
    using R = RowStore<DMAX>;
    // the lane index made opaque here, so that the address arithmetic below
    // is done at the store and not hoisted ahead of the tile loop into
    // registers that the loop needs
    asm volatile("" : "+v"(lane));
    const int h = lane >> 5, ln = lane & 31;
    const int c = lane % R::NCH, r0 = lane / R::NCH;
#pragma unroll
    for (int p = 0; p < R::NP; ++p) {
#pragma unroll
        for (int b4 = 0; b4 < R::DBP; ++b4) {
            const int db = p * R::DBP + b4;
            if (db < R::NDB) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int cw = 4 * b4 + qd;  // chunk of this lane's 4 values, half h
                    st8(ws + ln * R::ROWB + ((cw ^ (ln & (R::NCH - 1))) << 4) + 8 * h,
                        pack4<T>(acc[db][4 * qd] * mul, acc[db][4 * qd + 1] * mul, acc[db][4 * qd + 2] * mul,
                                 acc[db][4 * qd + 3] * mul));
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 32 / R::RPI; ++i) {
            const int r = i * R::RPI + r0;
            const u32x4 v = ld16(ws + r * R::ROWB + ((c ^ (r & (R::NCH - 1))) << 4));
            const int col = p * R::COLS + 8 * c;
            if (r < nrows && col < ncols) st16(base + (size_t)r * pitch + col, v);
        }
    }
}

// ===========================================================================
// Forward
// ===========================================================================
template <class T, int DMAX, int BKV, int RW, int DW, int NS> struct Fwd2Cfg {
    static constexpr int NW = RW * DW, NT = 64 * NW, BQ = 32 * RW;
    static constexpr int DS = DMAX / DW, SCH = DS / 8, NKG = SCH / 2, NDB = DS / 32;
    static constexpr int NKB = BKV / 32, NPG = BKV / 16;
    // K fragments in flight per batch of score MFMAs. A 256-wide d slice keeps
    // 64 registers of Q fragments and 128 of O accumulators per wave, which at
    // two waves per SIMD leaves room for one fragment ahead of its MFMA.
    static constexpr int FB = DS >= 256 ? 1 : NKG < 8 ? NKG : 8;
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BKV * ROWB, STAGEB = 2 * TILEB;
    static constexpr int RED = DW > 1 ? RW * DW * NKB * 16 * 64 * 4 : 0;
    static constexpr int LDS = NS * STAGEB + RED;
    static_assert(LDS <= kLdsBudget, "forward stages do not fit in LDS");
    static_assert(NS >= 2 && DMAX % 32 == 0 && DS % 32 == 0, "configuration");
};

template <class T, int DMAX, int BKV, int RW, int DW, int OCC, int NS, bool MASK>
__global__ __launch_bounds__(64 * RW * DW, OCC) void fa_fwd_lds_kernel(FwdArgs a) {
    using C = Fwd2Cfg<T, DMAX, BKV, RW, DW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS DMA destinations depend on it
    const int h = lane >> 5, ln = lane & 31;
    const int rw = w / DW, dw = w % DW;

    // logical order: (batch, kv head) group, then query tile heaviest first,
    // then the query heads of the group (which share every K/V tile)
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
    const int row = i0 + 32 * rw + ln;
    const int D = a.D, Dv = a.Dv;

    const size_t qhead = (size_t)(b * a.Hq + hq) * a.Lq * D;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const T*>(a.q) + qhead, (uint32_t)a.Lq * (uint32_t)D * 2u);
    const dsc_t rk = make_dsc(reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Lkv * D,
                                (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const dsc_t rv = make_dsc(reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Lkv * Dv,
                                (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    // Q fragments of this wave's 32 rows and d slice (B operand of S^T = K Q^T);
    // rows past Lq and the head-dim tail read as zero.
    u32x4 qf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        qf[gi] = buf_ld16(rq, c * 8 < D ? (uint32_t)((row * D + c * 8) * 2) : kOob);
    }
    float c = a.c;
    if (c < 0.f) {  // fold a negative scale into Q (exact), so that c >= 0 below
        c = -c;
#pragma unroll
        for (int gi = 0; gi < C::NKG; ++gi) qf[gi] ^= 0x80008000u;
    }
    // A zero scale becomes 1e-30: every allowed score then enters exp2 within
    // 1e-25 of the row max, so P is exactly 1 in fp32 as with scale 0, and
    // -inf (masked) times the factor stays -inf, so exp2 gives exactly 0 with
    // no further test.
    c = fmaxf(c, 1e-30f);

    f32x16 o[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) o[i] = zero16();
    float m_ref = -INFINITY, l_run = 0.f;

    const int i_last = min(i0 + C::BQ, a.Lq) - 1;
    const int j_lo = a.window ? max(0, i0 - a.window + 1) : 0;
    const int j_hi = a.causal ? min(i_last, a.Lkv - 1) : a.Lkv - 1;
    const int t_lo = j_lo / BKV;
    const int n_t = j_hi >= j_lo ? j_hi / BKV - t_lo + 1 : 0;

    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<BKV, DMAX, C::NW> dma;
    dma.init(lane, w, D);
    float* red = reinterpret_cast<float*>(smem + NS * C::STAGEB);
    const int cb = dw * C::SCH;  // chunk base of this wave's d slice

    auto issue = [&](int t, auto slot) {
        char* st = smem + decltype(slot)::value * C::STAGEB;
        dma.issue(rk, lds_of(st, smem), (t_lo + t) * BKV, D, w);
        if (Dv == D) dma.issue(rv, lds_of(st + C::TILEB, smem), (t_lo + t) * BKV, D, w);
        else dma.issue_pitch(rv, lds_of(st + C::TILEB, smem), (t_lo + t) * BKV, Dv, w, lane);
    };
    constexpr int LPT = 2 * DmaPlan<BKV, DMAX, C::NW>::NIW;  // DMA instructions per tile per wave

    unroll_slots<0, NS - 1>(0, n_t, issue);

    auto step = [&](int t, auto slot) {
        constexpr int SL = decltype(slot)::value;  // stage of tile t
            if (t + NS - 2 < n_t) wait_vm<(NS - 2) * LPT>();
            else wait_vm<0>();
            lds_barrier();  // tile t visible to all waves; every wave is done with tile t-1
            if (t + NS - 1 < n_t) issue(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});

            const char* kl = smem + SL * C::STAGEB;
            const char* vl = kl + C::TILEB;
            const int t0 = (t_lo + t) * BKV;
            // S^T = K Q^T in batches of FB fragments; each batch's K fragments are
            // requested before the previous batch's MFMAs
            f32x16 s[C::NKB];
            {
                constexpr int FB = C::FB, BPK = C::NKG / FB, NB = C::NKB * BPK;
                auto load = [&](int k, u32x4 (&f)[FB]) {
#pragma unroll
                    for (int i = 0; i < FB; ++i) f[i] = ld16(kl + to.natural(32 * (k / BPK), (k % BPK) * FB + i, cb));
                };
                u32x4 cur[FB];
                load(0, cur);
                prio_mfma<true>();
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    u32x4 nxt[FB];
                    if (k + 1 < NB) load(k + 1, nxt);
                    sched_fence();
                    const int kb = k / BPK, g0 = (k % BPK) * FB;
                    if (g0 == 0) s[kb] = zero16();
#pragma unroll
                    for (int i = 0; i < FB; ++i) Mma<T>::nat(s[kb], cur[i], qf[g0 + i]);
                    sched_fence();
                    if (k + 1 < NB) {
#pragma unroll
                        for (int i = 0; i < FB; ++i) cur[i] = nxt[i];
                    }
                }
            }
            prio_valu();
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

            // V^T fragments of the first output block, in flight during the softmax
            u32x4 vcur[C::NPG];
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg)
                vcur[gg] = rd_tr(vl + to.transposed(gg, 0, cb, 0), vl + to.transposed(gg, 0, cb, 1));

            const bool need = (t0 + BKV > a.Lkv) || (a.causal && t0 + BKV - 1 > i0) ||
                              (a.window && i_last - t0 >= a.window);
            if (need) {
                // the allowed keys of this lane's row form one run c in [clo, chi]
                // of the tile offsets c = 32 kb + 8(r/4) + r%4 (key t0 + 4h + c)
                const int base = row - t0 - 4 * h;
                int chi = a.Lkv - t0 - 4 * h - 1;
                if (a.causal) chi = min(chi, base);
                const int clo = a.window ? base - a.window + 1 : INT_MIN;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int cr = 32 * kb + 8 * (r >> 2) + (r & 3);
                        s[kb][r] = (cr >= clo && cr <= chi) ? s[kb][r] : -INFINITY;
                    }
            }
            constexpr int NSC = 16 * C::NKB;  // scores per lane
            auto sv = [&](int i) { return s[i / 16][i % 16]; };
            float mx = max3f(sv(0), sv(1), sv(2));
#pragma unroll
            for (int i = 3; i + 1 < NSC; i += 2) mx = max3f(mx, sv(i), sv(i + 1));
            mx = max3f(mx, sv(NSC - 1), sv(NSC - 1));
            mx = max_halves(mx);
            const float m_tile = mx * cs;  // -inf stays -inf (cs > 0)
            const bool upd = m_tile > m_ref + kRescaleLog2;
            if (OCC < 2 || __ballot(upd)) {
                const float m_new = upd ? m_tile : m_ref;
                const float alpha = upd ? fast_exp2(m_ref - m_new) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
                m_ref = m_new;
            }
            const float moff = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], cs, -moff));

            // O^T += V^T P^T, one 32-wide output block at a time; the next block's
            // fragments are requested before this block's MFMAs. The row sum l
            // adds the probabilities as rounded for the MFMA, two per instruction
            // (the same values that weight V).
            PF<T> pf[C::NPG];
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) pf[gg] = make_pf<T>(s[gg >> 1], gg & 1);
            {
                float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) {
                    ls0 = add_pair<T>(pf[gg].v[0], ls0);
                    ls1 = add_pair<T>(pf[gg].v[1], ls1);
                    ls0 = add_pair<T>(pf[gg].v[2], ls0);
                    ls1 = add_pair<T>(pf[gg].v[3], ls1);
                }
                l_run += ls0 + ls1;
            }
            prio_mfma<true>();
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                u32x4 vnxt[C::NPG];
                if (db + 1 < C::NDB) {
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg)
                        vnxt[gg] = rd_tr(vl + to.transposed(gg, db + 1, cb, 0), vl + to.transposed(gg, db + 1, cb, 1));
                }
                sched_fence();
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) Mma<T>::nat(o[db], vcur[gg], pf[gg].v);
                sched_fence();
                if (db + 1 < C::NDB) {
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) vcur[gg] = vnxt[gg];
                }
            }
            prio_valu();
    };
    for (int t = 0; t < n_t; t += NS) unroll_slots<0, NS>(t, n_t, step);

    const float l = sum_halves(l_run);
    // At D = 256 O goes through the stage that holds neither the last tile nor
    // a pending DMA (every wave is done with tile n_t - 2 since the last
    // barrier): 0.152 -> 0.145 ms on the 8192-token windowed workload. At
    // D <= 128 the same measured 0.1554 -> 0.1561 ms on the 2048-token
    // workload and 10.87 -> 11.31 ms at 32768 tokens, so there the lanes
    // store their own pieces.
    if constexpr (DW == 1 && DMAX >= 256) {
        static_assert(C::NW * RowStore<DMAX>::BYTES <= C::STAGEB, "output staging does not fit in a stage");
        const float inv = l > 0.f ? 1.f / l : 0.f;
        char* ws = smem + ((n_t + NS - 2) % NS) * C::STAGEB + w * RowStore<DMAX>::BYTES;
        const int r0 = i0 + 32 * rw;
        T* ob = reinterpret_cast<T*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Lq + r0) * Dv;
        store_rows<T, DMAX>(ws, o, inv, ob, (size_t)Dv, a.Lq - r0, Dv, lane);
        if (row < a.Lq && h == 0)
            a.lse[(size_t)(b * a.Hq + hq) * a.Lq + row] = l > 0.f ? (m_ref + fast_log2(l)) * kLn2 : -INFINITY;
    } else if (row < a.Lq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        T* op = reinterpret_cast<T*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Lq + row) * Dv;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < Dv)
                    store4<T>(op + d, o[db][4 * qd] * inv, o[db][4 * qd + 1] * inv, o[db][4 * qd + 2] * inv,
                              o[db][4 * qd + 3] * inv);
            }
        if (h == 0 && dw == 0)
            a.lse[(size_t)(b * a.Hq + hq) * a.Lq + row] = l > 0.f ? (m_ref + fast_log2(l)) * kLn2 : -INFINITY;
    }
}

// ===========================================================================
// dQ
// ===========================================================================
template <class T, int DMAX, int BKV, int RW, int DW, int NS> struct Dq2Cfg {
    static constexpr int NW = RW * DW, NT = 64 * NW, BQ = 32 * RW;
    static constexpr int DS = DMAX / DW, SCH = DS / 8, NKG = SCH / 2, NDB = DS / 32;
    static constexpr int NKB = BKV / 32, NPG = BKV / 16;
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BKV * ROWB, STAGEB = 2 * TILEB;
    static constexpr int RED = DW > 1 ? 2 * RW * DW * NKB * 16 * 64 * 4 : 0;
    static constexpr int LDS = NS * STAGEB + RED;
    static_assert(LDS <= kLdsBudget, "dQ stages do not fit in LDS");
    static_assert(NS >= 2 && DMAX % 32 == 0 && DS % 32 == 0, "configuration");
};

// VP: the value head dim differs from D (extended calls); the other
// instantiation takes Dv = D at compile time.
template <class T, int DMAX, int BKV, int RW, int DW, int OCC, int NS, bool MASK, bool VP>
__global__ __launch_bounds__(64 * RW * DW, OCC) void fa_dq_lds_kernel(BwdArgs a) {
    using C = Dq2Cfg<T, DMAX, BKV, RW, DW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, ln = lane & 31;
    const int rw = w / DW, dw = w % DW;

    // same logical order as the forward
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
    const int row = i0 + 32 * rw + ln;
    const int D = a.D, Dv = VP ? a.Dv : a.D;

    const size_t qhead = (size_t)(b * a.Hq + hq) * a.Lq * D;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const T*>(a.q) + qhead, (uint32_t)a.Lq * (uint32_t)D * 2u);
    const rsrc_t rdo = make_rsrc(reinterpret_cast<const T*>(a.dO) + (size_t)(b * a.Hq + hq) * a.Lq * Dv,
                                 (uint32_t)a.Lq * (uint32_t)Dv * 2u);
    const dsc_t rk = make_dsc(reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Lkv * D,
                                (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const dsc_t rv = make_dsc(reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Lkv * Dv,
                                (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    u32x4 qf[C::NKG], df[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        qf[gi] = buf_ld16(rq, c * 8 < D ? (uint32_t)((row * D + c * 8) * 2) : kOob);
        df[gi] = buf_ld16(rdo, c * 8 < Dv ? (uint32_t)((row * Dv + c * 8) * 2) : kOob);
    }
    const size_t lrow = (size_t)(b * a.Hq + hq) * a.Lq + row;
    const float lse2 = row < a.Lq ? (MASK ? lse_l2_masked(a.lse[lrow]) : a.lse[lrow] * kLog2e) : 0.f;
    const MaskRow mb = MASK ? mask_slice(a, b, hq) : MaskRow{nullptr, nullptr};
    const float dl = row < a.Lq ? a.delta[lrow] : 0.f;

    f32x16 acc[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) acc[i] = zero16();

    const int i_last = min(i0 + C::BQ, a.Lq) - 1;
    const int j_lo = a.window ? max(0, i0 - a.window + 1) : 0;
    const int j_hi = a.causal ? min(i_last, a.Lkv - 1) : a.Lkv - 1;
    const int t_lo = j_lo / BKV;
    const int n_t = j_hi >= j_lo ? j_hi / BKV - t_lo + 1 : 0;

    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<BKV, DMAX, C::NW> dma;
    dma.init(lane, w, D);
    float* red = reinterpret_cast<float*>(smem + NS * C::STAGEB);
    const int cb = dw * C::SCH;
    // allowed entries: row - key in [dlo, dhi)
    const int dlo = a.causal ? 0 : INT_MIN;
    const int dhi = a.window ? a.window : INT_MAX;

    auto issue = [&](int t) {
        char* st = smem + (t % NS) * C::STAGEB;
        dma.issue(rk, lds_of(st, smem), (t_lo + t) * BKV, D, w);
        if constexpr (VP) dma.issue_pitch(rv, lds_of(st + C::TILEB, smem), (t_lo + t) * BKV, Dv, w, lane);
        else dma.issue(rv, lds_of(st + C::TILEB, smem), (t_lo + t) * BKV, D, w);
    };
    constexpr int LPT = 2 * DmaPlan<BKV, DMAX, C::NW>::NIW;

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < n_t) issue(s);

    for (int t = 0; t < n_t; ++t) {
        if (t + NS - 2 < n_t) wait_vm<(NS - 2) * LPT>();
        else wait_vm<0>();
        lds_barrier();
        if (t + NS - 1 < n_t) issue(t + NS - 1);

        const char* kl = smem + (t % NS) * C::STAGEB;
        const char* vl = kl + C::TILEB;
        const int t0 = (t_lo + t) * BKV;
        const bool need = (t0 + BKV > a.Lkv) || (a.causal && t0 + BKV - 1 > i0) ||
                          (a.window && i_last - t0 >= a.window);
        f32x16 s[C::NKB], dp[C::NKB];
        if constexpr (DW == 1) {
            // S^T = K Q^T first, then dP^T = V dO^T with the exponentials of S^T
            // placed between its MFMAs; element masks are applied to P afterwards
            // (one MFMA code path for every tile). Fragments come in batches of FB,
            // each batch requested before the previous batch's MFMAs.
            f32x4 m4[C::NKB][4];
            if constexpr (MASK) {
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        m4[kb][qd] = mask4_l2(mb, row, t0 + 32 * kb + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
#pragma unroll
                        for (int i = 0; i < 4; ++i) m4[kb][qd][i] -= lse2;
                    }
            }
            constexpr int FB = C::NKG < FA2_DQ_FB ? C::NKG : FA2_DQ_FB, BPK = C::NKG / FB, NB = C::NKB * BPK;
            constexpr int NSC = 16 * C::NKB, EPB = (NSC + NB - 1) / NB;  // exponentials per dP^T batch
            auto loadf = [&](const char* base, int k, u32x4 (&f)[FB]) {
#pragma unroll
                for (int i = 0; i < FB; ++i) f[i] = ld16(base + to.natural(32 * (k / BPK), (k % BPK) * FB + i, cb));
            };
            u32x4 cur[FB];
            loadf(kl, 0, cur);
            prio_mfma();
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                u32x4 nxt[FB];
                if (k + 1 < NB) loadf(kl, k + 1, nxt);
                else loadf(vl, 0, nxt);
                sched_fence();
                const int kb = k / BPK, g0 = (k % BPK) * FB;
                if (g0 == 0) s[kb] = zero16();
#pragma unroll
                for (int i = 0; i < FB; ++i) Mma<T>::nat(s[kb], cur[i], qf[g0 + i]);
                sched_fence();
#pragma unroll
                for (int i = 0; i < FB; ++i) cur[i] = nxt[i];
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                u32x4 nxt[FB];
                if (k + 1 < NB) loadf(vl, k + 1, nxt);
                const int kb = k / BPK, g0 = (k % BPK) * FB;
                if (g0 == 0) dp[kb] = zero16();
#pragma unroll
                for (int i = 0; i < FB; ++i) Mma<T>::nat(dp[kb], cur[i], df[g0 + i]);
#pragma unroll
                for (int e = k * EPB; e < (k + 1) * EPB && e < NSC; ++e) {
                    const int sb = e / 16, r = e % 16;
                    s[sb][r] = fast_exp2(fmaf(s[sb][r], a.c, MASK ? m4[sb][r >> 2][r & 3] : -lse2));
                }
#pragma unroll
                for (int i = 0; i < FB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 2 * EPB / FB, 0);  // VALU
                }
                sched_fence();
                if (k + 1 < NB) {
#pragma unroll
                    for (int i = 0; i < FB; ++i) cur[i] = nxt[i];
                }
            }
            prio_valu();
            if (need) {
                // the allowed keys of this lane's row form one run [clo, chi] of the
                // tile offsets c = 32 kb + 8(r/4) + r%4 (key t0 + 4h + c)
                const int base = row - t0 - 4 * h;
                int chi = a.Lkv - t0 - 4 * h - 1;
                if (a.causal) chi = min(chi, base);
                const int clo = a.window ? base - a.window + 1 : INT_MIN;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int cr = 32 * kb + 8 * (r >> 2) + (r & 3);
                        s[kb][r] = (cr >= clo && cr <= chi) ? s[kb][r] : 0.f;
                    }
            }
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] *= dp[kb][r] - dl;  // dS^T
        } else {
            // d split over DW waves: partial S^T = K Q^T and dP^T = V dO^T over this
            // wave's d slice in batches of H fragments of each (a batch's K/V
            // fragments requested before the previous batch's MFMAs), summed
            // across the slices through LDS
            {
                constexpr int H = 2, BPK = C::NKG / H, NB = C::NKB * BPK;
                auto load = [&](int k, u32x4 (&kf)[H], u32x4 (&vf)[H]) {
    #pragma unroll
                    for (int i = 0; i < H; ++i) {
                        const int off = to.natural(32 * (k / BPK), (k % BPK) * H + i, cb);
                        kf[i] = ld16(kl + off);
                        vf[i] = ld16(vl + off);
                    }
                };
                u32x4 kcur[H], vcur[H];
                load(0, kcur, vcur);
                prio_mfma();
    #pragma unroll
                for (int k = 0; k < NB; ++k) {
                    u32x4 knxt[H], vnxt[H];
                    if (k + 1 < NB) load(k + 1, knxt, vnxt);
                    sched_fence();
                    const int kb = k / BPK, g0 = (k % BPK) * H;
                    if (g0 == 0) {
                        s[kb] = zero16();
                        dp[kb] = zero16();
                    }
    #pragma unroll
                    for (int i = 0; i < H; ++i) {
                        Mma<T>::nat(s[kb], kcur[i], qf[g0 + i]);
                        Mma<T>::nat(dp[kb], vcur[i], df[g0 + i]);
                    }
                    sched_fence();
                    if (k + 1 < NB) {
    #pragma unroll
                        for (int i = 0; i < H; ++i) {
                            kcur[i] = knxt[i];
                            vcur[i] = vnxt[i];
                        }
                    }
                }
            }
            prio_valu();
            if constexpr (DW > 1) {
                reduce_partials<DW, C::NKB>(s, red, rw * DW, dw, lane);
                reduce_partials<DW, C::NKB>(dp, red + RW * DW * C::NKB * 16 * 64, rw * DW, dw, lane);
            }

            f32x4 m4[C::NKB][4];
            if constexpr (MASK) {
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        m4[kb][qd] = mask4_l2(mb, row, t0 + 32 * kb + 8 * qd + 4 * h, a.Lq, a.Lkv, a.mvec);
    #pragma unroll
                        for (int i = 0; i < 4; ++i) m4[kb][qd][i] -= lse2;
                    }
            }
            auto dscore = [&](auto masked) {
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float p = fast_exp2(fmaf(s[kb][r], a.c, MASK ? m4[kb][r >> 2][r & 3] : -lse2));
                        if constexpr (decltype(masked)::value) {
                            const int j = t0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3), dd = row - j;
                            p = ((j < a.Lkv) & (dd >= dlo) & (dd < dhi)) ? p : 0.f;
                        }
                        s[kb][r] = p * (dp[kb][r] - dl);  // dS^T
                    }
            };
            if (need) dscore(std::true_type{});
            else dscore(std::false_type{});
        }
        PF<T> pf[C::NPG];
#pragma unroll
        for (int gg = 0; gg < C::NPG; ++gg) pf[gg] = make_pf<T>(s[gg >> 1], gg & 1);
        // dQ^T += K^T dS^T, one 32-wide output block at a time; the next block's
        // K^T fragments are requested before this block's MFMAs
        u32x4 kt[C::NPG];
#pragma unroll
        for (int gg = 0; gg < C::NPG; ++gg)
            kt[gg] = rd_tr(kl + to.transposed(gg, 0, cb, 0), kl + to.transposed(gg, 0, cb, 1));
        prio_mfma();
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            u32x4 knxt[C::NPG];
            if (db + 1 < C::NDB) {
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg)
                    knxt[gg] = rd_tr(kl + to.transposed(gg, db + 1, cb, 0), kl + to.transposed(gg, db + 1, cb, 1));
            }
            sched_fence();
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) Mma<T>::nat(acc[db], kt[gg], pf[gg].v);
            sched_fence();
            if (db + 1 < C::NDB) {
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) kt[gg] = knxt[gg];
            }
        }
        prio_valu();
    }

    if constexpr (DW == 1) {
        // dQ through the stage that holds neither the last tile nor a pending DMA
        // (0.1943 -> 0.1894 ms on the 2048-token workload)
        static_assert(C::NW * RowStore<DMAX>::BYTES <= C::STAGEB, "output staging does not fit in a stage");
        char* ws = smem + ((n_t + NS - 2) % NS) * C::STAGEB + w * RowStore<DMAX>::BYTES;
        const int r0 = i0 + 32 * rw;
        T* ob = reinterpret_cast<T*>(a.dq) + qhead + (size_t)r0 * D;
        store_rows<T, DMAX>(ws, acc, a.scale, ob, (size_t)D, a.Lq - r0, D, lane);
    } else if (row < a.Lq) {
        T* op = reinterpret_cast<T*>(a.dq) + qhead + (size_t)row * D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < D)
                    store4<T>(op + d, acc[db][4 * qd] * sc, acc[db][4 * qd + 1] * sc, acc[db][4 * qd + 2] * sc,
                              acc[db][4 * qd + 3] * sc);
            }
    }
}

// ===========================================================================
// dK/dV: the workgroup owns BKV = 32*KW keys of one kv head (one per lane) and
// walks every query tile of every query head of the group that can see them.
// ===========================================================================
template <class T, int DMAX, int BQ, int KW, int DW, int NS> struct Dkv2Cfg {
    static constexpr int NW = KW * DW, NT = 64 * NW, BKV = 32 * KW;
    static constexpr int DS = DMAX / DW, SCH = DS / 8, NKG = SCH / 2, NDB = DS / 32;
    static constexpr int NRB = BQ / 32, NPG = BQ / 16;
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BQ * ROWB;
    static constexpr int ROWSB = 2 * BQ * 4;                    // lse and delta of the tile's rows
    static constexpr int STAGEB = 2 * TILEB + ((ROWSB + 1023) / 1024) * 1024;
    static constexpr int RED1 = DW > 1 ? KW * DW * NRB * 16 * 64 * 4 : 0;
    // When two partial-sum buffers do not fit next to the stages, S and dP are
    // reduced one after the other through one buffer (one more barrier).
    static constexpr bool SEQ = NS * STAGEB + 2 * RED1 > kLdsBudget;
    static constexpr int RED = SEQ ? RED1 : 2 * RED1;
    static constexpr int LDS = NS * STAGEB + RED;
    static_assert(LDS <= kLdsBudget, "dK/dV stages do not fit in LDS");
    static_assert(NS >= 2 && DMAX % 32 == 0 && DS % 32 == 0 && BQ >= 32 && BQ <= 64, "configuration");
};

template <class T, int DMAX, int BQ, int KW, int DW, int OCC, int NS, bool MASK>
__global__ __launch_bounds__(64 * KW * DW, OCC) void fa_dkv_lds_kernel(BwdArgs a) {
    using C = Dkv2Cfg<T, DMAX, BQ, KW, DW, NS>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5, ln = lane & 31;
    const int kw = w / DW, dw = w % DW;

    // Key blocks in dispatch order, small blocks (the most work under causal)
    // first across all (batch, kv head) groups: grouping them per XCD would
    // pair heavy blocks on the same CU, and the Q/dO a group re-reads does
    // not fit one L2 anyway.
    const int BG = a.B * a.Hkv;
    const int kt_idx = blockIdx.x / BG;
    const int bg = blockIdx.x % BG;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int reps = a.Hq / a.Hkv;
    const int j0 = kt_idx * C::BKV;
    const int key = j0 + 32 * kw + ln;
    const int D = a.D, Dv = a.Dv;

    const size_t kvhead = (size_t)(b * a.Hkv + g) * a.Lkv * D, kvhead_v = (size_t)(b * a.Hkv + g) * a.Lkv * Dv;
    const uint32_t qbytes = (uint32_t)a.Lq * (uint32_t)D * 2u, obytes = (uint32_t)a.Lq * (uint32_t)Dv * 2u;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const T*>(a.k) + kvhead, (uint32_t)a.Lkv * (uint32_t)D * 2u);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const T*>(a.v) + kvhead_v, (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    // K and V fragments of this lane's key and this wave's d slice
    // (B operands of S = Q K^T and dP = dO V^T).
    u32x4 kf[C::NKG], vf[C::NKG];
#pragma unroll
    for (int gi = 0; gi < C::NKG; ++gi) {
        const int c = dw * C::SCH + 2 * gi + h;
        kf[gi] = buf_ld16(rk, c * 8 < D ? (uint32_t)((key * D + c * 8) * 2) : kOob);
        vf[gi] = buf_ld16(rv, c * 8 < Dv ? (uint32_t)((key * Dv + c * 8) * 2) : kOob);
    }

    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }

    const int j_last = min(j0 + C::BKV, a.Lkv) - 1;
    const int i_lo = a.causal ? j0 : 0;
    const int i_hi = a.window ? min(a.Lq - 1, j_last + a.window - 1) : a.Lq - 1;
    const int qt_lo = i_lo / BQ;
    const int nqt = i_hi >= i_lo ? i_hi / BQ - qt_lo + 1 : 0;
    const int n_it = nqt * reps;

    TileOffs<C::ROWB> to;
    to.init(lane);
    DmaPlan<BQ, DMAX, C::NW> dma;
    dma.init(lane, w, D);
    float* red = reinterpret_cast<float*>(smem + NS * C::STAGEB);
    const int cb = dw * C::SCH;
    // lse and delta of a query tile, one float per lane (rows past Lq read as
    // zero): wave 0 fetches lse, wave WD delta.
    constexpr int WD = C::NW > 1 ? 1 : 0;

    auto issue = [&](int it) {
        const int hq = g * reps + it / nqt;
        const int q0 = (qt_lo + it % nqt) * BQ;
        const dsc_t rq = make_dsc(reinterpret_cast<const T*>(a.q) + (size_t)(b * a.Hq + hq) * a.Lq * D, qbytes);
        const dsc_t rdo = make_dsc(reinterpret_cast<const T*>(a.dO) + (size_t)(b * a.Hq + hq) * a.Lq * Dv, obytes);
        char* st = smem + (it % NS) * C::STAGEB;
        dma.issue(rq, lds_of(st, smem), q0, D, w);
        if (Dv == D) dma.issue(rdo, lds_of(st + C::TILEB, smem), q0, D, w);
        else dma.issue_pitch(rdo, lds_of(st + C::TILEB, smem), q0, Dv, w, lane);
        const size_t lhead = (size_t)(b * a.Hq + hq) * a.Lq;
        if (w == 0) {
            const dsc_t rl = make_dsc(a.lse + lhead, (uint32_t)a.Lq * 4u);
            if (lane < BQ) dma4(rl, lds_of(st + 2 * C::TILEB, smem), (uint32_t)(q0 + lane) * 4u);
        }
        if (w == WD) {
            const dsc_t rd = make_dsc(a.delta + lhead, (uint32_t)a.Lq * 4u);
            if (lane < BQ) dma4(rd, lds_of(st + 2 * C::TILEB + BQ * 4, smem), (uint32_t)(q0 + lane) * 4u);
        }
    };
    constexpr int LPT = 2 * DmaPlan<BQ, DMAX, C::NW>::NIW;
    // DMA instructions per tile of this wave: the Q and dO pieces, plus lse
    // (wave 0) and delta (wave WD).
    const int extra = (w == 0) + (w == WD);

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < n_it) issue(s);

    for (int it = 0; it < n_it; ++it) {
        if (it + NS - 2 < n_it) {
            if (extra == 2) wait_vm<(NS - 2) * (LPT + 2)>();
            else if (extra == 1) wait_vm<(NS - 2) * (LPT + 1)>();
            else wait_vm<(NS - 2) * LPT>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();
        if (it + NS - 1 < n_it) issue(it + NS - 1);

        const char* ql = smem + (it % NS) * C::STAGEB;
        const char* dol = ql + C::TILEB;
        const float* lf = reinterpret_cast<const float*>(ql + 2 * C::TILEB);
        const int q0 = (qt_lo + it % nqt) * BQ;

        f32x16 s[C::NRB], dp[C::NRB];
#pragma unroll
        for (int rb = 0; rb < C::NRB; ++rb) {
            s[rb] = zero16();
            dp[rb] = zero16();
            constexpr int H = C::NKG > 4 ? C::NKG / 2 : C::NKG;  // fragments per batch
#pragma unroll
            for (int g0 = 0; g0 < C::NKG; g0 += H) {
                u32x4 qfr[H], dfr[H];
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    const int off = to.natural(32 * rb, g0 + i, cb);
                    qfr[i] = ld16(ql + off);
                    dfr[i] = ld16(dol + off);
                }
                sched_fence();
#pragma unroll
                for (int i = 0; i < H; ++i) {
                    Mma<T>::nat(s[rb], qfr[i], kf[g0 + i]);
                    Mma<T>::nat(dp[rb], dfr[i], vf[g0 + i]);
                }
            }
        }
        if constexpr (DW > 1) {
            reduce_partials<DW, C::NRB>(s, red, kw * DW, dw, lane);
            if constexpr (C::SEQ) {
                lds_barrier();  // every wave has read the S partials
                reduce_partials<DW, C::NRB>(dp, red, kw * DW, dw, lane);
            } else {
                reduce_partials<DW, C::NRB>(dp, red + KW * DW * C::NRB * 16 * 64, kw * DW, dw, lane);
            }
        }
        const bool need = (q0 + BQ > a.Lq) || (a.causal && j0 + C::BKV - 1 > q0) ||
                          (a.window && min(q0 + BQ, a.Lq) - 1 - j0 >= a.window);
#pragma unroll
        for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int rl = 32 * rb + 8 * qd + 4 * h;  // first of the 4 rows this lane holds
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lf + rl);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(lf + BQ + rl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * qd + i;
                    float p;
                    if constexpr (MASK) {
                        const MaskRow mb = mask_slice(a, b, g * reps + it / nqt);
                        p = fast_exp2(fmaf(s[rb][r], a.c, mask_l2(mb, q0 + rl + i, key, a.Lq, a.Lkv) -
                                                              lse_l2_masked(l4[i])));
                    } else {
                        p = fast_exp2(fmaf(s[rb][r], a.c, -l4[i] * kLog2e));
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
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            u32x4 dofr[C::NPG], qfr[C::NPG];
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) {
                const int o0 = to.transposed(gg, db, cb, 0), o1 = to.transposed(gg, db, cb, 1);
                dofr[gg] = rd_tr(dol + o0, dol + o1);
                qfr[gg] = rd_tr(ql + o0, ql + o1);
            }
            sched_fence();
#pragma unroll
            for (int gg = 0; gg < C::NPG; ++gg) {
                Mma<T>::nat(dv[db], dofr[gg], pf[gg].v);
                Mma<T>::nat(dk[db], qfr[gg], sf[gg].v);
            }
        }
    }

    if (key < a.Lkv) {
        T* kop = reinterpret_cast<T*>(a.dk) + kvhead + (size_t)key * D;
        T* vop = reinterpret_cast<T*>(a.dv) + kvhead_v + (size_t)key * Dv;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d = dw * C::DS + 32 * db + 8 * qd + 4 * h;
                if (d < D)
                    store4<T>(kop + d, dk[db][4 * qd] * sc, dk[db][4 * qd + 1] * sc, dk[db][4 * qd + 2] * sc,
                              dk[db][4 * qd + 3] * sc);
                if (d < Dv)
                    store4<T>(vop + d, dv[db][4 * qd], dv[db][4 * qd + 1], dv[db][4 * qd + 2], dv[db][4 * qd + 3]);
            }
    }
}

// ===========================================================================
// dK/dV on wave pairs with one barrier per query tile. For each 32-key block
// two waves share the work: the dV wave computes S = Q K^T, P = exp(S - LSE)
// (masked entries 0) and dV^T += dO^T P; the dK wave computes dP = dO V^T,
// takes P from its partner through LDS, forms dS = P (dP - Delta) and
// dK^T += Q^T dS. Each wave holds one of K/V, one accumulator set and one
// score block, so a SIMD runs one wave of each kind. Keys are owned by the
// workgroup alone (no atomics).
//
// Query tiles go through a three-slot LDS ring with one barrier per tile: it
// publishes P of tile t, makes tile t+1 (already landed) visible and frees
// the slot of tile t-1 for the DMA of tile t+2. The dK wave forms dP of tile
// t before that barrier and dS and its dK update after it. The dV wave runs
// one tile ahead: after the barrier of tile t it forms the scores of tile
// t+1, then updates dV from tile t with the exponentials of tile t+1 placed
// between those MFMAs, and stores P of tile t+1 before the next barrier. The
// LDS fragments of the next product are requested before the MFMAs of the
// current one.
//
// Under a causal mask without window a workgroup may take key blocks p and
// nkt-1-p, which gives every workgroup the same amount of work. Workgroups of
// one (batch, kv head) are placed on one XCD, and the query tiles are walked
// (heads innermost) in an order under which the workgroups of a group stream
// the same Q/dO tiles at about the same time through that XCD's L2.
// ===========================================================================
template <class T, int DMAX, int BQ, int KW> struct DkvPipeCfg {
    static constexpr int NS = 3;  // tile t (computing), t+1 (landed), t+2 (in flight)
    static constexpr int NW = 2 * KW, NT = 64 * NW, BKV = 32 * KW;
    static constexpr int NKG = DMAX / 16, NDB = DMAX / 32;
    static constexpr int NRB = BQ / 32, NPG = BQ / 16;
    static constexpr int ROWB = tile_row_bytes(DMAX), TILEB = BQ * ROWB;
    static constexpr int ROWSB = 2 * BQ * 4;  // lse and delta of the tile's rows
    static constexpr int STAGEB = 2 * TILEB + ((ROWSB + 1023) / 1024) * 1024;
    static constexpr int PBUF = KW * NPG * 64 * 16;  // P of every key block as MFMA operands, lane-major
    static constexpr int LDS = NS * STAGEB + 2 * PBUF;
    static_assert(LDS <= kLdsBudget, "dK/dV stages do not fit in LDS");
    static_assert(DMAX % 32 == 0 && (BQ == 32 || BQ == 64) && KW >= 2, "configuration");
};

template <class T, int DMAX, int BQ, int KW, int OCC, int PRIO, bool MASK>
__global__ __launch_bounds__(128 * KW, OCC) void fa_dkv_pipe_kernel(BwdArgs a, int pair) {
    using C = DkvPipeCfg<T, DMAX, BQ, KW>;
    using T8 = typename Vec8<T>::type;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: buffer descriptors below depend on it
    const int h = lane >> 5, ln = lane & 31;
    const bool vw = w < KW;  // dV wave (else dK wave)
    const int kw = w % KW;   // key block of this wave
    if (PRIO && vw) __builtin_amdgcn_s_setprio(1);

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
    // dV wave: K fragments (B of S = Q K^T); dK wave: V fragments (B of dP = dO V^T)
    const rsrc_t rkv = vw ? make_rsrc(reinterpret_cast<const T*>(a.k) + kvhead, (uint32_t)a.Lkv * (uint32_t)D * 2u)
                          : make_rsrc(reinterpret_cast<const T*>(a.v) + kvhead_v, (uint32_t)a.Lkv * (uint32_t)Dv * 2u);

    TileOffs<C::ROWB> to;
    to.init(lane);
    // Who streams the Q/dO tiles. A wave stalls while the CU's memory pipeline
    // takes its LDS-DMA requests, and the requests go out right after the
    // barrier, so they are left to the dV waves, which otherwise wait at the
    // next one (0.273 -> 0.268 ms on the 2048-token workload).
    DmaPlan<BQ, DMAX, KW> dma;
    dma.init(lane, vw ? w : 0, D);
    char* const pbase = smem + C::NS * C::STAGEB + (kw * C::NPG * 64 + lane) * 16;
    constexpr int cb = 0;  // chunk base of the tile columns (the head dim is not split)
    const int aoff = vw ? 0 : C::TILEB;  // phase-A operand: Q (dV wave) or dO (dK wave)
    const int toff = vw ? C::TILEB : 0;  // phase-B operand (transposed): dO or Q

    // The two wave kinds run separate copies of the loop (same barriers in the
    // same order), so each is register-allocated and scheduled on its own.
    auto run = [&](auto role) {
        constexpr bool V = decltype(role)::value;
        const int Db = V ? D : Dv;  // head dim of this wave's register operand (K or V)
        const int Do = V ? Dv : D;  // head dim of its output (dV or dK)
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int kt = pass ? kt1 : kt0;
            if (kt < 0) break;
            const int j0 = kt * C::BKV;
            const int key = j0 + 32 * kw + ln;

            u32x4 bf[C::NKG];
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) {
                const int c = cb + 2 * gi + h;
                bf[gi] = buf_ld16(rkv, c * 8 < Db ? (uint32_t)((key * Db + c * 8) * 2) : kOob);
            }
            f32x16 acc[C::NDB];  // dV^T (dV wave) or dK^T (dK wave)
#pragma unroll
            for (int i = 0; i < C::NDB; ++i) acc[i] = zero16();

            const int j_last = min(j0 + C::BKV, a.Lkv) - 1;
            const int i_lo = a.causal ? j0 : 0;
            const int i_hi = a.window ? min(a.Lq - 1, j_last + a.window - 1) : a.Lq - 1;
            const int qt_lo = i_lo / BQ, qt_hi = i_hi / BQ;
            const int nq = qt_hi - qt_lo + 1;
            const int n_it = i_hi >= i_lo ? nq * reps : 0;

            // Tiles in the order (query tile) x (head of the group), the query tiles
            // walked so that the workgroups of one kv head, which run at the same
            // pace, visit the same tile at about the same time and share it in L2:
            // under a causal mask without window every range ends at the last tile,
            // so the first key block of each workgroup walks down from it; the
            // second block of a causal pair walks up from its diagonal tile: a
            // workgroup starts it after the tiles of its first block, and the first
            // range is shorter by as many tiles as the second starts higher, so at
            // each step every workgroup in its second pass is on the same tile too.
            // Without causal mask every range starts at tile 0, so all walk up from
            // it; under causal + window the ranges have the same length nq and
            // different starts, so each walks up from the tile whose index is a
            // multiple of nq, wrapping to its first tile (at step s every workgroup
            // is on a tile congruent to s mod nq).
            const int tdir = a.causal && !a.window && !pass ? -1 : 1;
            const int trot = a.causal && a.window && nq > 0 ? (nq - qt_lo % nq) % nq : 0;
            auto tile_of = [&](int st) {  // query tile at position st of the walk
                int u = st + trot;
                if (u >= nq) u -= nq;
                return tdir < 0 ? qt_hi - u : qt_lo + u;
            };
            int hq_issue = g * reps, st_issue = 0, slot_issue = 0;
            auto issue = [&]() {
                const size_t qrow0 = (size_t)(b * a.Hq + hq_issue) * a.Lq;
                const dsc_t rq = make_dsc(reinterpret_cast<const T*>(a.q) + qrow0 * D, qbytes);
                const dsc_t rdo = make_dsc(reinterpret_cast<const T*>(a.dO) + qrow0 * Dv, obytes);
                char* st = smem + slot_issue * C::STAGEB;
                const int qrow = tile_of(st_issue) * BQ;
                if constexpr (V) {
                    dma.issue(rq, lds_of(st, smem), qrow, D, w);
                    if (Dv == D) dma.issue(rdo, lds_of(st + C::TILEB, smem), qrow, D, w);
                    else dma.issue_pitch(rdo, lds_of(st + C::TILEB, smem), qrow, Dv, w, lane);
                }
                const size_t lhead = (size_t)(b * a.Hq + hq_issue) * a.Lq;
                if (V && w == 0) {
                    const dsc_t rl = make_dsc(a.lse + lhead, (uint32_t)a.Lq * 4u);
                    if (lane < BQ) dma4(rl, lds_of(st + 2 * C::TILEB, smem), (uint32_t)(qrow + lane) * 4u);
                }
                if (V && w == 1) {
                    const dsc_t rd = make_dsc(a.delta + lhead, (uint32_t)a.Lq * 4u);
                    if (lane < BQ) dma4(rd, lds_of(st + 2 * C::TILEB + BQ * 4, smem), (uint32_t)(qrow + lane) * 4u);
                }
                if (++hq_issue == (g + 1) * reps) {
                    hq_issue = g * reps;
                    ++st_issue;
                }
                slot_issue = slot_issue == C::NS - 1 ? 0 : slot_issue + 1;
            };

            lds_barrier();  // the previous pass is done with every slot and P buffer
            if (n_it > 0) issue();
            if (n_it > 1) issue();
            wait_vm<0>();
            lds_barrier();

            // row block 0 of the phase-A operand of the tile being computed
            u32x4 fr0[C::NKG];
#pragma unroll
            for (int gi = 0; gi < C::NKG; ++gi) fr0[gi] = ld16(smem + aoff + to.natural(0, gi, cb));

            if constexpr (V) {
                // dV wave, pipelined across query tiles. After the barrier of tile it
                // come the score products of tile it+1 (visible since that barrier),
                // then dV^T += dO^T P of tile it with the exponentials of tile it+1
                // placed between its MFMAs, so that the exp phase of this wave runs
                // under matrix-core work instead of after it. P of each tile is stored
                // for the dK wave before the barrier that publishes it, as in the plain
                // order, and read back from there for this wave's own dV update; the
                // barrier sequence is the dK wave's.
                constexpr int HG = C::NKG / 2;
                f32x16 x[C::NRB];
                u32x4 nx[C::NDB];  // dO^T fragments of the row group multiplied next
                u32x4 px;          // P of that row group (operand of the dV update)
                int sa = 0, ha = 0;  // walk position and head (in the group) of the next scores

                // S = Q K^T of the tile whose phase-A operand is at `sa`; row block 0's
                // fragments are in fr0
                auto scores = [&](const char* sa) {
                    u32x4 fr1[C::NKG];
                    if constexpr (C::NRB == 2) {
#pragma unroll
                        for (int gi = 0; gi < HG; ++gi) fr1[gi] = ld16(sa + to.natural(32, gi, cb));
                    }
                    sched_fence();
                    x[0] = zero16();
#pragma unroll
                    for (int gi = 0; gi < C::NKG; ++gi) Mma<T>::nat(x[0], fr0[gi], bf[gi]);
                    sched_fence();
                    if constexpr (C::NRB == 2) {
#pragma unroll
                        for (int gi = HG; gi < C::NKG; ++gi) fr1[gi] = ld16(sa + to.natural(32, gi, cb));
                        sched_fence();
                        x[1] = zero16();
#pragma unroll
                        for (int gi = 0; gi < C::NKG; ++gi) Mma<T>::nat(x[1], fr1[gi], bf[gi]);
                    }
                    sched_fence();
                };
                // lse of the rows of row group gg (accumulator half gg%2 of row block
                // gg/2) of the tile in stage `sa`: rows 32(gg/2) + 8qd + 4h + i for
                // qd = 2(gg%2), 2(gg%2)+1
                auto rows = [&](const char* sa, int gg, f32x4 (&lg)[2]) {
                    const float* rowv = reinterpret_cast<const float*>(sa + 2 * C::TILEB) + 4 * h;
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        lg[k] = *reinterpret_cast<const f32x4*>(rowv + 32 * (gg >> 1) + 8 * (2 * (gg & 1) + k));
                };
                // P of row group gg as MFMA operand, from its scores and the rows' lse
                // (element masks are applied to the packed values by mask_p)
                auto probs = [&](int gg, const f32x4 (&lg)[2], int q0, int hq) {
                    const int rb = gg >> 1, hf = gg & 1;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 8 * hf + i;
                        const float l = lg[i >> 2][i & 3];
                        float e;
                        if constexpr (MASK) {
                            const MaskRow mb = mask_slice(a, b, hq);
                            e = mask_l2(mb, q0 + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3), key, a.Lq, a.Lkv) -
                                lse_l2_masked(l);
                        } else {
                            e = -l * kLog2e;
                        }
                        x[rb][r] = fast_exp2(fmaf(x[rb][r], a.c, e));
                    }
                    return make_pf<T>(x[rb], hf).v;
                };
                // Zero the packed probabilities of the rows this lane's key may not see.
                // Element r of row block rb is row q0 + 4h + rel with rel = 32 rb + 8(r/4)
                // + r%4; the allowed rows of a key form one run [lo, hi) of rel. Each
                // 32-bit word holds elements r (low half) and r+1 (high half, rel + 1).
                auto mask_p = [&](u32x4 (&pn)[C::NPG], int q0) {
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
                };
                auto needs_mask = [&](int q0) {
                    return (q0 + BQ > a.Lq) || (a.causal && j0 + C::BKV - 1 > q0) ||
                           (a.window && min(q0 + BQ, a.Lq) - 1 - j0 >= a.window);
                };
                auto next_tile = [&]() {
                    if (++ha == reps) {
                        ha = 0;
                        ++sa;
                    }
                };
                // dO^T fragments of row group gg of the tile whose dO is at `tb`
                auto dot_frags = [&](const char* tb, int gg, u32x4 (&f)[C::NDB]) {
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
                        f[db] = rd_tr(tb + to.transposed(gg, db, cb, 0), tb + to.transposed(gg, db, cb, 1));
                };

                // first tile: scores, P stored for the dK wave, its first dO^T row group
                if (n_it > 0) {
                    const int q0 = tile_of(sa) * BQ, hq = g * reps + ha;
                    scores(smem + aoff);
                    u32x4 pn[C::NPG];
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) {
                        f32x4 lg[2];
                        rows(smem, gg, lg);
                        pn[gg] = probs(gg, lg, q0, hq);
                    }
                    if (needs_mask(q0)) mask_p(pn, q0);
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) st16(pbase + gg * 1024, pn[gg]);
                    dot_frags(smem + toff, 0, nx);
                    next_tile();
                }
                // tiles 0 .. n_it-2: the dV update of tile it with the scores and P of
                // tile it+1 (one code path for every tile, so the accumulators stay in
                // place; element masks are applied to the packed P afterwards)
                int slot = 0;
                for (int it = 0; it + 1 < n_it; ++it) {
                    const int nslot = slot == C::NS - 1 ? 0 : slot + 1;
                    const char* tb = smem + slot * C::STAGEB + toff;  // dO of tile it
                    const char* sn = smem + nslot * C::STAGEB;        // tile it+1
                    const char* pcur = pbase + (it & 1) * C::PBUF;    // P of tile it
                    px = ld16(pcur);  // this wave's own P: read before the barrier, no wait after it
                    wait_vm<0>();     // this wave's share of tile it+1
                    lds_barrier();    // P of tile it visible; tile it+1 visible; tile it-1 done
                    if (it + 2 < n_it) issue();
                    const int q0 = tile_of(sa) * BQ, hq = g * reps + ha;
#pragma unroll
                    for (int gi = 0; gi < C::NKG; ++gi) fr0[gi] = ld16(sn + aoff + to.natural(0, gi, cb));
                    sched_fence();
                    // row group 0 of tile it while row block 0 of tile it+1 arrives
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) Mma<T>::nat(acc[db], nx[db], px);
                    sched_fence();
                    dot_frags(tb, 1, nx);
                    px = ld16(pcur + 1024);
                    scores(sn + aoff);
                    f32x4 lg[2][2];  // lse of row group k of tile it+1 in lg[k % 2]
                    rows(sn, 0, lg[0]);
                    u32x4 pn[C::NPG];  // P of tile it+1
                    // row groups 1.. of tile it, each group's MFMAs with the
                    // exponentials of one row group of tile it+1
#pragma unroll
                    for (int gg = 1; gg < C::NPG; ++gg) {
                        u32x4 nn[C::NDB], pq;
                        if (gg + 1 < C::NPG) {
                            dot_frags(tb, gg + 1, nn);
                            pq = ld16(pcur + (gg + 1) * 1024);
                        } else {
                            dot_frags(sn + toff, 0, nn);
                        }
                        rows(sn, gg, lg[gg & 1]);
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) Mma<T>::nat(acc[db], nx[db], px);
                        pn[gg - 1] = probs(gg - 1, lg[(gg - 1) & 1], q0, hq);
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // three LDS reads
                            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
                        }
                        sched_fence();
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) nx[db] = nn[db];
                        if (gg + 1 < C::NPG) px = pq;
                    }
                    pn[C::NPG - 1] = probs(C::NPG - 1, lg[(C::NPG - 1) & 1], q0, hq);
                    if (needs_mask(q0)) mask_p(pn, q0);
                    char* pb = pbase + ((it + 1) & 1) * C::PBUF;
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) st16(pb + gg * 1024, pn[gg]);
                    next_tile();
                    slot = nslot;
                }
                if (n_it > 0) {
                    // last tile: its dV update alone
                    const char* tb = smem + slot * C::STAGEB + toff;
                    const char* pcur = pbase + ((n_it - 1) & 1) * C::PBUF;
                    wait_vm<0>();
                    lds_barrier();
                    px = ld16(pcur);
#pragma unroll
                    for (int gg = 0; gg < C::NPG; ++gg) {
                        u32x4 nn[C::NDB], pq;
                        if (gg + 1 < C::NPG) {
                            dot_frags(tb, gg + 1, nn);
                            pq = ld16(pcur + (gg + 1) * 1024);
                        }
                        sched_fence();
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) Mma<T>::nat(acc[db], nx[db], px);
                        sched_fence();
                        if (gg + 1 < C::NPG) {
#pragma unroll
                            for (int db = 0; db < C::NDB; ++db) nx[db] = nn[db];
                            px = pq;
                        }
                    }
                }
            } else {
            // dK wave: dP of tile it, then (after the barrier that publishes the dV
            // wave's P of that tile) dS = P (dP - Delta) and dK^T += Q^T dS
            int slot = 0;
            for (int it = 0; it < n_it; ++it) {
                const char* st = smem + slot * C::STAGEB;
                const float* lf = reinterpret_cast<const float*>(st + 2 * C::TILEB);
                const char* tb = st + toff;
                const char* pb = pbase + (it & 1) * C::PBUF;

                // phase A: dP of this tile's rows x this lane's key.
                // Row block 0's fragments are already here; row block 1's arrive in two
                // halves, each requested one chain ahead of its use.
                f32x16 x[C::NRB];
                u32x4 nx[C::NDB];     // row group 0 of Q^T, all column blocks
                f32x4 rv[C::NRB][4];  // delta of the rows this lane holds
                {
                    constexpr int HG = C::NKG / 2;
                    u32x4 fr1[C::NKG];
                    if constexpr (C::NRB == 2) {
#pragma unroll
                        for (int gi = 0; gi < HG; ++gi) fr1[gi] = ld16(st + aoff + to.natural(32, gi, cb));
                    }
                    sched_fence();
                    x[0] = zero16();
#pragma unroll
                    for (int gi = 0; gi < C::NKG; ++gi) Mma<T>::nat(x[0], fr0[gi], bf[gi]);
                    sched_fence();
                    if constexpr (C::NRB == 2) {
#pragma unroll
                        for (int gi = HG; gi < C::NKG; ++gi) fr1[gi] = ld16(st + aoff + to.natural(32, gi, cb));
                    }
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
                        nx[db] = rd_tr(tb + to.transposed(0, db, cb, 0), tb + to.transposed(0, db, cb, 1));
                    sched_fence();
                    if constexpr (C::NRB == 2) {
                        x[1] = zero16();
#pragma unroll
                        for (int gi = 0; gi < C::NKG; ++gi) Mma<T>::nat(x[1], fr1[gi], bf[gi]);
                    }
                    sched_fence();
                    const float* rowv = lf + BQ + 4 * h;
#pragma unroll
                    for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd)
                            rv[rb][qd] = *reinterpret_cast<const f32x4*>(rowv + 32 * rb + 8 * qd);
                }
                // dP - Delta while the dV wave is still on its exp phase
#pragma unroll
                for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[rb][r] -= rv[rb][r >> 2][r & 3];
                wait_vm<0>();   // this wave's share of tile it+1
                lds_barrier();  // P visible; tile it+1 visible; every wave is done with tile it-1
                if (it + 2 < n_it) issue();

                // phase B: acc[db] += Q^T (column block db, row group gg) x dS of row
                // group gg, row groups outermost so that the NDB accumulator chains
                // alternate. The next row group's fragments (after the last group: the
                // next tile's phase-A fragments) are requested ahead of each group's
                // MFMAs; dS = P (dP - Delta) is formed one row group ahead.
                const int nslot = slot == C::NS - 1 ? 0 : slot + 1;
                PF<T> pf[C::NPG];
                // P of every row group requested at once, right after the barrier
                // that publishes it (one LDS wait instead of one per row group)
                u32x4 pp[C::NPG];
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) pp[gg] = ld16(pb + gg * 1024);
                auto ds_group = [&](int gg) {
                    const T8 pv = __builtin_bit_cast(T8, pp[gg]);
                    const int rb = gg >> 1, hf = gg & 1;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = 8 * hf + i;
                        x[rb][r] *= (float)pv[i];
                    }
                    pf[gg] = make_pf<T>(x[rb], hf);
                };
                ds_group(0);
#pragma unroll
                for (int gg = 0; gg < C::NPG; ++gg) {
                    u32x4 nn[C::NDB];
                    if (gg + 1 < C::NPG) {
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db)
                            nn[db] = rd_tr(tb + to.transposed(gg + 1, db, cb, 0), tb + to.transposed(gg + 1, db, cb, 1));
                    } else {
                        const char* an = smem + nslot * C::STAGEB + aoff;
#pragma unroll
                        for (int gi = 0; gi < C::NKG; ++gi) fr0[gi] = ld16(an + to.natural(0, gi, cb));
                    }
                    sched_fence();
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) Mma<T>::nat(acc[db], nx[db], pf[gg].v);
                    if (gg + 1 < C::NPG) ds_group(gg + 1);
                    sched_fence();
                    if (gg + 1 < C::NPG) {
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) nx[db] = nn[db];
                    }
                }
                slot = nslot;
            }
            }

            // dK or dV of the wave's 32 keys: each lane stores its key's row
            // pieces (staged through LDS as whole rows, measured slower here)
            if (key < a.Lkv) {
                T* op = reinterpret_cast<T*>(V ? a.dv : a.dk) + (V ? kvhead_v : kvhead) + (size_t)key * Do;
                const float sc = V ? 1.f : a.scale;
#pragma unroll
                for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const int d = 32 * db + 8 * qd + 4 * h;
                        if (d < Do)
                            store4<T>(op + d, acc[db][4 * qd] * sc, acc[db][4 * qd + 1] * sc,
                                      acc[db][4 * qd + 2] * sc, acc[db][4 * qd + 3] * sc);
                    }
            }
        }
    };
    if (vw) run(std::true_type{});
    else run(std::false_type{});
}

// ===========================================================================
// Launchers
// ===========================================================================
template <class T, int DMAX, int BKV, int RW, int DW, int OCC, int NS>
hipError_t launch_fwd2(const FwdArgs& a, hipStream_t s) {
    using C = Fwd2Cfg<T, DMAX, BKV, RW, DW, NS>;
    auto kern = (a.mask || a.bmask) ? fa_fwd_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, true>
                       : fa_fwd_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long grid = (long long)((a.Lq + C::BQ - 1) / C::BQ) * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}
template <class T, int DMAX, int BKV, int RW, int DW, int OCC, int NS>
hipError_t launch_dq2(const BwdArgs& a, hipStream_t s) {
    using C = Dq2Cfg<T, DMAX, BKV, RW, DW, NS>;
    auto kern = a.Dv != a.D ? ((a.mask || a.bmask) ? fa_dq_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, true, true>
                                      : fa_dq_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, false, true>)
                            : ((a.mask || a.bmask) ? fa_dq_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, true, false>
                                      : fa_dq_lds_kernel<T, DMAX, BKV, RW, DW, OCC, NS, false, false>);
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long grid = (long long)((a.Lq + C::BQ - 1) / C::BQ) * a.B * a.Hq;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}
template <class T, int DMAX, int BQ, int KW, int DW, int OCC, int NS>
hipError_t launch_dkv2(const BwdArgs& a, hipStream_t s) {
    using C = Dkv2Cfg<T, DMAX, BQ, KW, DW, NS>;
    auto kern = (a.mask || a.bmask) ? fa_dkv_lds_kernel<T, DMAX, BQ, KW, DW, OCC, NS, true>
                       : fa_dkv_lds_kernel<T, DMAX, BQ, KW, DW, OCC, NS, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long grid = (long long)((a.Lkv + C::BKV - 1) / C::BKV) * a.B * a.Hkv;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
    return hipGetLastError();
}

// Pairing key blocks p and nkt-1-p balances the work of a causal mask
// without window; it is used only while it still leaves a workgroup for each
// of the 256 CUs.
constexpr int kPairMinGrid = 256;
template <class T, int DMAX, int BQ, int KW, int OCC, int PRIO>
hipError_t launch_dkv_pipe(const BwdArgs& a, hipStream_t s) {
    using C = DkvPipeCfg<T, DMAX, BQ, KW>;
    auto kern = (a.mask || a.bmask) ? fa_dkv_pipe_kernel<T, DMAX, BQ, KW, OCC, PRIO, true>
                       : fa_dkv_pipe_kernel<T, DMAX, BQ, KW, OCC, PRIO, false>;
    hipError_t e = set_lds(kern, C::LDS);
    if (e != hipSuccess) return e;
    const long long nkt = (a.Lkv + C::BKV - 1) / C::BKV;
    const long long bg = (long long)a.B * a.Hkv;
    const int pair = a.causal && !a.window && nkt >= 2 && (nkt + 1) / 2 * bg >= kPairMinGrid;
    const long long grid = pair ? (nkt + 1) / 2 * bg : nkt * bg;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a, pair);
    return hipGetLastError();
}

// Head-dim buckets of the 16-bit path: D is served by the smallest of 32, 64,
// 96, 128, 256 and 512 that holds it (columns past D read as zero and are
// never stored; the 32 and 96 buckets keep padded LDS rows, see
// tile_row_bytes, but run their products over 32 and 96 columns).
inline int dmax16(int D) {
    return D <= 32 ? 32 : D <= 64 ? 64 : D <= 96 ? 96 : D <= 128 ? 128 : D <= 256 ? 256 : 512;
}

// <tile, waves along rows/keys, waves along d, min waves per SIMD, stages>.
// Overridable at build time for tuning sweeps (e.g. -DFA2_FWD_128=64,4,1,2,2).
#ifndef FA2_FWD_32
#define FA2_FWD_32 64, 4, 1, 2, 2
#endif
#ifndef FA2_FWD_64
#define FA2_FWD_64 64, 4, 1, 2, 2
#endif
#ifndef FA2_FWD_96
#define FA2_FWD_96 64, 4, 1, 2, 2
#endif
#ifndef FA2_FWD_128
#define FA2_FWD_128 64, 4, 1, 2, 2
#endif
#ifndef FA2_FWD_256
#define FA2_FWD_256 32, 4, 1, 2, 2
#endif
#ifndef FA2_FWD_512
#define FA2_FWD_512 32, 1, 4, 1, 2
#endif
#ifndef FA2_DQ_32
#define FA2_DQ_32 64, 4, 1, 2, 2
#endif
#ifndef FA2_DQ_64
#define FA2_DQ_64 64, 4, 1, 2, 2
#endif
#ifndef FA2_DQ_96
#define FA2_DQ_96 64, 4, 1, 2, 2
#endif
#ifndef FA2_DQ_128
#define FA2_DQ_128 64, 4, 1, 2, 2
#endif
#ifndef FA2_DQ_512
#define FA2_DQ_512 32, 1, 4, 1, 2
#endif
#ifndef FA2_DKV_512
#define FA2_DKV_512 32, 1, 4, 1, 2
#endif

// dK/dV on wave pairs (head dims up to 128): <query tile, key blocks of 32, min
// waves per SIMD, dV-wave priority>.
#ifndef FA2_DKVS_32
#define FA2_DKVS_32 64, 4, 2, 1
#endif
#ifndef FA2_DKVS_64
#define FA2_DKVS_64 64, 4, 2, 1
#endif
#ifndef FA2_DKVS_96
#define FA2_DKVS_96 64, 4, 2, 1
#endif
#ifndef FA2_DKVS_128
#define FA2_DKVS_128 64, 4, 2, 1
#endif

}  // namespace lds
}  // namespace fa
