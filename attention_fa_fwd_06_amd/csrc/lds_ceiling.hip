// Sustained LDS read rate of this GPU for the two operand-fragment reads of
// the 16-bit attention kernels: ds_read_b128 of a natural fragment (a lane
// reads 16 bytes of its own row) and ds_read_b64_tr_b16 (a transposing read),
// both at the kernels' swizzled addresses in tiles of 256-byte rows. Every
// wave runs only these reads (one XOR per result register to keep them live)
// from a 64 KB shared array, 256 x WPC workgroups of NT threads (WPC
// workgroups per CU). s_memtime / s_memrealtime around each wave's loop give
// the clock the chip ran at, so the rate is also reported per clock and CU:
// the figure to hold against the 128 bytes per clock and CU that one LDS
// operand per 32x32x16 MFMA needs at full matrix-core rate.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kLds = 64 * 1024;
constexpr int kRow = 256;  // bytes per tile row (head dim 128, 16-bit)

// chunk swizzle of 256-byte rows: the 16 rows of a natural fragment read and
// the 4 rows x 64 bytes of each half of a transposing read cover all banks once
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <bool TR>
__global__ __launch_bounds__(512) void lds_loop(unsigned* out, unsigned long long* clk, int iters) {
    __shared__ __attribute__((aligned(16))) unsigned char sm[kLds];
    for (int i = threadIdx.x * 16; i < kLds; i += blockDim.x * 16)
        *reinterpret_cast<u32x4*>(sm + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, ln = lane & 31, q = lane >> 4, m = lane & 15;
    // 16 distinct fragment offsets per iteration: two tiles of 32 rows x 256
    // bytes for the natural reads (8 fragments cover a tile), one tile for the
    // transposing reads (16 fragments cover it)
    int off[16];
    for (int u = 0; u < 16; ++u) {
        if constexpr (TR) {
            const int e = u & 1, x = (u >> 1) & 3, gg = (u >> 3) & 1;
            const int row = 16 * gg + 4 * h + (m >> 2) + 8 * e;
            off[u] = row * kRow + (((4 * x + 2 * (q & 1) + ((m & 3) >> 1)) ^ swz(row & 15)) << 4) + 8 * (m & 1);
        } else {
            off[u] = (u >> 3) * 32 * kRow + ln * kRow + (((2 * (u & 7) + h) ^ swz(ln)) << 4);
        }
    }
    constexpr int kStep = TR ? 8192 : 16384;  // bytes covered per iteration
    int tile = (w & 3) * kStep;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if constexpr (TR) {
                const u32x2 v = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(sm + tile + off[u])));
                acc[0] ^= v[0];
                acc[1] ^= v[1];
            } else {
                acc ^= *reinterpret_cast<const u32x4*>(sm + tile + off[u]);
            }
        }
        tile = (tile + kStep) & (kLds - 1);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

template <bool TR>
static int run(int nt, int wpc, unsigned* out, unsigned long long* clk, int iters) {
    const int grid = 256 * wpc;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    lds_loop<TR><<<grid, nt>>>(out, clk, iters);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    const int reps = 5;
    (void)hipEventRecord(e0);
    for (int r = 0; r < reps; ++r) lds_loop<TR><<<grid, nt>>>(out, clk, iters);
    (void)hipEventRecord(e1);
    if (hipEventSynchronize(e1) != hipSuccess) return 1;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    ms /= reps;
    unsigned long long h[2 * 512];
    if (hipMemcpy(h, clk, 2 * grid * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    double ratio = 0.0;
    for (int i = 0; i < grid; ++i) ratio += (double)h[2 * i] / (double)h[2 * i + 1];
    const double ghz = ratio / grid * 0.1;
    const double bytes = (double)grid * nt * iters * 16 * (TR ? 8 : 16);
    std::printf("{\"read\": \"%s\", \"threads\": %d, \"workgroups_per_cu\": %d, \"ms\": %.4f, \"tb_per_s\": %.1f, "
                "\"clock_ghz\": %.3f, \"bytes_per_clock_per_cu\": %.1f}\n",
                TR ? "ds_read_b64_tr_b16" : "ds_read_b128", nt, wpc, ms, bytes / ms / 1e9, ghz,
                bytes / (ms * 1e-3) / (ghz * 1e9) / 256);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return 0;
}

int main() {
    const int max_wpc = 2, iters = 4000;
    unsigned* out = nullptr;
    unsigned long long* clk = nullptr;
    if (hipMalloc(&out, (size_t)256 * max_wpc * 512 * 4) != hipSuccess ||
        hipMalloc(&clk, (size_t)256 * max_wpc * 2 * sizeof(unsigned long long)) != hipSuccess)
        return 1;
    int rc = 0;
    const int shapes[3][2] = {{256, 1}, {256, 2}, {512, 2}};  // 1, 2, 4 waves per SIMD
    for (const auto& s : shapes) {
        rc |= run<false>(s[0], s[1], out, clk, iters);
        rc |= run<true>(s[0], s[1], out, clk, iters);
    }
    (void)hipFree(out);
    (void)hipFree(clk);
    return rc;
}
