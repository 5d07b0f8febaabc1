// Sustained bf16 MFMA rate of this GPU with random operands: every wave runs
// chains of v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic
// in the loop), 256 x WPS workgroups of 4 waves (WPS waves per SIMD). The
// wave also reads s_memtime (shader clock) and s_memrealtime (100 MHz) around
// its loop, which gives the clock the chip actually ran at. This is the
// ceiling the attention kernels' MFMA phases can reach at most; the roofline
// peak stays the published dense figure.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int CHAINS>
__global__ __launch_bounds__(256) void mfma_loop(const u32x4* src, float* out, unsigned long long* clk, int iters) {
    const int lane = threadIdx.x & 63;
    u32x4 ra[4], rb[4];
    for (int i = 0; i < 4; ++i) {
        ra[i] = src[i * 64 + lane];
        rb[i] = src[(4 + i) * 64 + lane];
    }
    f32x16 acc[CHAINS];
    for (int c = 0; c < CHAINS; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int n = 0; n < 16 / CHAINS; ++n)
#pragma unroll
            for (int c = 0; c < CHAINS; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[(n + c) & 3]),
                                                                 __builtin_bit_cast(bf16x8, rb[(3 * n + c) & 3]),
                                                                 acc[c], 0, 0, 0);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int c = 0; c < CHAINS; ++c)
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

template <int CHAINS>
static int run(int wps, const u32x4* src, float* out, unsigned long long* clk, int iters) {
    const int grid = 256 * wps;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    mfma_loop<CHAINS><<<grid, 256>>>(src, out, clk, iters);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    const int reps = 5;
    (void)hipEventRecord(e0);
    for (int r = 0; r < reps; ++r) mfma_loop<CHAINS><<<grid, 256>>>(src, out, clk, iters);
    (void)hipEventRecord(e1);
    if (hipEventSynchronize(e1) != hipSuccess) return 1;
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    ms /= reps;
    std::vector<unsigned long long> h(2 * grid);
    if (hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    double ratio = 0.0;
    for (int i = 0; i < grid; ++i) ratio += (double)h[2 * i] / (double)h[2 * i + 1];
    ratio /= grid;
    const double flops = (double)grid * 4 * iters * 16 * 32768.0;
    std::printf("{\"chains\": %d, \"waves_per_simd\": %d, \"ms\": %.4f, \"tflops\": %.1f, \"clock_ghz\": %.3f}\n",
                CHAINS, wps, ms, flops / ms / 1e9, ratio * 0.1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return 0;
}

int main() {
    const int max_wps = 4, maxgrid = 256 * max_wps, iters = 4000;
    std::vector<unsigned> hs(8 * 64 * 4);
    std::mt19937 gen(7);
    std::normal_distribution<float> nd(0.f, 1.f);
    for (auto& x : hs) {  // two bf16 values (truncated N(0,1) floats) per word
        const float a = nd(gen), b = nd(gen);
        unsigned ua, ub;
        std::memcpy(&ua, &a, 4);
        std::memcpy(&ub, &b, 4);
        x = (ua >> 16) | (ub & 0xffff0000u);
    }
    u32x4* src = nullptr;
    float* out = nullptr;
    unsigned long long* clk = nullptr;
    if (hipMalloc(&src, hs.size() * 4) != hipSuccess || hipMalloc(&out, (size_t)maxgrid * 256 * 4) != hipSuccess ||
        hipMalloc(&clk, (size_t)maxgrid * 2 * sizeof(unsigned long long)) != hipSuccess)
        return 1;
    if (hipMemcpy(src, hs.data(), hs.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return 1;
    int rc = 0;
    for (int wps = 1; wps <= max_wps; wps *= 2) {
        rc |= run<1>(wps, src, out, clk, iters);
        rc |= run<2>(wps, src, out, clk, iters);
        rc |= run<4>(wps, src, out, clk, iters);
    }
    (void)hipFree(src);
    (void)hipFree(out);
    (void)hipFree(clk);
    return rc;
}
