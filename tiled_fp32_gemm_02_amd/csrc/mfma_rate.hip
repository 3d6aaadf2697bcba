// The fp32 matrix-core rate the chip sustains, as a ceiling to read GEMM timings against.
//
// Every wave issues rounds of eight independent v_mfma_f32_32x32x2_f32 (each 32*32*2
// multiply-adds, 64 cycles on one SIMD) with no memory traffic. Each workgroup also
// records its shader-clock cycles (s_memtime) and the 100 MHz reference clock
// (s_memrealtime) over its run, and the id of the accelerator die (XCD) it ran on, so the
// clock each XCD actually ran at is reported next to the rate. The published fp32 matrix
// peak of 157.3 TFLOP/s assumes 256 CUs at 2.4 GHz.
//
// Usage: mfma_rate [workgroups per CU = 2] [rounds = 100000] [repetitions = 10]
// (256-thread workgroups: one wave per SIMD each).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;          // independent accumulators per wave
constexpr int kBlock = 256;
constexpr int kCus = 256;
constexpr double kPeakTflops = 157.3;

__global__ __launch_bounds__(kBlock) void mfma_rounds(float *out, unsigned long long *stamps, int rounds, float x)
{
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    floatx16 acc[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0.f;
    const float a = x + threadIdx.x * 1e-7f, b = x - threadIdx.x * 1e-7f;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int i = 0; i < kAcc; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
        for (int e = 0; e < 16; ++e)
            s += acc[i][e];
    out[blockIdx.x * kBlock + threadIdx.x] = s;     // keeps the products live
    __syncthreads();
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        stamps[3 * blockIdx.x] = c1 - c0;
        stamps[3 * blockIdx.x + 1] = r1 - r0;
        stamps[3 * blockIdx.x + 2] = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 15;  // XCC_ID
    }
}

bool ok(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        fprintf(stderr, "mfma_rate: %s: %s\n", what, hipGetErrorString(e));
    return e == hipSuccess;
}

}  // namespace

int main(int argc, char **argv)
{
    const int per_cu = argc > 1 ? atoi(argv[1]) : 2;
    const int rounds = argc > 2 ? atoi(argv[2]) : 100000;
    const int reps = argc > 3 ? atoi(argv[3]) : 10;
    if (per_cu < 1 || per_cu > 8 || rounds < 1 || reps < 1) {
        fprintf(stderr, "usage: mfma_rate [workgroups per CU 1..8] [rounds >= 1] [repetitions >= 1]\n");
        return 2;
    }
    const int grid = kCus * per_cu;
    float *out = nullptr;
    unsigned long long *stamps = nullptr;
    if (!ok(hipMalloc(&out, sizeof(float) * grid * kBlock), "hipMalloc") ||
        !ok(hipMalloc(&stamps, sizeof(unsigned long long) * 3 * grid), "hipMalloc"))
        return 1;
    std::vector<unsigned long long> host(3 * grid);
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate"))
        return 1;
    const double flop = 2.0 * 32 * 32 * 2 * kAcc * (double)rounds * grid * (kBlock / 64);
    printf("mfma_rate: %d workgroups of %d threads, %d rounds of %d v_mfma_f32_32x32x2_f32 per wave\n", grid,
           kBlock, rounds, kAcc);
    for (int r = 0; r < reps; ++r) {
        if (!ok(hipEventRecord(e0), "hipEventRecord"))
            return 1;
        mfma_rounds<<<grid, kBlock>>>(out, stamps, rounds, 1.0f);
        if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "hipEventRecord") ||
            !ok(hipEventSynchronize(e1), "hipEventSynchronize"))
            return 1;
        float ms = 0.f;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime") ||
            !ok(hipMemcpy(host.data(), stamps, sizeof(unsigned long long) * 3 * grid, hipMemcpyDeviceToHost),
                "hipMemcpy"))
            return 1;
        double cyc = 0, ticks = 0, xcd_cyc[16] = {}, xcd_ticks[16] = {};
        for (int g = 0; g < grid; ++g) {
            cyc += host[3 * g];
            ticks += host[3 * g + 1];
            xcd_cyc[host[3 * g + 2]] += host[3 * g];
            xcd_ticks[host[3 * g + 2]] += host[3 * g + 1];
        }
        double lo = 1e9, hi = 0;
        for (int x = 0; x < 16; ++x)
            if (xcd_ticks[x] > 0) {
                const double ghz = xcd_cyc[x] / xcd_ticks[x] * 0.1;
                lo = ghz < lo ? ghz : lo;
                hi = ghz > hi ? ghz : hi;
            }
        const double tflops = flop / (ms * 1e-3) / 1e12;
        printf("rep %d: %.3f ms  %.1f TFLOP/s  %.1f%% of %.1f  clock %.3f GHz (XCDs %.3f..%.3f)\n", r, ms, tflops,
               100.0 * tflops / kPeakTflops, kPeakTflops, cyc / ticks * 0.1, lo, hi);
        fflush(stdout);
    }
    hipFree(out);
    hipFree(stamps);
    return 0;
}
