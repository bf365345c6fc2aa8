// fa_peak_probe.hip -- measurement aid of the benchmark, not part of the attention library:
// the device's compute-unit count and peak engine clock, and a loop of nothing but
// v_mfma_f32_32x32x16_bf16 that shows what dense bf16 MFMA rate the chip sustains and at
// which clock, next to the published 2516.6 TFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP/clk/CU).
//
// C entry points (loaded by bench.py through ctypes; built as libfa_probe.so):
//   int fa_probe_device(int* num_cus, int* max_clock_khz)
//       hipDeviceProp of the current device.  Returns 0 or a hipError_t code.
//   int fa_probe_mfma(int iters, double* tflops, double* clock_ghz)
//       Runs 512 workgroups of 4 waves (two waves per SIMD on 256 CUs), each wave issuing
//       16 * iters MFMAs on four independent accumulators; *tflops from hipEvent time,
//       *clock_ghz the median over waves of shader-clock cycles (s_memtime) divided by
//       real time (s_memrealtime, 100 MHz).  Allocates and frees its own buffers.
//       Returns 0 or a hipError_t code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBlocks = 512;
constexpr int kWaves = kBlocks * kThreads / 64;

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float* sink, uint64_t* ticks) {
    const int lane = threadIdx.x & 63;
    // Four pairs of pseudo-random operands in [-1, 1), one pair per accumulator, so that
    // consecutive MFMAs see different data (constant operands draw less power and would let
    // the clock run higher than on real data).  A small hash of (lane, pair, element).
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t h = (uint32_t)(lane * 131 + j * 17 + i) * 2654435761u;
            h ^= h >> 13;
            h *= 0x5bd1e995u;
            h ^= h >> 15;
            a[j][i] = (__bf16)((float)(h & 0xffff) / 32768.0f - 1.0f);
            b[j][i] = (__bf16)((float)(h >> 16) / 32768.0f - 1.0f);
        }
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    const uint64_t c0 = __builtin_readcyclecounter();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], acc3, 0, 0, 0);
        }
    }
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i] + acc2[i] + acc3[i];
    const int wave = (blockIdx.x * kThreads + threadIdx.x) / 64;
    sink[blockIdx.x * kThreads + threadIdx.x] = s;   // keeps the loop; never read
    if (lane == 0) {
        ticks[2 * wave] = c1 - c0;
        ticks[2 * wave + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" int fa_probe_device(int* num_cus, int* max_clock_khz) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return (int)e;
    *num_cus = prop.multiProcessorCount;
    *max_clock_khz = prop.clockRate;
    return 0;
}

extern "C" int fa_probe_mfma(int iters, double* tflops, double* clock_ghz) {
    if (iters < 1) return (int)hipErrorInvalidValue;
    float* sink = nullptr;
    uint64_t* ticks = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    std::vector<uint64_t> host(2 * kWaves);
    float ms = 0.0f;
    hipError_t e = hipMalloc(&sink, sizeof(float) * kBlocks * kThreads);
    if (e == hipSuccess) e = hipMalloc(&ticks, sizeof(uint64_t) * 2 * kWaves);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        // One short warm-up launch brings the clock up from idle.
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(kBlocks), dim3(kThreads), 0, nullptr, std::max(1, iters / 4),
                           sink, ticks);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e0, nullptr);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(mfma_loop_kernel, dim3(kBlocks), dim3(kThreads), 0, nullptr, iters, sink, ticks);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess) e = hipMemcpy(host.data(), ticks, sizeof(uint64_t) * 2 * kWaves, hipMemcpyDeviceToHost);
    if (e == hipSuccess) {
        const double flops = 2.0 * 32 * 32 * 16 * 16.0 * iters * kWaves;
        *tflops = flops / (ms * 1e-3) / 1e12;
        std::vector<double> ghz;
        ghz.reserve(kWaves);
        for (int w = 0; w < kWaves; ++w)
            if (host[2 * w + 1] > 0) ghz.push_back((double)host[2 * w] / ((double)host[2 * w + 1] / 100e6) / 1e9);
        std::sort(ghz.begin(), ghz.end());
        *clock_ghz = ghz.empty() ? 0.0 : ghz[ghz.size() / 2];
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (ticks) (void)hipFree(ticks);
    if (sink) (void)hipFree(sink);
    return (int)e;
}
