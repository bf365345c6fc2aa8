// fa_merge_kernel.hpp -- gfx950 merge of split-KV partial results.
//
// A split-KV launch of fa_fwd_kernel leaves, for every (batch, head, query) row and key
// range s, the range's normalised partial output O_s (fp32) and its log-sum-exp LSE_s.
// The merge is the online-softmax update of "Tuning Flash Attention for peak performance
// in NVIDIA CUDA Tile" (Part 1 "Online softmax update") applied across whole ranges:
//     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// where a range with no visible key has LSE_s = -inf and weight 0 (a row with none at all
// gets O = 0, LSE = -inf).
//
// One wave per row.  The lanes load the row's LSE_s in parallel (lane l holds ranges
// l, l + 64, ...), reduce max and sum across the wave, and keep their ranges' weights; then
// every lane accumulates its D/64 output elements over the ranges, reading each range's
// weight from the lane that holds it (v_readlane), with eight ranges' loads in flight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kMergeMaxSplits = 256;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <bool BF16>
__device__ __forceinline__ uint32_t merge_pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 x = {a, b};
    if constexpr (BF16) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));
    } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, h2));
    }
}

// One output row: the row's partial LSE values and weights across the wave, then its
// D outputs, D / 64 per lane.
template <int D, bool BF16>
__device__ __forceinline__ void fa_merge_row(const float* o_part, const float* lse_part, void* o, float* lse,
                                             size_t rows, int num_splits, size_t row) {
    constexpr int PER = D / 64;                  // output elements per lane
    constexpr int SPL = kMergeMaxSplits / 64;    // ranges held per lane
    const int lane = threadIdx.x & 63;
    constexpr float LOG2E = 1.44269504088896340736f;

    float ls[SPL];
    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < SPL; ++t) {
        const int sp = t * 64 + lane;
        ls[t] = sp < num_splits ? lse_part[(size_t)sp * rows + row] : -__builtin_inff();
        mx = fmaxf(mx, ls[t]);
    }
    mx = wave_max(mx);
    float wt[SPL];
    float total = 0.0f;
#pragma unroll
    for (int t = 0; t < SPL; ++t) {
        wt[t] = (ls[t] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f((ls[t] - mx) * LOG2E);
        total += wt[t];
    }
    total = wave_sum(total);

    float acc[PER] = {};
    const float* base = o_part + (size_t)row * D + lane * PER;
    const size_t sstride = (size_t)rows * D;
    typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int t = 0; t < SPL; ++t) {
        const int n = min(64, num_splits - t * 64);
        if (n <= 0) break;
        const int wbits = __float_as_int(wt[t]);
        // Batches of 8 ranges: all 8 loads are issued before the first is used.  Entries
        // past n re-read range n - 1 with weight 0.
        for (int r0 = 0; r0 < n; r0 += 8) {
            f2 x[8];
            float w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = min(r0 + u, n - 1);
                const float* src = base + (size_t)(t * 64 + r) * sstride;
                if constexpr (PER == 2) x[u] = *(const f2*)src;
                else x[u] = (f2){src[0], 0.0f};
                w[u] = r0 + u < n ? __int_as_float(__builtin_amdgcn_readlane(wbits, r)) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc[0] += w[u] * x[u][0];
                if constexpr (PER == 2) acc[1] += w[u] * x[u][1];
            }
        }
    }
    const float inv = total > 0.0f ? __builtin_amdgcn_rcpf(total) : 0.0f;
    uint16_t* orow = (uint16_t*)o + (size_t)row * D + lane * PER;
    if constexpr (PER == 2) {
        *(uint32_t*)orow = merge_pack2<BF16>(acc[0] * inv, acc[1] * inv);
    } else {
        orow[0] = (uint16_t)(merge_pack2<BF16>(acc[0] * inv, 0.0f) & 0xffffu);
    }
    if (lane == 0) lse[row] = total > 0.0f ? mx + __builtin_logf(total) : -__builtin_inff();
}

// o_part [S][rows][D] and lse_part [S][rows] fp32; o [rows][D] in the storage type, lse
// [rows] fp32.  Blocks of 256 threads, one wave per row, striding over the rows by the grid;
// num_splits <= 256.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* o_part, const float* lse_part,
                                                       void* o, float* lse, size_t rows, int num_splits) {
    for (size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (size_t)gridDim.x * 4)
        fa_merge_row<D, BF16>(o_part, lse_part, o, lse, rows, num_splits, row);
}

}  // namespace fa
