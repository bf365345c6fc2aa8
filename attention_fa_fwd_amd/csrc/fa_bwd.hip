// fa_bwd.hip -- host side of the backward pass: argument checks and the launches of
// fa_bwd_kernel.hpp (row statistics, dK/dV, the sum of dK/dV partials when the GQA group is
// split over workgroups, dQ), exported as fa_bwd.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "fa_bwd_kernel.hpp"
#include "fa_fwd.h"

namespace {

using fa::BwdParams;

constexpr int kNumCUs = 256;

bool overlaps(uintptr_t a, size_t na, uintptr_t b, size_t nb) {
    return a < b + nb && b < a + na;
}

__global__ void zero16(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

// Workgroups sharing one K/V block's query heads: the smallest divisor of the group size
// that gives the dK/dV grid at least two workgroups per CU (causal: uneven work per block,
// balanced by handing out the heaviest first) or one per CU (non-causal).
int group_split(int B, int Hq, int Hkv, int Skv, int causal) {
    const int group = Hq / Hkv;
    const long long n = (long long)((Skv + 127) / 128) * B * Hkv;
    const long long target = causal ? 2LL * kNumCUs : kNumCUs;
    for (int d = 1; d <= group; ++d)
        if (group % d == 0 && n * d >= target) return d;
    return group;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t stats_bytes(int B, int Hq, int Sq) { return round256((size_t)B * Hq * Sq * 8); }

size_t part_bytes(int gsplit, int B, int Hkv, int Skv, int D) {
    return gsplit > 1 ? (size_t)gsplit * 2 * B * Hkv * Skv * D * 4 : 0;
}

template <int D, bool BF16>
hipError_t launch_all(const BwdParams& p, int causal, hipStream_t s) {
    const size_t rows = (size_t)p.B * p.Hq * p.Sq;
    constexpr int RPB = 256 / (D / 8);
    const dim3 gd((unsigned)std::min<size_t>((rows + RPB - 1) / RPB, (size_t)1 << 20));
    hipLaunchKernelGGL((fa::fa_bwd_dot_kernel<D, BF16>), gd, dim3(256),
                       0, s, p.o, p.dout, p.lse, p.stats, rows, (float)(1.0 / (double)p.scale));
    BwdParams pk = p, pq = p;
    pk.n_tiles = (p.Skv + 127) / 128;
    pq.n_tiles = (p.Sq + 127) / 128;
    const dim3 gk((unsigned)((long long)pk.n_tiles * p.B * p.Hkv * p.gsplit));
    const dim3 gq((unsigned)((long long)pq.n_tiles * p.B * p.Hq));
    if (causal) hipLaunchKernelGGL((fa::fa_bwd_dkdv_pair_kernel<D, true, BF16>), gk, dim3(512), 0, s, pk);
    else hipLaunchKernelGGL((fa::fa_bwd_dkdv_pair_kernel<D, false, BF16>), gk, dim3(512), 0, s, pk);
    if (p.gsplit > 1) {
        const size_t n = (size_t)p.B * p.Hkv * p.Skv * D;
        const size_t threads = n / 4;   // 2 tensors x n / 8
        const dim3 gr((unsigned)std::min<size_t>((threads + 255) / 256, 8 * kNumCUs));
        hipLaunchKernelGGL((fa::fa_bwd_reduce_kernel<BF16>), gr, dim3(256), 0, s, (const float*)p.part, p.dk,
                           p.dv, n, p.gsplit, p.scale);
    }
    if (causal) hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<D, true, BF16>), gq, dim3(256), 0, s, pq);
    else hipLaunchKernelGGL((fa::fa_bwd_dq_kernel<D, false, BF16>), gq, dim3(256), 0, s, pq);
    return hipGetLastError();
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal) {
    if (B <= 0 || Hq <= 0 || Sq <= 0 || Hkv <= 0 || Skv <= 0 || Hq % Hkv != 0) return 0;
    if (D != 64 && D != 128) return 0;
    return stats_bytes(B, Hq, Sq) + part_bytes(group_split(B, Hq, Hkv, Skv, causal), B, Hkv, Skv, D);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv,
           int D, float scale, int causal, int input_pos, int window, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
    const bool q_empty = B <= 0 || Hq <= 0 || Sq <= 0;
    const bool kv_empty = B <= 0 || Hkv <= 0 || Skv <= 0;
    if ((!q_empty && (!q || !out || !lse || !dout || !dq)) || (!kv_empty && (!k || !v || !dk || !dv)))
        return FA_ERR_NULL_POINTER;
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    if ((long long)B * Hq > INT_MAX || (long long)B * Hkv > INT_MAX) return FA_ERR_INVALID_SHAPE;
    if ((double)B * Hq * Sq * 256.0 > 1125899906842624.0 ||
        (double)B * Hkv * Skv * 256.0 > 1125899906842624.0)
        return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_SCALE;
    if (input_pos < 0 || (long long)input_pos + Sq > INT_MAX) return FA_ERR_INVALID_INPUT_POS;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_WINDOW;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout |
         (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
        return FA_ERR_MISALIGNED;
    if ((uintptr_t)lse & 3u) return FA_ERR_MISALIGNED;
    const size_t qb = (size_t)B * Hq * Sq * D * 2, kb = (size_t)B * Hkv * Skv * D * 2;
    const size_t lb = (size_t)B * Hq * Sq * 4;
    // Outputs must not overlap an input or each other.
    const uintptr_t outs[3] = {(uintptr_t)dq, (uintptr_t)dk, (uintptr_t)dv};
    const size_t osz[3] = {qb, kb, kb};
    const uintptr_t ins[6] = {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)out,
                              (uintptr_t)lse, (uintptr_t)dout};
    const size_t isz[6] = {qb, kb, kb, qb, lb, qb};
    for (int i = 0; i < 3; ++i) {
        if (osz[i] == 0) continue;
        for (int j = 0; j < 6; ++j)
            if (isz[j] && overlaps(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (osz[j] && overlaps(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_ALIAS;
    }
    if (q_empty && kv_empty) return FA_OK;
    const size_t need = fa_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal);
    if (need > 0) {
        if (!workspace) return FA_ERR_NULL_POINTER;
        if ((uintptr_t)workspace & 15u) return FA_ERR_MISALIGNED;
        if (workspace_bytes < need) return FA_ERR_WORKSPACE;
        const uintptr_t w = (uintptr_t)workspace;
        for (int i = 0; i < 3; ++i)
            if (osz[i] && overlaps(w, need, outs[i], osz[i])) return FA_ERR_ALIAS;
        for (int j = 0; j < 6; ++j)
            if (isz[j] && overlaps(w, need, ins[j], isz[j])) return FA_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    if (q_empty) {
        // No query rows: every dK and dV is zero (a fill kernel, not a memset, so that the
        // call can be captured in a graph).
        const size_t n16 = kb / 16;
        const dim3 grid((unsigned)std::min<size_t>((n16 + 255) / 256, 65535));
        hipLaunchKernelGGL(zero16, grid, dim3(256), 0, s, (uint4*)dk, n16);
        hipLaunchKernelGGL(zero16, grid, dim3(256), 0, s, (uint4*)dv, n16);
        return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.dout = dout;
    p.lse = lse;
    p.stats = (float*)workspace;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Sq = Sq;
    p.Skv = Skv;
    p.causal = causal != 0;
    p.input_pos = causal ? input_pos : 0;
    p.window = causal ? window : 0;
    p.c = (float)((double)scale * 1.4426950408889634073599246810019);
    p.scale = scale;
    p.group = Hq / Hkv;
    p.gsplit = group_split(B, Hq, Hkv, Skv, causal);
    p.hpw = p.group / p.gsplit;
    p.part = p.gsplit > 1 ? (float*)((unsigned char*)workspace + stats_bytes(B, Hq, Sq)) : nullptr;
    p.n_tiles = 0;
    if ((long long)((Skv + 127) / 128) * B * Hkv * p.gsplit > 0x7fffffffLL ||
        (long long)((Sq + 127) / 128) * B * Hq > 0x7fffffffLL)
        return FA_ERR_INVALID_SHAPE;
    hipError_t e;
    const int bf16 = dtype == FA_DTYPE_BF16;
    if (D == 128) e = bf16 ? launch_all<128, true>(p, causal, s) : launch_all<128, false>(p, causal, s);
    else e = bf16 ? launch_all<64, true>(p, causal, s) : launch_all<64, false>(p, causal, s);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
