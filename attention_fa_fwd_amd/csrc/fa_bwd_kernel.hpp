// fa_bwd_kernel.hpp -- gfx950 (MI355X) backward pass of the attention forward kernel.
//
// Gradients of O = softmax(scale Q K^T + M) V for an upstream gradient dO.  The pages name
// the backward pass only as future work ("How I Beat PyTorch's Flash Attention", "Future
// work"); the formulas are the textbook softmax derivative, recomputing P from the LSE the
// forward pass returns instead of storing it:
//     P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),
//     dS = P * (dP - D),       dQ = scale dS K,  dK = scale dS^T Q.
//
// Kernels, no atomics, deterministic:
//  * fa_bwd_dot_kernel: per query row the pair {-LSE / scale (-inf for a row with no
//    visible key), -D} with D = dO . O, in fp32 -- the row statistics both gradient kernels
//    read.  The dK/dV kernel starts its S and dP accumulators at these values, so the MFMAs
//    produce S - LSE / scale and dP - D directly: P = exp2(c (S - LSE / scale)),
//    dS = P (dP - D).
//  * fa_bwd_dkdv_pair_kernel: two waves on one SIMD share 32 keys of one K/V head, one
//    holding K (S, P, dV), the other V (dP, dS, dK), P passing between them through LDS;
//    the workgroup streams 32-row tiles of Q, dO and the row statistics of the query heads
//    it covers and accumulates dK^T and dV^T in registers, so the grouped heads' sum
//    happens in place.  When there are too few K/V blocks to fill the chip, the group's
//    query heads are split over several workgroups, each writing an fp32 partial that
//    fa_bwd_reduce_kernel sums in a fixed order.
//  * fa_bwd_dq_kernel: a wave owns 32 query rows (Q and dO rows in registers); the
//    workgroup streams 32-key tiles of K and V and accumulates dQ^T; two workgroups share
//    a CU.
// Both use the forward kernel's MFMA formulation: the streamed tile is the A operand of
// v_mfma_f32_32x32x16 (row reads from LDS), the wave's own rows are the B operand, so the
// 32x32 accumulator gives each lane one of its own rows and 16 streamed rows; P and dS go
// from that accumulator straight into the B operand of the second product, whose A
// operand is the streamed tile transposed (ds_read_b64_tr_b16).  Since each streamed tile
// is read both ways, its LDS layout uses one XOR swizzle of the 16-byte chunks that a
// bank model finds conflict-free for both the row reads and the transposed reads.
//
// Pipeline: several LDS buffer sets.  A step loads a tile a few steps ahead, issues the
// S / dP products of the next tile into a second register set, then turns this tile's
// S / dP into P and dS and issues the transposed products -- so the exp2 work of one tile
// overlaps the matrix work of the next.  A step ends by waiting only for the tile the
// next step needs (later tiles' loads stay in flight) and one barrier.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;    // [B*Hq*Sq], natural log, -inf for rows with no visible key
    float* stats;        // [B*Hq*Sq][2]: -LSE / scale (-inf for an empty row), -D
    void* dq;
    void* dk;
    void* dv;
    float* part;         // gsplit > 1: fp32 partial dK, dV [gsplit][2][B*Hkv*Skv*D]
    int B, Hq, Hkv, Sq, Skv;
    int causal, input_pos, window;   // window > 0 only with causal
    float c;                         // scale * log2(e)
    float scale;
    int group;                       // Hq / Hkv
    int gsplit;                      // workgroups sharing one K/V block's query heads
    int hpw;                         // query heads per dK/dV workgroup (group / gsplit)
    int n_tiles;                     // 128-row blocks per head (queries for dQ, keys for dK/dV)
};

// XOR swizzle of the 16-byte chunks of row `row`, linear in the row's low four bits, found
// by an exhaustive search over such maps to be free of LDS bank conflicts both for row
// reads (32 rows x one chunk) and for the transposed reads of the P V style product.
template <int D>
__device__ __forceinline__ int b_swz(int row) {
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    if constexpr (D == 128) return (b0 ? 4 : 0) ^ (b1 ? 9 : 0) ^ (b2 ? 2 : 0) ^ (b3 ? 1 : 0);
    else return (b0 ? 1 : 0) ^ (b1 ? 4 : 0) ^ (b2 ? 2 : 0) ^ (b3 ? 1 : 0);
}

template <bool BF16>
__device__ __forceinline__ float half_to_f32(uint32_t x) {
    if constexpr (BF16) return __uint_as_float(x << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)x);
}

// Buffer resource whose base and size are wave-uniform by construction; passing them
// through readfirstlane lets the compiler keep the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, int nbytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane(nbytes);
    return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
}

// 4 bytes per lane from a buffer straight into LDS: lane i writes lds + 4*i.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                             voff, 0, 0, 0);
}

// Row statistics: stats[row] = {-LSE / scale or -inf for an empty row, -sum_d dO * O};
// D / 8 lanes per row, 16 bytes each, summed by a butterfly in a fixed order.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_dot_kernel(const void* o, const void* dout, const float* lse,
                                                         float* stats, size_t rows, float inv_scale) {
    constexpr int TPR = D / 8, RPB = 256 / TPR;
    const int t = threadIdx.x % TPR;
    for (size_t row0 = (size_t)blockIdx.x * RPB; row0 < rows; row0 += (size_t)gridDim.x * RPB) {
        const size_t row = row0 + threadIdx.x / TPR;
        float acc = 0.0f;
        if (row < rows) {
            const u32x4 a = ((const u32x4*)((const uint16_t*)o + row * D))[t];
            const u32x4 g = ((const u32x4*)((const uint16_t*)dout + row * D))[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = __builtin_fmaf(half_to_f32<BF16>(a[e] & 0xffffu), half_to_f32<BF16>(g[e] & 0xffffu), acc);
                acc = __builtin_fmaf(half_to_f32<BF16>(a[e] >> 16), half_to_f32<BF16>(g[e] >> 16), acc);
            }
        }
#pragma unroll
        for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
        if (row < rows && t == 0) {
            const float l = lse[row];
            const float nls = l == -__builtin_inff() ? -__builtin_inff() : -l * inv_scale;
            *(f32x2*)(stats + 2 * row) = (f32x2){nls, -acc};
        }
    }
}

// dK = scale * sum_g part[g][0], dV = sum_g part[g][1], rounded to the storage type; n
// elements per tensor (a multiple of 8), 8 per thread.
template <bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(const float* part, void* dk, void* dv, size_t n,
                                                            int gsplit, float scale) {
    const size_t n8 = n / 8;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n8; i += (size_t)gridDim.x * 256) {
        const int t = i >= n8;
        const size_t j = (i - (t ? n8 : 0)) * 8;
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, c = a;
        for (int g = 0; g < gsplit; ++g) {
            const float* s = part + (size_t)(2 * g + t) * n + j;
            a += *(const f32x4*)s;
            c += *(const f32x4*)(s + 4);
        }
        const float mul = t ? 1.0f : scale;
        a *= mul;
        c *= mul;
        const u32x4 wv = {pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]), pack2<BF16>(c[0], c[1]),
                          pack2<BF16>(c[2], c[3])};
        *(u32x4*)((uint16_t*)(t ? dv : dk) + j) = wv;
    }
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// dQ: a wave owns 32 query rows of one query head (its Q and dO rows in registers, its
// statistics in two registers); the workgroup streams 32-key tiles of K and V through LDS.
// S^T = K Q^T and dP^T = V dO^T come out with lane = query, and dQ^T += K^T dS^T.  Four LDS
// buffer sets: step j loads tile j + 3, so one tile's loads stay in flight across a step's
// closing wait; the S / dP register set alternates with the step's parity.
template <int D, bool CAUSAL, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
    constexpr int NT = 256, NW = 4;
    constexpr int BR = 32;               // streamed rows per tile
    constexpr int DK = D / 16, DB = D / 32;
    constexpr int ROWB = D * 2, TILE = BR * ROWB, CPR = D / 8;
    constexpr int LD = BR * CPR / NT;    // 16-byte chunks of a tile per thread
    constexpr int LOAD_STRIDE = NT * 16;
    constexpr int NL = 2 * LD;           // tile loads per lane per step
    static_assert(BR * CPR % NT == 0 && (64 * NW / CPR) % 16 == 0, "tile load layout");
    typedef uint16_t T;
    constexpr int NB = 4;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // Workgroup -> (batch, query head, 128-row block); causal: heaviest blocks first.
    const int wg = blockIdx.x;
    const int bh = wg % (p.B * p.Hq);
    const int trank = wg / (p.B * p.Hq);
    const int b = bh / p.Hq;
    const int head = bh - b * p.Hq;
    const int blk = CAUSAL ? p.n_tiles - 1 - trank : trank;
    const int r0 = blk * 128;                 // first own row of the workgroup
    const int rw0 = r0 + w * 32;              // first own row of the wave
    const bool win = CAUSAL && p.window > 0;
    const int W = p.window;

    // Own rows (B operands): the Q and dO rows of query head `head`.
    const int own_row = min(rw0 + l32, p.Sq - 1);
    const size_t own_head = (size_t)(b * p.Hq + head);
    const T* x1p = (const T*)p.q + (own_head * p.Sq + own_row) * D;
    const T* x2p = (const T*)p.dout + (own_head * p.Sq + own_row) * D;
    u32x4 x1[DK], x2[DK];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
        x1[dk] = ((const u32x4*)x1p)[dk * 2 + h];
        x2[dk] = ((const u32x4*)x2p)[dk * 2 + h];
    }
    // The lane's own query row statistics, as LSE * log2(e) (+inf for an empty row, so
    // that p = 0) and D.
    float lse2_own, d_own;
    {
        const f32x2 st = *(const f32x2*)(p.stats + 2 * (own_head * p.Sq + own_row));
        lse2_own = -st[0] * p.c;
        d_own = -st[1];
    }

    // Key tiles [tb, tb + n_steps) of K/V head head / group; tiles [ua, ub) need no mask:
    // a tile needs no mask when it lies inside the tensors, the workgroup's own rows do
    // too, and every (query, key) pair of the two blocks is visible (causal: key <=
    // input_pos + query; window: key >= input_pos + query - window + 1).
    const int kv_head = head / p.group;
    int n_steps, tb, ua, ub;
    {
        const int q_last = min(r0 + 128, p.Sq) - 1;
        const int Tc = CAUSAL ? (min(p.input_pos + q_last + 1, p.Skv) + BR - 1) / BR : (p.Skv + BR - 1) / BR;
        tb = win ? min(max(0, p.input_pos + r0 - W + 1) / BR, Tc) : 0;
        n_steps = Tc - tb;
        int a = tb, e = min(Tc, p.Skv / BR);
        if (CAUSAL) e = min(e, (p.input_pos + r0 + 1) / BR);
        if (win) {
            const int x = p.input_pos + r0 + 128 - W;
            if (x > 0) a = max(a, (x + BR - 1) / BR);
        }
        if (r0 + 128 > p.Sq) e = a;
        ua = min(a, Tc);
        ub = max(min(e, Tc), ua);
    }

    __shared__ __attribute__((aligned(16))) unsigned char t1_0[TILE], t1_1[TILE], t1_2[TILE], t1_3[TILE];
    __shared__ __attribute__((aligned(16))) unsigned char t2_0[TILE], t2_1[TILE], t2_2[TILE], t2_3[TILE];
    auto t1_of = [&](auto ph) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return t1_0;
        else if constexpr (P == 1) return t1_1;
        else if constexpr (P == 2) return t1_2;
        else return t1_3;
    };
    auto t2_of = [&](auto ph) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return t2_0;
        else if constexpr (P == 1) return t2_1;
        else if constexpr (P == 2) return t2_2;
        else return t2_3;
    };

    // Tile loads (direct to LDS): lane slot -> (row, physical chunk); it fetches the
    // logical chunk the swizzle places there.  Rows past the tensor's end read zero; steps
    // past the last one load nothing (zero-size range).
    int src_off;
    {
        const int slot = w * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        src_off = row * ROWB + ((pc ^ b_swz<D>(row)) << 4);
    }
    int f_s = 0;
    const size_t f_slab = (size_t)(b * p.Hkv + kv_head) * p.Skv;
    auto fetch_tiles = [&](unsigned char* d1, unsigned char* d2) FA_INLINE {
        const int row0 = (tb + f_s) * BR;
        const int rows = f_s < n_steps ? min(p.Skv - row0, BR) : 0;
        const size_t first = rows > 0 ? f_slab + row0 : 0;
        const __amdgpu_buffer_rsrc_t r1 = make_rsrc_uniform((const T*)p.k + first * D, rows * ROWB);
        const __amdgpu_buffer_rsrc_t r2 = make_rsrc_uniform((const T*)p.v + first * D, rows * ROWB);
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            buffer_load_lds16(r1, d1 + (i * NW + w) * 1024, src_off, i * LOAD_STRIDE);
            buffer_load_lds16(r2, d2 + (i * NW + w) * 1024, src_off, i * LOAD_STRIDE);
        }
        ++f_s;
    };

    // Row-read offsets (A operand rows l32, chunk 2dk + h) and transposed-read offsets.
    int off_r[DK];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) off_r[dk] = l32 * ROWB + (((2 * dk + h) ^ b_swz<D>(l32)) << 4);
    int off_t[2][DB];
    {
        const int vs = lane & 15, vj = vs >> 2, vq = vs & 3, vg = lane >> 4;
        const int row_in = 4 * (vg >> 1) + vj;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int row = row_in + 8 * rr;
                const int c = 4 * db + 2 * (vq & 1) + (vg & 1);
                off_t[rr][db] = row * ROWB + ((c ^ b_swz<D>(row)) << 4) + (vq >> 1) * 8;
            }
    }
    auto rows_mfma = [&](const unsigned char* tb_, const u32x4 (&x)[DK]) FA_INLINE {
        f32x16 acc = {};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            const u32x4 a = *(const u32x4*)(tb_ + off_r[dk]);
            acc = mfma32<BF16>(a, x[dk], acc);
        }
        return acc;
    };
    auto trans_mfma = [&](const unsigned char* tb_, const u32x4 (&pk)[2], f32x16 (&acc)[DB]) FA_INLINE {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x2 y0 = lds_read_tr16(tb_ + 16 * hf * ROWB + off_t[0][db]);
                const u32x2 y1 = lds_read_tr16(tb_ + 16 * hf * ROWB + off_t[1][db]);
                const u32x4 a = {y0[0], y0[1], y1[0], y1[1]};
                acc[db] = mfma32<BF16>(a, pk[hf], acc[db]);
            }
    };

    f32x16 acc1[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc1[db] = (f32x16){};
    f32x16 sc0 = {}, dp0 = {}, sc1 = {}, dp1 = {};   // S and dP of two consecutive tiles

    // s_waitcnt vmcnt(N) then s_barrier, as one asm statement (also a compiler memory
    // barrier): at the end of a step only the newest tile's loads stay in flight (the next
    // step's tile j + 2 has landed).
    auto wait_tiles = [&]() FA_INLINE {
        constexpr int N = (NB - 3) * NL;
        static_assert(N < 64, "vmcnt range");
        constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
        asm volatile("s_waitcnt %0\n\ts_barrier" ::"n"(imm) : "memory");
    };

    int c_row0 = tb * BR;   // first key of the step being computed

    // Step j: loads tile j + 3, issues S^T / dP^T of tile j + 1, then P and dS of tile j and
    // dQ^T += K(j)^T dS(j)^T.  Key tiles outside [ua, ub) are masked.
    auto step = [&](auto ph_tag) FA_INLINE {
        constexpr int PH = decltype(ph_tag)::value;
        const bool masked = c_row0 < ua * BR || c_row0 >= ub * BR;
        using PN = std::integral_constant<int, (PH + 1) % NB>;
        using PF = std::integral_constant<int, (PH + NB - 1) % NB>;
        using PC = std::integral_constant<int, PH>;
        f32x16& sc = (PH & 1) ? sc1 : sc0;
        f32x16& dp = (PH & 1) ? dp1 : dp0;
        f32x16& scn = (PH & 1) ? sc0 : sc1;
        f32x16& dpn = (PH & 1) ? dp0 : dp1;

        fetch_tiles(t1_of(PF{}), t2_of(PF{}));
        scn = rows_mfma(t1_of(PN{}), x1);
        dpn = rows_mfma(t2_of(PN{}), x2);

        // This tile: P and dS.  Element i of a lane is key c_row0 + 4h + ci(i).
        float pe[16], de[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c, -lse2_own));
            pe[i] = pv;
            de[i] = pv * (dp[i] - d_own);
        }
        // Mask (edge tiles only): the lane's element i is key c_row0 + 4h + ci(i),
        // ci(i) = 8(i/4) + i%4 < 32.  Visible elements form one range of ci, [lo, hi); bit
        // ci of `vis` is set inside it, and a one-bit signed extract turns that bit into an
        // all-ones / zero word that clears p and dS where masked.
        if (masked) {
            const int base = c_row0 + 4 * h;
            const int own = rw0 + l32;
            int lo = 0, hi = p.Skv - base;
            if (CAUSAL) hi = min(hi, p.input_pos + own - base + 1);    // key <= input_pos + query
            if (win) lo = p.input_pos + own - base - W + 1;            // key >= input_pos + query - W + 1
            if (own >= p.Sq) hi = 0;
            lo = min(max(lo, 0), 32);
            hi = min(max(hi, 0), 32);
            const uint32_t below_hi = hi >= 32 ? ~0u : (1u << hi) - 1u;
            const uint32_t below_lo = lo >= 32 ? ~0u : (1u << lo) - 1u;
            const uint32_t vis = hi > lo ? below_hi & ~below_lo : 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vis, 8 * (i >> 2) + (i & 3), 1);
                de[i] = __uint_as_float(__float_as_uint(de[i]) & keep);
            }
        }
        u32x4 dsk[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const float* f = de + 8 * hf;
            dsk[hf] = (u32x4){pack2<BF16>(f[0], f[1]), pack2<BF16>(f[2], f[3]), pack2<BF16>(f[4], f[5]),
                              pack2<BF16>(f[6], f[7])};
        }
        // Keep the transposed reads below this point: hoisted above, they would be live
        // alongside the next tile's S / dP and this tile's softmax temporaries.
        __builtin_amdgcn_sched_barrier(0);
        trans_mfma(t1_of(PC{}), dsk, acc1);
        wait_tiles();
        c_row0 += BR;
    };

    if (n_steps > 0) {
        // Prologue: tiles 0 .. NB-2 in flight, wait for 0 and 1, products of tile 0.
        static_for<NB - 1>([&](auto ph) FA_INLINE { fetch_tiles(t1_of(ph), t2_of(ph)); });
        wait_tiles();
        sc0 = rows_mfma(t1_0, x1);
        dp0 = rows_mfma(t2_0, x2);

        // Unrolled by NB so the buffer phase of each copy of the step is fixed.
        int i = 0;
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        using P3 = std::integral_constant<int, 3>;
        for (; i + NB - 1 < n_steps; i += NB) {
            step(P0{});
            step(P1{});
            step(P2{});
            step(P3{});
        }
        if (i < n_steps) { step(P0{}); ++i; }
        if (i < n_steps) { step(P1{}); ++i; }
        if (i < n_steps) { step(P2{}); ++i; }
        // The last steps issued loads past the range (zero-size): let them land before the
        // workgroup can end and its LDS be reused.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // Store: the wave's own rows; lane l holds 16 consecutive d of row rw0 + l32 per
    // 32-wide block (the forward pass's O^T layout).
    const int row = rw0 + l32;
    if (row < p.Sq) {
        T* orow = (T*)p.dq + (own_head * p.Sq + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x16 a = acc1[db] * p.scale;
            const u32x4 w0 = {pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]),
                              pack2<BF16>(a[4], a[5]), pack2<BF16>(a[6], a[7])};
            const u32x4 w1 = {pack2<BF16>(a[8], a[9]), pack2<BF16>(a[10], a[11]),
                              pack2<BF16>(a[12], a[13]), pack2<BF16>(a[14], a[15])};
            *(u32x4*)(orow + db * 32 + 16 * h) = w0;
            *(u32x4*)(orow + db * 32 + 16 * h + 8) = w1;
        }
    }
}

// dK / dV with paired waves.  One wave holding 32 keys' K and V rows and both accumulators
// (dK^T and dV^T) needs more than 256 registers and so runs alone on its SIMD, where nothing
// hides the latency between a tile's products and the exp2 / dS work that depends on them.
// Here the same 32 keys are shared by two waves on one SIMD (waves kw and kw + 4 of an 8-wave
// workgroup), each with half of the work and half of the registers:
//  * role 0 holds K: S = Q K^T (started at -LSE / scale), P = exp2(c S), masks, writes P in
//    fp32 to LDS for its partner, and accumulates dV^T += dO^T P;
//  * role 1 holds V: dP = dO V^T (started at -D), reads its partner's P of the previous
//    tile, dS = P (dP - D), and accumulates dK^T += Q^T dS.
// Each role issues 16 of a tile's 32 MFMAs, and a step's two waves per SIMD overlap one's
// exp2 / dS work with the other's products.  Role 0 loads the Q tiles, role 1 the dO tiles
// (direct to LDS); wave 0 also loads the row statistics.  Role 1 works one tile behind role
// 0 (it needs the P that role 0 wrote in the previous step), so a tile stays in LDS for
// three steps: NB = 6 buffer sets, step j loads tile j + 4, ends by waiting for tile j + 2,
// and writes P(j) to one of two exchange buffers that role 1 reads in step j + 1.
template <int D, bool CAUSAL, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_pair_kernel(BwdParams p) {
    constexpr int NW = 4;                // waves per role
    constexpr int BR = 32;               // streamed rows per tile
    constexpr int DK = D / 16, DB = D / 32;
    constexpr int ROWB = D * 2, TILE = BR * ROWB, CPR = D / 8;
    constexpr int LDT = BR * CPR / (NW * 64);   // 16-byte chunks of its tile per lane
    constexpr int LOAD_STRIDE = NW * 64 * 16;
    constexpr int STB = BR * 8;
    constexpr int NB = 6;
    constexpr int XB = 64 * 64;          // one wave's P: 64 lanes x 16 fp32
    static_assert(BR * CPR % (NW * 64) == 0 && (64 * NW / CPR) % 16 == 0, "tile load layout");
    typedef uint16_t T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = w >> 2;             // 0: S, P, dV; 1: dP, dS, dK
    const int kw = w & 3;                // the 32-key block of the pair
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const int nh = p.Hkv * p.gsplit;
    const int wg = blockIdx.x;
    const int bh = wg % (p.B * nh);
    const int trank = wg / (p.B * nh);
    const int b = bh / nh;
    const int hx = bh - b * nh;
    const int head = hx / p.gsplit;
    const int gp = hx - head * p.gsplit;
    const int r0 = trank * 128;
    const int rw0 = r0 + kw * 32;
    const bool win = CAUSAL && p.window > 0;
    const int W = p.window;

    // Own rows (B operand): K for role 0, V for role 1.
    const int own_row = min(rw0 + l32, p.Skv - 1);
    const size_t own_head = (size_t)(b * p.Hkv + head);
    const T* xp = (const T*)(role == 0 ? p.k : p.v) + (own_head * p.Skv + own_row) * D;
    u32x4 x[DK];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) x[dk] = ((const u32x4*)xp)[dk * 2 + h];

    // Query tiles [qt0, qt1) of each of the workgroup's hpw query heads; [qa, qb) need no mask.
    const int k_last = min(r0 + 128, p.Skv) - 1;
    int lo = 0, hi = p.Sq - 1;
    if (CAUSAL) {
        lo = max(0, r0 - p.input_pos);
        if (win) hi = min(hi, k_last + W - 1 - p.input_pos);
    }
    const int qt0 = lo / BR;
    const int qt1 = hi < lo ? qt0 : hi / BR + 1;
    const int n_steps = (qt1 - qt0) * p.hpw;
    int qa, qb;
    {
        int a = qt0, e = min(qt1, p.Sq / BR);
        if (CAUSAL) {
            const int xx = r0 + 127 - p.input_pos;
            if (xx > 0) a = max(a, (xx + BR - 1) / BR);
        }
        if (win) {
            const int y = r0 - p.input_pos + W - 32;
            e = min(e, y < 0 ? 0 : y / BR + 1);
        }
        if (r0 + 128 > p.Skv) e = a;
        qa = min(a, qt1);
        qb = max(min(e, qt1), qa);
    }

    __shared__ __attribute__((aligned(16))) unsigned char t1_0[TILE], t1_1[TILE], t1_2[TILE], t1_3[TILE], t1_4[TILE], t1_5[TILE];
    __shared__ __attribute__((aligned(16))) unsigned char t2_0[TILE], t2_1[TILE], t2_2[TILE], t2_3[TILE], t2_4[TILE], t2_5[TILE];
    __shared__ __attribute__((aligned(16))) unsigned char st_0[STB], st_1[STB], st_2[STB], st_3[STB], st_4[STB], st_5[STB];
    __shared__ __attribute__((aligned(16))) unsigned char xp_0[NW * XB], xp_1[NW * XB];
    auto t1_of = [&](auto ph) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return t1_0;
        else if constexpr (P == 1) return t1_1;
        else if constexpr (P == 2) return t1_2;
        else if constexpr (P == 3) return t1_3;
        else if constexpr (P == 4) return t1_4;
        else return t1_5;
    };
    auto t2_of = [&](auto ph) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return t2_0;
        else if constexpr (P == 1) return t2_1;
        else if constexpr (P == 2) return t2_2;
        else if constexpr (P == 3) return t2_3;
        else if constexpr (P == 4) return t2_4;
        else return t2_5;
    };
    auto st_of = [&](auto ph) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return st_0;
        else if constexpr (P == 1) return st_1;
        else if constexpr (P == 2) return st_2;
        else if constexpr (P == 3) return st_3;
        else if constexpr (P == 4) return st_4;
        else return st_5;
    };
    auto xp_of = [&](auto par) FA_INLINE -> unsigned char* {
        constexpr int P = decltype(par)::value;
        if constexpr (P == 0) return xp_0 + kw * XB;
        else return xp_1 + kw * XB;
    };

    // Tile loads: role 0 fetches the Q tile, role 1 the dO tile; lane slot -> (row,
    // physical chunk), fetching the logical chunk the swizzle places there.  Rows past the
    // tensor's end read zero; steps past the last one load nothing (zero-size range).
    int src_off;
    {
        const int slot = kw * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        src_off = row * ROWB + ((pc ^ b_swz<D>(row)) << 4);
    }
    const T* src = (const T*)(role == 0 ? p.q : p.dout);
    int f_s = 0, f_qt = qt0;
    size_t f_slab = (size_t)(b * p.Hq + head * p.group + gp * p.hpw) * p.Sq;
    size_t st_row = 0;
    int st_rows = 0;
    auto fetch = [&](unsigned char* d1, unsigned char* d2) FA_INLINE {
        const int row0 = f_qt * BR;
        const int rows = f_s < n_steps ? min(p.Sq - row0, BR) : 0;
        const size_t first = rows > 0 ? f_slab + row0 : 0;
        const __amdgpu_buffer_rsrc_t r = make_rsrc_uniform(src + first * D, rows * ROWB);
        unsigned char* d = role == 0 ? d1 : d2;
#pragma unroll
        for (int i = 0; i < LDT; ++i) buffer_load_lds16(r, d + (i * NW + kw) * 1024, src_off, i * LOAD_STRIDE);
        st_row = first;
        st_rows = rows;
        ++f_s;
        if (++f_qt == qt1) {
            f_qt = qt0;
            f_slab += p.Sq;
        }
    };
    // Wave 0: the statistics of the tile fetched last, as two planes (32 x -LSE / scale,
    // 32 x -D) by the per-lane source offsets.
    auto fetch_stats = [&](unsigned char* ds) FA_INLINE {
        const __amdgpu_buffer_rsrc_t r = make_rsrc_uniform(p.stats + 2 * st_row, st_rows * 8);
        buffer_load_lds4(r, ds, lane < 32 ? lane * 8 : (lane - 32) * 8 + 4);
    };

    int off_r[DK];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) off_r[dk] = l32 * ROWB + (((2 * dk + h) ^ b_swz<D>(l32)) << 4);
    int off_t[2][DB];
    {
        const int vs = lane & 15, vj = vs >> 2, vq = vs & 3, vg = lane >> 4;
        const int row_in = 4 * (vg >> 1) + vj;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int row = row_in + 8 * rr;
                const int c = 4 * db + 2 * (vq & 1) + (vg & 1);
                off_t[rr][db] = row * ROWB + ((c ^ b_swz<D>(row)) << 4) + (vq >> 1) * 8;
            }
    }
    auto stat_init = [&](const unsigned char* st, int plane) FA_INLINE {
        f32x16 v;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 u = *(const f32x4*)(st + plane + (8 * g4 + 4 * h) * 4);
            v[4 * g4 + 0] = u[0];
            v[4 * g4 + 1] = u[1];
            v[4 * g4 + 2] = u[2];
            v[4 * g4 + 3] = u[3];
        }
        return v;
    };
    auto rows_mfma_init = [&](const unsigned char* tb_, f32x16 acc) FA_INLINE {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            const u32x4 a = *(const u32x4*)(tb_ + off_r[dk]);
            acc = mfma32<BF16>(a, x[dk], acc);
        }
        return acc;
    };
    // acc[db] += (tile^T)[32 d of block db] x (packed B operand), the tile read transposed.
    auto trans_mfma = [&](const unsigned char* tb_, const u32x4 (&pk)[2], f32x16 (&acc)[DB]) FA_INLINE {
        u32x4 y[DB][2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x2 y0 = lds_read_tr16(tb_ + 16 * hf * ROWB + off_t[0][db]);
                const u32x2 y1 = lds_read_tr16(tb_ + 16 * hf * ROWB + off_t[1][db]);
                y[db][hf] = (u32x4){y0[0], y0[1], y1[0], y1[1]};
            }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) acc[db] = mfma32<BF16>(y[db][hf], pk[hf], acc[db]);
    };
    auto pack16 = [&](const float (&e)[16], u32x4 (&pk)[2]) FA_INLINE {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const float* f = e + 8 * hf;
            pk[hf] = (u32x4){pack2<BF16>(f[0], f[1]), pack2<BF16>(f[2], f[3]), pack2<BF16>(f[4], f[5]),
                             pack2<BF16>(f[6], f[7])};
        }
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
    f32x16 sd0 = {}, sd1 = {};   // role 0: S of two consecutive tiles; role 1: dP

    auto wait_barrier = [&](auto n_tag) FA_INLINE {
        constexpr int N = decltype(n_tag)::value;
        static_assert(N < 64, "vmcnt range");
        constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
        asm volatile("s_waitcnt %0\n\ts_barrier" ::"n"(imm) : "memory");
    };
    // End of a step: role 0 waits for its P writes (lgkmcnt) so that role 1 reads them
    // after the barrier; every wave waits until only the newest two tiles' loads are in
    // flight (tile j + 2 has landed), then the barrier.
    auto end_step = [&](auto pf) FA_INLINE {
        if (role == 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (w == 0) {
            fetch_stats(st_of(pf));
            wait_barrier(std::integral_constant<int, 2 * (LDT + 1)>{});
        } else {
            wait_barrier(std::integral_constant<int, 2 * LDT>{});
        }
    };

    // Role 0, step j (phase PH = j mod 6): loads tile j + 4; S(j + 1); P(j), written for the
    // partner; dV^T += dO(j)^T P(j).
    int c_qt = qt0;
    auto step0 = [&](auto ph_tag) FA_INLINE {
        constexpr int PH = decltype(ph_tag)::value;
        using PN = std::integral_constant<int, (PH + 1) % NB>;
        using PF = std::integral_constant<int, (PH + 4) % NB>;
        using PC = std::integral_constant<int, PH>;
        using PX = std::integral_constant<int, PH & 1>;
        f32x16& sc = (PH & 1) ? sd1 : sd0;
        f32x16& scn = (PH & 1) ? sd0 : sd1;
        const bool masked = c_qt < qa || c_qt >= qb;
        const int c_row0 = c_qt * BR;

        fetch(t1_of(PF{}), t2_of(PF{}));
        scn = rows_mfma_init(t1_of(PN{}), stat_init(st_of(PN{}), 0));
        float pe[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pe[i] = __builtin_amdgcn_exp2f(sc[i] * p.c);
        if (masked) {
            const int base = c_row0 + 4 * h;
            const int own = rw0 + l32;
            int lo_ = 0, hi_ = p.Sq - base;
            if (CAUSAL) lo_ = own - p.input_pos - base;
            if (win) hi_ = min(hi_, own - p.input_pos - base + W);
            if (own >= p.Skv) hi_ = 0;
            lo_ = min(max(lo_, 0), 32);
            hi_ = min(max(hi_, 0), 32);
            const uint32_t below_hi = hi_ >= 32 ? ~0u : (1u << hi_) - 1u;
            const uint32_t below_lo = lo_ >= 32 ? ~0u : (1u << lo_) - 1u;
            const uint32_t vis = hi_ > lo_ ? below_hi & ~below_lo : 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vis, 8 * (i >> 2) + (i & 3), 1);
                pe[i] = __uint_as_float(__float_as_uint(pe[i]) & keep);
            }
        }
        unsigned char* xb = xp_of(PX{});
        u32x4 pk[2];
        pack16(pe, pk);
        __builtin_amdgcn_sched_barrier(0);
        trans_mfma(t2_of(PC{}), pk, acc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *(f32x4*)(xb + c * 1024 + lane * 16) = (f32x4){pe[4 * c], pe[4 * c + 1], pe[4 * c + 2], pe[4 * c + 3]};
        end_step(PF{});
        if (++c_qt == qt1) c_qt = qt0;
    };
    // Role 1, step j: loads tile j + 4; dP(j); with DO_DK, dS(j - 1) = P(j - 1) (dP - D)
    // and dK^T += Q(j - 1)^T dS(j - 1).
    auto step1 = [&](auto ph_tag, auto dk_tag) FA_INLINE {
        constexpr int PH = decltype(ph_tag)::value;
        constexpr bool DO_DK = decltype(dk_tag)::value;
        using PP = std::integral_constant<int, (PH + NB - 1) % NB>;
        using PF = std::integral_constant<int, (PH + 4) % NB>;
        using PC = std::integral_constant<int, PH>;
        using PXP = std::integral_constant<int, (PH + 1) & 1>;
        f32x16& dpc = (PH & 1) ? sd1 : sd0;
        f32x16& dpp = (PH & 1) ? sd0 : sd1;

        fetch(t1_of(PF{}), t2_of(PF{}));
        dpc = rows_mfma_init(t2_of(PC{}), stat_init(st_of(PC{}), 128));
        if constexpr (DO_DK) {
            const unsigned char* xb = xp_of(PXP{});
            float de[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 pv = *(const f32x4*)(xb + c * 1024 + lane * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) de[4 * c + e] = pv[e] * dpp[4 * c + e];
            }
            u32x4 dsk[2];
            pack16(de, dsk);
            __builtin_amdgcn_sched_barrier(0);
            trans_mfma(t1_of(PP{}), dsk, acc);
        }
        end_step(PF{});
    };

    if (n_steps > 0) {
        // Prologue: tiles 0..3 in flight, wait for 0 and 1; role 0 computes S(0).
        static_for<4>([&](auto ph) FA_INLINE {
            fetch(t1_of(ph), t2_of(ph));
            if (w == 0) fetch_stats(st_of(ph));
        });
        if (w == 0) wait_barrier(std::integral_constant<int, 2 * (LDT + 1)>{});
        else wait_barrier(std::integral_constant<int, 2 * LDT>{});
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        using P3 = std::integral_constant<int, 3>;
        using P4 = std::integral_constant<int, 4>;
        using P5 = std::integral_constant<int, 5>;
        using Y = std::true_type;
        using N = std::false_type;
        if (role == 0) {
            sd0 = rows_mfma_init(t1_0, stat_init(st_0, 0));
            int i = 0;
            for (; i + NB - 1 < n_steps; i += NB) {
                step0(P0{}); step0(P1{}); step0(P2{}); step0(P3{}); step0(P4{}); step0(P5{});
            }
            if (i < n_steps) { step0(P0{}); ++i; }
            if (i < n_steps) { step0(P1{}); ++i; }
            if (i < n_steps) { step0(P2{}); ++i; }
            if (i < n_steps) { step0(P3{}); ++i; }
            if (i < n_steps) { step0(P4{}); ++i; }
        } else {
            step1(P0{}, N{});
            int i = 1;
            for (; i + NB - 1 < n_steps; i += NB) {
                step1(P1{}, Y{}); step1(P2{}, Y{}); step1(P3{}, Y{}); step1(P4{}, Y{}); step1(P5{}, Y{}); step1(P0{}, Y{});
            }
            if (i < n_steps) { step1(P1{}, Y{}); ++i; }
            if (i < n_steps) { step1(P2{}, Y{}); ++i; }
            if (i < n_steps) { step1(P3{}, Y{}); ++i; }
            if (i < n_steps) { step1(P4{}, Y{}); ++i; }
            if (i < n_steps) { step1(P5{}, Y{}); ++i; }
            // The last tile's dS and dK product (its P was written before the last barrier).
            const int jl = n_steps - 1;
            const int pl = jl % NB;
            const unsigned char* tq = pl == 0 ? t1_0 : pl == 1 ? t1_1 : pl == 2 ? t1_2 : pl == 3 ? t1_3 : pl == 4 ? t1_4 : t1_5;
            const unsigned char* xb = ((jl & 1) ? xp_1 : xp_0) + kw * XB;
            const f32x16 dpl = (jl & 1) ? sd1 : sd0;
            float de[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 pv = *(const f32x4*)(xb + c * 1024 + lane * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) de[4 * c + e] = pv[e] * dpl[4 * c + e];
            }
            u32x4 dsk[2];
            pack16(de, dsk);
            trans_mfma(tq, dsk, acc);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // Store: role 0 dV, role 1 dK (scaled); lane l holds 16 consecutive d of key rw0 + l32
    // per 32-wide block.
    const int row = rw0 + l32;
    if (row < p.Skv) {
        if (p.gsplit == 1) {
            T* orow = (T*)(role == 0 ? p.dv : p.dk) + (own_head * p.Skv + row) * D;
            const float mul = role == 0 ? 1.0f : p.scale;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x16 a = acc[db] * mul;
                const u32x4 w0 = {pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]),
                                  pack2<BF16>(a[4], a[5]), pack2<BF16>(a[6], a[7])};
                const u32x4 w1 = {pack2<BF16>(a[8], a[9]), pack2<BF16>(a[10], a[11]),
                                  pack2<BF16>(a[12], a[13]), pack2<BF16>(a[14], a[15])};
                *(u32x4*)(orow + db * 32 + 16 * h) = w0;
                *(u32x4*)(orow + db * 32 + 16 * h + 8) = w1;
            }
        } else {
            const size_t n = (size_t)p.B * p.Hkv * p.Skv * D;
            float* orow = p.part + (size_t)(2 * gp + (role == 0 ? 1 : 0)) * n + (own_head * p.Skv + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    *(f32x4*)(orow + db * 32 + 16 * h + 4 * v4) =
                        (f32x4){acc[db][4 * v4], acc[db][4 * v4 + 1], acc[db][4 * v4 + 2], acc[db][4 * v4 + 3]};
        }
    }
}

}  // namespace fa
