// fa_bwd_kernel.hpp -- gfx950 (MI355X) backward pass of the attention forward kernel.
//
// Gradients of O = softmax(scale Q K^T + M) V for an upstream gradient dO.  The pages name
// the backward pass only as future work ("How I Beat PyTorch's Flash Attention", "Future
// work"); the formulas are the textbook softmax derivative, recomputing P from the LSE the
// forward pass returns instead of storing it:
//     P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),
//     dS = P * (dP - D),       dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, no atomics, deterministic:
//  * fa_bwd_dot_kernel:  D_i = dO_i . O_i (fp32), one wave per row.
//  * fa_bwd_kernel<DKDV>: a wave owns 32 keys of one K/V head (K and V rows in registers);
//    the workgroup streams 32-row tiles of Q and dO of every query head of the GQA group
//    through LDS and accumulates dK^T and dV^T in registers -- the grouped heads' sum
//    happens in place.
//  * fa_bwd_kernel<DQ>: a wave owns 32 query rows (Q and dO rows in registers); the
//    workgroup streams 32-key tiles of K and V and accumulates dQ^T.
// Both use the forward kernel's MFMA formulation: the streamed tile is the A operand of
// v_mfma_f32_32x32x16 (row reads from LDS), the wave's own rows are the B operand, so the
// 32x32 accumulator gives each lane one of its own rows and 16 streamed rows; P and dS go
// from that accumulator straight into the B operand of the second product, whose A
// operand is the streamed tile transposed (ds_read_b64_tr_b16).  Since each streamed tile
// is read both ways, its LDS layout uses one XOR swizzle of the 16-byte chunks that a
// bank model finds conflict-free for both the row reads and the transposed reads.
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
    const float* dvec;   // D = rowsum(dO * O), fp32 [B*Hq*Sq]
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, Sq, Skv;
    int causal, input_pos, window;   // window > 0 only with causal
    float c;                         // scale * log2(e)
    float scale;
    int group;                       // Hq / Hkv
    int n_tiles;                     // 128-row blocks per head (queries for DQ, keys for DKDV)
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
__device__ __forceinline__ float half_to_f32(uint16_t x) {
    if constexpr (BF16) return __uint_as_float((uint32_t)x << 16);
    else return (float)__builtin_bit_cast(_Float16, x);
}

// D_i = sum_d dO[i][d] * O[i][d] in fp32; rows = B*Hq*Sq; 4 rows per 256-thread block.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_dot_kernel(const void* o, const void* dout, float* dvec,
                                                         int rows) {
    constexpr int PER = D / 64;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const uint16_t* op = (const uint16_t*)o + (size_t)row * D + lane * PER;
    const uint16_t* dp = (const uint16_t*)dout + (size_t)row * D + lane * PER;
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc += half_to_f32<BF16>(op[e]) * half_to_f32<BF16>(dp[e]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) dvec[row] = acc;
}

enum BwdMode { BWD_DQ = 0, BWD_DKDV = 1 };

template <int D, bool CAUSAL, bool BF16, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(MODE == BWD_DQ ? 2 : 1, MODE == BWD_DQ ? 2 : 1)))
void fa_bwd_kernel(BwdParams p) {
    constexpr int NT = 256, NW = 4;
    constexpr int BR = 32;               // streamed rows per tile
    constexpr int DK = D / 16, DB = D / 32;
    constexpr int ROWB = D * 2, TILE = BR * ROWB, CPR = D / 8;
    constexpr int LD = BR * CPR / NT;    // 16-byte chunks of a tile per thread
    constexpr int LOAD_STRIDE = NT * 16;
    static_assert(BR * CPR % NT == 0 && (64 * NW / CPR) % 16 == 0, "tile load layout");
    constexpr bool DKDV = MODE == BWD_DKDV;
    typedef uint16_t T;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // Workgroup -> (batch, head, 128-row block); causal: the heaviest blocks first.
    const int nh = DKDV ? p.Hkv : p.Hq;
    const int wg = blockIdx.x;
    const int bh = wg % (p.B * nh);
    const int trank = wg / (p.B * nh);
    const int b = bh / nh, head = bh - b * nh;
    const int blk = CAUSAL ? (DKDV ? trank : p.n_tiles - 1 - trank) : trank;
    const int r0 = blk * 128;                 // first own row of the workgroup
    const int rw0 = r0 + w * 32;              // first own row of the wave
    const bool win = CAUSAL && p.window > 0;

    // Own rows (B operands): DQ: Q and dO rows of query head `head`; DKDV: K and V rows.
    const int n_own = DKDV ? p.Skv : p.Sq;
    const int own_row = min(rw0 + l32, n_own - 1);
    const size_t own_head = DKDV ? (size_t)(b * p.Hkv + head) : (size_t)(b * p.Hq + head);
    const T* x1p = (const T*)(DKDV ? p.k : p.q) + (own_head * n_own + own_row) * D;
    const T* x2p = (const T*)(DKDV ? p.v : p.dout) + (own_head * n_own + own_row) * D;
    u32x4 x1[DK], x2[DK];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
        x1[dk] = ((const u32x4*)x1p)[dk * 2 + h];
        x2[dk] = ((const u32x4*)x2p)[dk * 2 + h];
    }
    // DQ: the lane's query row statistics (LSE in the exp2 domain, +inf for an empty row
    // so that p = 0; and D).
    float lse2_own = 0.0f, d_own = 0.0f;
    if constexpr (!DKDV) {
        const size_t rr = (size_t)(b * p.Hq + head) * p.Sq + own_row;
        const float l = p.lse[rr];
        lse2_own = l == -__builtin_inff() ? __builtin_inff() : l * 1.44269504088896340736f;
        d_own = p.dvec[rr];
    }

    // Streamed tiles: DQ: K (t1) and V (t2) of head `head / group`; DKDV: Q (t1) and dO
    // (t2) of each query head of the group.  Steps s = 0 .. n_steps-1.
    int n_steps, s_first;   // DQ: key tiles [s_first, s_first + n_steps); DKDV: see below
    int qt0 = 0, qt1 = 0;   // DKDV: query tiles [qt0, qt1) per head
    const int kv_head = DKDV ? head : head / p.group;
    if constexpr (!DKDV) {
        const int q_last = min(r0 + 128, p.Sq) - 1;
        const int Tc = CAUSAL ? (min(p.input_pos + q_last + 1, p.Skv) + BR - 1) / BR
                              : (p.Skv + BR - 1) / BR;
        const int tb = win ? min(max(0, p.input_pos + r0 - p.window + 1) / BR, Tc) : 0;
        s_first = tb;
        n_steps = Tc - tb;
    } else {
        // Query rows that see some key of [r0, min(r0 + 128, Skv)).
        const int k_last = min(r0 + 128, p.Skv) - 1;
        int lo = 0, hi = p.Sq - 1;
        if (CAUSAL) {
            lo = max(0, r0 - p.input_pos);
            if (win) hi = min(hi, k_last + p.window - 1 - p.input_pos);
        }
        qt0 = lo / BR;
        qt1 = hi < lo ? qt0 : hi / BR + 1;
        s_first = 0;
        n_steps = (qt1 - qt0) * p.group;
    }

    __shared__ __attribute__((aligned(16))) unsigned char t1_lds0[TILE], t1_lds1[TILE];
    __shared__ __attribute__((aligned(16))) unsigned char t2_lds0[TILE], t2_lds1[TILE];

    // Tile loads (direct to LDS): lane slot -> (row, physical chunk); it fetches the
    // logical chunk the swizzle places there.  Rows past the tensor's end read zero.
    int src_off;
    {
        const int slot = w * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        src_off = row * ROWB + ((pc ^ b_swz<D>(row)) << 4);
    }
    // Step s -> (tile start row, head slab) of the streamed tensors.
    auto tile_of = [&](int s, int& row0, size_t& slab) FA_INLINE {
        if constexpr (!DKDV) {
            row0 = (s_first + s) * BR;
            slab = (size_t)(b * p.Hkv + kv_head) * p.Skv;
        } else {
            const int nq = qt1 - qt0;
            const int hl = s / nq;
            row0 = (qt0 + (s - hl * nq)) * BR;
            slab = (size_t)(b * p.Hq + kv_head * p.group + hl) * p.Sq;
        }
    };
    const int n_stream = DKDV ? p.Sq : p.Skv;
    auto fetch = [&](int s, unsigned char* d1, unsigned char* d2) FA_INLINE {
        int row0;
        size_t slab;
        tile_of(s, row0, slab);
        const int rows = max(0, min(n_stream - row0, BR));
        const T* s1 = (const T*)(DKDV ? p.q : p.k) + (slab + min(row0, n_stream)) * D;
        const T* s2 = (const T*)(DKDV ? p.dout : p.v) + (slab + min(row0, n_stream)) * D;
        const __amdgpu_buffer_rsrc_t r1 = make_rsrc(s1, rows * ROWB);
        const __amdgpu_buffer_rsrc_t r2 = make_rsrc(s2, rows * ROWB);
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            buffer_load_lds16(r1, d1 + (i * NW + w) * 1024, src_off, i * LOAD_STRIDE);
            buffer_load_lds16(r2, d2 + (i * NW + w) * 1024, src_off, i * LOAD_STRIDE);
        }
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
    auto rows_mfma = [&](const unsigned char* tb, const u32x4 (&x)[DK]) FA_INLINE {
        f32x16 acc = {};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            const u32x4 a = *(const u32x4*)(tb + off_r[dk]);
            acc = mfma32<BF16>(a, x[dk], acc);
        }
        return acc;
    };
    auto trans_mfma = [&](const unsigned char* tb, const u32x4 (&pk)[2], f32x16 (&acc)[DB]) FA_INLINE {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x2 y0 = lds_read_tr16(tb + 16 * hf * ROWB + off_t[0][db]);
                const u32x2 y1 = lds_read_tr16(tb + 16 * hf * ROWB + off_t[1][db]);
                const u32x4 a = {y0[0], y0[1], y1[0], y1[1]};
                acc[db] = mfma32<BF16>(a, pk[hf], acc[db]);
            }
    };

    f32x16 acc1[DB], acc2[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        acc1[db] = (f32x16){};
        acc2[db] = (f32x16){};
    }

    auto step = [&](int s, const unsigned char* t1, const unsigned char* t2) FA_INLINE {
        int row0;
        size_t slab;
        tile_of(s, row0, slab);
        // DKDV: the statistics of the 16 streamed rows this lane holds.
        float lse2[16], dv16[16];
        if constexpr (DKDV) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = min(row0 + 8 * g4 + 4 * h + e, p.Sq - 1);
                    const float l = p.lse[slab + r];
                    lse2[4 * g4 + e] = l == -__builtin_inff() ? __builtin_inff() : l * 1.44269504088896340736f;
                    dv16[4 * g4 + e] = p.dvec[slab + r];
                }
            }
        }
        f32x16 sc = rows_mfma(t1, x1);    // DQ: S^T (lane = query); DKDV: S (lane = key)
        f32x16 dp = rows_mfma(t2, x2);    // DQ: dP^T; DKDV: dP
        // Mask: streamed row index and own row index of each element.
        const int own = rw0 + l32;
        u32x4 pk[2], dsk[2];
        float pe[16], de[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int sr = row0 + 8 * (i >> 2) + 4 * h + (i & 3);   // streamed row
            const int qrow = DKDV ? sr : own;
            const int key = DKDV ? own : sr;
            bool vis = key < p.Skv && qrow < p.Sq;
            if (CAUSAL) {
                vis = vis && key <= p.input_pos + qrow;
                if (win) vis = vis && key >= p.input_pos + qrow - p.window + 1;
            }
            const float l2 = DKDV ? lse2[i] : lse2_own;
            const float dd = DKDV ? dv16[i] : d_own;
            const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c, -l2)) : 0.0f;
            pe[i] = pv;
            de[i] = pv * (dp[i] - dd);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const float* e = pe + 8 * hf;
            const float* f = de + 8 * hf;
            pk[hf] = (u32x4){pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]), pack2<BF16>(e[4], e[5]),
                             pack2<BF16>(e[6], e[7])};
            dsk[hf] = (u32x4){pack2<BF16>(f[0], f[1]), pack2<BF16>(f[2], f[3]), pack2<BF16>(f[4], f[5]),
                              pack2<BF16>(f[6], f[7])};
        }
        trans_mfma(t1, dsk, acc1);        // DQ: dQ^T += K^T dS^T; DKDV: dK^T += Q^T dS
        if constexpr (DKDV) trans_mfma(t2, pk, acc2);   // dV^T += dO^T P
    };

    if (n_steps > 0) {
        fetch(0, t1_lds0, t2_lds0);
        __syncthreads();
        int s = 0;
        for (; s + 1 < n_steps; s += 2) {
            fetch(s + 1, t1_lds1, t2_lds1);
            step(s, t1_lds0, t2_lds0);
            __syncthreads();
            if (s + 2 < n_steps) fetch(s + 2, t1_lds0, t2_lds0);
            step(s + 1, t1_lds1, t2_lds1);
            __syncthreads();
        }
        if (s < n_steps) step(s, t1_lds0, t2_lds0);
    }

    // Store: the wave's own rows; lane l holds 16 consecutive d of row rw0 + l32 per
    // 32-wide block (the forward pass's O^T layout).
    const int row = rw0 + l32;
    if (row < n_own) {
        auto store = [&](void* base, size_t head_rows, const f32x16 (&acc)[DB], float mul) FA_INLINE {
            T* orow = (T*)base + (head_rows * n_own + row) * D;
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
        };
        if constexpr (DKDV) {
            store(p.dk, own_head, acc1, p.scale);
            store(p.dv, own_head, acc2, 1.0f);
        } else {
            store(p.dq, own_head, acc1, p.scale);
        }
    }
}

}  // namespace fa
