// fa_fwd_kernel.hpp -- gfx950 (MI355X) FlashAttention-style forward kernel.
//
// What is computed follows "Tuning Flash Attention for peak performance in NVIDIA CUDA
// Tile" (NVIDIA cuTile post), Part 1: a workgroup owns a tile of query rows, keeps them
// resident, streams K/V tiles through on-chip memory, and folds every tile into a running
// row max m, row sum l and fp32 accumulator ("Understanding online softmax", "Online
// softmax update"), normalising once at the end ("Final normalization and store").
// Causal tiles past the diagonal are never visited and only diagonal/tail tiles build a
// mask (Part 2 "K-loop split"); heavy causal tiles are launched first (Part 2 "ProgramId
// remapping"); exp2 is used with log2(e) folded into the scale (Part 1 "Initializing
// accumulators"; "How I Beat PyTorch's Flash Attention", "Phase 4").
//
// The CDNA4 design (not the pages' sm_80/Blackwell one):
//  * A wave owns 32*QB query rows of one head.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_{f16,bf16}: K is the A operand (from LDS),
//    the wave's queries are the B operand (held in VGPRs for the whole loop).  In the
//    32x32 accumulator lane l holds 16 keys of query (l mod 32), so a row max / row sum
//    is an in-lane reduction plus one v_permlane32_swap with lane l^32.
//  * The output is accumulated transposed too, O^T += V^T P^T.  The accumulator layout of
//    S^T is exactly the B-operand layout P^T needs (keys 16*half + 8*(j/4) + 4*(l/32) +
//    j%4 in slot j), so P goes from exp2 straight into the PV MFMA with no LDS round trip.
//    V^T comes from LDS, where each V tile is stored transposed (d-major) with its rows
//    in MFMA order, so each lane's 16 output values are 16 consecutive d (two 128-bit
//    stores).
//  * K/V tiles are double-buffered in LDS through registers: tile j+1 is fetched from
//    HBM with 128-bit loads while tile j is computed.  Both LDS layouts are XOR-swizzled
//    so the MFMA operand reads and the tile writes are bank-conflict free.
//  * The running max is rescaled lazily: m is only raised (and acc, l rescaled) when some
//    row's max grows by more than 2^8 in the exp2 domain; otherwise the stale max is
//    kept.  softmax is invariant to the shift, p stays <= 2^8, and the normalisation at
//    the end uses the same m for acc and l, so the result is the same softmax.
//  * A workgroup is HPW heads x WPH position blocks.  HPW > 1 packs query heads of one
//    GQA group into a workgroup: they share every K/V tile ("Grouped-query attention").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Kernel arguments (one struct, passed by value).
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Sq, Skv;
    int input_pos;   // causal: query i sits at position input_pos + i
    float c;         // scale * log2(e): exp(scale*s - m) = exp2(c*s - m')
    int group;       // Hq / Hkv
    int n_tiles;     // query tiles per (batch, head group)
    int n_hgroups;   // Hq / HPW
};

// Compile-time configuration of one kernel instance.
template <int D_, int BN_, int QB_, int WPH_, int HPW_, bool CAUSAL_, bool BF16_>
struct Cfg {
    static constexpr int D = D_;        // head dim
    static constexpr int BN = BN_;      // keys per K/V tile
    static constexpr int QB = QB_;      // 32-row query blocks per wave
    static constexpr int WPH = WPH_;    // waves per head (along positions)
    static constexpr int HPW = HPW_;    // heads per workgroup
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr bool BF16 = BF16_;
    static constexpr int NW = WPH * HPW;
    static constexpr int NT = 64 * NW;
    static constexpr int BMP = 32 * QB * WPH;   // query positions per workgroup
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN == 64 || BN == 128, "key tile");
    static_assert(QB == 1 || QB == 2, "query blocks per wave");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value over lanes l and l^32 (the two halves hold the same query).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> one packed pair of the storage type, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2 x = {a, b};
    if constexpr (BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
    }
}

// D(32x32, fp32) += A(32x16) * B(16x32): A rows / B columns are lane mod 32; the 8
// k-elements of a lane are its half (lane / 32) of the k-range, same order in A and B.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Low / high 16-bit halves of x (low half of the result) and y (high half).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// --- LDS layouts -----------------------------------------------------------------------
// K tile: [BN][D] row-major, 16-byte chunks XOR-swizzled by (row mod 8).
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk16) {
    return row * (D * 2) + ((chunk16 ^ (row & 7)) << 4);
}
// V^T tile: [D][BN]; row R holds d = vt_row_to_d(R) so that MFMA row m of output block db
// is d = db*32 + 16*(m/4 mod 2) + 4*(m/8) + m%4, i.e. a lane's accumulator values are 16
// consecutive d.  8-byte chunks (4 keys) are XOR-swizzled per row.
__device__ __forceinline__ int d_to_vt_row(int d) {
    const int x = d & 31;                // x = 16*hh + 4*g + e
    const int hh = x >> 4, g = (x >> 2) & 3, e = x & 3;
    return (d & ~31) | (g << 3) | (hh << 2) | e;
}
template <int BN>
__device__ __forceinline__ int vt_swz(int R) {
    const int u = (R >> 4) & 7;
    const int phi = (u & 3) | ((u & 4) << 1);
    return ((R & 15) ^ phi) & (BN / 4 - 1);
}
template <int BN>
__device__ __forceinline__ int vt_off(int R, int chunk8) {
    return R * (BN * 2) + ((chunk8 ^ vt_swz<BN>(R)) << 3);
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::NT, C::NT), amdgpu_waves_per_eu(1, 1)))
void fa_fwd_kernel(Params p) {
    constexpr int D = C::D, BN = C::BN, QB = C::QB, NT = C::NT, WPH = C::WPH, HPW = C::HPW;
    constexpr bool CAUSAL = C::CAUSAL, BF16 = C::BF16;
    constexpr int KB = BN / 32;          // 32-key blocks per tile
    constexpr int DK = D / 16;           // k-steps of Q K^T
    constexpr int DB = D / 32;           // 32-wide d blocks of O
    constexpr int K_BYTES = BN * D * 2;
    constexpr int BUF = 2 * K_BYTES;     // K tile + V^T tile
    constexpr int KCH = BN * D / 8;      // 16-byte chunks per K tile
    constexpr int KLD = KCH / NT;
    constexpr int VBL = (BN / 4) * (D / 8);   // 4-key x 8-d blocks per V tile
    constexpr int VLD = (VBL + NT - 1) / NT;
    constexpr float TAU = 8.0f;          // lazy-rescale threshold (log2 domain)
    constexpr float LN2 = 0.69314718055994530942f;
    static_assert(KCH % NT == 0, "K tile chunks per thread");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // Workgroup -> (query tile, batch, head group).  Causal: heaviest tiles first.
    const int bg = p.B * p.n_hgroups;
    int tile = blockIdx.x / bg;
    const int rem = blockIdx.x - tile * bg;
    if (CAUSAL) tile = p.n_tiles - 1 - tile;
    const int b = rem / p.n_hgroups;
    const int hg = rem - b * p.n_hgroups;
    const int hq = hg * HPW + w / WPH;
    const int kvh = (hg * HPW) / p.group;
    const int q0 = tile * C::BMP;
    const int qw0 = q0 + (w % WPH) * (32 * QB);

    typedef uint16_t T;
    const T* qp = (const T*)p.q + (size_t)(b * p.Hq + hq) * p.Sq * D;
    const T* kp = (const T*)p.k + (size_t)(b * p.Hkv + kvh) * p.Skv * D;
    const T* vp = (const T*)p.v + (size_t)(b * p.Hkv + kvh) * p.Skv * D;

    // Queries of this wave, as the B operand of S^T = K Q^T: lane l holds row l%32 of
    // query block qb, elements dk*16 + 8*(l/32) .. +8.
    u32x4 qf[QB][DK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + qb * 32 + l32;
        const u32x4* src = (const u32x4*)(qp + (size_t)row * D);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            qf[qb][dk] = row < p.Sq ? src[dk * 2 + h] : (u32x4){0u, 0u, 0u, 0u};
        }
    }

    // Loop bounds.  Workgroup: Tc tiles.  Wave: tiles >= wave_tc are fully masked for
    // its rows; tiles >= wave_ms need the mask (diagonal or key tail).
    const int q_last = min(q0 + C::BMP, p.Sq) - 1;
    const int Tc = CAUSAL ? (min(p.input_pos + q_last + 1, p.Skv) + BN - 1) / BN
                          : (p.Skv + BN - 1) / BN;
    const int qw_last = min(qw0 + 32 * QB, p.Sq) - 1;
    int wave_tc;
    if (qw_last < qw0) {
        wave_tc = 0;
    } else if (CAUSAL) {
        wave_tc = (min(p.input_pos + qw_last + 1, p.Skv) + BN - 1) / BN;
    } else {
        wave_tc = Tc;
    }
    const int wave_ms = CAUSAL ? min((p.input_pos + qw0) / BN, p.Skv / BN) : p.Skv / BN;

    // Running state: m (exp2 domain, possibly stale), l, acc (= O^T blocks).
    float m_run[QB], l_run[QB];
    f32x16 acc[DB][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -__builtin_inff();
        l_run[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] = (f32x16){};
    }

    // Register staging of the next tile.
    u32x4 kreg[KLD];
    u32x4 vreg[VLD][4];

    auto fetch = [&](int j) {
        const int j0 = j * BN;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int cid = tid + i * NT;
            const int row = cid / (D / 8), c = cid % (D / 8);
            const int key = j0 + row;
            kreg[i] = key < p.Skv ? *(const u32x4*)(kp + (size_t)key * D + c * 8)
                                  : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int bid = tid + i * NT;
            if (VBL % NT == 0 || bid < VBL) {
                const int c = bid % (D / 8), r = bid / (D / 8);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int key = j0 + 4 * r + kk;
                    vreg[i][kk] = key < p.Skv ? *(const u32x4*)(vp + (size_t)key * D + c * 8)
                                              : (u32x4){0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto stash = [&](int buf) {
        unsigned char* kb = smem + buf * BUF;
        unsigned char* vb = kb + K_BYTES;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int cid = tid + i * NT;
            const int row = cid / (D / 8), c = cid % (D / 8);
            *(u32x4*)(kb + k_off<D>(row, c)) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int bid = tid + i * NT;
            if (VBL % NT == 0 || bid < VBL) {
                const int c = bid % (D / 8), r = bid / (D / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int wd = e >> 1;
                    uint32_t lo, hi;
                    if (e & 1) {
                        lo = pack_hi16(vreg[i][0][wd], vreg[i][1][wd]);
                        hi = pack_hi16(vreg[i][2][wd], vreg[i][3][wd]);
                    } else {
                        lo = pack_lo16(vreg[i][0][wd], vreg[i][1][wd]);
                        hi = pack_lo16(vreg[i][2][wd], vreg[i][3][wd]);
                    }
                    const int R = d_to_vt_row(8 * c + e);
                    *(u32x2*)(vb + vt_off<BN>(R, r)) = (u32x2){lo, hi};
                }
            }
        }
    };

    auto compute = [&](int j, int buf, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const unsigned char* kb = smem + buf * BUF;
        const unsigned char* vb = kb + K_BYTES;

        // S^T = K Q^T for this tile.
        f32x16 s[KB][QB];
#pragma unroll
        for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb2][qb] = (f32x16){};
            const int row = kb2 * 32 + l32;
#pragma unroll
            for (int dk = 0; dk < DK; ++dk) {
                const u32x4 a = *(const u32x4*)(kb + k_off<D>(row, 2 * dk + h));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[kb2][qb] = mfma32<BF16>(a, qf[qb][dk], s[kb2][qb]);
            }
        }

        if constexpr (MASKED) {
            const int j0 = j * BN;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qpos = p.input_pos + qw0 + qb * 32 + l32;
#pragma unroll
                for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = j0 + kb2 * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                        const bool vis = key < p.Skv && (!CAUSAL || key <= qpos);
                        if (!vis) s[kb2][qb][i] = -__builtin_inff();
                    }
                }
            }
        }

        // Online softmax update per query block.
        u32x4 pk[KB][QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][qb][i]);
            mx = xhalf_max(mx);
            const float m_new = fmaxf(m_run[qb], mx * p.c);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run[qb] + TAU) != 0) {
                const float alpha = fast_exp2(m_run[qb] - m_new);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
            }
            const float neg_m = -m_run[qb];
            float ls = 0.0f;
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = fast_exp2(__builtin_fmaf(s[kb2][qb][i], p.c, neg_m));
                    s[kb2][qb][i] = pv;
                    ls += pv;
                }
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    pk[kb2][qb][hf] = (u32x4){
                        pack2<BF16>(s[kb2][qb][8 * hf + 0], s[kb2][qb][8 * hf + 1]),
                        pack2<BF16>(s[kb2][qb][8 * hf + 2], s[kb2][qb][8 * hf + 3]),
                        pack2<BF16>(s[kb2][qb][8 * hf + 4], s[kb2][qb][8 * hf + 5]),
                        pack2<BF16>(s[kb2][qb][8 * hf + 6], s[kb2][qb][8 * hf + 7])};
                }
            }
            l_run[qb] += xhalf_sum(ls);
        }

        // O^T += V^T P^T.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int R = db * 32 + l32;
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int ch0 = kb2 * 8 + 4 * hf + h;
                    const u32x2 x0 = *(const u32x2*)(vb + vt_off<BN>(R, ch0));
                    const u32x2 x1 = *(const u32x2*)(vb + vt_off<BN>(R, ch0 + 2));
                    const u32x4 a = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = mfma32<BF16>(a, pk[kb2][qb][hf], acc[db][qb]);
                }
            }
        }
    };

    fetch(0);
    stash(0);
    __syncthreads();
    for (int j = 0; j < Tc; ++j) {
        const int buf = j & 1;
        if (j + 1 < Tc) fetch(j + 1);
        if (j < wave_tc) {
            if (j >= wave_ms) compute(j, buf, std::true_type{});
            else compute(j, buf, std::false_type{});
        }
        if (j + 1 < Tc) stash(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = acc / l (v_rcp_f32), rounded to the storage type; LSE = ln2 (m + log2 l).
    T* op = (T*)p.o + (size_t)(b * p.Hq + hq) * p.Sq * D;
    float* lp = p.lse + (size_t)(b * p.Hq + hq) * p.Sq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + qb * 32 + l32;
        if (row < p.Sq) {
            const float inv = __builtin_amdgcn_rcpf(l_run[qb]);
            T* orow = op + (size_t)row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x16 a = acc[db][qb] * inv;
                const u32x4 w0 = {pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]),
                                  pack2<BF16>(a[4], a[5]), pack2<BF16>(a[6], a[7])};
                const u32x4 w1 = {pack2<BF16>(a[8], a[9]), pack2<BF16>(a[10], a[11]),
                                  pack2<BF16>(a[12], a[13]), pack2<BF16>(a[14], a[15])};
                *(u32x4*)(orow + db * 32 + 16 * h) = w0;
                *(u32x4*)(orow + db * 32 + 16 * h + 8) = w1;
            }
            if (h == 0) lp[row] = (m_run[qb] + __builtin_amdgcn_logf(l_run[qb])) * LN2;
        }
    }
}

}  // namespace fa
