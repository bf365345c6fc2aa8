// fa_fwd_kernel.hpp -- gfx950 (MI355X) FlashAttention-style forward kernel.
//
// What is computed follows "Tuning Flash Attention for peak performance in NVIDIA CUDA
// Tile" (NVIDIA cuTile post), Part 1: a workgroup owns a tile of query rows, keeps them
// resident, streams K/V tiles through on-chip memory, and folds every tile into a running
// row max m, row sum l and fp32 accumulator ("Understanding online softmax", "Online
// softmax update"), normalising once at the end ("Final normalization and store").
// Causal tiles past the diagonal are never visited, and the K loop is split into a
// mask-free loop and a masked loop over the diagonal / key-tail tiles (Part 2 "K-loop
// split"); heavy causal tiles are launched first (Part 2 "ProgramId remapping"); exp2 is
// used with log2(e) folded into the scale (Part 1 "Initializing accumulators"; "How I
// Beat PyTorch's Flash Attention", "Phase 4").
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
//    V stays row-major in LDS; ds_read_b64_tr_b16 delivers V^T fragments: in each group
//    of 16 lanes, lane i receives element (i mod 4) of the 8-byte rows addressed by lanes
//    4j + i/4, j = 0..3.  The d-order of the fragments is chosen so that each lane ends
//    with 16 consecutive d of its query per 32-wide block.  In the plain call the
//    epilogue stages O through LDS and writes whole 128-byte row segments with
//    non-temporal stores; split partials are stored from the registers.
//  * K and V tiles are triple-buffered in LDS and move there straight from HBM with
//    gfx950's 128-bit buffer loads to LDS: no staging registers, no LDS write instructions
//    (staging through registers measured 5% slower).  The buffer range ends at key Skv,
//    so a ragged key tail lands as zeros.  The K loop is a three-stage software pipeline:
//    step j issues the MFMAs of S(j+1) in the same block as the softmax of tile j together
//    with the P V of tile j-1, so all matrix work of a step is independent of its exp2 work
//    and can overlap it.  K is loaded three tiles and V two tiles ahead of their use, so a
//    load has two steps to land; each step waits only for the previous step's loads.
//    16-byte chunks are XOR-swizzled per row so that tile writes, K operand reads and V
//    transpose reads are bank-conflict free.
//  * Register use is held to 256 per lane so that two waves share each SIMD: one wave's
//    softmax and memory latency overlap the other's MFMAs.
//  * The running max is kept lazily: p = exp2(c s - m) is computed with the current m and
//    m is only raised (acc and l rescaled, p recomputed) when a lane's partial row sum of
//    p exceeds 2^15 -- on the first tile and on a large jump of the max.  softmax is
//    invariant to the shift, p stays <= 2^15 (exact range in bf16 / fp16), and the
//    normalisation at the end uses the same m for acc and l, so the result is the same
//    softmax; the common path computes no row max at all.
//  * A workgroup is HPW heads x WPH position blocks.  HPW > 1 packs query heads of one
//    GQA group into a workgroup: they share every K/V tile ("Grouped-query attention").
//  * Workgroups are dispatched round-robin over the 8 XCDs.  The workgroup id is remapped
//    so that each XCD works on whole (batch, K/V head) groups, keeping their K/V tiles in
//    its own L2, and within an XCD the heaviest causal tiles come first.
//  * Split-KV (for grids too small to fill 256 CUs, e.g. decoding with one query row --
//    the pages' "too few tiles" case, cuTile post Part 2 "Autotuning", "How I Beat PyTorch's
//    Flash Attention" Phase 5): each query tile's visible K/V tiles are cut into num_splits
//    tile-aligned ranges, one workgroup each.  A workgroup stores its range's normalised
//    partial O (fp32) and LSE; fa_merge_kernel (fa_merge_kernel.hpp) folds the partials
//    with the online-softmax rescale ("Online softmax update") applied across ranges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

// The K-loop lambdas must be inlined: an outlined step is a call with its state on the
// stack (private memory), several times slower.
#define FA_INLINE __attribute__((always_inline))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kNumXcd = 8;

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
    int hsub;        // head groups per K/V head: group / HPW
    int map_mode;    // workgroup -> XCD mapping: 0 plain, 1 groups per XCD, 2 XCDs per group
    int map_arg;     // mode 1: groups per XCD; mode 2: XCDs per group
    int window;      // causal sliding window: keys input_pos + i - window + 1 .. ; 0 = none
    int num_splits;  // key ranges per query tile; > 1 writes partials for the merge kernel
    float* o_part;   // num_splits > 1: normalised partial O, fp32 [num_splits][B*Hq*Sq][D]
    float* lse_part; // num_splits > 1: partial LSE, fp32 [num_splits][B*Hq*Sq]
    float o_scale;   // fp8 V: its dequantisation factor, applied to O; 1 otherwise
};

// Compile-time configuration of one kernel instance.
template <int D_, int BN_, int QB_, int WPH_, int HPW_, bool CAUSAL_, bool BF16_, bool QK8_ = false,
          bool V8_ = false, int KS_ = 1>
struct Cfg {
    static constexpr int D = D_;        // head dim
    static constexpr int BN = BN_;      // keys per K/V tile
    static constexpr int QB = QB_;      // 32-row query blocks per wave
    static constexpr int WPH = WPH_;    // waves per head (along positions)
    static constexpr int HPW = HPW_;    // heads per workgroup
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr bool BF16 = BF16_;    // V / O element type: bf16, else fp16
    static constexpr bool QK8 = QK8_;      // Q and K in fp8 e4m3 (S = K Q^T on the fp8 MFMA)
    static constexpr bool V8 = V8_;        // V in fp8 e4m3 too (widened to BF16 ? bf16 : fp16)
    static constexpr int KS = KS_;         // key parts: KS sets of WPH x HPW waves, each taking
                                           // 1/KS of the key tiles, merged at the end
    static constexpr int NWQ = WPH * HPW;  // waves per key part
    static constexpr int NW = NWQ * KS;
    static constexpr int NT = 64 * NW;
    static constexpr int BMP = 32 * QB * WPH;   // query positions per workgroup
    static constexpr int WAVES_PER_SIMD = QB == 1 ? 2 : 1;  // register budget 256 / 512
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN == 32 || BN == 64, "key tile");
    static_assert(QB == 1 || QB == 2, "query blocks per wave");
    static_assert(NW == 4 || NW == 8, "waves per workgroup");
    static_assert(!QK8 || ((D == 128 && BN == 32) || (D == 64 && BN == 64)) && QB == 1,
                  "fp8 Q/K: head dim 128 with 32-key tiles or head dim 64 with 64-key tiles");
    static_assert(!V8 || QK8, "fp8 V comes with fp8 Q and K");
    static_assert(KS == 1 || (KS == 2 && !CAUSAL && !QK8 && QB == 1),
                  "key parts: non-causal fp16 / bf16, one query block per wave");
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

// D(32x32, fp32) += A(32x64) * B(64x32) with fp8 e4m3 A and B (unit block scales).  Lane l
// holds row / column l mod 32 and the 32 k-elements 32*(l/32) .. +31 of the 64, in order, in
// its 8 registers; any ordering of k works as long as A and B share it (probe-checked).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f, 0, 0x7f);
}

// 8 bytes (4 x 16 bit) of a transposed LDS read; see the header comment for the lanes.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// 8 bytes of an 8-bit transposed LDS read.  Measured lane rule: in each group of 16 lanes,
// lane i receives byte (i mod 8) of the 8-byte pieces addressed by lanes 2j + i/8,
// j = 0..7, in that order.
__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char* p) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Two fp8 e4m3 codes (bytes 0, 1 of x, or 2, 3 when HI) widened exactly to bf16 / fp16:
// low half from the lower byte.
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t fp8x2_widen(uint32_t x) {
    if constexpr (BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
    }
}

// Balanced reductions of N floats held in registers: a max tree of v_max3 and a pairwise
// sum tree, so the dependency depth is log(N) rather than N.  `a` is overwritten.
template <int N>
struct Tree {
    __device__ __forceinline__ static float max(float* a) {
        constexpr int M = (N + 2) / 3;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            if (3 * i + 2 < N) a[i] = fmaxf(fmaxf(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
            else if (3 * i + 1 < N) a[i] = fmaxf(a[3 * i], a[3 * i + 1]);
            else a[i] = a[3 * i];
        }
        return Tree<M>::max(a);
    }
    __device__ __forceinline__ static float sum(float* a) {
        constexpr int M = (N + 1) / 2;
#pragma unroll
        for (int i = 0; i < M; ++i) a[i] = (2 * i + 1 < N) ? a[2 * i] + a[2 * i + 1] : a[2 * i];
        return Tree<M>::sum(a);
    }
};
template <>
struct Tree<1> {
    __device__ __forceinline__ static float max(float* a) { return a[0]; }
    __device__ __forceinline__ static float sum(float* a) { return a[0]; }
};

// Buffer resource for a raw byte range (gfx9-family descriptor: stride 0, 32-bit records).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes lds + 16*i.  A device
// function of its own, so the host compilation pass never sees the builtin.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff,
                                                  int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             voff, soff, 0, 0);
}

// --- LDS tile layout: [BN][D] row-major, 16-byte chunks XOR-swizzled per row ------------
// K rows (read 32 rows x one chunk per MFMA operand): chunk ^ (row mod 16) for D=128;
// for D=64 (8 chunks) the swizzle also folds row bit 3 so 16 consecutive rows differ.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D == 128) return row & 15;
    else if constexpr (D == 64) return (row & 7) ^ ((row >> 3) & 1);
    else return (row >> 2) & 3;   // 64-byte rows (fp8, head dim 64): 16 rows on 16 bank groups
}
// V rows: a swizzle taken from key mod 4.  A transposed read serves 32 lanes per pass: 4
// consecutive keys x 4 chunks x 16 bytes = 256 bytes, which must fall on the 64 distinct
// 4-byte banks.  Head dim 128 (256-byte rows, all four keys on the same banks): the four keys
// take chunk XORs {0, 4, 9, 13}.  Head dim 64 (128-byte rows, keys k and k + 2 on the same
// banks): XORs {0, 1, 4, 5}, so keys k and k + 2 use opposite halves of the row.  Both also
// keep each 16-lane half of a pass on distinct banks.
template <int D>
__device__ __forceinline__ int v_swz_of(int key_mod4) {
    if constexpr (D == 128)
        return ((key_mod4 & 1) << 2) | ((key_mod4 >> 1) & 1) | (((key_mod4 >> 1) & 1) << 3);
    else
        return (((key_mod4 >> 1) & 1) << 2) | (key_mod4 & 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    return v_swz_of<D>(row & 3);
}
// fp8 V rows (128 bytes, 8 chunks), read 8 bytes at a time by the 8-bit transposed read:
// one read covers, for each half of the wave, 8 keys (rows r with r mod 16 in {0..3, 8..11}
// or {4..7, 12..15}) x 2 chunks x 16 bytes.  Chunk XOR 2 * (bit 1 of r | bit 3 of r << 1)
// gives the four even and the four odd rows of each half distinct 32-byte bank windows,
// so the 256 bytes of a half land on the 64 banks once.
// fp8 V rows of 64 bytes (head dim 64, 4 chunks): rows r and r + 8 share banks, so chunk XOR
// 2 * (bit 3 of r) puts them on opposite chunk pairs; the other rows of a half already fall
// on distinct banks.
template <int D>
__device__ __forceinline__ int v8_swz(int row) {
    if constexpr (D == 128) return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
    else return 2 * ((row >> 3) & 1);
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::NT, C::NT), amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD)))
void fa_fwd_kernel(Params p) {
    constexpr int D = C::D, BN = C::BN, QB = C::QB, WPH = C::WPH, HPW = C::HPW;
    constexpr bool CAUSAL = C::CAUSAL, BF16 = C::BF16;
    constexpr int KB = BN / 32;          // 32-key blocks per tile
    constexpr int DK = D / 16;           // k-steps of Q K^T
    constexpr int DB = D / 32;           // 32-wide d blocks of O
    constexpr bool QK8 = C::QK8;
    constexpr bool V8 = C::V8;
    constexpr int ROWB = D * 2;          // bytes per fp16 / bf16 row
    constexpr int ROWV = V8 ? D : ROWB;  // bytes per V row
    constexpr int TILE = BN * ROWV;      // bytes per V tile
    constexpr int CPR = ROWV / 16;       // 16-byte chunks per V row
    constexpr int NLV = BN * CPR / 64;   // 64-lane loads per V tile
    constexpr int NWV = NLV < C::NWQ ? NLV : C::NWQ; // waves of a key part that load V (its last NWV)
    constexpr int LD = NLV / NWV;        // V loads per loading thread
    static_assert(NLV % NWV == 0, "V tile loads per wave");
    constexpr int ROWK = QK8 ? D : ROWB; // bytes per K row
    constexpr int TILEK = BN * ROWK;     // bytes per K tile
    constexpr int CPRK = ROWK / 16;      // 16-byte chunks per K row
    constexpr int NLK = BN * CPRK / 64;  // 64-lane loads per K tile
    constexpr int NWK = NLK < C::NWQ ? NLK : C::NWQ; // waves of a key part that load K
    constexpr int LDK = NLK / NWK;       // K loads per loading thread
    static_assert(NLK % NWK == 0, "K tile loads per wave");
    constexpr float P_LIMIT = 32768.0f;  // lazy max: largest partial row sum of p allowed
    constexpr float LN2 = 0.69314718055994530942f;
    static_assert(TILE % (NWV * 1024) == 0, "each load fills whole 1 KiB wave slots");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int kpart = C::KS == 1 ? 0 : w / C::NWQ;   // key part of the wave (0 unless KS > 1)
    const int wq = C::KS == 1 ? w : w % C::NWQ;      // its place among the part's query blocks
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // Workgroup -> (batch, K/V head, query tile, head subgroup, key split); see the header
    // comment.  The splits of one query tile are adjacent work items.
    const int ngrp = p.B * p.Hkv;
    int grp, item;
    {
        const int wg = blockIdx.x;
        if (p.map_mode == 1) {
            const int x = wg % kNumXcd, s = wg / kNumXcd;
            grp = x * p.map_arg + s % p.map_arg;
            item = s / p.map_arg;
        } else if (p.map_mode == 2) {
            const int x = wg % kNumXcd, s = wg / kNumXcd;
            grp = x / p.map_arg;
            item = s * p.map_arg + x % p.map_arg;
        } else {
            grp = wg % ngrp;
            item = wg / ngrp;
        }
    }
    const int b = grp / p.Hkv;
    const int kvh = grp - b * p.Hkv;
    const int split = item % p.num_splits;
    item /= p.num_splits;
    const int trank = item / p.hsub;
    const int hs = item - trank * p.hsub;
    const int tile = CAUSAL ? p.n_tiles - 1 - trank : trank;
    const int hq = kvh * p.group + hs * HPW + wq / WPH;
    const int q0 = tile * C::BMP;
    const int qw0 = q0 + (wq % WPH) * (32 * QB);

    typedef uint16_t T;
    constexpr int QE = QK8 ? 1 : 2;   // bytes per Q / K element
    const unsigned char* qp = (const unsigned char*)p.q + (size_t)(b * p.Hq + hq) * p.Sq * D * QE;
    const unsigned char* kp = (const unsigned char*)p.k + (size_t)(b * p.Hkv + kvh) * p.Skv * D * QE;
    const unsigned char* vp = (const unsigned char*)p.v + (size_t)(b * p.Hkv + kvh) * p.Skv * ROWV;

    // Queries of this wave, as the B operand of S^T = K Q^T: lane l holds row l%32 of
    // query block qb, elements dk*16 + 8*(l/32) .. +8.  Rows past Sq read row Sq-1; their
    // results are never stored.
    // fp8: lane l holds bytes 64*dk + 32*(l/32) .. +31 of its row for the fp8 MFMA's k-range.
    constexpr int DK8 = D / 64;
    u32x4 qf[QK8 ? 1 : QB][QK8 ? 1 : DK];
    i32x8 qf8[QK8 ? QB : 1][DK8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + qb * 32 + l32, p.Sq - 1);
        const u32x4* src = (const u32x4*)(qp + (size_t)row * D * QE);
        if constexpr (QK8) {
#pragma unroll
            for (int dk = 0; dk < DK8; ++dk) {
                const u32x4 lo = src[dk * 4 + 2 * h], hi = src[dk * 4 + 2 * h + 1];
                qf8[qb][dk] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        } else {
#pragma unroll
            for (int dk = 0; dk < DK; ++dk) qf[qb][dk] = src[dk * 2 + h];
        }
    }

    // Loop bounds.  Workgroup: tiles [tb, Tc); tiles [f0, f1) need no mask (K-loop split),
    // those before f0 (sliding-window edge) and from f1 on (diagonal, key tail) do.  Wave:
    // tiles outside [wave_lo, wave_tc) are fully masked for its rows and skipped.
    const bool win = CAUSAL && p.window > 0;
    const int q_last = min(q0 + C::BMP, p.Sq) - 1;
    const int Tc = CAUSAL ? (min(p.input_pos + q_last + 1, p.Skv) + BN - 1) / BN
                          : (p.Skv + BN - 1) / BN;
    const int tb = win ? min(max(0, p.input_pos + q0 - p.window + 1) / BN, Tc) : 0;
    const int f1 = min(CAUSAL ? min((p.input_pos + q0) / BN, p.Skv / BN) : p.Skv / BN, Tc);
    // First tile above every row's window edge.  When masked tiles precede it, it is run
    // as a masked step too, so that every unmasked step follows an unmasked one (or is the
    // first step) and P V of its predecessor needs no per-wave check.
    int f0 = win ? max(tb, (p.input_pos + q_last - p.window + BN) / BN) : tb;
    if (f0 > tb) ++f0;
    const int qw_last = min(qw0 + 32 * QB, p.Sq) - 1;
    const int wave_tc = qw_last < qw0 ? 0
                        : CAUSAL ? (min(p.input_pos + qw_last + 1, p.Skv) + BN - 1) / BN
                                 : Tc;
    const int wave_lo = win ? max(0, p.input_pos + qw0 - p.window + 1) / BN : 0;
    // This workgroup's key split: tiles [r0, r1) of [tb, Tc), tile-aligned, so no mask is
    // needed at split boundaries.  An empty range (more splits than tiles) leaves the state
    // empty: the partial is O = 0, LSE = -inf.
    int r0 = tb + (int)((long long)(Tc - tb) * split / p.num_splits);
    int r1 = tb + (int)((long long)(Tc - tb) * (split + 1) / p.num_splits);
    if constexpr (C::KS > 1) {
        // Key parts: consecutive, equal runs of the range's tiles (the host launches key parts
        // only for even tile counts), so every wave of the workgroup runs the same number of
        // steps, and of barriers.
        const int part = (r1 - r0) / C::KS;
        r0 += kpart * part;
        r1 = r0 + part;
    }
    const int t0 = r0, t1 = r1;
    const int nt = t1 - t0;                    // tiles in this range
    // Local step bands: [0, ua) masked, [ua, ub) unmasked, [ub, nt) masked.
    const int ua = min(max(f0 - t0, 0), nt);
    const int ub = max(ua, min(f1 - t0, nt));
    const int kend = min(p.Skv, t1 * BN);

    // Running state: m (exp2 domain, possibly stale), l, acc (= O^T blocks).
    float m_run[QB], l_run[QB];
    f32x16 acc[DB][QB];
    // Each S block starts from -m/c (0 while m = -inf) instead of 0, so that the MFMAs
    // deliver s - m/c and p = exp2(c (s - m/c)) costs one multiply before the exp2.
    f32x16 negm[QB];
    const float inv_c = 1.0f / p.c;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        negm[qb] = (f32x16){};
        m_run[qb] = -__builtin_inff();
        l_run[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] = (f32x16){};
    }

    // LDS: K(t0+i) lives in k_lds[i%3] and V(t0+i) in v_lds[i%3].  Six separate arrays, so
    // the compiler can tell a direct-to-LDS load into one from reads of another and does
    // not wait for the load before those reads; the step-end barrier publishes it.
    // With key parts, part k uses bytes [k TILE, (k+1) TILE) of each array.
    __shared__ __attribute__((aligned(16))) unsigned char k_lds0[TILEK * C::KS], k_lds1[TILEK * C::KS],
        k_lds2[TILEK * C::KS];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILE * C::KS], v_lds1[TILE * C::KS],
        v_lds2[TILE * C::KS];
    // fp8 V: the tile buffers (4 KiB each) are too small to stage O in the epilogue; it gets
    // its own 4 KiB per wave.
    __shared__ __attribute__((aligned(16))) unsigned char o_stage[V8 && C::KS == 1 ? C::NW * 4096 : 16];
    auto kl = [&](auto ph) -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        return (P == 0 ? k_lds0 : P == 1 ? k_lds1 : k_lds2) + kpart * TILEK;
    };
    auto vl = [&](auto ph) -> unsigned char* {
        constexpr int P = decltype(ph)::value;
        return (P == 0 ? v_lds0 : P == 1 ? v_lds1 : v_lds2) + kpart * TILE;
    };

    // Tiles move from HBM straight into LDS (buffer_load_dwordx4 ... lds): in load i, wave
    // w fills the 1 KiB of LDS at chunk slots (i*NW + w)*64 + lane, so each lane fetches
    // the chunk that the row swizzle places in its slot.  The buffer range ends at key Skv:
    // rows past Skv, and whole tiles past the end, are out of range and land as zeros.
    // The row of a slot advances by 64*NW/CPR rows per load i; that is a multiple of 16, so
    // the swizzles (row mod 16) do not depend on i: one per-lane offset plus i * stride.
    static_assert((64 * NWV / CPR) % 16 == 0, "load stride keeps the swizzle");
    static_assert((64 * NWK / CPRK) % 16 == 0, "K load stride keeps the swizzle");
    constexpr int LOAD_STRIDE = 64 * NWV * 16;     // bytes of V tile per load i
    constexpr int LOAD_STRIDE_K = 64 * NWK * 16;   // bytes of K tile per load i
    // fp8 K rows (D bytes) use the swizzle of a bf16 row of the same length: head dim 128
    // takes the 8-chunk map of the head-dim-64 layout, head dim 64 a 4-chunk map.
    constexpr int KSWZ_D = QK8 ? D / 2 : D;
    auto kswz = [&](int row) { return k_swz<KSWZ_D>(row); };
    // Waves that load V tiles are the last NWV of their key part; those that load K the first
    // NWK.  Each key part streams its own tiles into its own half of the buffers.
    const int vw = wq - (C::NWQ - NWV);
    const bool ld_v = NWV == C::NWQ || vw >= 0;
    const bool ld_k = NWK == C::NWQ || wq < NWK;
    int ksrc, vsrc;
    {
        const int slot = (ld_v ? vw : 0) * 64 + lane;
        const int row = slot / CPR, pc = slot % CPR;
        if constexpr (V8) vsrc = row * ROWV + ((pc ^ v8_swz<D>(row)) << 4);
        else vsrc = row * ROWV + ((pc ^ v_swz<D>(row)) << 4);
        const int slotk = wq * 64 + lane;
        const int rowk = slotk / CPRK, pck = slotk % CPRK;
        ksrc = rowk * ROWK + ((pck ^ kswz(rowk)) << 4);
    }
    // One buffer resource for K and one for V from tile jb to the range's last valid key
    // kend; a load adds the tile's byte offset from jb plus i * stride as the scalar offset.
    // gfx950's range check covers voffset + soffset, so every load past the end of the range
    // -- the ragged key tail, tiles past the end, keys of the next split -- reads zero.  jb
    // moves up (rebase) only once a range has run RB tiles past it, which keeps offsets and
    // record counts below 2^31: never, unless the range holds more than 2^30 bytes of K or V.
    constexpr int RB = (1 << 30) / (TILEK > TILE ? TILEK : TILE);
    int jb = t0;
    __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, 0), rv = make_rsrc(vp, 0);
    auto rebase = [&](int j) FA_INLINE {
        jb = j;
        const int k0 = min(j * BN, kend);
        const int n = min(kend - k0, (RB + 16) * BN);
        rk = make_rsrc(kp + (size_t)k0 * ROWK, n * ROWK);
        rv = make_rsrc(vp + (size_t)k0 * ROWV, n * ROWV);
    };
    auto fetch = [&](int j, unsigned char* dst) FA_INLINE {
        if (ld_v) {
#pragma unroll
            for (int i = 0; i < LD; ++i)
                buffer_load_lds16(rv, dst + (i * NWV + vw) * 1024, vsrc, (j - jb) * TILE + i * LOAD_STRIDE);
        }
    };
    // K tiles: waves wq < NWK load LDK chunks per lane (all waves unless fp8).
    auto fetch_k = [&](int j, unsigned char* dst) FA_INLINE {
        if (ld_k) {
#pragma unroll
            for (int i = 0; i < LDK; ++i)
                buffer_load_lds16(rk, dst + (i * NWK + wq) * 1024, ksrc, (j - jb) * TILEK + i * LOAD_STRIDE_K);
        }
    };

    // Per-lane LDS offsets.  K operand: row kb*32 + l32, chunk (2dk + h) ^ k_swz(row); the
    // swizzle depends only on l32, so chunk = (2dk) ^ ku with ku = h ^ k_swz(l32).
    // fp8: chunks 4dk + 2h and 4dk + 2h + 1 of row l32 (physical chunks c and c ^ 1, since
    // 4dk + 2h is even) hold the lane's 32 k-bytes.
    const int ku = h ^ k_swz<D>(l32);
    int koff[QK8 ? DK8 : DK];
#pragma unroll
    for (int dk = 0; dk < (QK8 ? DK8 : DK); ++dk)
        koff[dk] = QK8 ? l32 * ROWK + (((4 * dk + 2 * h) ^ kswz(l32)) << 4)
                       : l32 * ROWB + (((2 * dk) ^ ku) << 4);
    // V^T operand (two transpose reads per MFMA): this lane addresses key
    // 4*h + jj (+ kb*32 + 16*hf + 8*r) and the 8-byte piece of d = db*32 + 16*(qq&1) +
    // 8*(g&1) + 4*(qq>>1), with jj, qq from the lane's index in its 16-lane group g.
    const int vs = lane & 15, vj = vs >> 2, vq = vs & 3, vg = lane >> 4;
    const int v_lane_row = 4 * (vg >> 1) + vj;
    const int vu = (2 * (vq & 1) + (vg & 1)) ^ v_swz_of<D>(vj);   // chunk ^ 4*db
    int voff[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        voff[db] = v_lane_row * ROWB + (vq >> 1) * 8 + (((4 * db) ^ vu) << 4);
    // fp8 V^T operand (one 8-bit transposed read per MFMA): the A operand of lane l holds,
    // for d = l mod 32 of its 32-wide block (so, unlike the 16-bit path, accumulator row m
    // is d = m and the epilogue stores accordingly), the same 8 keys as P^T's lane: keys
    // 4h + e and 8 + 4h + e, e = 0..3 (h = l / 32) of the 16-key half.  By the read's lane
    // rule, the lanes 2j + p of each 16-lane group g address key j of that list (d bytes
    // 16 (g mod 2) + 8p of the block), so lane i receives key j's byte for its own d as
    // element j.
    int voff8[DB];
    {
        const int g8 = lane >> 4, a8 = lane & 15, j8 = a8 >> 1, p8 = a8 & 1;
        const int key = 4 * (g8 >> 1) + j8 + (j8 >= 4 ? 4 : 0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
            voff8[db] = key * ROWV + (((2 * db + (g8 & 1)) ^ v8_swz<D>(key)) << 4) + 8 * p8;
    }

    // S^T = K Q^T of the tile in K buffer `kb`.
    auto qk = [&](const unsigned char* kb, f32x16 (&s)[KB][QB]) FA_INLINE {
#pragma unroll
        for (int k2 = 0; k2 < KB; ++k2) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[k2][qb] = negm[qb];
            if constexpr (QK8) {
#pragma unroll
                for (int dk = 0; dk < DK8; ++dk) {
                    const u32x4 lo = *(const u32x4*)(kb + k2 * 32 * ROWK + koff[dk]);
                    const u32x4 hi = *(const u32x4*)(kb + k2 * 32 * ROWK + (koff[dk] ^ 16));
                    const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[k2][qb] = mfma32_fp8(a, qf8[qb][dk], s[k2][qb]);
                }
            } else {
#pragma unroll
                for (int dk = 0; dk < DK; ++dk) {
                    const u32x4 a = *(const u32x4*)(kb + k2 * 32 * ROWB + koff[dk]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[k2][qb] = mfma32<BF16>(a, qf[qb][dk], s[k2][qb]);
                }
            }
        }
    };

    // O^T += V^T P^T for the tile whose V sits in `vb` and whose packed P is `pk`.
    auto pv = [&](const unsigned char* vb, const u32x4 (&pk)[KB][QB][2]) FA_INLINE {
        if constexpr (V8) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const u32x2 x = lds_read_tr8(vb + voff8[db] + (k2 * 32 + 16 * hf) * ROWV);
                            const u32x4 a = {fp8x2_widen<BF16, false>(x[0]), fp8x2_widen<BF16, true>(x[0]),
                                             fp8x2_widen<BF16, false>(x[1]), fp8x2_widen<BF16, true>(x[1])};
                            acc[db][qb] = mfma32<BF16>(a, pk[k2][qb][hf], acc[db][qb]);
                        }
            return;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const unsigned char* pr = vb + voff[db] + (k2 * 32 + 16 * hf) * ROWB;
                        const u32x2 x0 = lds_read_tr16(pr);
                        const u32x2 x1 = lds_read_tr16(pr + 8 * ROWB);
                        const u32x4 a = {x0[0], x0[1], x1[0], x1[1]};
                        acc[db][qb] = mfma32<BF16>(a, pk[k2][qb][hf], acc[db][qb]);
                    }
    };

    // Register sets that rotate with the phase of the step: S and packed P.
    f32x16 s0[KB][QB], s1[KB][QB], s2[KB][QB];
    u32x4 pk0[KB][QB][2], pk1[KB][QB][2], pk2[KB][QB][2];
    auto pick = [](auto ph, auto& a, auto& b, auto& c) -> auto& {
        constexpr int P = decltype(ph)::value;
        if constexpr (P == 0) return a;
        else if constexpr (P == 1) return b;
        else return c;
    };
    // End of a step: wait until this wave's loads issued one step earlier have landed
    // (the loads of this step, 2*LD of them, may stay in flight), then the workgroup
    // barrier.  The asm is a compiler memory barrier as well.
    // s_waitcnt vmcnt(N) then s_barrier, as one asm statement (also a compiler memory
    // barrier).
    auto wait_barrier = [&](auto n_tag) FA_INLINE {
        constexpr int N = decltype(n_tag)::value;
        static_assert(N < 64, "vmcnt range");
        constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
        asm volatile("s_waitcnt %0\n\ts_barrier" ::"n"(imm) : "memory");
    };
    // Wait until at most KN (for a wave that loads K) plus VN (for a wave that loads V) of
    // this wave's loads are in flight, then the barrier.
    auto wait_loads = [&](auto kn, auto vn) FA_INLINE {
        constexpr int KN = decltype(kn)::value, VN = decltype(vn)::value;
        if (ld_k && ld_v) wait_barrier(std::integral_constant<int, KN + VN>{});
        else if (ld_k) wait_barrier(std::integral_constant<int, KN>{});
        else if (ld_v) wait_barrier(std::integral_constant<int, VN>{});
        else wait_barrier(std::integral_constant<int, 0>{});
    };
    // A wave issues LDK K loads (if it loads K) and LD V loads (if it loads V) per step.
    auto end_step = [&]() FA_INLINE {
        wait_loads(std::integral_constant<int, LDK>{}, std::integral_constant<int, LD>{});
    };

    // One K-loop step for tile j (phase PH = (j - t0) % 3), a three-stage software
    // pipeline.  The step issues the MFMAs of S(j+1) = K(j+1) Q^T and of O^T += V(j-1)^T
    // P(j-1)^T -- neither depends on this step's softmax -- in the same straight-line
    // block as the softmax of S(j) into P(j), so all matrix work can overlap the exp2
    // work.  Loads: K(j+3) into k_lds[PH] (K(j) was used by the previous step) and V(j+1)
    // into v_lds[PH+1] (V(j-2) was used by the previous step); the step reads
    // k_lds[PH+1] = K(j+1) and v_lds[PH+2] = V(j-1), so no buffer is written while it is
    // read, and one barrier per step suffices.
    auto step = [&](int j, auto ph_tag, auto masked_tag, auto first_tag) FA_INLINE {
        constexpr int PH = decltype(ph_tag)::value;        // (j - t0) % 3
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr bool FIRST = decltype(first_tag)::value; // j == t0: no P(j-1) yet
        using N1 = std::integral_constant<int, (PH + 1) % 3>;
        using N2 = std::integral_constant<int, (PH + 2) % 3>;
        auto& s_cur = pick(ph_tag, s0, s1, s2);
        auto& s_nxt = pick(N1{}, s0, s1, s2);
        auto& pk_cur = pick(ph_tag, pk0, pk1, pk2);
        auto& pk_prev = pick(N2{}, pk0, pk1, pk2);
        fetch_k(j + 3, kl(ph_tag));
        fetch(j + 1, vl(N1{}));
        const bool do_sm = !MASKED || (j >= wave_lo && j < wave_tc);   // softmax of tile j
        const bool do_pv = !FIRST && (!MASKED || (j - 1 >= wave_lo && j - 1 < wave_tc));   // P V of tile j-1
        if (do_sm) {
            if constexpr (MASKED) {
                const int j0 = j * BN;
                // A band tile that every row of this wave sees whole (below its diagonal, above
                // its window edge, before the key tail) needs no mask: skip it for the wave.
                const bool whole = j0 + BN - 1 <= (CAUSAL ? min(p.input_pos + qw0, p.Skv - 1) : p.Skv - 1) &&
                                   (!win || j0 >= p.input_pos + qw0 + 32 * QB - p.window);
                if (!whole)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int qpos = p.input_pos + qw0 + qb * 32 + l32;
                    const int lim = CAUSAL ? min(qpos, p.Skv - 1) : p.Skv - 1;   // last visible key
                    const int lo = win ? qpos - p.window + 1 : 0;                 // first visible key
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = j0 + k2 * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                            if (key > lim || key < lo) s_cur[k2][qb][i] = -__builtin_inff();
                        }
                }
            }
        }
        // Scheduling: the backend's MFMA / LDS-read interleave (one fragment read between
        // MFMAs) for this step's block.  Same instructions; measured 0.5% faster on the causal
        // GQA shapes and 5-10% on the grids with one or two waves per SIMD and long key loops.
        __builtin_amdgcn_iglp_opt(0);
        // Matrix work of this step: S(j+1), and P V of tile j-1.
        qk(kl(N1{}), s_nxt);
        if constexpr (!FIRST) {
            if (!MASKED || do_pv) pv(vl(N2{}), pk_prev);
        }
        if (do_sm) {
            // P = exp2(c s - m) with the running max m, packed to the storage type, and the
            // lane's partial row sums in fp32 (each 16-key block summed as soon as it is
            // packed).  Summing the rounded bf16 p instead would move LSE by ~1e-3 on rows
            // with few visible keys.
            float ts[QB];
            auto make_p = [&]() FA_INLINE {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float psum[KB];
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2) {
                        float t[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            t[i] = fast_exp2(s_cur[k2][qb][i] * p.c);
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const float* e = t + 8 * hf;
                            pk_cur[k2][qb][hf] = (u32x4){pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]),
                                                         pack2<BF16>(e[4], e[5]), pack2<BF16>(e[6], e[7])};
                        }
                        psum[k2] = Tree<16>::sum(t);
                    }
                    ts[qb] = Tree<KB>::sum(psum);
                }
            };
            make_p();
            // Lazy max.  Every p is at most its lane's partial sum, so while those sums stay
            // <= 2^15 the running max m may lag the true row max: p fits the storage type and
            // the softmax is unchanged, since acc and l share m.  Otherwise (a jump of the
            // max, or m still -inf: the row's first tile) raise m to the row max, rescale acc
            // (which already holds P V up to tile j-1) and l, and recompute P.  No row max on
            // the common path.
            bool bad = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                bad |= !(ts[qb] <= P_LIMIT) || ((MASKED || FIRST) && m_run[qb] == -__builtin_inff());
            if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float t[KB * 16];
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
                        for (int i = 0; i < 16; ++i) t[k2 * 16 + i] = s_cur[k2][qb][i];
                    // S holds s - m_used/c, m_used = m (0 while m = -inf).
                    const float m_used = m_run[qb] == -__builtin_inff() ? 0.0f : m_run[qb];
                    const float m_new = fmaxf(m_run[qb], m_used + xhalf_max(Tree<KB * 16>::max(t)) * p.c);
                    // A row with no visible key yet keeps m = -inf and its (zero) state.
                    const float alpha = m_new == -__builtin_inff() ? 1.0f : fast_exp2(m_run[qb] - m_new);
                    m_run[qb] = m_new;
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
                    // S(j) and S(j+1) started from -m_used/c: move both to the new m.
                    const float nm = (m_new == -__builtin_inff() ? 0.0f : -m_new) * inv_c;
                    const float delta = m_used * inv_c + nm;
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2) {
                        s_cur[k2][qb] += delta;
                        s_nxt[k2][qb] += delta;
                    }
                    negm[qb] = nm;
                }
                make_p();
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_run[qb] += ts[qb];
        }
        end_step();
    };

    // Prologue: K(t0), K(t0+1), K(t0+2) and V(t0) to LDS; S(t0) once K(t0) has landed.
    // Local step i handles tile t0+i with buffers and register sets of phase i % 3.
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using F = std::false_type;
    using TT = std::true_type;
    if (nt > 0) {
        rebase(t0);
        fetch_k(t0, kl(Q0{}));
        fetch_k(t0 + 1, kl(Q1{}));
        fetch_k(t0 + 2, kl(Q2{}));
        fetch(t0, vl(Q0{}));
        // K(t0) landed; K(t0+1), K(t0+2) and V(t0) may be in flight.
        wait_loads(std::integral_constant<int, 2 * LDK>{}, std::integral_constant<int, LD>{});
        qk(kl(Q0{}), s0);
        end_step();   // K(t0+1) and K(t0+2) landed

        // The K loop in bands (K-loop split): window-edge tiles, tiles needing no mask,
        // then the diagonal / key-tail tiles.  Unrolled by three so the phase of i --
        // buffers and register roles -- is fixed at compile time in every copy of the step.
        if (ua == 0 && ub > 0) step(t0, Q0{}, F{}, TT{});
        else step(t0, Q0{}, TT{}, TT{});
        int i = 1;
        auto run = [&](int end, auto masked) FA_INLINE {
            if (i < end && i % 3 == 1) { step(t0 + i, Q1{}, masked, F{}); ++i; }
            if (i < end && i % 3 == 2) { step(t0 + i, Q2{}, masked, F{}); ++i; }
            for (; i + 2 < end; i += 3) {
                // At most RB + 8 tiles past jb before the next check: the rest of this
                // iteration, up to four peeled steps, and the loads three tiles ahead.
                if (t0 + i - jb >= RB) rebase(t0 + i);
                step(t0 + i, Q0{}, masked, F{});
                step(t0 + i + 1, Q1{}, masked, F{});
                step(t0 + i + 2, Q2{}, masked, F{});
            }
            if (i < end) { step(t0 + i, Q0{}, masked, F{}); ++i; }
            if (i < end) { step(t0 + i, Q1{}, masked, F{}); ++i; }
        };
        run(ua, TT{});
        run(ub, F{});
        run(nt, TT{});
        // The last steps issued loads past the range (zero-size, landing as zeros): let
        // them land before the workgroup can end and its LDS be reused.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // Drain: P V of the last tile (its V landed by the end of the last step).
        if (t1 - 1 >= wave_lo && t1 - 1 < wave_tc) {
            const int ph = (nt - 1) % 3;
            if (ph == 0) pv(vl(Q0{}), pk0);
            else if (ph == 1) pv(vl(Q1{}), pk1);
            else pv(vl(Q2{}), pk2);
        }
    }

    // l_run holds each lane's half of its row's keys: add the two halves.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] = xhalf_sum(l_run[qb]);

    if constexpr (C::KS > 1) {
        // Merge the two key parts' states through LDS, whose tile buffers are free once every
        // wave has done its last P V: part 1 stores (m, l, acc); part 0 folds them into its
        // own with the online-softmax rescale (both m in the same exp2 units) and goes on to
        // the epilogue; part 1 ends here.
        static_assert(C::KS == 2 && C::NWQ <= 4, "two key parts of at most four waves");
        static_assert(DB * 16 * 64 * 4 <= TILEK * C::KS && DB * 16 * 64 * 4 <= TILE * C::KS &&
                          C::NWQ * 64 * 8 <= TILE * C::KS,
                      "a wave's state fits one buffer array");
        __syncthreads();
        unsigned char* xa = wq == 0 ? k_lds0 : wq == 1 ? k_lds1 : wq == 2 ? k_lds2 : v_lds0;
        float* xml = (float*)v_lds1 + 2 * (wq * 64 + lane);
        if (kpart == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db) *(f32x16*)(xa + (db * 64 + lane) * 64) = acc[db][0];
            xml[0] = m_run[0];
            xml[1] = l_run[0];
        }
        __syncthreads();
        if (kpart == 1) return;
        const float m1 = xml[0], l1 = xml[1], m0 = m_run[0];
        const float m = fmaxf(m0, m1);
        const float a0 = m0 == -__builtin_inff() ? 0.0f : fast_exp2(m0 - m);
        const float a1 = m1 == -__builtin_inff() ? 0.0f : fast_exp2(m1 - m);
        m_run[0] = m;
        l_run[0] = a0 * l_run[0] + a1 * l1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            acc[db][0] = acc[db][0] * a0 + *(const f32x16*)(xa + (db * 64 + lane) * 64) * a1;
    }

    // Epilogue of a one-split, one-part call: O leaves through LDS so that every global
    // store writes whole 128-byte row segments.  A lane holds 16 consecutive d of one row
    // per 32-wide block (fp8 V: four runs of four), so direct stores would put 16-byte (8-byte)
    // pieces of each line into separate instructions; staged, eight lanes store one 128-byte
    // segment.  The stores are non-temporal: nothing reads O back, and it need not displace
    // K/V in L2.  Each wave stages its 32 rows x 64 d (4 KiB) in its own part of the tile
    // buffers, free once every wave is past its last P V (fp8 V: in o_stage); 16-byte chunks
    // XOR-swizzled by row / 2.
    if constexpr (C::KS == 1 && QB == 1) {
        if (p.num_splits == 1) {
            static_assert(V8 || (TILE >= 8192 && TILEK >= 4096 && C::NW <= 8), "eight 4 KiB stages");
            const size_t head_row0 = (size_t)(b * p.Hq + hq) * p.Sq;
            const float l = l_run[0];
            float inv = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;
            if constexpr (V8) inv *= p.o_scale;   // V's dequantisation factor
            if (h == 0 && qw0 + l32 < p.Sq)
                p.lse[head_row0 + qw0 + l32] =
                    l > 0.0f ? (m_run[0] + __builtin_amdgcn_logf(l)) * LN2 : -__builtin_inff();
            // Two stages per 8 KiB buffer (fp8 keys: 4 KiB K buffers, one stage each).
            unsigned char* sb;
            if constexpr (V8)
                sb = o_stage + w * 4096;
            else if constexpr (TILEK >= 8192)
                sb = (w >> 1 == 0 ? k_lds0 : w >> 1 == 1 ? k_lds1 : w >> 1 == 2 ? k_lds2 : v_lds0) + (w & 1) * 4096;
            else
                sb = w < 6 ? (w >> 1 == 0 ? v_lds0 : w >> 1 == 1 ? v_lds1 : v_lds2) + (w & 1) * 4096
                           : (w == 6 ? k_lds0 : k_lds1);
            __syncthreads();
#pragma unroll
            for (int ps = 0; ps < D / 64; ++ps) {
                if (ps > 0) __syncthreads();   // this wave's reads of the previous pass are done
#pragma unroll
                for (int dh = 0; dh < 2; ++dh) {
                    const f32x16 a = acc[2 * ps + dh][0] * inv;
                    const int sw = (l32 >> 1) & 7;
                    if constexpr (V8) {
                        // d = 32 db + 8t + 4h + 0..3 in slots 4t .. 4t+3: half h of chunk 4 dh + t.
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            *(u32x2*)(sb + l32 * 128 + (((4 * dh + t) ^ sw) << 4) + 8 * h) =
                                (u32x2){pack2<BF16>(a[4 * t], a[4 * t + 1]), pack2<BF16>(a[4 * t + 2], a[4 * t + 3])};
                    } else {
                        const u32x4 w0 = {pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]),
                                          pack2<BF16>(a[4], a[5]), pack2<BF16>(a[6], a[7])};
                        const u32x4 w1 = {pack2<BF16>(a[8], a[9]), pack2<BF16>(a[10], a[11]),
                                          pack2<BF16>(a[12], a[13]), pack2<BF16>(a[14], a[15])};
                        const int c = 4 * dh + 2 * h;
                        *(u32x4*)(sb + l32 * 128 + ((c ^ sw) << 4)) = w0;
                        *(u32x4*)(sb + l32 * 128 + (((c + 1) ^ sw) << 4)) = w1;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = 8 * k + (lane >> 3), c = lane & 7;
                    const u32x4 x = *(const u32x4*)(sb + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
                    if (qw0 + r < p.Sq)
                        __builtin_nontemporal_store(x, (u32x4*)((T*)p.o + (head_row0 + qw0 + r) * D + 64 * ps + 8 * c));
                }
            }
            return;
        }
    }

    // Epilogue: O = acc / l (v_rcp_f32); LSE = ln2 (m + log2 l), -inf for a row with no
    // visible key (l = 0, O = 0).  One split: O rounded to the storage type.  Several
    // splits: the normalised partial O in fp32 and its LSE, for the merge kernel.
    const size_t head_row0 = (size_t)(b * p.Hq + hq) * p.Sq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + qb * 32 + l32;
        if (row < p.Sq) {
            const float l = l_run[qb];
            float inv = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;
            if constexpr (V8) inv *= p.o_scale;   // V's dequantisation factor
            const float lse = l > 0.0f ? (m_run[qb] + __builtin_amdgcn_logf(l)) * LN2 : -__builtin_inff();
            if constexpr (V8) {
                // fp8 V: accumulator row m is d = 32 db + m, so the lane holds, for t = 0..3,
                // the four consecutive d = 32 db + 8t + 4h + 0..3 in slots 4t .. 4t+3.
                if (p.num_splits == 1) {
                    T* orow = (T*)p.o + (head_row0 + row) * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const f32x16 a = acc[db][qb] * inv;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            *(u32x2*)(orow + db * 32 + 8 * t + 4 * h) =
                                (u32x2){pack2<BF16>(a[4 * t], a[4 * t + 1]), pack2<BF16>(a[4 * t + 2], a[4 * t + 3])};
                    }
                    if (h == 0) p.lse[head_row0 + row] = lse;
                } else {
                    const size_t rows = (size_t)p.B * p.Hq * p.Sq;
                    float* orow = p.o_part + ((size_t)split * rows + head_row0 + row) * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const f32x16 a = acc[db][qb] * inv;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            *(f32x4*)(orow + db * 32 + 8 * t + 4 * h) =
                                (f32x4){a[4 * t], a[4 * t + 1], a[4 * t + 2], a[4 * t + 3]};
                    }
                    if (h == 0) p.lse_part[(size_t)split * rows + head_row0 + row] = lse;
                }
            } else if (p.num_splits == 1) {
                T* orow = (T*)p.o + (head_row0 + row) * D;
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
                if (h == 0) p.lse[head_row0 + row] = lse;
            } else {
                const size_t rows = (size_t)p.B * p.Hq * p.Sq;
                float* orow = p.o_part + ((size_t)split * rows + head_row0 + row) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const f32x16 a = acc[db][qb] * inv;
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4)
                        *(f32x4*)(orow + db * 32 + 16 * h + 4 * v4) =
                            (f32x4){a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]};
                }
                if (h == 0) p.lse_part[(size_t)split * rows + head_row0 + row] = lse;
            }
        }
    }
}

}  // namespace fa
