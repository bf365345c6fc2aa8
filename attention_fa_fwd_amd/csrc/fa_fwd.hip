// fa_fwd.hip -- host side of the attention forward library: argument validation, the
// static dispatch table, kernel launch, and the exported C ABI declared in fa_fwd.h.
//
// The dispatch table replaces the runtime autotuner of "Tuning Flash Attention for peak
// performance in NVIDIA CUDA Tile" (Part 2 "Autotuning") and the length threshold of
// "How I Beat PyTorch's Flash Attention" ("Phase 5: Adaptive Tile Dispatch"): a fixed
// list of compiled tile configurations and a deterministic rule that picks one from the
// problem shape, so the same call always runs the same kernel.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "fa_fwd.h"
#include "fa_configs.h"
#include "fa_fwd_kernel.hpp"
#include "fa_launch.hpp"
#include "fa_merge_kernel.hpp"

namespace {

using fa::Cfg;
using fa::Params;

typedef hipError_t (*LaunchFn)(const Params&, hipStream_t);

struct ConfigEntry {
    const char* name;
    int D, bf16, causal, qk8, v8;
    int BN, QB, WPH, HPW, KS;
    LaunchFn launch;
};

#define FA_TABLE_ENTRY(D, BN, QB, WPH, HPW, C, B, Q, V8, KS, CNAME, TNAME)                    \
    ConfigEntry{"D" FA_STR(D) "_BN" FA_STR(BN) "_Mw" FA_STR(QB) "x32_WPH" FA_STR(WPH)        \
                "_HPW" FA_STR(HPW) "_" CNAME "_" TNAME,                                        \
                D, B, C, Q, V8, BN, QB, WPH, HPW, KS,                                           \
                &fa_host::launch_cfg<Cfg<D, BN, QB, WPH, HPW, C, B, Q, V8, KS>>},
#define FA_STR2(x) #x
#define FA_STR(x) FA_STR2(x)

// Every compiled configuration (fa_configs.h), in table order.
const ConfigEntry kConfigs[] = {FA_LIST_ALL(FA_TABLE_ENTRY)};
constexpr int kNumConfigs = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));

// Largest split count: bounds the merge kernel's loop and the workspace.
constexpr int kMaxSplits = fa::kMergeMaxSplits;
// CUs of an MI355X, and the resident workgroups that fill it (two four-wave workgroups
// per CU).
constexpr long long kNumCUs = 256;
// Shortest key range for which the dispatch takes two key parts (see select).
constexpr int kKeyPartsMinKeys = 4096;
constexpr long long kFullGrid = 512;

hipError_t launch_merge(const Params& p, int D, int bf16, hipStream_t s) {
    const size_t rows = (size_t)p.B * p.Hq * p.Sq;
    const dim3 grid((unsigned)std::min<size_t>((rows + 3) / 4, (size_t)1 << 20)), block(256);
    if (D == 128) {
        if (bf16) hipLaunchKernelGGL((fa::fa_merge_kernel<128, true>), grid, block, 0, s, p.o_part, p.lse_part, p.o, p.lse, rows, p.num_splits);
        else hipLaunchKernelGGL((fa::fa_merge_kernel<128, false>), grid, block, 0, s, p.o_part, p.lse_part, p.o, p.lse, rows, p.num_splits);
    } else {
        if (bf16) hipLaunchKernelGGL((fa::fa_merge_kernel<64, true>), grid, block, 0, s, p.o_part, p.lse_part, p.o, p.lse, rows, p.num_splits);
        else hipLaunchKernelGGL((fa::fa_merge_kernel<64, false>), grid, block, 0, s, p.o_part, p.lse_part, p.o, p.lse, rows, p.num_splits);
    }
    return hipGetLastError();
}

bool overlaps(uintptr_t a, size_t na, uintptr_t b, size_t nb) {
    return a < b + nb && b < a + na;
}

// One call's arguments.  dtype is the element type of out (and of v unless v8, of q, k
// unless qk8); qk8: q and k are fp8 e4m3 with per-tensor dequantisation factors; v8: v
// too.
struct Call {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int B, Hq, Hkv, Sq, Skv, D;
    float scale;
    int causal, input_pos, window, dtype;
    int qk8, v8;
    float q_descale, k_descale, v_descale;
};

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

// Pure host validation: no HIP call.  Returns FA_OK or the first failing check.
int validate(const Call& a) {
    const int B = a.B, Hq = a.Hq, Hkv = a.Hkv, Sq = a.Sq, Skv = a.Skv, D = a.D;
    // A pointer may be NULL only when its tensor has no elements (an empty problem).
    const bool q_empty = B <= 0 || Hq <= 0 || Sq <= 0;
    const bool kv_empty = B <= 0 || Hkv <= 0 || Skv <= 0;
    if ((!q_empty && (!a.q || !a.out || !a.lse)) || (!kv_empty && (!a.k || !a.v)))
        return FA_ERR_NULL_POINTER;
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    // Head indices b*H + h are 32-bit in the kernel; byte sizes stay below 2^50.
    if ((long long)B * Hq > INT_MAX || (long long)B * Hkv > INT_MAX) return FA_ERR_INVALID_SHAPE;
    const double qe = (double)B * Hq * Sq * 128.0 * 2.0;
    const double ke = (double)B * Hkv * Skv * 128.0 * 2.0;
    if (qe > 1125899906842624.0 || ke > 1125899906842624.0) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (a.dtype != FA_DTYPE_FP16 && a.dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (!finite_pos(a.scale)) return FA_ERR_INVALID_SCALE;
    if (a.qk8 && (!finite_pos(a.q_descale) || !finite_pos(a.k_descale))) return FA_ERR_INVALID_SCALE;
    if (a.qk8 && !finite_pos(a.scale * a.q_descale * a.k_descale)) return FA_ERR_INVALID_SCALE;
    if (a.v8 && !finite_pos(a.v_descale)) return FA_ERR_INVALID_SCALE;
    if (a.input_pos < 0 || (long long)a.input_pos + Sq > INT_MAX) return FA_ERR_INVALID_INPUT_POS;
    if (a.window < 0 || (a.window > 0 && !a.causal)) return FA_ERR_INVALID_WINDOW;
    if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.out) & 15u)
        return FA_ERR_MISALIGNED;
    if ((uintptr_t)a.lse & 3u) return FA_ERR_MISALIGNED;
    const size_t qke = a.qk8 ? 1 : 2;
    const size_t qb = (size_t)B * Hq * Sq * D * qke, kb = (size_t)B * Hkv * Skv * D * qke;
    const size_t ob = (size_t)B * Hq * Sq * D * 2, vb = (size_t)B * Hkv * Skv * D * (a.v8 ? 1 : 2);
    const size_t lb = (size_t)B * Hq * Sq * 4;
    const uintptr_t o = (uintptr_t)a.out, l = (uintptr_t)a.lse;
    const uintptr_t q = (uintptr_t)a.q, k = (uintptr_t)a.k, v = (uintptr_t)a.v;
    if (ob > 0 && (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb) ||
                   overlaps(o, ob, l, lb) || overlaps(l, lb, q, qb) || overlaps(l, lb, k, kb) ||
                   overlaps(l, lb, v, vb)))
        return FA_ERR_ALIAS;
    return FA_OK;
}

bool applicable(const ConfigEntry& c, int Hq, int Hkv, int D, int causal, int dtype, int qk8,
                int v8) {
    const int group = Hq / Hkv;
    return c.D == D && c.bf16 == (dtype == FA_DTYPE_BF16) && c.causal == (causal != 0) &&
           c.qk8 == (qk8 != 0) && c.v8 == (v8 != 0) && group % c.HPW == 0;
}

int find(int D, int bf16, int causal, int qk8, int v8, int BN, int QB, int WPH, int HPW, int KS = 1) {
    for (int i = 0; i < kNumConfigs; ++i) {
        const ConfigEntry& c = kConfigs[i];
        if (c.D == D && c.bf16 == bf16 && c.causal == causal && c.qk8 == qk8 && c.v8 == v8 &&
            c.BN == BN && c.QB == QB && c.WPH == WPH && c.HPW == HPW && c.KS == KS)
            return i;
    }
    return -1;
}

// A configuration with two key parts splits each workgroup's key tiles into two equal runs:
// it needs one key split and an even number of key tiles.
bool key_parts_fit(const ConfigEntry& c, int Skv, int num_splits) {
    return c.KS == 1 || (num_splits == 1 && ((Skv + c.BN - 1) / c.BN) % c.KS == 0);
}

// Workgroups of the unsplit grid of configuration c.
long long grid_of(const ConfigEntry& c, int B, int Hq, int Hkv, int Sq) {
    const int bmp = 32 * c.QB * c.WPH;
    return (long long)((Sq + bmp - 1) / bmp) * (Hq / Hkv / c.HPW) * B * Hkv;
}

// The dispatch rule, from a sweep of every configuration on the named workloads (timed
// after the GPU has reached its working clock): 32-key tiles for head dim 128 (fewer live
// registers, so the pipelined loop hides more latency), 64-key tiles for head dim 64.
// Grouped-query problems pack 4 (or 2) query heads of a group into one workgroup, so each
// K/V tile is read once for all of them.  An 8-wave workgroup (a whole CU: its K/V tiles
// shared by twice the waves) beats two 4-wave ones when it still forms at least one
// workgroup per CU; smaller grids use 4-wave workgroups for more of them.
int select(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, int dtype, int qk8, int v8 = 0) {
    const int bf16 = dtype == FA_DTYPE_BF16;
    const int cz = causal != 0;
    const int q8 = qk8 != 0;
    const int x8 = v8 != 0;
    const int group = Hq / Hkv;
    const int bn = D == 128 ? 32 : 64;
    int big, small;
    if (group % 8 == 0 && D == 128) {
        // All eight heads of a group on one 32-row block: the K/V tile is shared by eight
        // waves as with 2 x 4, and the waves reach the causal diagonal together.
        big = find(D, bf16, cz, q8, x8, bn, 1, 1, 8);
        small = find(D, bf16, cz, q8, x8, bn, 1, 1, 4);
    } else if (group % 4 == 0) {
        big = find(D, bf16, cz, q8, x8, bn, 1, 2, 4);
        small = find(D, bf16, cz, q8, x8, bn, 1, 1, 4);
    } else if (group % 2 == 0) {
        big = find(D, bf16, cz, q8, x8, bn, 1, 4, 2);
        small = find(D, bf16, cz, q8, x8, bn, 1, 2, 2);
    } else {
        big = find(D, bf16, cz, q8, x8, bn, 1, 8, 1);
        small = find(D, bf16, cz, q8, x8, bn, 1, 4, 1);
    }
    if (big >= 0 && grid_of(kConfigs[big], B, Hq, Hkv, Sq) >= kNumCUs) return big;
    // At most one four-wave workgroup per CU leaves one wave per SIMD, so nothing overlaps one
    // wave's softmax with another's MFMAs.  A non-causal call over at least kKeyPartsMinKeys
    // keys whose key tiles split evenly takes the two-key-part twin instead: the same
    // workgroups with twice the waves, each half of them on half of the keys.  Measured against
    // the one-part kernel: 8% faster at 16K keys with 256 workgroups, 17-19% with 64-128, 2-6%
    // at 4K keys, and 4% slower at 1K keys, where the doubled tile loads and the merge are not
    // paid back.
    if (!cz && !q8 && !x8 && small >= 0 && Skv >= kKeyPartsMinKeys &&
        grid_of(kConfigs[small], B, Hq, Hkv, Sq) <= kNumCUs) {
        const ConfigEntry& c = kConfigs[small];
        const int twin = find(D, bf16, cz, q8, x8, bn, 1, c.WPH, c.HPW, 2);
        if (twin >= 0 && key_parts_fit(kConfigs[twin], Skv, 1)) return twin;
    }
    return small;
}

// Workgroup -> XCD mapping.  The hardware hands workgroup w to XCD w % 8.  Mode 1 gives
// each XCD whole (batch, K/V head) groups; mode 2 spreads each group over 8/ngrp XCDs.
void xcd_mapping(int ngrp, int items_per_group, int* mode, int* arg) {
    const long long n = (long long)ngrp * items_per_group;
    *mode = 0;
    *arg = 0;
    if (n % fa::kNumXcd != 0) return;
    if (ngrp % fa::kNumXcd == 0) {
        *mode = 1;
        *arg = ngrp / fa::kNumXcd;
    } else if (fa::kNumXcd % ngrp == 0 && items_per_group % (fa::kNumXcd / ngrp) == 0) {
        *mode = 2;
        *arg = fa::kNumXcd / ngrp;
    }
}

// Bytes of split-KV workspace: the fp32 partial O [S][B*Hq*Sq][D], then the fp32 partial
// LSE [S][B*Hq*Sq].  Zero for one split.
size_t workspace_bytes_for(int B, int Hq, int Sq, int D, int num_splits) {
    if (num_splits <= 1 || B <= 0 || Hq <= 0 || Sq <= 0) return 0;
    return (size_t)num_splits * B * Hq * Sq * (size_t)(D + 1) * sizeof(float);
}

// Tiles of the longest key range of any query tile (all keys, the causal extent, or a
// sliding window plus the query tile's own positions).
int max_key_tiles(const ConfigEntry& c, int Sq, int Skv, int causal, int input_pos, int window) {
    long long vis = causal ? std::min<long long>((long long)input_pos + Sq, Skv) : Skv;
    if (causal && window > 0) vis = std::min<long long>(vis, (long long)window + 32 * c.QB * c.WPH);
    return (int)((vis + c.BN - 1) / c.BN);
}

// Split count for num_splits = 0.  Splitting pays only when the plain grid leaves CUs idle
// (fewer workgroups than CUs): then enough ranges for about kFullGrid workgroups, with at
// least 8 key tiles per range, and no more ranges than keep the partials' fp32 traffic
// (written once, read once by the merge) within the K/V bytes the kernel reads.  Chosen
// from measured sweeps: decoding with 8 to 128 workgroups runs fastest at ~512 after the
// split; a 256-workgroup prefill loses to the partial traffic.
int auto_splits(const ConfigEntry& c, const Call& a) {
    const long long wgs = grid_of(c, a.B, a.Hq, a.Hkv, a.Sq);
    if (wgs <= 0 || wgs >= kNumCUs) return 1;
    const long long want = (kFullGrid + wgs - 1) / wgs;
    const int tiles = max_key_tiles(c, a.Sq, a.Skv, a.causal, a.causal ? a.input_pos : 0,
                                    a.causal ? a.window : 0);
    const long long by_len = tiles / 8;
    const double kv_elem_bytes = (a.qk8 ? 1.0 : 2.0) + (a.v8 ? 1.0 : 2.0);   // K + V bytes
    const double kv_bytes = kv_elem_bytes * a.B * a.Hkv * std::min<double>(a.Skv, (double)tiles * c.BN) * c.D;
    const double part_bytes = 8.0 * a.B * a.Hq * (double)a.Sq * (c.D + 1);   // per range
    const long long by_traffic = (long long)(kv_bytes / part_bytes);
    return (int)std::max(1LL, std::min({want, by_len, by_traffic, (long long)kMaxSplits}));
}

int resolve_config(int config, const Call& a) {
    if (config < -1 || config >= kNumConfigs) return FA_ERR_INVALID_CONFIG;
    if (config == -1) config = select(a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D, a.causal, a.dtype, a.qk8, a.v8);
    if (config < 0) return FA_ERR_INVALID_CONFIG;
    if (!applicable(kConfigs[config], a.Hq, a.Hkv, a.D, a.causal, a.dtype, a.qk8, a.v8) ||
        !key_parts_fit(kConfigs[config], a.Skv, 1))
        return FA_ERR_INVALID_CONFIG;
    return config;
}

// Configuration and split count of a split-KV call (num_splits 0 = the split rule).  A
// two-key-part configuration runs one split: when the call splits keys, the table's choice
// falls back to its one-part twin, and a forced two-part configuration is an error.
int plan_splitkv(const Call& a, int config, int num_splits, int* config_out, int* splits_out) {
    const int forced = config;
    config = resolve_config(config, a);
    if (config < 0) return config;
    if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID_SPLITS;
    const ConfigEntry& c = kConfigs[config];
    if (num_splits == 0) num_splits = auto_splits(c, a);   // the grid does not depend on KS
    if (c.KS > 1 && num_splits > 1) {
        if (forced != -1) return FA_ERR_INVALID_CONFIG;
        config = find(c.D, c.bf16, c.causal, c.qk8, c.v8, c.BN, c.QB, c.WPH, c.HPW, 1);
        if (config < 0) return FA_ERR_INVALID_CONFIG;
    }
    *config_out = config;
    *splits_out = num_splits;
    return FA_OK;
}

// num_splits: 1 = the plain forward pass (out / lse written by the attention kernel);
// > 1 = partials into `workspace`, then the merge kernel.  Arguments already validated.
int launch(const Call& a, int config, int num_splits, void* workspace, void* stream) {
    const ConfigEntry& c = kConfigs[config];
    const int bmp = 32 * c.QB * c.WPH;
    Params p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.out;
    p.lse = a.lse;
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.Sq = a.Sq;
    p.Skv = a.Skv;
    p.input_pos = a.causal ? a.input_pos : 0;
    p.window = a.causal ? a.window : 0;
    // scale * log2(e), with the fp8 dequantisation factors of q and k folded in.
    double c2 = (double)a.scale * 1.4426950408889634073599246810019;
    if (a.qk8) c2 *= (double)a.q_descale * (double)a.k_descale;
    p.c = (float)c2;
    p.group = a.Hq / a.Hkv;
    p.n_tiles = (a.Sq + bmp - 1) / bmp;
    p.hsub = p.group / c.HPW;
    p.num_splits = num_splits;
    p.o_part = nullptr;
    p.lse_part = nullptr;
    p.o_scale = a.v8 ? a.v_descale : 1.0f;
    if (num_splits > 1) {
        const size_t rows = (size_t)a.B * a.Hq * a.Sq;
        p.o_part = (float*)workspace;
        p.lse_part = (float*)workspace + (size_t)num_splits * rows * c.D;
    }
    const long long wgs = (long long)p.n_tiles * p.hsub * a.B * a.Hkv * num_splits;
    if (wgs > 0x7fffffffLL) return FA_ERR_INVALID_SHAPE;
    xcd_mapping(a.B * a.Hkv, p.n_tiles * p.hsub * num_splits, &p.map_mode, &p.map_arg);
    hipStream_t s = (hipStream_t)stream;
    if (c.launch(p, s) != hipSuccess) return FA_ERR_LAUNCH;
    if (num_splits > 1 && launch_merge(p, c.D, c.bf16, s) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
}

int run(const Call& a, void* stream, int config) {
    int rc = validate(a);
    if (rc != FA_OK) return rc;
    config = resolve_config(config, a);
    if (config < 0) return config;
    if ((long long)a.B * a.Hq * a.Sq == 0) return FA_OK;
    return launch(a, config, 1, nullptr, stream);
}

int run_splitkv(const Call& a, int num_splits, int config, void* workspace,
                size_t workspace_bytes, void* stream) {
    int rc = validate(a);
    if (rc != FA_OK) return rc;
    rc = plan_splitkv(a, config, num_splits, &config, &num_splits);
    if (rc != FA_OK) return rc;
    if ((long long)a.B * a.Hq * a.Sq == 0) return FA_OK;
    if (num_splits > 1) {
        const size_t need = workspace_bytes_for(a.B, a.Hq, a.Sq, a.D, num_splits);
        if (!workspace) return FA_ERR_NULL_POINTER;
        if ((uintptr_t)workspace & 15u) return FA_ERR_MISALIGNED;
        if (workspace_bytes < need) return FA_ERR_WORKSPACE;
        const size_t qke = a.qk8 ? 1 : 2;
        const size_t qb = (size_t)a.B * a.Hq * a.Sq * a.D * qke;
        const size_t kb = (size_t)a.B * a.Hkv * a.Skv * a.D * qke;
        const size_t ob = (size_t)a.B * a.Hq * a.Sq * a.D * 2;
        const size_t vb = (size_t)a.B * a.Hkv * a.Skv * a.D * (a.v8 ? 1 : 2);
        const size_t lb = (size_t)a.B * a.Hq * a.Sq * 4;
        const uintptr_t w = (uintptr_t)workspace;
        if (overlaps(w, need, (uintptr_t)a.q, qb) || overlaps(w, need, (uintptr_t)a.k, kb) ||
            overlaps(w, need, (uintptr_t)a.v, vb) || overlaps(w, need, (uintptr_t)a.out, ob) ||
            overlaps(w, need, (uintptr_t)a.lse, lb))
            return FA_ERR_ALIAS;
    }
    return launch(a, config, num_splits, workspace, stream);
}

// --- Scratch of fa_fwd_splitkv_noalloc --------------------------------------------------
// The split-KV partials of callers that cannot allocate device memory live in this array.
// Each GPU the library runs on holds its own copy, at its own address, until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device memory: the
// address of a device's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)FA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return FA_ERR_LAUNCH;
    }
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
                (void)hipGetLastError();
                return FA_ERR_LAUNCH;
            }
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return FA_OK;
}

// fa_fwd_splitkv with the partials in `scratch` instead of a caller's workspace.
int run_splitkv_noalloc(const Call& a, int num_splits, int config, void* stream) {
    int rc = validate(a);
    if (rc != FA_OK) return rc;
    rc = plan_splitkv(a, config, num_splits, &config, &num_splits);
    if (rc != FA_OK) return rc;
    if ((long long)a.B * a.Hq * a.Sq == 0) return FA_OK;
    void* ws = nullptr;
    if (num_splits > 1) {
        if (workspace_bytes_for(a.B, a.Hq, a.Sq, a.D, num_splits) > kScratchBytes)
            return FA_ERR_SCRATCH;
        rc = scratch_address(&ws);
        if (rc != FA_OK) return rc;
    }
    return launch(a, config, num_splits, ws, stream);
}

Call make_call(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
               int Hkv, int Sq, int Skv, int D, float scale, int causal, int input_pos,
               int window, int dtype) {
    Call a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Skv = Skv;
    a.D = D;
    a.scale = scale;
    a.causal = causal;
    a.input_pos = input_pos;
    a.window = window;
    a.dtype = dtype;
    a.qk8 = 0;
    a.v8 = 0;
    a.q_descale = 1.0f;
    a.k_descale = 1.0f;
    a.v_descale = 1.0f;
    return a;
}

Call make_call_fp8qkv(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                      int Hq, int Hkv, int Sq, int Skv, int D, float scale, float q_descale,
                      float k_descale, float v_descale, int causal, int input_pos, int window,
                      int out_dtype) {
    Call a = make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, input_pos,
                       window, out_dtype);
    a.qk8 = 1;
    a.v8 = 1;
    a.q_descale = q_descale;
    a.k_descale = k_descale;
    a.v_descale = v_descale;
    return a;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
           int Hkv, int Sq, int Skv, int D, float scale, int causal, int input_pos, int dtype,
           void* stream) {
    return run(make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, input_pos, 0,
                         dtype),
               stream, -1);
}

int fa_fwd_config(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                  int input_pos, int dtype, void* stream, int config) {
    return run(make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, input_pos, 0,
                         dtype),
               stream, config);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, float scale, int input_pos,
                  int window, int dtype, void* stream, int config) {
    // window < 1 is invalid here; -1 lets validate() report it in its documented place.
    return run(make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, 1, input_pos,
                         window < 1 ? -1 : window, dtype),
               stream, config);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
               int Hq, int Hkv, int Sq, int Skv, int D, float scale, float q_descale,
               float k_descale, int causal, int input_pos, int window, int v_dtype,
               void* stream, int config) {
    Call a = make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, input_pos,
                       window, v_dtype);
    a.qk8 = 1;
    a.q_descale = q_descale;
    a.k_descale = k_descale;
    return run(a, stream, config);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                   int input_pos, int window, int dtype, int num_splits, int config,
                   void* workspace, size_t workspace_bytes, void* stream) {
    return run_splitkv(make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal,
                                 input_pos, window, dtype),
                       num_splits, config, workspace, workspace_bytes, stream);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                           int causal, int input_pos, int window, int dtype, int num_splits,
                           int config, void* stream) {
    return run_splitkv_noalloc(make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale,
                                         causal, input_pos, window, dtype),
                               num_splits, config, stream);
}

int fa_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int D, float scale, float q_descale,
                       float k_descale, int causal, int input_pos, int window, int v_dtype,
                       int num_splits, int config, void* workspace, size_t workspace_bytes,
                       void* stream) {
    Call a = make_call(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, input_pos,
                       window, v_dtype);
    a.qk8 = 1;
    a.q_descale = q_descale;
    a.k_descale = k_descale;
    return run_splitkv(a, num_splits, config, workspace, workspace_bytes, stream);
}
int fa_splitkv_num_splits_fp8(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                              int input_pos, int window, int v_dtype, int config) {
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (v_dtype != FA_DTYPE_FP16 && v_dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (input_pos < 0 || (long long)input_pos + Sq > INT_MAX) return FA_ERR_INVALID_INPUT_POS;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_WINDOW;
    Call a = make_call(nullptr, nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Sq, Skv, D, 1.0f,
                       causal, input_pos, window, v_dtype);
    a.qk8 = 1;
    int splits = 0;
    const int rc = plan_splitkv(a, config, 0, &config, &splits);
    return rc != FA_OK ? rc : splits;
}
int fa_fwd_fp8qkv(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, float scale, float q_descale,
                  float k_descale, float v_descale, int causal, int input_pos, int window,
                  int out_dtype, void* stream, int config) {
    return run(make_call_fp8qkv(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, q_descale,
                                k_descale, v_descale, causal, input_pos, window, out_dtype),
               stream, config);
}

int fa_fwd_splitkv_fp8qkv(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                          float q_descale, float k_descale, float v_descale, int causal,
                          int input_pos, int window, int out_dtype, int num_splits, int config,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return run_splitkv(make_call_fp8qkv(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale,
                                        q_descale, k_descale, v_descale, causal, input_pos,
                                        window, out_dtype),
                       num_splits, config, workspace, workspace_bytes, stream);
}

int fa_splitkv_num_splits_fp8qkv(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                                 int input_pos, int window, int out_dtype, int config) {
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (out_dtype != FA_DTYPE_FP16 && out_dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (input_pos < 0 || (long long)input_pos + Sq > INT_MAX) return FA_ERR_INVALID_INPUT_POS;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_WINDOW;
    const Call a = make_call_fp8qkv(nullptr, nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Sq,
                                    Skv, D, 1.0f, 1.0f, 1.0f, 1.0f, causal, input_pos, window,
                                    out_dtype);
    int splits = 0;
    const int rc = plan_splitkv(a, config, 0, &config, &splits);
    return rc != FA_OK ? rc : splits;
}

int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                          int input_pos, int window, int dtype, int config) {
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (input_pos < 0 || (long long)input_pos + Sq > INT_MAX) return FA_ERR_INVALID_INPUT_POS;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_WINDOW;
    const Call a = make_call(nullptr, nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Sq, Skv, D,
                             1.0f, causal, input_pos, window, dtype);
    int splits = 0;
    const int rc = plan_splitkv(a, config, 0, &config, &splits);
    return rc != FA_OK ? rc : splits;
}

size_t fa_splitkv_workspace_size(int B, int Hq, int Sq, int D, int num_splits) {
    if (D != 64 && D != 128) return 0;
    return workspace_bytes_for(B, Hq, Sq, D, num_splits);
}

int fa_select_config(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, int input_pos,
                     int dtype) {
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1 || Skv < 1) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    if (input_pos < 0) return FA_ERR_INVALID_INPUT_POS;
    const int c = select(B, Hq, Hkv, Sq, Skv, D, causal, dtype, 0);
    return c < 0 ? FA_ERR_INVALID_CONFIG : c;
}

int fa_select_config_fp8(int B, int Hq, int Hkv, int Sq, int D, int causal, int v_dtype) {
    if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 1) return FA_ERR_INVALID_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (v_dtype != FA_DTYPE_FP16 && v_dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED_DTYPE;
    const int c = select(B, Hq, Hkv, Sq, 1, D, causal, v_dtype, 1);
    return c < 0 ? FA_ERR_INVALID_CONFIG : c;
}

int fa_num_configs(void) { return kNumConfigs; }

const char* fa_config_name(int config) {
    return (config >= 0 && config < kNumConfigs) ? kConfigs[config].name : nullptr;
}

const char* fa_strerror(int code) {
    switch (code) {
        case FA_OK: return "success";
        case FA_ERR_NULL_POINTER: return "a tensor pointer is NULL";
        case FA_ERR_INVALID_SHAPE: return "invalid sizes (B, Hq, Sq >= 0; Hkv, Skv >= 1; sizes too large)";
        case FA_ERR_HEAD_GROUP: return "Hq is not a multiple of Hkv";
        case FA_ERR_UNSUPPORTED_HEAD_DIM: return "head dim must be 64 or 128";
        case FA_ERR_UNSUPPORTED_DTYPE: return "dtype must be FA_DTYPE_FP16 or FA_DTYPE_BF16";
        case FA_ERR_INVALID_SCALE: return "scale must be finite and > 0";
        case FA_ERR_INVALID_INPUT_POS: return "input_pos must be >= 0 and input_pos + Sq must fit in int";
        case FA_ERR_MISALIGNED: return "q/k/v/out must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_ALIAS: return "out or lse overlaps an input or each other";
        case FA_ERR_INVALID_CONFIG: return "kernel configuration id out of range or not applicable to this call";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_INVALID_SPLITS: return "num_splits must be in 0..256";
        case FA_ERR_WORKSPACE: return "workspace smaller than fa_splitkv_workspace_size() / fa_bwd_workspace_size()";
        case FA_ERR_INVALID_WINDOW: return "window must be >= 0, needs causal masking, and >= 1 for fa_fwd_window";
        case FA_ERR_SCRATCH: return "split-KV partials larger than the fixed scratch of fa_fwd_splitkv_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status code";
    }
}

}  // extern "C"
