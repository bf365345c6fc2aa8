// fa_configs.h -- the compiled forward-kernel configurations, as X-macro lists.
//
// X(D, BN, QB, WPH, HPW, CAUSAL, BF16, QK8, V8, KS, CNAME, TNAME) is applied to every
// configuration; fa_fwd.hip builds its dispatch table from the lists and the fa_inst_*.hip
// files instantiate the kernels (one list per file, so they compile in parallel).  The
// lists' order is the order of the table (configuration ids).
#pragma once

// Head dim 64: 64-key tiles; 4 or 8 waves (WPH position blocks x HPW query heads).
#define FA_SHAPES_BN64Q(X, D, C, B, Q, V8, CN, TN)                                             \
    X(D, 64, 1, 1, 4, C, B, Q, V8, 1, CN, TN) X(D, 64, 1, 2, 4, C, B, Q, V8, 1, CN, TN)             \
    X(D, 64, 1, 2, 2, C, B, Q, V8, 1, CN, TN) X(D, 64, 1, 4, 2, C, B, Q, V8, 1, CN, TN)             \
    X(D, 64, 1, 4, 1, C, B, Q, V8, 1, CN, TN) X(D, 64, 1, 8, 1, C, B, Q, V8, 1, CN, TN)
#define FA_SHAPES_BN64(X, D, C, B, CN, TN) FA_SHAPES_BN64Q(X, D, C, B, false, false, CN, TN)

// Head dim 128: 32-key tiles (a 32 x 64 tile is too small to split over 512 threads, and
// with three LDS buffers and three register sets a 64-key tile does not fit two waves per
// SIMD).  1 x 8: all eight query heads of a GQA-8 group on one 32-row block.
#define FA_SHAPES_BN32(X, C, B, Q, V8, CN, TN)                                                 \
    X(128, 32, 1, 1, 4, C, B, Q, V8, 1, CN, TN) X(128, 32, 1, 2, 4, C, B, Q, V8, 1, CN, TN)       \
    X(128, 32, 1, 2, 2, C, B, Q, V8, 1, CN, TN) X(128, 32, 1, 4, 2, C, B, Q, V8, 1, CN, TN)       \
    X(128, 32, 1, 4, 1, C, B, Q, V8, 1, CN, TN) X(128, 32, 1, 8, 1, C, B, Q, V8, 1, CN, TN)       \
    X(128, 32, 1, 1, 8, C, B, Q, V8, 1, CN, TN)

#define FA_LIST_D64(X)                                                                      \
    FA_SHAPES_BN64(X, 64, true, true, "causal", "bf16")                                     \
    FA_SHAPES_BN64(X, 64, false, true, "full", "bf16")                                      \
    FA_SHAPES_BN64(X, 64, true, false, "causal", "fp16")                                    \
    FA_SHAPES_BN64(X, 64, false, false, "full", "fp16")
#define FA_LIST_D128_BF16(X)                                                                \
    FA_SHAPES_BN32(X, true, true, false, false, "causal", "bf16")                                  \
    FA_SHAPES_BN32(X, false, true, false, false, "full", "bf16")
#define FA_LIST_D128_FP16(X)                                                                \
    FA_SHAPES_BN32(X, true, false, false, false, "causal", "fp16")                                 \
    FA_SHAPES_BN32(X, false, false, false, false, "full", "fp16")
// "fp8qk": Q and K in fp8 E4M3.
#define FA_LIST_FP8_BF16(X)                                                                 \
    FA_SHAPES_BN32(X, true, true, true, false, "causal", "fp8qk_bf16")                             \
    FA_SHAPES_BN32(X, false, true, true, false, "full", "fp8qk_bf16")
#define FA_LIST_FP8_FP16(X)                                                                 \
    FA_SHAPES_BN32(X, true, false, true, false, "causal", "fp8qk_fp16")                            \
    FA_SHAPES_BN32(X, false, false, true, false, "full", "fp8qk_fp16")

// "fp8qkv": Q, K and V in fp8 E4M3; O (and P) in bf16 / fp16.
#define FA_LIST_FP8QKV_BF16(X)                                                              \
    FA_SHAPES_BN32(X, true, true, true, true, "causal", "fp8qkv_bf16")                      \
    FA_SHAPES_BN32(X, false, true, true, true, "full", "fp8qkv_bf16")
#define FA_LIST_FP8QKV_FP16(X)                                                              \
    FA_SHAPES_BN32(X, true, false, true, true, "causal", "fp8qkv_fp16")                     \
    FA_SHAPES_BN32(X, false, false, true, true, "full", "fp8qkv_fp16")

// fp8 at head dim 64 (64-key tiles): "fp8qk" and "fp8qkv", bf16 and fp16 output.
#define FA_LIST_FP8_D64(X)                                                                  \
    FA_SHAPES_BN64Q(X, 64, true, true, true, false, "causal", "fp8qk_bf16")                 \
    FA_SHAPES_BN64Q(X, 64, false, true, true, false, "full", "fp8qk_bf16")                  \
    FA_SHAPES_BN64Q(X, 64, true, false, true, false, "causal", "fp8qk_fp16")                \
    FA_SHAPES_BN64Q(X, 64, false, false, true, false, "full", "fp8qk_fp16")
#define FA_LIST_FP8QKV_D64(X)                                                               \
    FA_SHAPES_BN64Q(X, 64, true, true, true, true, "causal", "fp8qkv_bf16")                 \
    FA_SHAPES_BN64Q(X, 64, false, true, true, true, "full", "fp8qkv_bf16")                  \
    FA_SHAPES_BN64Q(X, 64, true, false, true, true, "causal", "fp8qkv_fp16")                \
    FA_SHAPES_BN64Q(X, 64, false, false, true, true, "full", "fp8qkv_fp16")

// Two key parts (KS = 2): the four-wave shapes doubled, the second set of waves taking the
// second half of the key tiles and the two states merged at the end -- two waves per SIMD for
// non-causal grids that leave one wave per SIMD otherwise.  Non-causal fp16 / bf16 only.
#define FA_SHAPES_KS2(X, D, BN, B, TN)                                                      \
    X(D, BN, 1, 1, 4, false, B, false, false, 2, "KS2_full", TN)                            \
    X(D, BN, 1, 2, 2, false, B, false, false, 2, "KS2_full", TN)                            \
    X(D, BN, 1, 4, 1, false, B, false, false, 2, "KS2_full", TN)
#define FA_LIST_KS2(X)                                                                      \
    FA_SHAPES_KS2(X, 128, 32, true, "bf16") FA_SHAPES_KS2(X, 128, 32, false, "fp16")        \
    FA_SHAPES_KS2(X, 64, 64, true, "bf16") FA_SHAPES_KS2(X, 64, 64, false, "fp16")

#define FA_LIST_ALL(X)                                                                      \
    FA_LIST_D64(X) FA_LIST_D128_BF16(X) FA_LIST_D128_FP16(X) FA_LIST_FP8_BF16(X)            \
    FA_LIST_FP8_FP16(X) FA_LIST_FP8QKV_BF16(X) FA_LIST_FP8QKV_FP16(X) FA_LIST_FP8_D64(X)    \
    FA_LIST_FP8QKV_D64(X) FA_LIST_KS2(X)
