/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) FlashAttention-style attention forward pass.
 *
 * The operation (sources cited by page title and section):
 *   "Tuning Flash Attention for peak performance in NVIDIA CUDA Tile" (NVIDIA cuTile post):
 *     "What is attention?"        O = softmax(scale * Q K^T + M) V per (batch, query head);
 *     "Causal attention"          M = 0 where key j <= input_pos + i, -inf elsewhere;
 *     "Grouped-query attention"   query head h reads K/V head h / (Hq / Hkv);
 *     Part 1 "Initializing accumulators" / "The main loop over K/V tiles": the query
 *       position carries an offset input_pos (a chunk of new queries against a cache);
 *     "Launching the kernel: Host-side code": contiguous [B, H, S, D] tensors, an output
 *       of the query's dtype, default scale 1/sqrt(D), launch on the caller's stream.
 *   The log-sum-exp output is on no page: LSE[b,h,i] = ln sum_{j visible} exp(scale q_i.k_j),
 *   the natural-log normaliser of each softmax row.
 *
 * Layout (row-major, contiguous, no strides):
 *   q, out : [B, Hq,  Sq,  D]  elements of `dtype` (out has q's dtype)
 *   k, v   : [B, Hkv, Skv, D]  elements of `dtype`
 *   lse    : [B, Hq,  Sq]      float32
 * All pointers are device pointers.  q, k, v and out must be 16-byte aligned (the kernels
 * move 128-bit vectors); lse must be 4-byte aligned.  out and lse must not overlap the
 * inputs or each other.
 *
 * Ownership: the caller owns every buffer (including fa_fwd_splitkv's workspace).  The
 * library allocates nothing, keeps no state besides constant tables, and may be called
 * from several host threads at once.
 *
 * Asynchrony: the call validates its arguments on the host (no HIP call), enqueues its
 * kernels (fa_fwd: one; fa_fwd_splitkv(_fp8): two; fa_bwd: three, or four when the GQA group is
 * split) on `stream` (a hipStream_t passed as void*; NULL = the null stream) and returns
 * without synchronising.  Faults inside a kernel surface on the next synchronisation.
 *
 * Errors: a nonzero return leaves every output untouched and launches nothing, except
 * FA_ERR_LAUNCH, which reports a failed launch.  Checks run in the order of the codes below,
 * except that the window check (FA_ERR_INVALID_WINDOW) follows the input_pos check.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and out.  Scores, softmax state and the accumulator are fp32. */
enum fa_dtype {
    FA_DTYPE_FP16 = 0,
    FA_DTYPE_BF16 = 1
};

/* Status codes, in the order the arguments are checked. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = -1,         /* a pointer is NULL although its tensor is not empty  */
    FA_ERR_INVALID_SHAPE = -2,        /* B, Hq, Sq < 0; Hkv, Skv < 1; B*H > INT_MAX; >= 2^50 B */
    FA_ERR_HEAD_GROUP = -3,           /* Hq is not a multiple of Hkv                          */
    FA_ERR_UNSUPPORTED_HEAD_DIM = -4, /* D not in {64, 128}                                   */
    FA_ERR_UNSUPPORTED_DTYPE = -5,    /* dtype not an fa_dtype                                */
    FA_ERR_INVALID_SCALE = -6,        /* scale not finite or not > 0                          */
    FA_ERR_INVALID_INPUT_POS = -7,    /* input_pos < 0, or input_pos + Sq overflows int       */
    FA_ERR_MISALIGNED = -8,           /* q/k/v/out not 16-byte or lse not 4-byte aligned      */
    FA_ERR_ALIAS = -9,                /* out or lse overlaps an input or each other           */
    FA_ERR_INVALID_CONFIG = -10,      /* fa_fwd_config: config id unknown or not applicable  */
    FA_ERR_LAUNCH = -11,              /* the kernel launch failed (hipGetLastError)           */
    FA_ERR_INVALID_SPLITS = -12,      /* fa_fwd_splitkv: num_splits outside 0..256            */
    FA_ERR_WORKSPACE = -13,           /* fa_fwd_splitkv, fa_bwd: workspace_bytes too small    */
    FA_ERR_INVALID_WINDOW = -14,      /* window < 0, window > 0 without causal masking, or    */
                                      /* fa_fwd_window with window < 1                        */
    FA_ERR_SCRATCH = -15              /* fa_fwd_splitkv_noalloc: partials exceed its scratch  */
};

/*
 * Attention forward pass: out = softmax(scale * q k^T + mask) v and lse, per (b, hq).
 *
 *   B, Hq, Hkv, Sq, Skv, D   sizes as in the layouts above; Hq % Hkv == 0, D in {64, 128}.
 *   scale                    multiplies q.k before the softmax; finite and > 0 (1/sqrt(D)
 *                            is the usual value).
 *   causal                   nonzero: query i sees key j iff j <= input_pos + i.
 *                            zero: every key is visible and input_pos is ignored.
 *   input_pos                position of query 0 (>= 0); input_pos = Skv - Sq aligns the
 *                            last query with the last key (a new chunk against a cache).
 *   dtype                    an fa_dtype.
 *   stream                   hipStream_t to enqueue on (NULL = null stream).
 * B*Hq*Sq == 0 returns FA_OK without a launch; pointers of empty tensors may then be NULL.
 * Returns an fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
           int causal, int input_pos, int dtype, void* stream);

/*
 * Same as fa_fwd, but runs kernel configuration `config` (0 <= config < fa_num_configs())
 * instead of the one the dispatch table picks; config = -1 uses the table.  A configuration
 * whose head dim, dtype, causality or head grouping does not fit the call returns
 * FA_ERR_INVALID_CONFIG, and so does a two-key-part one ("_KS2_" in its name: non-causal,
 * the key tiles split between two sets of waves) when ceil(Skv / its key tile) is odd.
 * Meant for tests and tile sweeps.
 */
int fa_fwd_config(const void* q, const void* k, const void* v, void* out, float* lse,
                  int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                  int causal, int input_pos, int dtype, void* stream, int config);

/*
 * Sliding-window causal attention: query i sees key j iff
 *     input_pos + i - window + 1 <= j <= input_pos + i,
 * the `window` most recent keys up to its own position.  The pages only name sliding-window
 * attention ("How I Beat PyTorch's Flash Attention", "Future work"); this is the usual
 * causal reading.  A query row whose window holds no key (input_pos + i - window + 1 >= Skv)
 * gets out = 0 and lse = -inf.  The kernel visits only the key tiles inside some row's window
 * and masks the window edge like the causal diagonal.
 *
 *   window    >= 1 (window >= input_pos + Sq gives plain causal attention).
 *   config    as for fa_fwd_config; -1 = the dispatch table.
 *   the rest  as for fa_fwd (causal masking is implied).
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse,
                  int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                  int input_pos, int window, int dtype, void* stream, int config);

/*
 * Attention with fp8 queries and keys: q [B,Hq,Sq,D] and k [B,Hkv,Skv,D] hold fp8 E4M3
 * codes (the OCP "E4M3FN" format gfx950's MFMA reads: 1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, largest finite value 448); v and out are fp16 / bf16
 * (v_dtype); lse fp32.  The real inputs are q_descale * q and k_descale * k (one factor per
 * tensor), so
 *     S = (scale * q_descale * k_descale) * (q_codes . k_codes)
 * and the rest is fa_fwd's (masking, window, softmax, P in v_dtype, O, LSE).  The pages give
 * no low-precision scaling rule; per-tensor dequantisation factors are the plainest one.
 * S = K Q^T runs on gfx950's fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales)
 * with fp32 accumulation, so the scores are the exact products of the fp8 values up to
 * fp32 rounding; P V stays on the fp16 / bf16 MFMA.
 *
 *   D          64 or 128 (FA_ERR_UNSUPPORTED_HEAD_DIM otherwise).
 *   q_descale, k_descale   finite and > 0 (FA_ERR_INVALID_SCALE), checked after scale.
 *   window     0 = none, >= 1 = sliding window (needs causal), as for fa_fwd_splitkv.
 *   config     -1 = the dispatch table (fa_select_config_fp8), else an fp8 configuration.
 *   the rest   as for fa_fwd; q and k need 16-byte alignment like the other tensors.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
               float q_descale, float k_descale, int causal, int input_pos, int window,
               int v_dtype, void* stream, int config);

/* Configuration fa_fwd_fp8 picks for these sizes (v_dtype: an fa_dtype), or a negative
 * fa_status. */
int fa_select_config_fp8(int B, int Hq, int Hkv, int Sq, int D, int causal, int v_dtype);

/*
 * Split-KV forward pass, for grids too small to fill the GPU (few heads or short query
 * blocks; decoding with Sq = 1).  The pages motivate it by launches with too few tiles for
 * the processors ("Tuning Flash Attention for peak performance in NVIDIA CUDA Tile", Part 2
 * "Autotuning"; "How I Beat PyTorch's Flash Attention", "Phase 5: Adaptive Tile
 * Dispatch"); they do not split the key loop, this library does: the visible key tiles of
 * each query tile (inside the window, if any) are cut into num_splits tile-aligned ranges,
 * each handled by its own workgroup, which writes the range's normalised partial output
 * O_s (fp32) and LSE_s.  A
 * second kernel merges them with the online-softmax rescale of the cuTile post ("Online
 * softmax update") applied across ranges:
 *     LSE = ln sum_s exp(LSE_s),   out = sum_s exp(LSE_s - LSE) O_s
 * (a range with no visible key has LSE_s = -inf and weight 0).  The result is the same
 * attention as fa_fwd up to rounding order; out is rounded to `dtype` once, after the merge.
 *
 *   q .. input_pos   as for fa_fwd.
 *   window           0 = none; >= 1 = a sliding window as in fa_fwd_window (needs causal).
 *   dtype            as for fa_fwd.
 *   num_splits       0 = choose (fa_splitkv_num_splits), 1 = no split (same kernels as
 *                    fa_fwd; workspace unused, may be NULL), 2..256 = that many ranges.
 *                    Ranges beyond the number of key tiles are empty and harmless.
 *   config           as for fa_fwd_config; -1 = the dispatch table (whose two-key-part
 *                    choices give way to their one-part twins when more than one range
 *                    runs).  A forced two-key-part configuration runs one range only:
 *                    more is FA_ERR_INVALID_CONFIG.
 *   workspace        device memory of >= fa_splitkv_workspace_size(B, Hq, Sq, D, splits)
 *                    bytes, 16-byte aligned, owned by the caller, overlapping no tensor.
 *                    Its contents on entry do not matter; on return it holds the partials.
 *                    Two calls in flight at once need two workspaces.
 *   workspace_bytes  size of workspace.
 *   stream           both kernels are enqueued on it, in order; no synchronisation.
 * Checks: those of fa_fwd_config, then num_splits (FA_ERR_INVALID_SPLITS), then -- only
 * when more than one split runs and B*Hq*Sq > 0 -- workspace NULL (FA_ERR_NULL_POINTER),
 * misaligned (FA_ERR_MISALIGNED), too small (FA_ERR_WORKSPACE), overlapping (FA_ERR_ALIAS).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                   int causal, int input_pos, int window, int dtype, int num_splits,
                   int config, void* workspace, size_t workspace_bytes, void* stream);

/* Split count fa_fwd_splitkv uses for num_splits = 0: 1 when the plain grid has at least
 * one workgroup per CU (256); else enough ranges for about 512 workgroups, capped so that
 * each range has >= 8 key tiles, the fp32 partials' traffic stays within the K/V bytes,
 * and there are at most 256 ranges.  Negative fa_status on invalid sizes. */
int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                          int input_pos, int window, int dtype, int config);

/*
 * Split-KV forward pass with fp8 E4M3 queries and keys, the two entry points above
 * combined: q, k, v, scale, q_descale, k_descale, window and v_dtype as for fa_fwd_fp8;
 * num_splits, config, workspace and workspace_bytes as for fa_fwd_splitkv (the workspace
 * size does not depend on the input types: fa_splitkv_workspace_size).  Decoding against
 * an fp8 key cache reads 3 bytes per K/V element instead of 4.  Checks: those of
 * fa_fwd_fp8, then those of fa_fwd_splitkv's split and workspace arguments.
 */
int fa_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                       float q_descale, float k_descale, int causal, int input_pos, int window,
                       int v_dtype, int num_splits, int config, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Split count fa_fwd_splitkv_fp8 uses for num_splits = 0 (the rule of
 * fa_splitkv_num_splits, with 3 bytes per K/V element), or a negative fa_status. */
int fa_splitkv_num_splits_fp8(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                              int input_pos, int window, int v_dtype, int config);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split-KV partials live in a fixed scratch array inside the library, one
 * copy per GPU, FA_NOALLOC_SCRATCH_BYTES bytes, held by each GPU the library runs on until
 * the process ends.  The call itself allocates nothing: no hipMalloc, no hipFree.
 *
 *   q .. config, stream   as for fa_fwd_splitkv; the kernels run on the current device,
 *                         which `stream` must belong to.
 * Checks: those of fa_fwd_splitkv up to num_splits; then, only when more than one split
 * runs and B*Hq*Sq > 0, fa_splitkv_workspace_size(B, Hq, Sq, D, splits) >
 * FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_SCRATCH.  The first call on a device that runs
 * more than one split looks up that device's copy of the array (hipGetSymbolAddress; a
 * failure returns FA_ERR_LAUNCH): make that first call outside graph capture.
 * Every call on one GPU shares that GPU's array and leaves its partials there: calls that
 * overlap in time on one GPU (two streams, two threads) race and may return wrong results;
 * serialise them, or use fa_fwd_splitkv with a workspace each.  Nothing in the array needs
 * to start at zero: every partial the merge reads is written by the same call.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                           int causal, int input_pos, int window, int dtype, int num_splits,
                           int config, void* stream);

/*
 * Attention forward pass with fp8 E4M3 queries, keys and values (OCP "E4M3FN": 1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; largest finite value 448), each with one
 * per-tensor dequantisation factor: the attention of q = q_descale * q_codes, k =
 * k_descale * k_codes, v = v_descale * v_codes.  "How I Beat PyTorch's Flash Attention"
 * names FP8 tensor cores as its next step ("What's Next"); no page gives a format or a
 * scaling rule, so this is the plainest one.  Q K^T runs on the fp8 MFMA; each V fragment
 * is widened exactly to bf16 / fp16 (every E4M3 value is representable there) and P V runs
 * on the bf16 / fp16 MFMA with P in that type; v_descale is applied to the fp32 result
 * before it is rounded.  K and V together move 2 bytes per element instead of 4.
 *
 *   q, k, v      fp8 E4M3 codes, one byte per element, layouts as for fa_fwd.
 *   out          [B, Hq, Sq, D] of out_dtype (an fa_dtype); lse as for fa_fwd.
 *   q_descale, k_descale, v_descale   finite and > 0 (FA_ERR_INVALID_SCALE), checked
 *                after scale, in this order.
 *   D            64 or 128 (FA_ERR_UNSUPPORTED_HEAD_DIM otherwise).
 *   other arguments as for fa_fwd_fp8 (config: an "fp8qkv" configuration or -1).
 * Checks and errors as for fa_fwd_fp8.
 */
int fa_fwd_fp8qkv(const void* q, const void* k, const void* v, void* out, float* lse,
                  int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                  float q_descale, float k_descale, float v_descale, int causal,
                  int input_pos, int window, int out_dtype, void* stream, int config);

/* Split-KV form of fa_fwd_fp8qkv (decoding against an fp8 K/V cache): arguments as for
 * fa_fwd_fp8qkv, then num_splits, config, workspace and workspace_bytes as for
 * fa_fwd_splitkv (fa_splitkv_workspace_size gives the size).  Checks: those of
 * fa_fwd_fp8qkv, then those of fa_fwd_splitkv's split and workspace arguments. */
int fa_fwd_splitkv_fp8qkv(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                          float q_descale, float k_descale, float v_descale, int causal,
                          int input_pos, int window, int out_dtype, int num_splits,
                          int config, void* workspace, size_t workspace_bytes, void* stream);

/* Split count fa_fwd_splitkv_fp8qkv uses for num_splits = 0 (the rule of
 * fa_splitkv_num_splits, with 2 bytes per K/V element), or a negative fa_status. */
int fa_splitkv_num_splits_fp8qkv(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                                 int input_pos, int window, int out_dtype, int config);

/* Workspace bytes fa_fwd_splitkv needs for num_splits ranges:
 * num_splits * B * Hq * Sq * (D + 1) * 4 (fp32 partial O, then fp32 partial LSE), 0 when
 * num_splits <= 1, the problem is empty or D is unsupported. */
size_t fa_splitkv_workspace_size(int B, int Hq, int Sq, int D, int num_splits);

/*
 * Backward pass: the gradients dq, dk, dv of out = attention(q, k, v) (as computed by fa_fwd
 * / fa_fwd_window with the same arguments) for an upstream gradient dout.  The pages name the
 * backward pass only as future work ("How I Beat PyTorch's Flash Attention", "Future work");
 * the formulas are the softmax derivative, with P recomputed from the forward's lse:
 *     P = exp(scale q k^T - lse) (0 where masked),  dv = P^T dout,  dP = dout v^T,
 *     D = rowsum(dout * out),  dS = P * (dP - D),  dq = scale dS k,  dk = scale dS^T q;
 * under grouped-query attention dk and dv of a K/V head sum over its query heads.  Rows
 * with lse = -inf (no visible key) contribute nothing.
 *
 *   q, k, v, out, lse   the forward pass's inputs and outputs (layouts as for fa_fwd).
 *   dout                [B, Hq, Sq, D] in `dtype`.
 *   dq / dk, dv         outputs, [B, Hq, Sq, D] / [B, Hkv, Skv, D] in `dtype`; they must not
 *                       overlap any input, each other or the workspace.
 *   scale .. window     as for fa_fwd_splitkv (window needs causal).
 *   workspace           >= fa_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal) bytes of
 *                       device memory, 16-byte aligned, owned by the caller (it receives
 *                       the row statistics -LSE / scale and -D, D = rowsum(dout * out), and
 *                       fp32 partial dk / dv sums when the head group is split).
 *   stream              the kernels (row statistics, dk/dv, the partial sum if any, dq)
 *                       are enqueued on it in order.
 * Checks: as for fa_fwd (pointers, sizes, head group, head dim, dtype, scale, input_pos,
 * window, alignment, aliasing), then the workspace (NULL, misaligned, too small,
 * overlapping).  B*Hq*Sq == 0 with K/V rows present writes zero dk and dv.
 * Deterministic: no atomics; every gradient element is summed in a fixed order.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
           int causal, int input_pos, int window, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd needs (0 for an empty or invalid problem): the row statistics,
 * B * Hq * Sq * 8 rounded up to 256, plus, when the dK/dV grid would have fewer than two
 * workgroups per CU (causal) or one (non-causal) and the head group allows it, fp32
 * partial sums of dk and dv for each of the g parts the group's query heads are split
 * into (g * 2 * B * Hkv * Skv * D * 4; g = the smallest divisor of Hq / Hkv that reaches
 * that grid size, else Hq / Hkv). */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal);

/* Configuration the dispatch table picks for these arguments, or a negative fa_status. */
int fa_select_config(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                     int input_pos, int dtype);

/* Number of kernel configurations compiled into the library. */
int fa_num_configs(void);

/* Static description of configuration `config` (tile sizes, waves, head packing, dtype,
 * head dim, causality), or NULL for an unknown id.  The string is owned by the library. */
const char* fa_config_name(int config);

/* Static, human-readable text for an fa_status code.  Never NULL. */
const char* fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
