// fa_inst_fp8qkv_d64.hip -- compiles the forward-kernel configurations of FA_LIST_FP8QKV_D64
// (fa_configs.h): fp8 E4M3 queries, keys and values at head dim 64, bf16 / fp16 output; the dispatch table in fa_fwd.hip refers to them.
#define FA_LAUNCH_DEFINE
#include "fa_launch.hpp"
#include "fa_configs.h"

FA_LIST_FP8QKV_D64(FA_INSTANTIATE)
