// fa_inst_fp8qkv_bf16.hip -- compiles the forward-kernel configurations of
// FA_LIST_FP8QKV_BF16 (fa_configs.h): fp8 E4M3 queries, keys and values, bf16 output; the
// dispatch table in fa_fwd.hip refers to them.
#define FA_LAUNCH_DEFINE
#include "fa_launch.hpp"
#include "fa_configs.h"

FA_LIST_FP8QKV_BF16(FA_INSTANTIATE)
