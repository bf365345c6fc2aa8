// fa_inst_fp8_bf16.hip -- compiles the forward-kernel configurations of FA_LIST_FP8_BF16
// (fa_configs.h); the dispatch table in fa_fwd.hip refers to them.
#define FA_LAUNCH_DEFINE
#include "fa_launch.hpp"
#include "fa_configs.h"

FA_LIST_FP8_BF16(FA_INSTANTIATE)
