// fa_inst_ks2.hip -- compiles the forward-kernel configurations of FA_LIST_KS2
// (fa_configs.h): two key parts per workgroup, non-causal, head dims 64 and 128; the dispatch
// table in fa_fwd.hip refers to them.
#define FA_LAUNCH_DEFINE
#include "fa_launch.hpp"
#include "fa_configs.h"

FA_LIST_KS2(FA_INSTANTIATE)
