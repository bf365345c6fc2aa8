// fa_launch.hpp -- launcher of one forward-kernel configuration.  fa_fwd.hip sees only
// the declaration; the fa_inst_*.hip files include the definition and instantiate it.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.hpp"

namespace fa_host {

// Launch configuration C of fa_fwd_kernel on stream s: n_tiles * hsub * B * Hkv * num_splits
// workgroups of C::NT threads.
template <class C>
hipError_t launch_cfg(const fa::Params& p, hipStream_t s);

#ifdef FA_LAUNCH_DEFINE
template <class C>
hipError_t launch_cfg(const fa::Params& p, hipStream_t s) {
    const long long wgs = (long long)p.n_tiles * p.hsub * p.B * p.Hkv * p.num_splits;
    hipLaunchKernelGGL(fa::fa_fwd_kernel<C>, dim3((unsigned)wgs), dim3(C::NT), 0, s, p);
    return hipGetLastError();
}
#endif

}  // namespace fa_host

#define FA_INSTANTIATE(D, BN, QB, WPH, HPW, C, B, Q, V8, KS, CN, TN)                         \
    template hipError_t fa_host::launch_cfg<fa::Cfg<D, BN, QB, WPH, HPW, C, B, Q, V8, KS>>(  \
        const fa::Params&, hipStream_t);
