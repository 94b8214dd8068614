// intra_bwd_v.hip -- the intra-chunk kernel in the gradient mode for
// dv: mirrored chunks, state read out-major.
#include "intra_impl.hpp"

namespace tfla {

hipError_t launch_intra_dv(const Problem& p, const void* q, const void* k, const void* v,
                          const float* fgate_pre, const Workspace& ws, void* out, float scale,
                          hipStream_t stream)
{
    if (intra_sweeps_dv(p)) return launch_intra_sweep_dv(p, q, k, v, fgate_pre, ws, out, scale, stream);
    return dispatch_type<kMirror>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

}  // namespace tfla
