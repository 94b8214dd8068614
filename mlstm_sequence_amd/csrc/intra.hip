// intra.hip -- the intra-chunk kernel of the forward pass.
#include "intra_impl.hpp"

namespace tfla {

hipError_t launch_intra(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                        const Workspace& ws, void* h, hipStream_t stream)
{
    if (intra_sweeps(p)) return launch_intra_sweep(p, q, k, v, fgate_pre, ws, h, stream);
    const float scale = 1.0f / sqrtf((float)p.dqk);
    if (p.bf16 && p.st32) return dispatch_gate<bf16, kStateF32>(p, q, k, v, fgate_pre, ws, h, scale, stream);
    return dispatch_type<0>(p, q, k, v, fgate_pre, ws, h, scale, stream);
}

int intra_value_tile(const Problem& p) { return intra_bv(p); }

}  // namespace tfla
