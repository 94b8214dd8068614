// intra_bwd_k.hip -- the intra-chunk kernel in the gradient mode for
// dk: mirrored chunks, state read contraction-major.
#include "intra_impl.hpp"

namespace tfla {

hipError_t launch_intra_dk(const Problem& p, const void* q, const void* k, const void* v,
                          const float* fgate_pre, const Workspace& ws, void* out, float scale,
                          hipStream_t stream)
{
    return dispatch_type<kNatState | kMirror | kRowDots>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

hipError_t launch_intra_dk_p(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                             const Workspace& ws, void* out, float scale, hipStream_t stream)
{
    return dispatch_type<kNatState | kMirror | kRowDots | kGivenP>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

}  // namespace tfla
