// intra_bwd_q.hip -- the intra-chunk kernel in the gradient mode for
// dq: causal, state read contraction-major (S computed, or the shared P read).
#include "intra_impl.hpp"

namespace tfla {

hipError_t launch_intra_dq(const Problem& p, const void* q, const void* k, const void* v,
                          const float* fgate_pre, const Workspace& ws, void* out, float scale,
                          hipStream_t stream)
{
    return dispatch_type<kNatState | kRowDots>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

hipError_t launch_intra_dq_p(const Problem& p, const void* q, const void* k, const void* v, const float* fgate_pre,
                             const Workspace& ws, void* out, float scale, hipStream_t stream)
{
    return dispatch_type<kNatState | kRowDots | kGivenP>(p, q, k, v, fgate_pre, ws, out, scale, stream);
}

}  // namespace tfla
