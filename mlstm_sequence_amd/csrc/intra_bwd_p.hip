// intra_bwd_p.hip -- the intra-chunk kernel in the mode that writes the
// shared P of the dq and dk products (and its mirrored transpose).
#include "intra_impl.hpp"

namespace tfla {

hipError_t launch_intra_p(const Problem& p, const void* q, const void* k, const float* fgate_pre,
                          const Workspace& ws, hipStream_t stream)
{
    // the values are not read; k stands in for them
    return dispatch_type<kEmitP>(p, q, k, k, fgate_pre, ws, nullptr, 1.0f, stream);
}

}  // namespace tfla
