// libgdn: the chunk-64 forward kernel instances that also save the
// chunk-start states and the per-token deltas, built with the ILP machine
// scheduler like the plain forward (gdn_forward.hip).
#include "gdn_forward_dispatch.h"

namespace gdn {

gdn_status enqueue_forward_states_c64(const gdn_problem *pr, FwdParams &fp, int grid,
                                      hipStream_t s) {
    return forward_k<64, true>(pr, fp, grid, s);
}

}  // namespace gdn
