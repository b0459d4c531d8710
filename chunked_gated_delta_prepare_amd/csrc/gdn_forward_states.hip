// libgdn: the chunk-32 forward kernel instances that also save the
// chunk-start states and the per-token deltas (the four-wave kernel's; the
// pipelined kernel's are dispatched from here into their own units).  Built
// with the default machine scheduler: the ILP scheduler crashes the compiler
// on them.  Chunk 64 is in gdn_forward_states_c64.hip.
#include "gdn_forward_dispatch.h"

namespace gdn {

gdn_status enqueue_forward_states(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    return pr->chunk == 32 ? forward_k<32, true>(pr, fp, grid, s)
                           : enqueue_forward_states_c64(pr, fp, grid, s);
}

}  // namespace gdn
