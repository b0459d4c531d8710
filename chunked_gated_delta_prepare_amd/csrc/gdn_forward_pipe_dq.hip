// libgdn: the scalar-gate pipelined kernel as the backward's re-scan (the
// DQ instances: chunk-start states, v' and dq's chunk-start-state term),
// built with the ILP machine scheduler.
#include "gdn_forward_pipe.h"
#include "gdn_internal.h"

namespace gdn {

namespace {
template <int C, int K>
const void *dq_fn(bool o_f32) {
    return o_f32 ? (const void *)&forward_pipe_kernel<C, K, float, true, false, true>
                 : (const void *)&forward_pipe_kernel<C, K, bf16_t, true, false, true>;
}
}  // namespace

gdn_status enqueue_forward_pipe_dq(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                   hipStream_t s) {
    const void *fn = C == 32 ? (K == 64 ? dq_fn<32, 64>(o_f32) : dq_fn<32, 128>(o_f32))
                             : (K == 64 ? dq_fn<64, 64>(o_f32) : dq_fn<64, 128>(o_f32));
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}

}  // namespace gdn
