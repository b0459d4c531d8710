// libgdn: the pipelined forward kernel instances that the ILP machine
// scheduler crashes the compiler on (every chunk-32 instance: plain and
// saving states), built with the default scheduler (see gdn_forward_pipe.hip).
#include "gdn_forward_pipe.h"
#include "gdn_internal.h"

namespace gdn {

gdn_status enqueue_forward_pipe_c32(int K, bool o_f32, FwdParams &fp, int grid, hipStream_t s) {
    const void *fn;
    if (K == 64)
        fn = o_f32 ? (const void *)&forward_pipe_kernel<32, 64, float>
                   : (const void *)&forward_pipe_kernel<32, 64, bf16_t>;
    else
        fn = o_f32 ? (const void *)&forward_pipe_kernel<32, 128, float>
                   : (const void *)&forward_pipe_kernel<32, 128, bf16_t>;
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}

gdn_status enqueue_forward_pipe_c32_states(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s) {
    const void *fn;
    if (K == 64)
        fn = o_f32 ? (const void *)&forward_pipe_kernel<32, 64, float, true>
                   : (const void *)&forward_pipe_kernel<32, 64, bf16_t, true>;
    else
        fn = o_f32 ? (const void *)&forward_pipe_kernel<32, 128, float, true>
                   : (const void *)&forward_pipe_kernel<32, 128, bf16_t, true>;
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}

}  // namespace gdn
