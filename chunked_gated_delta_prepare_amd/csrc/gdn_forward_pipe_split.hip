// libgdn: the sequence-split (SP) instances of the pipelined forward kernel
// (gdn_forward_pipe.h), built with the ILP scheduler; gdn_split.hip launches
// them and finishes the second segment.
#include "gdn_forward_pipe.h"
#include "gdn_internal.h"

namespace gdn {

gdn_status enqueue_forward_pipe_split(int K, bool o_f32, FwdParams &fp, int grid, hipStream_t s) {
    const void *fn = K == 64 ? (o_f32 ? (const void *)&forward_pipe_kernel<64, 64, float, false, false, false, true>
                                      : (const void *)&forward_pipe_kernel<64, 64, bf16_t, false, false, false, true>)
                             : (o_f32 ? (const void *)&forward_pipe_kernel<64, 128, float, false, false, false, true>
                                      : (const void *)&forward_pipe_kernel<64, 128, bf16_t, false, false, false, true>);
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}

}  // namespace gdn
