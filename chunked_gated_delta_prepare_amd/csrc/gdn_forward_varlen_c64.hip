// libgdn: the chunk-64 kernel instances over packed sequences (both kernels),
// built with the ILP machine scheduler like the plain forward.
#include "gdn_forward_dispatch.h"
#include "gdn_forward_pipe.h"

namespace gdn {

namespace {
template <int C, int K>
gdn_status pipe_varlen(bool o_f32, FwdParams &fp, int grid, hipStream_t s) {
    const void *fn = o_f32 ? (const void *)&forward_pipe_kernel<C, K, float, false, true>
                           : (const void *)&forward_pipe_kernel<C, K, bf16_t, false, true>;
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}
}  // namespace

gdn_status enqueue_forward_varlen_c64(const gdn_problem *pr, FwdParams &fp, int grid,
                                      hipStream_t s) {
    return forward_k<64, false, true>(pr, fp, grid, s);
}

gdn_status enqueue_forward_pipe_varlen_c64(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s) {
    return K == 64 ? pipe_varlen<64, 64>(o_f32, fp, grid, s) : pipe_varlen<64, 128>(o_f32, fp, grid, s);
}

}  // namespace gdn
