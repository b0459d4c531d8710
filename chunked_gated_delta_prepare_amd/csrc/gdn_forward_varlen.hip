// libgdn: the chunk-32 kernel instances over packed sequences (both kernels),
// built with the default machine scheduler: the ILP scheduler crashes the
// compiler on them.  Chunk 64 is in gdn_forward_varlen_c64.hip.
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

gdn_status enqueue_forward_varlen(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    return pr->chunk == 32 ? forward_k<32, false, true>(pr, fp, grid, s)
                           : enqueue_forward_varlen_c64(pr, fp, grid, s);
}

gdn_status enqueue_forward_pipe_varlen_c32(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s) {
    return K == 64 ? pipe_varlen<32, 64>(o_f32, fp, grid, s) : pipe_varlen<32, 128>(o_f32, fp, grid, s);
}

}  // namespace gdn
