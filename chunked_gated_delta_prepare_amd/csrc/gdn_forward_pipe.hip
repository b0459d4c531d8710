// libgdn: dispatch of the pipelined forward kernel.  Compiled with the ILP
// machine scheduler, which issues fragment loads well ahead of the matrix
// instructions that use them; the chunk-32 / key-128 instance lives in
// gdn_forward_pipe_c32.hip because that scheduler crashes the compiler on it,
// and so do the chunk-32 instances that save states.
#include "gdn_forward_pipe.h"
#include "gdn_internal.h"

namespace gdn {

namespace {
template <int C, int K, bool ST>
gdn_status pipe_o(bool o_f32, FwdParams &fp, int grid, hipStream_t s) {
    const void *fn = o_f32 ? (const void *)&forward_pipe_kernel<C, K, float, ST>
                           : (const void *)&forward_pipe_kernel<C, K, bf16_t, ST>;
    return launch_kernel(fn, grid, &fp, s, kPipeThreads);
}
}  // namespace

gdn_status enqueue_forward_pipe(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                hipStream_t s) {
    if (fp.dq) return enqueue_forward_pipe_dq(C, K, o_f32, fp, grid, s);
    if (fp.cu) return C == 32 ? enqueue_forward_pipe_varlen_c32(K, o_f32, fp, grid, s)
                              : enqueue_forward_pipe_varlen_c64(K, o_f32, fp, grid, s);
    const bool st = fp.hck != nullptr;
    if (C == 32) {
        if (st) return enqueue_forward_pipe_c32_states(K, o_f32, fp, grid, s);
        return enqueue_forward_pipe_c32(K, o_f32, fp, grid, s);
    }
    if (st) return K == 64 ? pipe_o<64, 64, true>(o_f32, fp, grid, s)
                           : pipe_o<64, 128, true>(o_f32, fp, grid, s);
    return K == 64 ? pipe_o<64, 64, false>(o_f32, fp, grid, s)
                   : pipe_o<64, 128, false>(o_f32, fp, grid, s);
}

}  // namespace gdn
