// libgdn: dispatch of the pipelined forward kernel for the per-key gate
// (gdn_forward_pipe_kda.h), plain, saving states (ST), over packed
// sequences (VL) or as the backward's re-scan (DQ).
#include "gdn_forward_pipe_kda.h"
#include "gdn_internal.h"

namespace gdn {

namespace {
template <int C, int K, bool ST, bool VL, bool DQ = false>
const void *kda_fn(bool o_f32) {
    return o_f32 ? (const void *)&forward_pipe_kda_kernel<C, K, float, ST, VL, DQ>
                 : (const void *)&forward_pipe_kda_kernel<C, K, bf16_t, ST, VL, DQ>;
}

template <int C, int K>
const void *kda_mode(bool o_f32, const FwdParams &fp, int &threads) {
    threads = kda_threads<C, K, false>();
    if (fp.dq) {
        threads = kda_threads<C, K, true>();
        return kda_fn<C, K, true, false, true>(o_f32);
    }
    if (fp.hck) return kda_fn<C, K, true, false>(o_f32);
    if (fp.cu) return kda_fn<C, K, false, true>(o_f32);
    return kda_fn<C, K, false, false>(o_f32);
}
}  // namespace

gdn_status enqueue_forward_pipe_kda(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                    hipStream_t s) {
    int threads = 0;
    const void *fn = C == 32 ? (K == 64 ? kda_mode<32, 64>(o_f32, fp, threads) : kda_mode<32, 128>(o_f32, fp, threads))
                             : (K == 64 ? kda_mode<64, 64>(o_f32, fp, threads) : kda_mode<64, 128>(o_f32, fp, threads));
    return launch_kernel(fn, grid, &fp, s, threads);
}

}  // namespace gdn
