// libgdn: gdn_backward dispatch for the per-key gate (kernels in
// gdn_backward_kda.h): the per-chunk factors, the reverse scan, the matrix
// products of the gradients, the decay-weighted sums.
#include "gdn_backward_kda.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int C, int K, int V>
gdn_status launch_backward_kda(BwdParams &bp, hipStream_t s) {
    const int gch = bp.B * bp.H * bp.NT;
    gdn_status st;
    if (bp.NT > 0) {
        st = launch_kernel((const void *)&bwd_prep_kda_kernel<C, K>, gch, &bp, s, 256);
        if (st != GDN_OK) return st;
    }
    st = launch_kernel((const void *)&bwd_dh_kda_kernel<C, K>, bp.B * bp.H * bp.nvt, &bp, s, 256);
    if (st != GDN_OK || bp.NT == 0) return st;
    st = launch_kernel((const void *)&bwd_grad_kda_kernel<C, K, V>, gch, &bp, s, 256);
    if (st != GDN_OK) return st;
    return launch_kernel((const void *)&bwd_dec_kda_kernel<C, K>, gch, &bp, s, 64 * BwdDecLayout<C, K>::NW);
}

template <int C, int K>
gdn_status backward_kda_v(const gdn_problem *pr, BwdParams &bp, hipStream_t s) {
    return pr->V == 64 ? launch_backward_kda<C, K, 64>(bp, s) : launch_backward_kda<C, K, 128>(bp, s);
}

template <int C>
gdn_status backward_kda_k(const gdn_problem *pr, BwdParams &bp, hipStream_t s) {
    return pr->K == 64 ? backward_kda_v<C, 64>(pr, bp, s) : backward_kda_v<C, 128>(pr, bp, s);
}

}  // namespace

int64_t backward_kda_slot_bytes(int64_t chunk, int64_t K) {
    if (chunk == 32) return K == 64 ? BwdSlotK<32, 64>::kBytes : BwdSlotK<32, 128>::kBytes;
    return K == 64 ? BwdSlotK<64, 64>::kBytes : BwdSlotK<64, 128>::kBytes;
}

gdn_status enqueue_backward_kda(const gdn_problem *pr, BwdParams &bp, hipStream_t s) {
    return pr->chunk == 32 ? backward_kda_k<32>(pr, bp, s) : backward_kda_k<64>(pr, bp, s);
}

}  // namespace gdn
