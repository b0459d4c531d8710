// libgdn: gdn_backward dispatch -- the reverse scan of the state's gradient,
// then the per-chunk gradients (kernels in gdn_backward.h).
#include "gdn_backward.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int C, int K, int V>
gdn_status launch_backward(BwdParams &bp, hipStream_t s) {
    gdn_status st;
    if (bp.NT > 0) {
        st = launch_kernel((const void *)&bwd_prep_kernel<C, K>, bp.B * bp.H * bp.NT, &bp, s, 256);
        if (st != GDN_OK) return st;
    }
    st = launch_kernel((const void *)&bwd_dh_kernel<C, K>, bp.B * bp.H * bp.nvt, &bp, s, 256);
    if (st != GDN_OK || bp.NT == 0) return st;
    // eight waves (two per SIMD) where the register pieces divide among 512
    // threads: chunk 64
    constexpr int NW = C == 64 ? 8 : 4;
    return launch_kernel((const void *)&bwd_grad_kernel<C, K, V, NW>, bp.B * bp.H * bp.NT, &bp, s, 64 * NW);
}

template <int C, int K>
gdn_status backward_v(const gdn_problem *pr, BwdParams &bp, hipStream_t s) {
    return pr->V == 64 ? launch_backward<C, K, 64>(bp, s) : launch_backward<C, K, 128>(bp, s);
}

template <int C>
gdn_status backward_k(const gdn_problem *pr, BwdParams &bp, hipStream_t s) {
    return pr->K == 64 ? backward_v<C, 64>(pr, bp, s) : backward_v<C, 128>(pr, bp, s);
}

}  // namespace

static int64_t slot_bytes(const gdn_problem *pr) {
    if (pr->gate == GDN_GATE_KEY) return backward_kda_slot_bytes(pr->chunk, pr->K);
    return pr->chunk == 32 ? BwdSlot<32>::kBytes : BwdSlot<64>::kBytes;
}

int64_t backward_workspace_bytes(const gdn_problem *pr) {
    const int64_t nt = (pr->T + pr->chunk - 1) / pr->chunk;
    int64_t bytes = pr->B * pr->T * pr->H * pr->V * 4 + pr->B * nt * pr->H * pr->K * pr->V * 4 +
                    pr->B * nt * pr->H * slot_bytes(pr);
    if (pr->gate == GDN_GATE_KEY) bytes += pr->B * nt * pr->H * 2 * pr->chunk * pr->chunk * 4;
    return bytes;
}

gdn_status enqueue_backward(const gdn_problem *pr, const void *q, const void *k, const void *v,
                            const float *beta, const float *g, const void *dout, const float *dhT,
                            const void *hck, const void *vnew, float *dq, float *dk, float *dv,
                            float *dbeta, float *dg, float *dh0, void *ws, hipStream_t s) {
    BwdParams bp;
    bp.q = q; bp.k = k; bp.v = v; bp.dout = dout; bp.beta = beta; bp.g = g; bp.dhT = dhT;
    bp.hck = hck; bp.vnew = vnew;
    bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dbeta = dbeta; bp.dg = dg; bp.dh0 = dh0;
    bp.B = (int)pr->B; bp.T = (int)pr->T; bp.H = (int)pr->H; bp.V = (int)pr->V;
    bp.nvt = (int)(pr->V / 64);
    bp.NT = (int)((pr->T + pr->chunk - 1) / pr->chunk);
    bp.dR = (float *)ws;
    bp.dhe = ws ? (float *)ws + pr->B * pr->T * pr->H * pr->V : nullptr;
    bp.prep = ws ? (void *)(bp.dhe + pr->B * bp.NT * pr->H * pr->K * pr->V) : nullptr;
    bp.dpa = ws ? (float *)((char *)bp.prep + pr->B * bp.NT * pr->H * slot_bytes(pr)) : nullptr;
    bp.swizzle = ((int64_t)bp.B * bp.H * bp.nvt) % 8 == 0 ? 1 : 0;
    if (pr->gate == GDN_GATE_KEY) return enqueue_backward_kda(pr, bp, s);
    return pr->chunk == 32 ? backward_k<32>(pr, bp, s) : backward_k<64>(pr, bp, s);
}

}  // namespace gdn
