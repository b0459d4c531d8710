// libgdn: dispatch of kda_gram_kernel (gdn_kda_gram.h), the per-key gate's
// exact Gram products and triangular factors for every chunk, into the
// workspace that the re-scan kernels read.
#include "gdn_internal.h"
#include "gdn_kda_gram.h"

namespace gdn {

namespace {
template <int C, int K, typename IO>
gdn_status gram_vl(GramParams &gp, bool vl, int items, hipStream_t s) {
    const void *fn = vl ? (const void *)&kda_gram_kernel<C, K, IO, true>
                        : (const void *)&kda_gram_kernel<C, K, IO, false>;
    return launch_kernel(fn, items, &gp, s);
}

template <int C, typename IO>
gdn_status gram_k(const gdn_problem *pr, GramParams &gp, bool vl, int grid, hipStream_t s) {
    return pr->K == 64 ? gram_vl<C, 64, IO>(gp, vl, grid, s) : gram_vl<C, 128, IO>(gp, vl, grid, s);
}

template <typename IO>
gdn_status gram_c(const gdn_problem *pr, GramParams &gp, bool vl, int grid, hipStream_t s) {
    return pr->chunk == 32 ? gram_k<32, IO>(pr, gp, vl, grid, s) : gram_k<64, IO>(pr, gp, vl, grid, s);
}
}  // namespace

int64_t kda_slot_bytes_host(const gdn_problem *pr) {
    const int64_t C = pr->chunk, K = pr->K;
    return pr->io_dtype == GDN_F32 ? 2 * C * C * 4 : 2 * C * C * 2 + 3 * C * K * 2 + K * 4;
}

int64_t kda_workspace_bytes(const gdn_problem *pr, int64_t n_seqs) {
    if (pr->gate != GDN_GATE_KEY || pr->T == 0) return 0;
    const int64_t nt = (pr->T + pr->chunk - 1) / pr->chunk;
    const int64_t slots = n_seqs > 0 ? nt + n_seqs : pr->B * nt;
    return slots * pr->H * kda_slot_bytes_host(pr);
}

gdn_status enqueue_kda_gram(const gdn_problem *pr, const void *q, const void *k,
                            const float *beta, const float *g, void *ws, const int32_t *cu,
                            int64_t n_seqs, hipStream_t s) {
    GramParams gp;
    gp.q = q; gp.k = k; gp.beta = beta; gp.g = g; gp.ws = ws; gp.cu = cu;
    gp.B = (int)(cu ? n_seqs : pr->B);
    gp.T = (int)pr->T;
    gp.H = (int)pr->H;
    gp.nt = (int)((pr->T + pr->chunk - 1) / pr->chunk);
    const int64_t slots = cu ? gp.nt + n_seqs : (int64_t)gp.B * gp.nt;
    if (slots * pr->H > ((int64_t)1 << 30)) return GDN_ERR_UNSUPPORTED;
    const int grid = (int)(slots * pr->H);
    return pr->io_dtype == GDN_F32 ? gram_c<float>(pr, gp, cu != nullptr, grid, s)
                                   : gram_c<bf16_t>(pr, gp, cu != nullptr, grid, s);
}

}  // namespace gdn
