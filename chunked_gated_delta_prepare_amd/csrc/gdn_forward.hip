// libgdn: launch planning and dispatch for the fused forward kernel.  Built
// as its own translation unit so it can carry its own scheduling flags (the
// instances that save states are in gdn_forward_states.hip).
#include <algorithm>
#include <cstdlib>

#include "gdn_forward_dispatch.h"

namespace gdn {

// The fused kernel addresses one (batch, head) stream of each tensor with
// 32-bit byte offsets from that stream's first token.
static bool fits_32bit_streams(const gdn_problem *pr) {
    const int64_t sio = pr->io_dtype == GDN_F32 ? 4 : 2, so = pr->o_dtype == GDN_F32 ? 4 : 2;
    const int64_t th = pr->T * pr->H;
    const int64_t gdim = pr->gate == GDN_GATE_KEY ? pr->K : 1;
    const int64_t worst = std::max({th * pr->K * sio, th * pr->V * sio, th * pr->V * so,
                                    th * gdim * 4});
    // per-key gate: one stream's workspace slots for all heads
    const int64_t nt = (pr->T + pr->chunk - 1) / pr->chunk;
    const int64_t ws = pr->gate == GDN_GATE_KEY ? nt * pr->H * kda_slot_bytes_host(pr) : 0;
    return worst < ((int64_t)1 << 32) && ws < ((int64_t)1 << 32);
}

gdn_status enqueue_forward(const gdn_problem *pr, const void *q, const void *k,
                           const void *v, const float *beta, const float *g,
                           const float *h0, void *o, float *hT, void *hck, void *vnew,
                           const int32_t *cu, int64_t n_seqs, void *ws, hipStream_t s,
                           const void *dout, float *dq) {
    if (!fits_32bit_streams(pr)) return GDN_ERR_UNSUPPORTED;
    // the re-scan with dq is a pipelined kernel only (bf16 io): refused
    // before anything is enqueued
    if (dq && (pr->io_dtype != GDN_BF16 || pipe_disabled())) return GDN_ERR_UNSUPPORTED;
    // per-key gate: the chunks' exact Gram products and triangular factors
    // first, all chunks at once, into the workspace the re-scan reads
    if (pr->gate == GDN_GATE_KEY && pr->T > 0) {
        const gdn_status st = enqueue_kda_gram(pr, q, k, beta, g, ws, cu, n_seqs, s);
        if (st != GDN_OK) return st;
    }
    FwdParams fp;
    fp.q = q; fp.k = k; fp.v = v; fp.beta = beta; fp.g = g; fp.h0 = h0;
    fp.o = o; fp.hT = hT; fp.hck = hck; fp.vnew = vnew; fp.cu = cu;
    fp.dout = dout; fp.dq = dq; fp.ws = ws;
    fp.wait_count = wait_count_ptr();
    wait_params(fp.wait_limit, fp.wait_bias);
    // packed sequences: one stream per sequence over the [1, T, H, .] tensors
    const int64_t streams = cu ? n_seqs : pr->B;
    fp.B = (int)streams; fp.T = (int)pr->T; fp.H = (int)pr->H; fp.V = (int)pr->V;
    fp.nvt = (int)(pr->V / 64);
    const int pairs = (int)(streams * pr->H);
    fp.swizzle = (pairs % 8 == 0) ? 1 : 0;
    if (const char *e = std::getenv("GDN_NO_SWIZZLE")) fp.swizzle = (*e == '1') ? 0 : fp.swizzle;
    const int grid = pairs * fp.nvt;
    if (hck) return enqueue_forward_states(pr, fp, grid, s);
    if (cu) return enqueue_forward_varlen(pr, fp, grid, s);
    return pr->chunk == 32 ? forward_k<32, false>(pr, fp, grid, s)
                           : forward_k<64, false>(pr, fp, grid, s);
}

}  // namespace gdn
