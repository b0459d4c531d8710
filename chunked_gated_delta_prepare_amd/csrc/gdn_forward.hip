// libgdn: launch planning and dispatch for the fused forward kernel.  Built
// as its own translation unit so it can carry its own scheduling flags.
#include <algorithm>
#include <cstdlib>

#include "gdn_forward.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

bool pipe_disabled() {
    const char *e = std::getenv("GDN_FORWARD_FOUR_WAVE");
    return e && *e == '1';
}

// ---------------------------------------------------------------------------
// forward (fused)
// ---------------------------------------------------------------------------
template <int C, int K, typename IO, typename OT, bool KG>
gdn_status run_forward(FwdParams &fp, int grid, hipStream_t s) {
    if constexpr (FwdLayout<C, K, IO, KG>::kBytes > kLdsBytesMax) {
        return GDN_ERR_LDS_BUDGET;
    } else {
        return launch_kernel((const void *)&forward_kernel<C, K, IO, OT, KG>, grid, &fp, s);
    }
}

// Scalar gate with bf16 io runs the pipelined kernel (prepare and re-scan on
// separate waves); the per-key gate and fp32 io run the four-wave kernel.
template <int C, int K, typename IO, typename OT>
gdn_status forward_gate(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    if (pr->gate == GDN_GATE_KEY) return run_forward<C, K, IO, OT, true>(fp, grid, s);
    if constexpr (sizeof(IO) == 2) {
        if (!pipe_disabled()) return enqueue_forward_pipe(C, K, sizeof(OT) == 4, fp, grid, s);
    }
    return run_forward<C, K, IO, OT, false>(fp, grid, s);
}

template <int C, int K>
gdn_status forward_dt(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    if (pr->io_dtype == GDN_F32) return forward_gate<C, K, float, float>(pr, fp, grid, s);
    if (pr->o_dtype == GDN_F32) return forward_gate<C, K, bf16_t, float>(pr, fp, grid, s);
    return forward_gate<C, K, bf16_t, bf16_t>(pr, fp, grid, s);
}

template <int C>
gdn_status forward_k(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    return pr->K == 64 ? forward_dt<C, 64>(pr, fp, grid, s) : forward_dt<C, 128>(pr, fp, grid, s);
}

}  // namespace

// The fused kernel addresses one (batch, head) stream of each tensor with
// 32-bit byte offsets from that stream's first token.
static bool fits_32bit_streams(const gdn_problem *pr) {
    const int64_t sio = pr->io_dtype == GDN_F32 ? 4 : 2, so = pr->o_dtype == GDN_F32 ? 4 : 2;
    const int64_t th = pr->T * pr->H;
    const int64_t gdim = pr->gate == GDN_GATE_KEY ? pr->K : 1;
    const int64_t worst = std::max({th * pr->K * sio, th * pr->V * sio, th * pr->V * so,
                                    th * gdim * 4});
    return worst < ((int64_t)1 << 32);
}

gdn_status enqueue_forward(const gdn_problem *pr, const void *q, const void *k,
                           const void *v, const float *beta, const float *g,
                           const float *h0, void *o, float *hT, hipStream_t s) {
    if (!fits_32bit_streams(pr)) return GDN_ERR_UNSUPPORTED;
    FwdParams fp;
    fp.q = q; fp.k = k; fp.v = v; fp.beta = beta; fp.g = g; fp.h0 = h0;
    fp.o = o; fp.hT = hT;
    fp.B = (int)pr->B; fp.T = (int)pr->T; fp.H = (int)pr->H; fp.V = (int)pr->V;
    fp.nvt = (int)(pr->V / 64);
    const int pairs = (int)(pr->B * pr->H);
    fp.swizzle = (pairs % 8 == 0) ? 1 : 0;
    if (const char *e = std::getenv("GDN_NO_SWIZZLE")) fp.swizzle = (*e == '1') ? 0 : fp.swizzle;
    const int grid = pairs * fp.nvt;
    return pr->chunk == 32 ? forward_k<32>(pr, fp, grid, s) : forward_k<64>(pr, fp, grid, s);
}

}  // namespace gdn
