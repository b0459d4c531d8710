// libgdn: dispatch of a validated forward problem onto the kernel template
// instances, for the plain forward (ST = false), the forward that also saves
// states (ST = true) and the one over packed sequences (VL = true); each is
// instantiated in its own translation units.
#pragma once

#include <cstdlib>

#include "gdn_forward.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

inline bool pipe_disabled() {
    const char *e = std::getenv("GDN_FORWARD_FOUR_WAVE");
    return e && *e == '1';
}

template <int C, int K, typename IO, typename OT, bool KG, bool ST, bool VL>
gdn_status run_forward(FwdParams &fp, int grid, hipStream_t s) {
    if constexpr (FwdLayout<C, K, IO, KG>::kBytes > kLdsBytesMax) {
        return GDN_ERR_LDS_BUDGET;
    } else {
        return launch_kernel((const void *)&forward_kernel<C, K, IO, OT, KG, ST, VL>, grid, &fp, s);
    }
}

// bf16 io runs the pipelined kernels (prepare and re-scan on separate waves),
// one for the scalar gate and one for the per-key gate; fp32 io runs the
// four-wave kernel (as does bf16 io with GDN_FORWARD_FOUR_WAVE=1).
template <int C, int K, typename IO, typename OT, bool ST, bool VL>
gdn_status forward_gate(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    const bool key = pr->gate == GDN_GATE_KEY;
    if constexpr (sizeof(IO) == 2) {
        if (!pipe_disabled())
            return key ? enqueue_forward_pipe_kda(C, K, sizeof(OT) == 4, fp, grid, s)
                       : enqueue_forward_pipe(C, K, sizeof(OT) == 4, fp, grid, s);
    }
    if (fp.dq) return GDN_ERR_UNSUPPORTED;   // the re-scan with dq is a pipelined kernel only
    return key ? run_forward<C, K, IO, OT, true, ST, VL>(fp, grid, s)
               : run_forward<C, K, IO, OT, false, ST, VL>(fp, grid, s);
}

template <int C, int K, bool ST, bool VL>
gdn_status forward_dt(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    if (pr->io_dtype == GDN_F32) return forward_gate<C, K, float, float, ST, VL>(pr, fp, grid, s);
    if (pr->o_dtype == GDN_F32) return forward_gate<C, K, bf16_t, float, ST, VL>(pr, fp, grid, s);
    return forward_gate<C, K, bf16_t, bf16_t, ST, VL>(pr, fp, grid, s);
}

template <int C, bool ST, bool VL = false>
gdn_status forward_k(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s) {
    return pr->K == 64 ? forward_dt<C, 64, ST, VL>(pr, fp, grid, s)
                       : forward_dt<C, 128, ST, VL>(pr, fp, grid, s);
}

}  // namespace
}  // namespace gdn
