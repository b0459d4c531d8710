// libgdn C ABI: argument validation, launch planning and dispatch onto the
// kernel template instances.  Everything here runs on the host, enqueues on
// the caller's stream and returns; nothing allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cxxabi.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/libgdn.h"
#include "gdn_internal.h"
#include "gdn_prepare.h"
#include "gdn_scan.h"

namespace gdn {

bool tracing();      // GDN_TRACE (below, beside launch_kernel)

namespace {

constexpr int kBV = 64;            // V tile per scan workgroup

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

gdn_status check_problem(const gdn_problem *pr) {
    if (!pr) return GDN_ERR_NULL_ARG;
    if (pr->B < 1 || pr->H < 1 || pr->K < 1 || pr->V < 1 || pr->T < 0 || pr->chunk < 1)
        return GDN_ERR_BAD_SHAPE;
    if (pr->io_dtype != GDN_F32 && pr->io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (pr->o_dtype != GDN_F32 && pr->o_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (pr->io_dtype == GDN_F32 && pr->o_dtype != GDN_F32) return GDN_ERR_UNSUPPORTED;
    if (pr->gate != GDN_GATE_HEAD && pr->gate != GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
    if (pr->K != 64 && pr->K != 128) return GDN_ERR_UNSUPPORTED;
    if (pr->V != 64 && pr->V != 128) return GDN_ERR_UNSUPPORTED;
    if (pr->chunk != 32 && pr->chunk != 64) return GDN_ERR_UNSUPPORTED;
    // index arithmetic inside the kernels: token rows and grid sizes in int
    const int64_t rows = pr->B * pr->T * pr->H;
    if (pr->T > (1 << 30) || rows > ((int64_t)1 << 31) / 8 || pr->B * pr->H > (1 << 24))
        return GDN_ERR_UNSUPPORTED;

    return GDN_OK;
}

gdn_status check_ptrs(std::initializer_list<const void *> required,
                      std::initializer_list<const void *> optional) {
    for (const void *p : required)
        if (!p) return GDN_ERR_NULL_ARG;
    for (const void *p : required)
        if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
    for (const void *p : optional)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    return GDN_OK;
}

// The workspace a forward entry point needs, checked before any launch.
gdn_status check_workspace(const gdn_problem *pr, int64_t n_seqs, const void *ws, size_t ws_bytes) {
    const int64_t need = kda_workspace_bytes(pr, n_seqs);
    if (need == 0) return GDN_OK;
    if (!ws || ws_bytes < (size_t)need) return GDN_ERR_WORKSPACE;
    if (!aligned16(ws)) return GDN_ERR_ALIGNMENT;
    return GDN_OK;
}

// check_problem, and with GDN_TRACE the entry point and its problem
gdn_status check_and_trace(const char *entry, const gdn_problem *pr) {
    const gdn_status st = check_problem(pr);
    if (tracing()) {
        if (pr)
            std::fprintf(stderr,
                         "gdn_trace %s: B=%lld T=%lld H=%lld K=%lld V=%lld chunk=%d io=%s o=%s gate=%s"
                         " V tiles=%lld status=%d\n",
                         entry, (long long)pr->B, (long long)pr->T, (long long)pr->H, (long long)pr->K,
                         (long long)pr->V, pr->chunk, pr->io_dtype == GDN_BF16 ? "bf16" : "fp32",
                         pr->o_dtype == GDN_BF16 ? "bf16" : "fp32", pr->gate == GDN_GATE_KEY ? "key" : "head",
                         (long long)((pr->V + kBV - 1) / kBV), (int)st);
        else
            std::fprintf(stderr, "gdn_trace %s: no problem\n", entry);
    }
    return st;
}

// gdn_forward_split's extra conditions on a validated problem.
gdn_status check_split(const gdn_problem *pr, int64_t t_split) {
    if (pr->gate != GDN_GATE_HEAD || pr->io_dtype != GDN_BF16 || pr->chunk != 64)
        return GDN_ERR_UNSUPPORTED;
    if (t_split <= 0 || t_split >= pr->T || t_split % pr->chunk != 0) return GDN_ERR_BAD_SHAPE;
    const int64_t th = pr->T * pr->H;
    if (th * std::max(pr->K, pr->V) * 4 >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
    if (pr->B * pr->H * (pr->V / 64 + pr->V / 64 + pr->K / 64) >= ((int64_t)1 << 31))
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// Where gdn_forward cuts its streams (0: a single pass).  Each stream is
// serial over its chunks, one workgroup per compute unit: the single pass
// keeps F = B H V/64 units busy for all of T.  The split runs the first
// segment's F workgroups beside the second segment's S = B H (V/64 + K/64)
// (zero-start V tiles and identity-start K tiles) on the other kCUs - F
// units, in R = ceil(S / (kCUs - F)) rounds of T - t_split each, so the two
// segments end together at t_split = T R / (R + 1).  Measured on gdn-shaped
// problems (B H from 8 to 64, K = V = 128), the split took 0.56-0.74 of the
// single pass's time at R = 1 from 128 chunks up and 0.86-0.89 at R = 2 from
// 256 chunks up, and was slower at R = 2 with 64 chunks (the combine
// launches and the ramp cost about 40 us).  Scalar gate, bf16 io, chunk 64
// only (the split's instances); GDN_FORWARD_NO_SPLIT=1 turns it off.
constexpr int64_t kCUs = 256;          // compute units of a gfx950 device
int64_t auto_split_point(const gdn_problem *pr) {
    if (pr->gate != GDN_GATE_HEAD || pr->io_dtype != GDN_BF16 || pr->chunk != 64) return 0;
    if (const char *e = std::getenv("GDN_FORWARD_NO_SPLIT"))
        if (*e == '1') return 0;
    const int64_t nc = (pr->T + pr->chunk - 1) / pr->chunk;
    const int64_t F = pr->B * pr->H * (pr->V / 64), S = pr->B * pr->H * (pr->V / 64 + pr->K / 64);
    if (F >= kCUs) return 0;
    const int64_t R = (S + kCUs - F - 1) / (kCUs - F);
    if (!((R == 1 && nc >= 128) || (R == 2 && nc >= 256))) return 0;
    int64_t t = (pr->T * R / (R + 1) + pr->chunk / 2) / pr->chunk * pr->chunk;
    t = std::min(std::max(t, (int64_t)pr->chunk), (nc - 1) * pr->chunk);
    return check_split(pr, t) == GDN_OK ? t : 0;
}

gdn_status launch(const void *fn, int grid, void *params, size_t psize, hipStream_t s) {
    (void)psize;
    return launch_kernel(fn, grid, params, s);
}

// ---------------------------------------------------------------------------
// prepare
// ---------------------------------------------------------------------------
template <int C, int K, typename IO, bool KG>
gdn_status run_prepare(PrepParams &pp, int grid, hipStream_t s) {
    if constexpr (PrepLayout<C, K, IO, KG>::kBytes > kLdsBytesMax) {
        return GDN_ERR_LDS_BUDGET;
    } else {
        return launch((const void *)&prepare_kernel<C, K, IO, KG>, grid, &pp, sizeof(pp), s);
    }
}

template <int C, int K, typename IO>
gdn_status prepare_gate(const gdn_problem *pr, PrepParams &pp, int grid, hipStream_t s) {
    return pr->gate == GDN_GATE_KEY ? run_prepare<C, K, IO, true>(pp, grid, s)
                                    : run_prepare<C, K, IO, false>(pp, grid, s);
}

template <int C, typename IO>
gdn_status prepare_k(const gdn_problem *pr, PrepParams &pp, int grid, hipStream_t s) {
    return pr->K == 64 ? prepare_gate<C, 64, IO>(pr, pp, grid, s)
                       : prepare_gate<C, 128, IO>(pr, pp, grid, s);
}

template <typename IO>
gdn_status prepare_c(const gdn_problem *pr, PrepParams &pp, int grid, hipStream_t s) {
    return pr->chunk == 32 ? prepare_k<32, IO>(pr, pp, grid, s)
                           : prepare_k<64, IO>(pr, pp, grid, s);
}

gdn_status enqueue_prepare(const gdn_problem *pr, const void *k, const void *v,
                           const float *beta, const float *g, float *w, float *u,
                           float *gcum, hipStream_t s) {
    PrepParams pp;
    pp.k = k; pp.v = v; pp.beta = beta; pp.g = g;
    pp.w = w; pp.u = u; pp.gcum = gcum;
    pp.B = (int)pr->B; pp.T = (int)pr->T; pp.H = (int)pr->H; pp.V = (int)pr->V;
    pp.nt = (int)((pr->T + pr->chunk - 1) / pr->chunk);
    const int grid = (int)(pr->B * pr->H) * pp.nt;
    return pr->io_dtype == GDN_F32 ? prepare_c<float>(pr, pp, grid, s)
                                   : prepare_c<bf16_t>(pr, pp, grid, s);
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
template <int C, int K, typename IO, typename OT, bool KG>
gdn_status run_scan(ScanParams &sp, int grid, hipStream_t s) {
    if constexpr (ScanLayout<C, K, kBV, IO, KG>::kBytes > kLdsBytesMax) {
        return GDN_ERR_LDS_BUDGET;
    } else {
        return launch((const void *)&scan_kernel<C, K, kBV, IO, OT, KG>, grid, &sp, sizeof(sp), s);
    }
}

template <int C, int K, typename IO, typename OT>
gdn_status scan_gate(const gdn_problem *pr, ScanParams &sp, int grid, hipStream_t s) {
    return pr->gate == GDN_GATE_KEY ? run_scan<C, K, IO, OT, true>(sp, grid, s)
                                    : run_scan<C, K, IO, OT, false>(sp, grid, s);
}

template <int C, int K>
gdn_status scan_dt(const gdn_problem *pr, ScanParams &sp, int grid, hipStream_t s) {
    if (pr->io_dtype == GDN_F32) return scan_gate<C, K, float, float>(pr, sp, grid, s);
    if (pr->o_dtype == GDN_F32) return scan_gate<C, K, bf16_t, float>(pr, sp, grid, s);
    return scan_gate<C, K, bf16_t, bf16_t>(pr, sp, grid, s);
}

template <int C>
gdn_status scan_k(const gdn_problem *pr, ScanParams &sp, int grid, hipStream_t s) {
    return pr->K == 64 ? scan_dt<C, 64>(pr, sp, grid, s) : scan_dt<C, 128>(pr, sp, grid, s);
}

gdn_status enqueue_scan(const gdn_problem *pr, const void *q, const void *k,
                        const float *w, const float *u, const float *gcum,
                        const float *h0, void *o, float *hT, hipStream_t s) {
    ScanParams sp;
    sp.q = q; sp.k = k; sp.w = w; sp.u = u; sp.gcum = gcum; sp.h0 = h0;
    sp.o = o; sp.hT = hT;
    sp.B = (int)pr->B; sp.T = (int)pr->T; sp.H = (int)pr->H; sp.V = (int)pr->V;
    sp.nvt = (int)(pr->V / kBV);
    const int pairs = (int)(pr->B * pr->H);
    sp.swizzle = (pairs % 8 == 0) ? 1 : 0;
    if (const char *e = std::getenv("GDN_NO_SWIZZLE")) sp.swizzle = (*e == '1') ? 0 : sp.swizzle;
    const int grid = pairs * sp.nvt;
    return pr->chunk == 32 ? scan_k<32>(pr, sp, grid, s) : scan_k<64>(pr, sp, grid, s);
}

}  // namespace

// The count of bounded LDS waits that gave up (see WaitCtl), one word per
// device.  Its device address is looked up once per device, with that
// device current, and kept: host code passes that address, never the
// symbol's name, to the kernels.
__device__ unsigned gdn_wait_timeout_word;

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_wait_mu;
unsigned *g_wait_addr[kMaxDevices];
bool g_wait_looked_up[kMaxDevices];
}  // namespace

unsigned *wait_count_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_wait_mu);
    if (!g_wait_looked_up[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(gdn_wait_timeout_word)) != hipSuccess) p = nullptr;
        g_wait_addr[dev] = (unsigned *)p;
        g_wait_looked_up[dev] = true;
    }
    return g_wait_addr[dev];
}

// Device memory for gdn_forward_noalloc: the per-key gate's Gram workspace
// lives in this file-scope array instead of caller memory.  Each device
// that loads the library holds its own copy until the process ends; its
// address is looked up once per device, with that device current, and only
// that address (never the array's name, which on the host is a stand-in)
// is handed to kernels.  Every no-alloc call on a device shares the array:
// the Gram kernel writes every slot the re-scan reads before the re-scan
// starts (same stream), so nothing needs clearing, but calls that overlap
// in time on one device (other streams, other threads) race.
constexpr size_t kNoAllocScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scr_mu;
void *g_scr_addr[kMaxDevices];
bool g_scr_looked_up[kMaxDevices];
}  // namespace

void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if (!g_scr_looked_up[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess) ptr = nullptr;
        g_scr_addr[dev] = ptr;
        g_scr_looked_up[dev] = true;
    }
    return g_scr_addr[dev];
}

void wait_params(unsigned &limit, unsigned &bias) {
    // GDN_WAIT_FORCE_TIMEOUT=1 makes every bounded wait give up after a few
    // polls (a test of the timeout path; results are then garbage)
    const char *e = std::getenv("GDN_WAIT_FORCE_TIMEOUT");
    const bool force = e && *e == '1';
    limit = force ? 4u : (1u << 16);
    bias = force ? (1u << 30) : 0u;
}

// GDN_TRACE (environment, read at every call; unset, empty or "0" is off)
// prints each entry point's problem and each launch's plan to stderr: the
// kernel instance, grid, workgroup size, static LDS bytes, registers per
// lane and scratch bytes per lane as the runtime reports them.
bool tracing() {
    const char *e = std::getenv("GDN_TRACE");
    return e && *e && std::strcmp(e, "0") != 0;
}

void trace_launch(const void *fn, int grid, int threads, hipStream_t s) {
    hipFuncAttributes a;
    std::memset(&a, 0, sizeof(a));
    const bool have = hipFuncGetAttributes(&a, fn) == hipSuccess;
    const char *raw = hipKernelNameRefByPtr(fn, s);
    int dst = -1;
    char *nice = raw ? abi::__cxa_demangle(raw, nullptr, nullptr, &dst) : nullptr;
    std::fprintf(stderr, "gdn_trace   launch %s grid=%d block=%d", nice ? nice : (raw ? raw : "?"), grid,
                 threads);
    if (have)
        std::fprintf(stderr, " lds=%zu regs=%d scratch=%zu\n", a.sharedSizeBytes, a.numRegs, a.localSizeBytes);
    else
        std::fprintf(stderr, " (attributes unavailable)\n");
    std::free(nice);
}

gdn_status launch_kernel(const void *fn, int grid, void *params, hipStream_t s, int threads) {
    if (grid <= 0) return GDN_OK;
    if (tracing()) trace_launch(fn, grid, threads, s);
    void *args[] = {params};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, s);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

gdn_status gdn_prepare(const gdn_problem *problem, const void *k, const void *v,
                       const float *beta, const float *g, float *w, float *u,
                       float *gcum, void *stream) {
    gdn_status st = check_and_trace("gdn_prepare", problem);
    if (st != GDN_OK) return st;
    if (problem->T == 0) return GDN_OK;
    st = check_ptrs({k, v, beta, g, w, u, gcum}, {});
    if (st != GDN_OK) return st;
    return enqueue_prepare(problem, k, v, beta, g, w, u, gcum, (hipStream_t)stream);
}

gdn_status gdn_scan(const gdn_problem *problem, const void *q, const void *k,
                    const float *w, const float *u, const float *gcum,
                    const float *h0, void *o, float *hT, void *stream) {
    gdn_status st = check_and_trace("gdn_scan", problem);
    if (st != GDN_OK) return st;
    if (problem->T == 0) {
        st = check_ptrs({}, {h0, hT});
        if (st != GDN_OK) return st;
    } else {
        st = check_ptrs({q, k, w, u, gcum, o}, {h0, hT});
        if (st != GDN_OK) return st;
    }
    if (problem->T == 0 && !hT) return GDN_OK;
    return enqueue_scan(problem, q, k, w, u, gcum, h0, o, hT, (hipStream_t)stream);
}

size_t gdn_workspace_bytes(const gdn_problem *problem) {
    if (check_problem(problem) != GDN_OK) return 0;
    const int64_t t_split = auto_split_point(problem);
    if (t_split > 0) return (size_t)split_workspace_bytes(problem, t_split);
    return (size_t)kda_workspace_bytes(problem, 0);
}

int64_t gdn_forward_split_point(const gdn_problem *problem) {
    if (check_problem(problem) != GDN_OK) return 0;
    return auto_split_point(problem);
}

size_t gdn_workspace_bytes_varlen(const gdn_problem *problem, int64_t n_seqs) {
    if (check_problem(problem) != GDN_OK || n_seqs < 1) return 0;
    return (size_t)kda_workspace_bytes(problem, n_seqs);
}

gdn_status gdn_forward(const gdn_problem *problem, const void *q, const void *k,
                       const void *v, const float *beta, const float *g,
                       const float *h0, void *o, float *hT, void *workspace,
                       size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_forward", problem);
    if (st != GDN_OK) return st;
    if (problem->T == 0) {
        st = check_ptrs({}, {h0, hT});
        if (st != GDN_OK) return st;
        if (!hT) return GDN_OK;
    } else {
        st = check_ptrs({q, k, v, beta, g, o}, {h0, hT});
        if (st != GDN_OK) return st;
        st = check_workspace(problem, 0, workspace, workspace_bytes);
        if (st != GDN_OK) return st;
        // long streams on a partly idle device: the sequence split, when the
        // workspace holds it (else the single pass)
        const int64_t t_split = auto_split_point(problem);
        if (t_split > 0 && workspace && aligned16(workspace) &&
            workspace_bytes >= (size_t)split_workspace_bytes(problem, t_split))
            return enqueue_forward_split(problem, t_split, q, k, v, beta, g, h0, o, hT, workspace,
                                         (hipStream_t)stream);
    }
    return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, nullptr, nullptr, nullptr, 0,
                           workspace, (hipStream_t)stream);
}

gdn_status gdn_forward_noalloc(const gdn_problem *problem, const void *q, const void *k,
                               const void *v, const float *beta, const float *g,
                               const float *h0, void *o, float *hT, void *stream) {
    gdn_status st = check_and_trace("gdn_forward_noalloc", problem);
    if (st != GDN_OK) return st;
    if (problem->T == 0) {
        st = check_ptrs({}, {h0, hT});
        if (st != GDN_OK) return st;
        if (!hT) return GDN_OK;
        return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, nullptr, nullptr, nullptr,
                               0, nullptr, (hipStream_t)stream);
    }
    st = check_ptrs({q, k, v, beta, g, o}, {h0, hT});
    if (st != GDN_OK) return st;
    const int64_t need = kda_workspace_bytes(problem, 0);
    if (need > (int64_t)kNoAllocScratchBytes) return GDN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws) return GDN_ERR_HIP;
    }
    return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, nullptr, nullptr, nullptr, 0, ws,
                           (hipStream_t)stream);
}

// The split forward's own conditions: scalar gate, bf16 io, chunk 64, a cut
// at a chunk boundary strictly inside the sequence.
size_t gdn_workspace_bytes_split(const gdn_problem *problem, int64_t t_split) {
    if (check_problem(problem) != GDN_OK || check_split(problem, t_split) != GDN_OK) return 0;
    return (size_t)split_workspace_bytes(problem, t_split);
}

gdn_status gdn_forward_split(const gdn_problem *problem, int64_t t_split, const void *q,
                             const void *k, const void *v, const float *beta, const float *g,
                             const float *h0, void *o, float *hT, void *workspace,
                             size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_forward_split", problem);
    if (st != GDN_OK) return st;
    st = check_split(problem, t_split);
    if (st != GDN_OK) return st;
    st = check_ptrs({q, k, v, beta, g, o, workspace}, {h0, hT});
    if (st != GDN_OK) return st;
    if (workspace_bytes < (size_t)split_workspace_bytes(problem, t_split)) return GDN_ERR_WORKSPACE;
    return enqueue_forward_split(problem, t_split, q, k, v, beta, g, h0, o, hT, workspace,
                                 (hipStream_t)stream);
}

gdn_status gdn_forward_states(const gdn_problem *problem, const void *q, const void *k,
                              const void *v, const float *beta, const float *g,
                              const float *h0, void *o, float *hT, void *hck, void *vnew,
                              void *workspace, size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_forward_states", problem);
    if (st != GDN_OK) return st;
    if (problem->T == 0) {
        // no chunk, so no checkpoint and no token: only hT = h0 (or zero)
        st = check_ptrs({}, {h0, hT, hck, vnew});
        if (st != GDN_OK) return st;
        if (!hT) return GDN_OK;
        return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, nullptr, nullptr, nullptr,
                               0, nullptr, (hipStream_t)stream);
    }
    st = check_ptrs({q, k, v, beta, g, o, hck, vnew}, {h0, hT});
    if (st != GDN_OK) return st;
    st = check_workspace(problem, 0, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, hck, vnew, nullptr, 0, workspace,
                           (hipStream_t)stream);
}

gdn_status gdn_rescan_dq(const gdn_problem *problem, const void *q, const void *k,
                         const void *v, const float *beta, const float *g, const float *h0,
                         const void *dout, float *hT, void *hck, void *vnew, float *dq,
                         void *workspace, size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_rescan_dq", problem);
    if (st != GDN_OK) return st;
    if (problem->io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (problem->T == 0) {
        st = check_ptrs({}, {h0, hT, hck, vnew, dq, dout});
        if (st != GDN_OK) return st;
        if (!hT) return GDN_OK;
        return enqueue_forward(problem, q, k, v, beta, g, h0, nullptr, hT, nullptr, nullptr,
                               nullptr, 0, nullptr, (hipStream_t)stream);
    }
    st = check_ptrs({q, k, v, beta, g, dout, hck, vnew, dq}, {h0, hT});
    if (st != GDN_OK) return st;
    st = check_workspace(problem, 0, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    return enqueue_forward(problem, q, k, v, beta, g, h0, nullptr, hT, hck, vnew, nullptr, 0,
                           workspace, (hipStream_t)stream, dout, dq);
}

gdn_status gdn_chunk_dq(const gdn_problem *problem, const void *dout, const void *hck, float *dq,
                        void *stream) {
    gdn_status st = check_and_trace("gdn_chunk_dq", problem);
    if (st != GDN_OK) return st;
    if (problem->io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (problem->T == 0) return GDN_OK;
    st = check_ptrs({dout, hck, dq}, {});
    if (st != GDN_OK) return st;
    // one chunk's token rows of dO and dq are addressed with 32-bit offsets
    const int64_t row_bytes = problem->H * std::max(2 * problem->V, 4 * problem->K);
    if ((int64_t)problem->chunk * row_bytes >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
    return enqueue_chunk_dq(problem, dout, hck, dq, (hipStream_t)stream);
}

gdn_status gdn_forward_varlen(const gdn_problem *problem, const int32_t *cu_seqlens,
                              int64_t n_seqs, const void *q, const void *k, const void *v,
                              const float *beta, const float *g, const float *h0, void *o,
                              float *hT, void *workspace, size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_forward_varlen", problem);
    if (st != GDN_OK) return st;
    if (problem->B != 1 || n_seqs < 1 || n_seqs * problem->H > (1 << 24)) return GDN_ERR_BAD_SHAPE;
    if (!cu_seqlens) return GDN_ERR_NULL_ARG;
    if (((uintptr_t)cu_seqlens & 3u) != 0) return GDN_ERR_ALIGNMENT;
    if (problem->T == 0) {
        // every sequence is empty: hT = h0 (or zero) per sequence
        st = check_ptrs({}, {h0, hT});
        if (st != GDN_OK) return st;
        if (!hT) return GDN_OK;
    } else {
        st = check_ptrs({q, k, v, beta, g, o}, {h0, hT});
        if (st != GDN_OK) return st;
        st = check_workspace(problem, n_seqs, workspace, workspace_bytes);
        if (st != GDN_OK) return st;
    }
    return enqueue_forward(problem, q, k, v, beta, g, h0, o, hT, nullptr, nullptr, cu_seqlens,
                           n_seqs, workspace, (hipStream_t)stream);
}

size_t gdn_workspace_bytes_backward(const gdn_problem *problem) {
    if (check_problem(problem) != GDN_OK) return 0;
    return (size_t)backward_workspace_bytes(problem);
}

gdn_status gdn_backward(const gdn_problem *problem, const void *q, const void *k, const void *v,
                        const float *beta, const float *g, const void *dout, const float *dhT,
                        const void *hck, const void *vnew, float *dq, float *dk, float *dv,
                        float *dbeta, float *dg, float *dh0, void *workspace,
                        size_t workspace_bytes, void *stream) {
    gdn_status st = check_and_trace("gdn_backward", problem);
    if (st != GDN_OK) return st;
    if (problem->io_dtype != GDN_BF16 || problem->o_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    // per-stream 32-bit byte offsets: fp32 [T, H, K | V] rows and one head's K x V block
    const int64_t row_bytes = problem->H * 4 * std::max(problem->K, problem->V);
    if (problem->T * row_bytes >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
    if (problem->T == 0) {
        // no tokens: dh0 = dhT (or zero)
        st = check_ptrs({}, {dhT, dh0});
        if (st != GDN_OK) return st;
        if (!dh0) return GDN_OK;
        return enqueue_backward(problem, q, k, v, beta, g, dout, dhT, hck, vnew, dq, dk, dv, dbeta,
                                dg, dh0, nullptr, (hipStream_t)stream);
    }
    st = check_ptrs({q, k, v, beta, g, dout, hck, vnew, dq, dk, dv, dbeta, dg}, {dhT, dh0});
    if (st != GDN_OK) return st;
    const int64_t need = backward_workspace_bytes(problem);
    if (!workspace || workspace_bytes < (size_t)need) return GDN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GDN_ERR_ALIGNMENT;
    return enqueue_backward(problem, q, k, v, beta, g, dout, dhT, hck, vnew, dq, dk, dv, dbeta, dg,
                            dh0, workspace, (hipStream_t)stream);
}

gdn_status gdn_wait_timeouts(uint32_t *count, int reset) {
    if (!count) return GDN_ERR_NULL_ARG;
    unsigned *p = wait_count_ptr();
    if (!p) return GDN_ERR_HIP;
    unsigned v = 0;
    if (hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return GDN_ERR_HIP;
    *count = v;
    if (reset) {
        const unsigned zero = 0;
        if (hipMemcpy(p, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

const char *gdn_status_str(gdn_status status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_ARG: return "GDN_ERR_NULL_ARG: a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: invalid problem size";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: shape or dtype not implemented";
        case GDN_ERR_ALIGNMENT: return "GDN_ERR_ALIGNMENT: pointer not 16-byte aligned";
        case GDN_ERR_LDS_BUDGET: return "GDN_ERR_LDS_BUDGET: kernel LDS need exceeds 160 KiB";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime call failed";
    }
    return "unknown gdn_status";
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
