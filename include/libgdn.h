/*
 * libgdn -- forward pass of the chunked gated delta rule on AMD Instinct
 * MI355X (gfx950).
 *
 * The method: per (batch, head) a state S_t (V x K) follows
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,            a_t = exp(g_t),
 * with one log-gate g_t per (token, head) for Gated DeltaNet, or one per
 * (token, head, key dimension) for Kimi-Delta-Attention (KDA), in which case
 * Diag(a_t) scales the key index of S.  The sequence is cut into chunks of C
 * tokens; a chunk's tokens are folded into WY factors (w, u) by a unit lower
 * triangular inverse, and a serial scan carries the state across chunks.
 *   - gdn_prepare follows the TileOPs gated deltanet "fused prepare" kernel
 *     (page "Reuse P as beta tiles in gated deltanet fused prepare": A_g, its
 *     inverse, then w = A_g^-1 k_beta and u = A_g^-1 v_beta).
 *   - gdn_scan follows the per-chunk algebra of the kernel_fun KDA forward
 *     re-scan (bwd_scan.py, KdaB1ScanKernel docstring: v' = u - w h,
 *     h <- exp(gd) h + kg^T v'), plus the output read-out.
 *   - gdn_forward is the two fused: q, k, v, beta, g (and h0) in, o and the
 *     final state out.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts are dense and row-major (the innermost index is contiguous):
 *     q, k, w     [B, T, H, K]       v, u, o   [B, T, H, V]
 *     beta        [B, T, H]          g, gcum   [B, T, H]  (GDN_GATE_HEAD)
 *                                              [B, T, H, K] (GDN_GATE_KEY)
 *     h0, hT      [B, H, K, V]  with hT[b,h,i,j] = S_T[j,i]  (fp32)
 * q, k, v use the problem's io dtype; o uses its o dtype; beta, g, gcum, w,
 * u, h0 and hT are always fp32.  g is the natural-log gate (g <= 0 for a
 * decaying state); gcum is its chunk-local inclusive cumulative sum.
 *
 * Numerics: state, accumulation and the triangular inverse are fp32.  With
 * bf16 io, matrix-core operands are fp16 (raw bf16 inputs convert exactly for
 * magnitudes in [2^-14, 65504]; derived operands are rounded once); with
 * fp32 io they are fp32.  Inputs and the state must keep |x| < 65504 with
 * bf16 io.  Any gate g <= 0 is supported, however strong: every decay
 * factor that enters an operand or a product is a decay (at most 1), for
 * both gates -- within a chunk each pair's decay e^(gcum_r - gcum_s) is
 * split at a row between r and s (the per-key gate by halving the chunk,
 * see gdn_forward), and operands are referenced to the chunk's start or end.
 * A factor that underflows only drops contributions below the operands'
 * precision.
 *
 * Ownership and execution: the caller allocates every buffer (device
 * memory) and owns it; the library never allocates, frees or synchronises.
 * Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 * default stream) and returns.  Argument, shape, alignment and resource
 * errors are reported before anything is enqueued; a failed launch returns
 * GDN_ERR_HIP; faults during execution surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 *
 * Diagnostics: with the environment variable GDN_TRACE set (to anything but
 * "" or "0"; read at every call) each entry point that takes a problem
 * prints it and its validation status to stderr, and each kernel launch
 * prints its plan: the kernel instance, grid, workgroup size, static LDS
 * bytes, registers and scratch bytes per lane.  libgdn_poison.so, built
 * beside libgdn.so from the same sources, exports this same interface; its
 * pipelined kernels fill each LDS stage with NaN once its last reader is
 * done with it, so that a read that overtakes the write it must wait for
 * shows up as NaN.  With every wait in place it returns exactly libgdn.so's
 * results, more slowly.
 *
 * Requirements: all pointers 16-byte aligned; K, V in {64, 128}; chunk in
 * {32, 64}; B, H >= 1; T >= 0 (any T: a short last chunk is exact).  Shapes
 * outside this set return GDN_ERR_UNSUPPORTED; there is no fallback path.
 * o must not alias any input; hT may alias h0 only in gdn_forward,
 * gdn_forward_split and gdn_scan (each state tile is read completely before
 * it is written).
 *
 * Thread safety: stateless; calls from several host threads are safe.
 */
#ifndef LIBGDN_H
#define LIBGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 10

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,     /* negative or zero size where >= 1 is needed */
    GDN_ERR_UNSUPPORTED = 3,   /* valid but not implemented (K, V, chunk, dtype) */
    GDN_ERR_ALIGNMENT = 4,     /* a pointer is not 16-byte aligned */
    GDN_ERR_LDS_BUDGET = 5,    /* the kernel's LDS need exceeds 160 KiB per CU */
    GDN_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required */
    GDN_ERR_HIP = 7            /* a HIP runtime call failed (see hipGetLastError) */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_gate {
    GDN_GATE_HEAD = 0,         /* Gated DeltaNet: g [B,T,H] */
    GDN_GATE_KEY = 1           /* KDA: g [B,T,H,K] */
} gdn_gate;

typedef struct gdn_problem {
    int64_t B, T, H, K, V;     /* batch, tokens, heads, key dim, value dim */
    int32_t chunk;             /* chunk size C: 32 or 64 */
    int32_t io_dtype;          /* gdn_dtype of q, k, v */
    int32_t o_dtype;           /* gdn_dtype of o */
    int32_t gate;              /* gdn_gate */
} gdn_problem;

/*
 * gdn_prepare -- per-chunk WY factors (fully parallel over chunks).
 * For each (b, h) and chunk of C tokens (r, s index the chunk's rows):
 *   gcum[r] = sum_{j<=r} g[j]                      (chunk-local, inclusive)
 *   A[r,s]  = beta_r sum_d k[r,d] k[s,d] exp(gcum[r,d]-gcum[s,d]),  s < r
 *   Tm      = (I + A)^-1                           (unit lower triangular)
 *   w       = Tm diag(beta) (exp(gcum) * k)        (row r of k scaled by
 *                                                   beta_r exp(gcum[r]))
 *   u       = Tm diag(beta) v
 * (TileOPs "Reuse P as beta tiles in gated deltanet fused prepare": A_g,
 * S_shared = its inverse, w/u from k_beta/v_beta; the exp(gcum) factor on w
 * is what makes the scan's v' = u - w h use the chunk-start state.)
 * Inputs k [B,T,H,K], v [B,T,H,V] in io dtype; beta, g fp32.
 * Outputs w [B,T,H,K], u [B,T,H,V], gcum (g's shape), all fp32, written in
 * full.  problem->o_dtype is ignored.
 */
gdn_status gdn_prepare(const gdn_problem *problem, const void *k, const void *v,
                       const float *beta, const float *g, float *w, float *u,
                       float *gcum, void *stream);

/*
 * gdn_scan -- the serial inter-chunk scan, given gdn_prepare's outputs.
 * For each (b, h), starting from h = h0[b,h] (K x V; zero if h0 is NULL),
 * per chunk (kernel_fun KDA re-scan, per-chunk algebra of KdaB1ScanKernel):
 *   v'  = u - w h
 *   o   = (q * exp(gcum)) h + tril_incl((q k^T) * decay) v'
 *            decay[r,s] = exp(gcum[r] - gcum[s])  (per key dim for KDA)
 *   h  <- exp(gcum_last) * h + (k * exp(gcum_last - gcum))^T v'
 * and finally hT[b,h] = h.  Inputs q, k in io dtype; w, u, gcum, h0 fp32.
 * o [B,T,H,V] in o dtype; hT may be NULL (not written) or alias h0.
 */
gdn_status gdn_scan(const gdn_problem *problem, const void *q, const void *k,
                    const float *w, const float *u, const float *gcum,
                    const float *h0, void *o, float *hT, void *stream);

/*
 * gdn_forward -- the whole forward pass: o and the final state from q, k, v,
 * beta, g and an optional h0 (NULL = zero state).  Results equal
 * gdn_prepare followed by gdn_scan up to rounding.  hT may be NULL or alias
 * h0.
 * Workspace: `workspace` must hold gdn_workspace_bytes(problem) bytes of
 * device memory, 16-byte aligned (it may be NULL when that is 0, or for the
 * scalar gate); its contents on entry do not matter, and it is free again
 * once the call's work on `stream` is done.  Otherwise GDN_ERR_WORKSPACE
 * (missing or too small) or GDN_ERR_ALIGNMENT before any launch.
 * Scalar gate: when gdn_forward_split_point(problem) is nonzero (long
 * streams that leave compute units idle, bf16 io, chunk 64) and the
 * workspace holds gdn_workspace_bytes(problem) bytes, the call runs
 * gdn_forward_split at that point (three launches); with a smaller or no
 * workspace it runs the single pass.  Either way the results agree up to
 * rounding.
 * For the per-key gate the call is two launches: a kernel over every chunk at
 * once forms each chunk's decayed Gram products (A, and P of the read-out)
 * with every pair's decay split at a row between the two tokens, found by
 * halving the chunk (TileOPs fused-prepare page: A_g and its inverse), and
 * the 16-token blocks of (I + A)^-1; with bf16 io also the re-scan's
 * operands q e^gcum, k e^gcum and k e^(gl - gcum), all decays referenced to
 * the chunk's ends.  Every factor is a product of per-token decays e^g <= 1.
 * It leaves them in the workspace, one slot per (chunk, head) (see
 * gdn_workspace_bytes); the re-scan then reads them (kernel-fun KDA re-scan
 * page's per-chunk algebra).
 */
gdn_status gdn_forward(const gdn_problem *problem, const void *q, const void *k,
                       const void *v, const float *beta, const float *g,
                       const float *h0, void *o, float *hT, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * gdn_forward_split_point -- where gdn_forward cuts each stream of this
 * problem into two segments run side by side (see gdn_forward_split), or 0
 * for a single pass.  Every (batch, head, 64-wide V tile) stream is serial
 * over its chunks and takes one compute unit, so a problem with F = B H V/64
 * streams leaves 256 - F units of a gfx950 device idle.  The split runs the
 * second segment as S = B H (V/64 + K/64) streams (zero-start V tiles and
 * identity-start K tiles) on those units in R = ceil(S / (256 - F)) rounds,
 * and cuts at T R / (R + 1), rounded to a chunk, so both segments end
 * together.  Nonzero for the scalar gate with bf16 io and chunk 64 when
 * R = 1 and T spans at least 128 chunks, or R = 2 and at least 256 chunks
 * (where it measured faster); 0 otherwise, for bad arguments, or with the
 * environment variable GDN_FORWARD_NO_SPLIT=1.
 */
int64_t gdn_forward_split_point(const gdn_problem *problem);

/*
 * gdn_forward_states -- gdn_forward that also saves what a backward pass
 * re-reads: the state at the start of every chunk and the delta each token
 * writes into the state (kernel_fun KDA re-scan page, bwd_scan.py: the h
 * checkpoints [B,NT,HV,K,V] and v_new [B,T,HV,V] of its host wrapper
 * chunk_gated_delta_rule_fwd_h and of KdaB1ScanKernel's per-chunk algebra).
 *   hck  [B, NT, H, K, V], NT = ceil(T / chunk): hck[b,c,h] is h (the K x V
 *        state, h = S^T) before token c*chunk is applied; hck[b,0,h] = h0
 *        (or zero).
 *   vnew [B, T, H, V]: the chunk form's v' = u - w h, which equals
 *        beta_t (v_t - S' k_t) with S' the state after token t's decay, so
 *        that h_t = Diag(a_t) h_{t-1} + k_t vnew_t^T.
 * Both are written in full, in the problem's o dtype (bf16 rounds to
 * nearest even).  o, hT and every other argument are as in gdn_forward;
 * hck and vnew must be non-NULL and 16-byte aligned when T > 0 (with T = 0
 * nothing is written to them and they may be NULL).  hck, vnew and o must
 * not alias each other or any input.  Workspace as in gdn_forward.
 */
gdn_status gdn_forward_states(const gdn_problem *problem, const void *q, const void *k,
                              const void *v, const float *beta, const float *g,
                              const float *h0, void *o, float *hT, void *hck, void *vnew,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_rescan_dq -- the backward pass's forward re-scan (kernel_fun KDA re-scan
 * page, bwd_scan.py: its CuTe kernel re-runs the state recurrence to save
 * the h checkpoints and v_new and, fused in, forms dq's only dependence on
 * the state, DQ = dO h_c^T, raw: no gate and no scale).  Here with bf16 io,
 * for the scalar gate (Gated DeltaNet) and the per-key gate (KDA), chunk 32
 * or 64:
 *   hck, vnew  as in gdn_forward_states (problem->o_dtype);
 *   dq [B,T,H,K] fp32: dq[t] += h_c dO_t for token t of chunk c, h_c the
 *              state at the chunk's start (K x V), dO [B,T,H,V] in the io
 *              dtype.  dq is accumulated into (the V tiles of a head add up
 *              there, in an order that does not change the sum for V <= 128),
 *              so the caller zeroes it first.
 * No o is produced (q is still read).  hT, h0 as in gdn_forward.  fp32 io
 * returns GDN_ERR_UNSUPPORTED.
 * With T = 0 only hT is
 * written.  Pointers as in gdn_forward_states; dq must not alias any input.
 * Workspace as in gdn_forward.
 */
gdn_status gdn_rescan_dq(const gdn_problem *problem, const void *q, const void *k,
                         const void *v, const float *beta, const float *g, const float *h0,
                         const void *dout, float *hT, void *hck, void *vnew, float *dq,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_backward -- the gradients of gdn_forward's outputs with respect to
 * every input, for either gate (one per head, Gated DeltaNet; one per key
 * dimension, KDA) with bf16 io, from what
 * gdn_forward_states (or gdn_rescan_dq) saved: the kernel_fun KDA re-scan
 * page has its re-scan keep the h checkpoints and v_new for the backward's
 * later stage (bwd_scan.py module docstring); this is that stage, with the
 * state's gradient carried backwards through the chunks.  For the loss
 * L = sum_t o_t . dO_t + sum hT * dhT:
 *   dout [B,T,H,V] bf16   dO
 *   dhT  [B,H,K,V] fp32   the final state's gradient, or NULL (zero)
 *   hck, vnew             bf16, as gdn_forward_states writes them for the
 *                         same inputs and chunk (problem->o_dtype must be
 *                         GDN_BF16: they are read in that dtype)
 *   dq, dk [B,T,H,K], dv [B,T,H,V], dbeta [B,T,H], dg (g's shape: [B,T,H]
 *        or [B,T,H,K])   fp32, written in full
 *   dh0  [B,H,K,V] fp32   h0's gradient, or NULL (not written)
 * Scalar gate: three launches on the stream: one workgroup per (chunk, head) forms each
 * chunk's factors of the reverse scan (the decayed Gram products, T^T and
 * P^T, the row factors); the reverse scan (one workgroup per (batch, head,
 * 64-wide V tile), serial over chunks) writes dR (v's gradient before the
 * beta factor) and the gradient of every chunk's end state into the
 * workspace, and dv and dh0; then one workgroup per (chunk, head) forms dq,
 * dk, dbeta and dg.  Workspace: gdn_workspace_bytes_backward(problem)
 * bytes, 16-byte aligned: dR [B,T,H,V] fp32, then the chunk-end gradients
 * [B,NT,H,K,V] fp32, then the per-chunk factors.  The per-key gate adds a
 * fourth launch for its decay-weighted sums (the decay of every pair of
 * tokens is per key, inside the C x C x K sums), and its workspace also
 * holds dP and dA per (chunk, head).  Results are deterministic (no
 * atomics).  Outputs must
 * not alias inputs or each other.  With T = 0 only dh0 is written (= dhT or
 * zero).  GDN_ERR_UNSUPPORTED for fp32 io, an fp32 o_dtype, or a stream
 * whose fp32 rows exceed 4 GiB.
 */
gdn_status gdn_backward(const gdn_problem *problem, const void *q, const void *k, const void *v,
                        const float *beta, const float *g, const void *dout, const float *dhT,
                        const void *hck, const void *vnew, float *dq, float *dk, float *dv,
                        float *dbeta, float *dg, float *dh0, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Workspace gdn_backward needs: B T H V 4 + B NT H K V 4 bytes (NT =
 * ceil(T / chunk)) + B NT H slot bytes, a slot being 8 C^2 + 16 C + 16
 * bytes (per-key gate: 8 C^2 + 4 C K + 4 C + 4 K, plus 8 C^2 more per
 * (chunk, head) for dP and dA); 0 on bad arguments. */
size_t gdn_workspace_bytes_backward(const gdn_problem *problem);

/*
 * gdn_chunk_dq -- dq's chunk-start-state term on its own, from states that
 * gdn_forward_states saved: the DQ = dO h^T product that the kernel_fun KDA
 * re-scan page fuses into its re-scan, whose own measurements found the
 * fused form slower (its section on the dq fusion); gdn_rescan_dq is the
 * fused form here.
 *   dout [B,T,H,V] in the io dtype (bf16 only);
 *   hck  [B,NT,H,K,V] in problem->o_dtype (bf16 or fp32), NT = ceil(T/chunk),
 *        as gdn_forward_states writes it;
 *   dq   [B,T,H,K] fp32, written (not accumulated): dq[t] = h_c dO_t for
 *        token t of chunk c, raw (no gate, no scale; the same for either
 *        gate).  fp32 states enter the product as bf16 high and low parts
 *        (~16 bits), bf16 states exactly; fp32 accumulation.
 * problem->gate is not used.  fp32 io returns GDN_ERR_UNSUPPORTED.  With
 * T = 0 nothing is done and the pointers may be NULL; otherwise all three
 * are required and 16-byte aligned, and dq must not alias the others.
 * Needs no workspace; one kernel launch, deterministic.
 */
gdn_status gdn_chunk_dq(const gdn_problem *problem, const void *dout, const void *hck, float *dq,
                        void *stream);

/*
 * gdn_forward_varlen -- gdn_forward over packed sequences of different
 * lengths (the kernel_fun re-scan page's host wrapper takes only T a
 * multiple of 64 and falls back otherwise; here any lengths run in the one
 * kernel, each sequence from its own initial state).
 *   problem->B must be 1 and problem->T is the total token count; q, k, v,
 *   beta, g, o use the [1, T, H, .] layouts of gdn_forward.
 *   cu_seqlens: n_seqs + 1 int32 token offsets in device memory (4-byte
 *   aligned), cu_seqlens[0] = 0, nondecreasing, cu_seqlens[n_seqs] = T;
 *   sequence n is tokens [cu_seqlens[n], cu_seqlens[n+1]).  The kernel
 *   clamps each offset into [0, T] (a malformed list gives wrong results,
 *   never an access outside the tensors); it must hold n_seqs + 1 entries.
 *   h0, hT: [n_seqs, H, K, V] fp32, the initial and final state of each
 *   sequence; h0 NULL means zero states, hT NULL means not written.
 * The state never crosses from one sequence into the next; results equal
 * separate gdn_forward calls per sequence.  Returns GDN_ERR_BAD_SHAPE if
 * problem->B != 1 or n_seqs < 1.  Workspace as in gdn_forward, of
 * gdn_workspace_bytes_varlen(problem, n_seqs) bytes.
 */
gdn_status gdn_forward_varlen(const gdn_problem *problem, const int32_t *cu_seqlens,
                              int64_t n_seqs, const void *q, const void *k, const void *v,
                              const float *beta, const float *g, const float *h0, void *o,
                              float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_wait_timeouts -- diagnostics of the bf16-io kernels' internal waits.
 * Inside a workgroup, the waves that prepare a chunk and the waves that scan
 * the previous one hand tiles over through LDS counters.  Every such wait is
 * bounded (2^16 polls, a few milliseconds): a wait that runs out lets the
 * wave go on instead of hanging the GPU, and adds one to a per-device count.
 * A launch during which the count grew has results that must not be
 * trusted.  This call stores the current device's count in *count and, if
 * `reset` is nonzero, sets it back to zero.  Unlike every other entry point
 * it is synchronous: it copies from device memory with hipMemcpy, so it
 * waits for the device's outstanding work.  Returns GDN_ERR_NULL_ARG for a
 * NULL count and GDN_ERR_HIP if the device word cannot be read.
 * (Setting the environment variable GDN_WAIT_FORCE_TIMEOUT=1 before a
 * launch makes every such wait give up after a few polls: a test of this
 * path only; the results of that launch are garbage, and every kernel still
 * ends normally.)
 */
gdn_status gdn_wait_timeouts(uint32_t *count, int reset);

/*
 * gdn_forward_split -- gdn_forward for the scalar gate (bf16 io, chunk 64)
 * with every stream cut at token t_split (a multiple of 64, 0 < t_split < T)
 * into two segments that run at the same time.  The recurrence is affine in
 * the state: from a start state h_in a segment ends in N + M h_in and
 * outputs o0_t + h_in^T oI_t, where N and o0 come from a zero start and M
 * and oI (a K-vector per token) from the identity start with v = 0 (the
 * chunk-parallel form of the scan the kernel-fun KDA re-scan page runs
 * serially).  One launch runs the first segment from h0 beside the second
 * segment's zero-start and identity-start passes; two small launches then
 * add h_in^T oI_t to the second segment's outputs and form hT = N + M h_in.
 * With one workgroup per compute unit the two segments fill the device
 * together when the first holds about twice the second's chunks.  Results
 * equal gdn_forward's up to rounding (the o of the second segment is
 * rounded to the o dtype twice when that is bf16).  Arguments as in
 * gdn_forward; hT may be NULL or alias h0 (h0 is read by the first launch
 * only, hT written by the last).  Workspace:
 * gdn_workspace_bytes_split(problem, t_split) bytes, 16-byte aligned.
 * GDN_ERR_UNSUPPORTED for the per-key gate, fp32 io or chunk 32;
 * GDN_ERR_BAD_SHAPE for a t_split outside those bounds.
 */
gdn_status gdn_forward_split(const gdn_problem *problem, int64_t t_split, const void *q,
                             const void *k, const void *v, const float *beta, const float *g,
                             const float *h0, void *o, float *hT, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Workspace gdn_forward_split needs: B H K V 4 (the first segment's end
 * state) + B H K V 4 (N) + B H K K 4 (M) + B H K V 4 (that end state
 * transposed in two bf16 parts) + B (T - t_split) H K times the o dtype's
 * size (oI).  0 on bad or unsupported arguments. */
size_t gdn_workspace_bytes_split(const gdn_problem *problem, int64_t t_split);

/*
 * gdn_forward_noalloc -- gdn_forward for callers that cannot allocate device
 * memory (code under stream capture into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * gdn_forward, without the workspace: the per-key gate's Gram workspace is
 * taken from a static device array of GDN_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on each device it runs on until the process ends.  The
 * scalar gate always runs the single pass here (never the sequence split,
 * whose workspace grows with T).  The call allocates nothing and frees
 * nothing.  Returns GDN_ERR_WORKSPACE, before anything is enqueued, when the
 * per-key gate's workspace, gdn_workspace_bytes(problem), exceeds that size
 * (the scalar gate uses none here and is never refused for it), and
 * GDN_ERR_HIP if the array's device address cannot be looked up (done once
 * per device, on the first call that needs it, with the current device).
 * All calls on one device share the array: calls that may run at the same
 * time on one device (different streams or host threads without ordering
 * between them) race and corrupt each other's results; calls ordered on one
 * stream are safe.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gdn_status gdn_forward_noalloc(const gdn_problem *problem, const void *q, const void *k,
                               const void *v, const float *beta, const float *g,
                               const float *h0, void *o, float *hT, void *stream);

/* Workspace gdn_forward, gdn_forward_states and gdn_rescan_dq need for this
 * problem.  Per-key gate: one slot per (chunk, head), B * ceil(T / chunk) * H
 * slots of 2 * chunk^2 * 4 bytes (fp32 io: the solve tile and P) or
 * 2 * chunk^2 * 2 + 3 * chunk * K * 2 + 4 * K bytes (bf16 io: the same in
 * fp16, the re-scan's three fp16 operand tiles and the chunk's per-key
 * decay).  Scalar gate: gdn_workspace_bytes_split(problem, t) when
 * t = gdn_forward_split_point(problem) is nonzero (what gdn_forward's split
 * uses; gdn_forward_states and gdn_rescan_dq need none and ignore it), else
 * 0.  0 for T = 0 and on bad arguments. */
size_t gdn_workspace_bytes(const gdn_problem *problem);

/* The same for gdn_forward_varlen over n_seqs packed sequences (the per-key
 * gate: (ceil(T / chunk) + n_seqs) * H slots). */
size_t gdn_workspace_bytes_varlen(const gdn_problem *problem, int64_t n_seqs);

/* Static, human-readable name of a status code. */
const char *gdn_status_str(gdn_status status);

/* GDN_ABI_VERSION of the library that was loaded. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_H */
