// Host-side declarations shared by the translation units of libgdn.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/libgdn.h"

namespace gdn {

// Device address of this device's count of bounded LDS waits that gave up
// (NULL if it cannot be looked up), and the poll limit and target bias the
// pipelined kernels take (normal: 2^16 polls, bias 0).
unsigned *wait_count_ptr();
void wait_params(unsigned &limit, unsigned &bias);

// Launch a kernel with one by-value parameter struct (256 threads per block
// unless stated).
gdn_status launch_kernel(const void *fn, int grid, void *params, hipStream_t s,
                         int threads = 256);

// Enqueue the fused forward kernel (validated problem, non-empty work).
// hck and vnew are both NULL, or both set for the instance that also saves
// the chunk-start states and the per-token deltas.  cu (n_seqs + 1 device
// int32 offsets) selects packed sequences over a B = 1 problem, or is NULL.
// Enqueue dq = dO h_c^T per chunk from saved states (validated problem, T > 0).
gdn_status enqueue_chunk_dq(const gdn_problem *pr, const void *dout, const void *hck, float *dq,
                            hipStream_t s);

gdn_status enqueue_forward(const gdn_problem *pr, const void *q, const void *k,
                           const void *v, const float *beta, const float *g,
                           const float *h0, void *o, float *hT, void *hck, void *vnew,
                           const int32_t *cu, int64_t n_seqs, void *ws, hipStream_t s,
                           const void *dout = nullptr, float *dq = nullptr);

// Per-key gate: the workspace the forward entry points need (kda_gram_kernel's
// Tmb and P per chunk and head; 0 for the scalar gate or T = 0), for a
// fixed-length batch (n_seqs = 0) or n_seqs packed sequences; and the launch
// of kda_gram_kernel into it.
int64_t kda_workspace_bytes(const gdn_problem *pr, int64_t n_seqs);
// bytes of one (chunk, head) slot of that workspace (kda_slot_bytes)
int64_t kda_slot_bytes_host(const gdn_problem *pr);

// gdn_forward_split (gdn_split.hip): its workspace and its launches
int64_t split_workspace_bytes(const gdn_problem *pr, int64_t t_split);
gdn_status enqueue_forward_split(const gdn_problem *pr, int64_t t_split, const void *q, const void *k,
                                 const void *v, const float *beta, const float *g, const float *h0,
                                 void *o, float *hT, void *ws, hipStream_t s);
gdn_status enqueue_kda_gram(const gdn_problem *pr, const void *q, const void *k,
                            const float *beta, const float *g, void *ws, const int32_t *cu,
                            int64_t n_seqs, hipStream_t s);

// gdn_backward (gdn_backward.hip): its workspace and its two launches
int64_t backward_workspace_bytes(const gdn_problem *pr);
gdn_status enqueue_backward(const gdn_problem *pr, const void *q, const void *k, const void *v,
                            const float *beta, const float *g, const void *dout, const float *dhT,
                            const void *hck, const void *vnew, float *dq, float *dk, float *dv,
                            float *dbeta, float *dg, float *dh0, void *ws, hipStream_t s);

struct BwdParams;
// the per-key gate's backward (gdn_backward_kda.hip): slot size and launches
int64_t backward_kda_slot_bytes(int64_t chunk, int64_t K);
gdn_status enqueue_backward_kda(const gdn_problem *pr, BwdParams &bp, hipStream_t s);

struct FwdParams;
// Dispatch a forward problem whose FwdParams carry hck and vnew.
gdn_status enqueue_forward_states(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s);
gdn_status enqueue_forward_states_c64(const gdn_problem *pr, FwdParams &fp, int grid,
                                      hipStream_t s);
// Dispatch a forward problem whose FwdParams carry packed-sequence offsets.
gdn_status enqueue_forward_varlen(const gdn_problem *pr, FwdParams &fp, int grid, hipStream_t s);
gdn_status enqueue_forward_varlen_c64(const gdn_problem *pr, FwdParams &fp, int grid,
                                      hipStream_t s);
gdn_status enqueue_forward_pipe_varlen_c32(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s);
gdn_status enqueue_forward_pipe_varlen_c64(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s);
// Launch the pipelined forward kernel (scalar gate, bf16 io) for chunk C,
// key dim K and fp32 (else bf16) output.
gdn_status enqueue_forward_pipe(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                hipStream_t s);
gdn_status enqueue_forward_pipe_c32(int K, bool o_f32, FwdParams &fp, int grid, hipStream_t s);
// the sequence-split (SP) instances, chunk 64 (gdn_forward_pipe_split.hip)
gdn_status enqueue_forward_pipe_split(int K, bool o_f32, FwdParams &fp, int grid, hipStream_t s);
// The pipelined kernel for the per-key gate (plain, ST or VL by fp.hck / fp.cu).
gdn_status enqueue_forward_pipe_kda(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                    hipStream_t s);
// The scalar-gate pipelined kernel as the backward's re-scan (fp.dq set).
gdn_status enqueue_forward_pipe_dq(int C, int K, bool o_f32, FwdParams &fp, int grid,
                                   hipStream_t s);
// Chunk 32, saving the chunk-start states and the per-token deltas.
gdn_status enqueue_forward_pipe_c32_states(int K, bool o_f32, FwdParams &fp, int grid,
                                           hipStream_t s);

}  // namespace gdn
