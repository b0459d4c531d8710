// Host-side declarations shared by the translation units of libgdn.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/libgdn.h"

namespace gdn {

// Launch a kernel with 256 threads per block and one by-value parameter struct.
gdn_status launch_kernel(const void *fn, int grid, void *params, hipStream_t s);

// Enqueue the fused forward kernel (validated problem, non-empty work).
gdn_status enqueue_forward(const gdn_problem *pr, const void *q, const void *k,
                           const void *v, const float *beta, const float *g,
                           const float *h0, void *o, float *hT, hipStream_t s);

}  // namespace gdn
