// Host interface of the matrix-core GQA kernel for large head groups (gqa_mfma.hip).
#pragma once

#include "da_launch.h"

namespace da {

// q bf16, K/V bf16 or fp8, head_dim 64 or 128; up to 16 (row, head) members
// per KV head (a.q_rows rows of q_heads / kv_heads heads, any count).  The
// partial slots hold the members padded to a power of two, as the merge
// kernel reads them.
hipError_t launch_gqa_mfma(int kv_dtype, int head_dim, const GqaArgs& a, hipStream_t s, const KernelEvents& ev);
// Workers (one wavefront each) of that kernel that run on one CU by default (0 if none).
int gqa_mfma_workers_per_cu(int kv_dtype, int head_dim);

}  // namespace da
