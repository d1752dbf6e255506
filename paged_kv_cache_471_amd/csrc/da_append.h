// Host/device interface of the paged KV append kernels (append.hip).
#pragma once

#include "da_launch.h"

namespace da {

// GQA: k_new / v_new [batch][kv_heads][head_dim] of in_dtype into
// kv [num_pages][2][kv_heads][page_size][head_dim] of kv_dtype.
// MLA: k_new is the bf16 latent [batch][576], kv is [num_pages][page_size][576].
struct AppendArgs {
    const void* k_new;
    const void* v_new;
    void* kv;
    const int32_t* page_table;
    const int32_t* positions;   // [batch]; negative: no append
    const float* k_scale;       // fp8: [kv_heads]
    const float* v_scale;
    int batch, kv_heads, head_dim, page_size, max_pages;
    int in_dtype, kv_dtype;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s, const KernelEvents& ev);
hipError_t launch_kv_append_mla(const AppendArgs& a, hipStream_t s, const KernelEvents& ev);

}  // namespace da
