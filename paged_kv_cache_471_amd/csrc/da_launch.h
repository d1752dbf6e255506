// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Bounds of the single-workgroup planner: its LDS holds cp [batch + 1], the
// cuts [workers + 1] and a 1024-entry scan buffer within 64 KiB.
constexpr int kPlanMaxBatch = 8192;
constexpr int kPlanMaxWorkers = 6144;

struct PlanArgs {
    const int32_t* seq_lens;
    int batch, page_size, units, workers, snap;
    int32_t* cp;            // [batch + 1]
    int32_t* cuts;          // [workers + 1]
    int4* cursors;          // [workers + 1]
    int32_t* first_worker;  // [batch * units]
    int32_t* split_list;    // [workers]
    int32_t* split_count;   // [1]
    // outputs of empty requests (L == 0) are written here: out = 0, lse = -inf
    void* out;              // may be null (planner-only runs)
    int out_elem_bytes;
    float* lse;             // may be null
    int heads;              // query heads per request
    int out_dim;            // values per head
};

struct GqaArgs {
    const void* q;
    const void* kv;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const float* k_scale;
    const float* v_scale;
    float scale_log2;       // softmax scale * log2(e)
    int batch, q_heads, kv_heads, page_size, max_pages, workers;
    const int32_t* cuts;
    const int4* cursors;
    void* out;
    float* lse;
    float* o_part;          // [2 * workers][group][head_dim]
    float* lse_part;        // [2 * workers][group]   (log2 domain)
};

struct MergeArgs {
    const int32_t* seq_lens;
    int batch, page_size, units, workers;
    int group;              // heads per stream
    int dim;                // values per head
    int q_heads;            // heads per request in out/lse
    const int32_t* cp;
    const int32_t* cuts;
    const int32_t* first_worker;
    const int32_t* split_list;
    const int32_t* split_count;
    const float* o_part;
    const float* lse_part;
    void* out;
    int out_is_bf16;
    float* lse;
};

struct GatherArgs {
    const void* kv;
    const int32_t* page_table;
    const int32_t* seq_lens;
    void* dense;
    int batch, kv_heads, head_dim, page_size, max_pages, elem_bytes, mla;
};

// Optional start/stop events for the main attention kernel: when set, the
// kernel is launched with hipExtLaunchKernelGGL, whose dispatch records them.
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int grid, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// Returns hipErrorInvalidValue if no kernel exists for this combination.
hipError_t launch_gqa(int q_dtype, int kv_dtype, int head_dim, int group, const GqaArgs& a, hipStream_t s,
                      const KernelEvents& ev);
// Wavefronts of the GQA kernel that fit on one CU at once (0 if no kernel).
int gqa_waves_per_cu(int q_dtype, int kv_dtype, int head_dim, int group);
constexpr int kGqaBlock = 256;   // 4 wavefronts per workgroup, each an independent worker

}  // namespace da
