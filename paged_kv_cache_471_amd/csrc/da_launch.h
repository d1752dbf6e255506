// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Largest batch the wave planner accepts: each lane scans ceil(B / 64) requests.
constexpr int kMaxBatch = 8192;
// Largest number of workers (waves for GQA, workgroups for MLA) per launch.
constexpr int kMaxWorkers = 16384;

// Debug run of the wave planner: worker g writes what its share would be.
struct PlanArgs {
    const int32_t* seq_lens;
    int batch, page_size, units, workers;
    int32_t* active;        // [1]
    int32_t* cuts;          // [workers + 1]; W for g >= active
    int4* cursors;          // [workers + 1]; (batch, 0, 0, 0) at W
    int32_t* first_worker;  // [batch * units]
    int32_t* piece_count;   // [batch * units]
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
    // The kernels work in tiles of 16 tokens; a page holds 2^tile_shift of
    // them (page_size = 16 << tile_shift), so tile t of a history lies in
    // page-table entry t >> tile_shift, from token 16 (t mod 2^tile_shift)
    // of that page.
    int tile_shift;
    // Query rows per request (q, out [batch][q_rows][q_heads][head_dim]): row i
    // sees history positions t <= len - q_rows + i.  The kernel's head group
    // GS holds the q_rows x (q_heads / kv_heads) (row, head) pairs of one KV
    // head, row-major, padded to a power of two; group_log2 = log2 of the
    // query heads per KV head, read by the vector kernel only (powers of two);
    // the matrix-core kernel takes any count q_heads / kv_heads.
    int q_rows, group_log2;
    int2* plan_info;        // [1]: (W, active workers), written by worker 0
    int2* stream_info;      // [batch * kv_heads]: (first unit, pieces) of each non-empty stream
    void* out;
    float* lse;             // [batch][q_rows][q_heads] or null
    float* o_part;          // [2 * workers][GS][head_dim]
    float* lse_part;        // [2 * workers][GS]   (log2 domain)
};

// Absorbed MLA: one head-shared latent of kMlaLatent bf16 values per token;
// values are its first kMlaV entries.  Tokens are processed in chunks of
// kMlaChunk (pages are a multiple of it).
constexpr int kMlaLatent = 576;
constexpr int kMlaV = 512;
constexpr int kMlaChunk = 32;
constexpr int kMlaMaxHeads = 128;
// Each MLA worker may leave two partial slots of [heads][512] fp32 (256 KiB at
// 128 heads); this bounds the workspace at 1 GiB.
constexpr int kMlaMaxWorkers = 2048;

struct MlaArgs {
    const void* q;          // bf16 [batch][heads][576]
    const void* kv;         // bf16 [num_pages][page_size][576]
    const int32_t* page_table;
    const int32_t* seq_lens;
    float scale_log2;       // softmax scale * log2(e)
    int batch, heads, page_size, max_pages, workers;
    int2* plan_info;        // [1]: (W, active workers), written by worker 0
    int2* stream_info;      // [batch]: (first unit, pieces) of each non-empty request
    void* out;              // bf16 [batch][heads][512]
    float* lse;             // fp32 [batch][heads] or null
    float* o_part;          // [2 * workers][heads][512]
    float* lse_part;        // [2 * workers][heads]   (log2 domain)
    // The 128-head kernel (mla_wave.hip) uses instead one slot per piece,
    // index b + worker: o_part [batch + workers][128][512] raw accumulator
    // tiles, lse_part [batch + workers][128][2] (running max in log2, sum),
    // and o_tmp [workers][128][512] as scratch.
    float* o_tmp;
    // Several query rows per request (128-head kernel): request e of the
    // expanded batch is row e / row_batch of request e % row_batch, whose q,
    // out and lse rows sit at (e % row_batch) * rows + e / row_batch; rows = 1
    // means request e itself.
    int row_batch, rows;
};

// Log-sum-exp merge of the partial slots of split streams.  One workgroup per
// (stream, group of heads_per_block heads, 1/col_chunks of their columns);
// streams that are empty or were not split return at once.
struct MergeArgs {
    const int32_t* seq_lens;
    const int2* plan_info;
    const int2* stream_info;
    const float* o_part;    // [2 * workers][group][dim]
    const float* lse_part;  // [2 * workers][group]  (log2 domain)
    void* out;              // [batch][rows][units * heads_per_unit][dim], bf16 or fp32
    float* lse;             // [batch][rows][units * heads_per_unit] or null
    int units;              // streams per request (KV heads, or 1 for MLA)
    int group;              // (row, head) slots per stream in the partials
    int dim;                // values per head
    int heads_per_block;    // divides group
    int col_chunks;         // power of two dividing heads_per_block * dim / 4 (1: whole heads)
    int out_is_bf16;
    int rows;               // query rows per request; slot h is row h / heads_per_unit
    int heads_per_unit;     // query heads per stream (any count)
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

hipError_t launch_plan_debug(const PlanArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int streams, hipStream_t s);

hipError_t launch_mla(const MlaArgs& a, hipStream_t s, const KernelEvents& ev);
// The 128-head kernel (mla_wave.hip) and its merge, which normalises every
// request from its per-piece slots (whole requests included).
hipError_t launch_mla_wave(const MlaArgs& a, hipStream_t s, const KernelEvents& ev);
hipError_t launch_mla_wave_merge(const MlaArgs& a, hipStream_t s);
int mla_wave_blocks_per_cu();
constexpr int kMlaWaveHeads = 128;
// Workgroups of the MLA kernel that fit on one CU at once.
int mla_blocks_per_cu();
// Head counts with an MLA kernel (16, 32, 64, 128).
bool mla_heads_supported(int heads);
// Workgroups that share one MLA worker's share (one per 64-head group).
int mla_blocks_per_worker(int heads);

// Returns hipErrorInvalidValue if no kernel exists for this combination.
// members: the kernel's head group (GqaArgs); a.group_log2 selects the
// single-row (members == 2^group_log2) or multi-row variant.
hipError_t launch_gqa(int q_dtype, int kv_dtype, int head_dim, int members, const GqaArgs& a, hipStream_t s,
                      const KernelEvents& ev);
// Workers of the GQA kernel that fit on one CU at once (0 if no kernel); a
// worker is one wavefront, or two for multi-row groups of 8 members.
int gqa_workers_per_cu(int q_dtype, int kv_dtype, int head_dim, int members, int group_log2);
constexpr int kGqaBlock = 256;   // 4 wavefronts per workgroup, each an independent worker

}  // namespace da
