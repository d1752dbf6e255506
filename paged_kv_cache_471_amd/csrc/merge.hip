// Log-sum-exp merge of split pieces, and the debug gather copy.
//
// A history split into disjoint token ranges is recombined exactly: with
// per-piece normalised outputs o_i and log-sum-exps lse_i,
//     lse = log sum_i exp(lse_i),   o = sum_i exp(lse_i - lse) o_i.
// This is the same attention result up to floating-point reduction order
// ("SPLASH: Switching Parallel Layouts of Attention with Seamless Handoff for
// LLM Serving", §3, Computation, and §6 on context-parallel attention that
// distributes within-context work).  Pieces are visited in token order, in a
// fixed reduction tree, so the result is deterministic.
#include "da_common.h"
#include "da_launch.h"

namespace da {
namespace {

constexpr int kMergeThreads = 256;

__device__ float block_max(float v, float* red) {
    const int t = threadIdx.x;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) v = fmaxf(v, __shfl_xor(v, x, 64));
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

__device__ float block_sum(float v, float* red) {
    const int t = threadIdx.x;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x, 64);
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) r += red[w];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
    __shared__ float red[kMergeThreads / 64];
    extern __shared__ float part[];     // [kMergeThreads]  partial dim sums
    const int t = threadIdx.x;
    const int G = a.workers;
    const int U = a.units;
    const int total = *a.split_count * a.group;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int s = a.split_list[item / a.group];
        const int hh = item % a.group;
        const int b = s / U, j = s % U;
        const int pages = a.cp[b + 1] - a.cp[b];
        const int start = U * a.cp[b] + j * pages;
        const int end = start + pages;
        const int gf = a.first_worker[s];

        // slot of worker g's piece of this stream, or -1 if the worker is empty
        auto slot_of = [&](int g) -> int {
            if (g == gf) return (a.cuts[g] == start) ? g : G + g;
            return (a.cuts[g + 1] > a.cuts[g]) ? g : -1;
        };
        auto in_stream = [&](int g) -> bool { return g < G && (g == gf || a.cuts[g] < end); };

        float mx = -__builtin_inff();
        for (int g = gf + t; in_stream(g); g += kMergeThreads) {
            const int sl = slot_of(g);
            if (sl >= 0) mx = fmaxf(mx, a.lse_part[static_cast<int64_t>(sl) * a.group + hh]);
        }
        const float M = block_max(mx, red);
        float z = 0.0f;
        for (int g = gf + t; in_stream(g); g += kMergeThreads) {
            const int sl = slot_of(g);
            if (sl >= 0) z += __builtin_amdgcn_exp2f(a.lse_part[static_cast<int64_t>(sl) * a.group + hh] - M);
        }
        const float Z = block_sum(z, red);
        const float invZ = 1.0f / Z;

        // weighted sum of the pieces' outputs; (kMergeThreads / dim) piece lanes per dim
        const int lanes = a.dim >= kMergeThreads ? 1 : kMergeThreads / a.dim;
        const int grp = t / (kMergeThreads / lanes);
        const int d0 = t % (kMergeThreads / lanes);
        const int64_t out_row = (static_cast<int64_t>(b) * a.q_heads + j * a.group + hh) * a.dim;
        for (int dbase = 0; dbase < a.dim; dbase += kMergeThreads / lanes) {
            const int d = dbase + d0;
            float accv = 0.0f;
            for (int g = gf + grp; in_stream(g); g += lanes) {
                const int sl = slot_of(g);
                if (sl < 0) continue;
                const float w = __builtin_amdgcn_exp2f(a.lse_part[static_cast<int64_t>(sl) * a.group + hh] - M);
                accv = __builtin_fmaf(w, a.o_part[(static_cast<int64_t>(sl) * a.group + hh) * a.dim + d], accv);
            }
            part[t] = accv;
            __syncthreads();
            if (grp == 0) {
                float r = part[d0];
                for (int q = 1; q < lanes; ++q) r += part[q * (kMergeThreads / lanes) + d0];
                r *= invZ;
                if (a.out_is_bf16) static_cast<uint16_t*>(a.out)[out_row + d] = f32_to_bf16_bits(r);
                else static_cast<float*>(a.out)[out_row + d] = r;
            }
            __syncthreads();
        }
        if (t == 0 && a.lse != nullptr)
            a.lse[static_cast<int64_t>(b) * a.q_heads + j * a.group + hh] = (M + __builtin_log2f(Z)) * kLn2;
    }
}

// One block per (page, request): copies the page's live tokens to the dense
// array through the kernels' address functions.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    const int p = blockIdx.x, b = blockIdx.y;
    const int L = a.seq_lens[b];
    const int P = a.page_size;
    if (p * P >= L) return;
    const int pg = a.page_table[static_cast<int64_t>(b) * a.max_pages + p];
    const int live = min(P, L - p * P);
    const int row_words = a.head_dim * a.elem_bytes / 4;
    const int64_t maxT = static_cast<int64_t>(a.max_pages) * P;
    const uint32_t* src = static_cast<const uint32_t*>(a.kv);
    uint32_t* dst = static_cast<uint32_t*>(a.dense);
    if (a.mla) {
        for (int i = threadIdx.x; i < live * row_words; i += blockDim.x) {
            const int slot = i / row_words, w = i % row_words;
            const int64_t so = mla_kv_offset(pg, slot, P, a.head_dim) * a.elem_bytes / 4 + w;
            const int64_t dofs = ((static_cast<int64_t>(b) * maxT + p * P + slot) * a.head_dim) * a.elem_bytes / 4 + w;
            dst[dofs] = src[so];
        }
    } else {
        const int per_slot = 2 * a.kv_heads * row_words;
        for (int i = threadIdx.x; i < live * per_slot; i += blockDim.x) {
            const int slot = i / per_slot;
            const int rem = i % per_slot;
            const int sel = rem / (a.kv_heads * row_words);
            const int j = (rem / row_words) % a.kv_heads;
            const int w = rem % row_words;
            const int64_t so = gqa_kv_offset(pg, sel, j, slot, a.kv_heads, P, a.head_dim) * a.elem_bytes / 4 + w;
            const int64_t dofs =
                ((((static_cast<int64_t>(b) * maxT + p * P + slot) * 2 + sel) * a.kv_heads + j) * a.head_dim) *
                    a.elem_bytes / 4 + w;
            dst[dofs] = src[so];
        }
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int grid, hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kMergeThreads), kMergeThreads * sizeof(float), s, a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(gather_kernel, dim3(a.max_pages, a.batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
