// Debug copy of the paged cache into dense (request, token) order through the
// kernels' address functions.  A bitwise copy with no arithmetic; it exists so
// that the address generation of the paged layout (page table entry of token
// t = page_table[b][t / P], slot t % P; OpWeave §8, paged KV-cache management)
// can be compared bit for bit with plain indexing.
#include "da_common.h"
#include "da_launch.h"

namespace da {
namespace {

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
    } else if (a.elem_bytes == 1) {
        // fp8: K rows copied as words; V blocks are tiled (fp8_v_byte), so
        // their codes are copied one by one into token order
        const int D = a.head_dim;
        const uint8_t* src8 = static_cast<const uint8_t*>(a.kv);
        uint8_t* dst8 = static_cast<uint8_t*>(a.dense);
        const int per_slot = 2 * a.kv_heads * D;
        for (int i = threadIdx.x; i < live * per_slot; i += blockDim.x) {
            const int slot = i / per_slot;
            const int rem = i % per_slot;
            const int sel = rem / (a.kv_heads * D);
            const int j = (rem / D) % a.kv_heads;
            const int d = rem % D;
            const int64_t block = gqa_kv_offset(pg, sel, j, 0, a.kv_heads, P, D);
            const int64_t so = block + (sel == 0 ? static_cast<int64_t>(slot) * D + d : fp8_v_byte(slot, d, D));
            const int64_t dofs = (((static_cast<int64_t>(b) * maxT + p * P + slot) * 2 + sel) * a.kv_heads + j) * D + d;
            dst8[dofs] = src8[so];
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

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(gather_kernel, dim3(a.max_pages, a.batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
