// Device helpers shared by the absorbed-MLA kernels (mla.hip, mla_wave.hip):
// the latent-chunk cursor, the global-to-LDS chunk loads and their waits, the
// row-swap reductions and the matrix-core wrappers.
//
// A latent row is 576 bf16 values = 1152 bytes ("Analytical Provisioning for
// Attention-FFN Disaggregated LLM Serving under Stochastic Workloads", App. B.1
// and B.2.1), held once per token with no head axis (SPLASH, §1 and §2).
#pragma once

#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kMlaRowBytes = kMlaLatent * 2;                 // 1152 bytes per token in HBM
constexpr int kMlaXB = kMlaRowBytes / 16;                    // 72 16-byte blocks per token
constexpr int kMlaSlotBytes = kMlaXB * kMlaChunk * 16;       // 36864: one 32-token chunk
constexpr int kMlaSlotLoads = kMlaSlotBytes / 1024;          // 36 wave-wide 16-byte loads

// Compute/load cursor over the chunks of a worker's share.  Wave-uniform.
struct MlaCursor {
    int b, p, ci;      // request, page, chunk within the page
    int len, pages;    // request length and page count
    int nch;           // chunks of page p holding live tokens
    int k;             // unit (page) index within the share
};

__device__ __forceinline__ int mla_chunks_of_page(int len, int p, int P) {
    const int live = min(P, len - p * P);
    return (live + kMlaChunk - 1) / kMlaChunk;
}

__device__ __forceinline__ void mla_cursor_init(MlaCursor& c, const WaveShare& sh, const int32_t* seq_lens, int P) {
    c.b = sh.b;
    c.p = sh.p;
    c.ci = 0;
    c.len = sload_i32(seq_lens + c.b);
    c.pages = (c.len + P - 1) / P;
    c.nch = mla_chunks_of_page(c.len, c.p, P);
    c.k = 0;
}

// Advance one chunk.  Moving past the share's last unit leaves k == n and
// reads nothing.
__device__ __forceinline__ void mla_cursor_next(MlaCursor& c, const int32_t* seq_lens, int P, int n) {
    if (++c.ci < c.nch) return;
    c.ci = 0;
    if (++c.k >= n) return;
    if (++c.p >= c.pages) {
        c.p = 0;
        do {
            ++c.b;
            c.len = sload_i32(seq_lens + c.b);
            c.pages = (c.len + P - 1) / P;
        } while (c.pages == 0);
    }
    c.nch = mla_chunks_of_page(c.len, c.p, P);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Written as inline assembly so that the compiler, which cannot tell which
// LDS bytes such a load writes, does not drain every outstanding load before
// each LDS access; completion is tracked with mla_wait_vmcnt below instead.
// m0 is listed as clobbered (the compiler warns that it is a reserved
// register): on gfx950 LDS instructions do not read m0, and the built kernels
// contain no m0 access other than these blocks' own writes.
__device__ __forceinline__ void mla_lds_dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_addr)
                 : "memory", "m0");
}

// The same load with the non-temporal hint: for loads that each bring whole
// 128-byte lines that nothing reads again.
__device__ __forceinline__ void mla_lds_dma16_nt(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds_addr)
                 : "memory", "m0");
}

// Wait until at most N vector memory operations of this wave are outstanding.
// Loads complete in issue order, so this makes every load issued before the
// last N complete.
template <int N>
__device__ __forceinline__ void mla_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only (does not wait for global loads).
__device__ __forceinline__ void mla_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Start the scalar read of *next_pid, wait until at most N vector memory
// operations of this wave are outstanding (the chunk about to be computed has
// landed), then meet the workgroup at a barrier.  The page-id read overlaps
// the wait for the chunk instead of stalling the wave on its own.
template <int N>
__device__ __forceinline__ int mla_wait_chunk_barrier(const int32_t* next_pid) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt vmcnt(%2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                 : "=s"(v)
                 : "s"(next_pid), "n"(N)
                 : "memory");
    return v;
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) with the gfx950
// row swaps: after swapping a value with itself, the two results hold the
// values of both lanes of each pair, in one order or the other, so max and
// sum of the two are the pairwise max and sum (no LDS round trip).
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values -> packed bf16 pair (round to nearest even), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_t));
}

// Transposing 8-byte LDS read (gfx950, ds_read_b64_tr_b16): in each group of
// 16 lanes, lane 4a+e receives element e of the 8-byte rows addressed by lanes
// a, 4+a, 8+a, 12+a (in that order).
__device__ __forceinline__ short4v ds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

__device__ __forceinline__ floatx16_t mfma32(bf16x8_t a, bf16x8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace da
