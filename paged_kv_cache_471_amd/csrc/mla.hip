// Paged absorbed-MLA decode attention, split-KV worker kernel (gfx950).
//
// What it computes: MLA keeps one latent per token with no head axis, shared by
// every query head (SPLASH: Switching Parallel Layouts of Attention with
// Seamless Handoff for LLM Serving, §1 and §2); the latent is d_c + d_rope =
// 512 + 64 = 576 values, 1152 bytes per token in bf16 ("Analytical
// Provisioning for Attention-FFN Disaggregated LLM Serving under Stochastic
// Workloads", App. B.1 and B.2.1).  With the up-projections absorbed into the
// query, head h of request b computes
//     s_t = scale * <q[b][h], c_t>,   out[b][h] = sum_t softmax(s)_t c_t[0:512]
// over the request's whole paged history (one decode row per request; OpWeave,
// App. A.2).  All heads read the same latent, so per token the work is a dense
// [heads x 576] x [576] product and a [heads] x [512] update: the contraction
// runs on MFMA.
//
// Design (one 512-thread workgroup = one worker of the device partition; one
// workgroup per CU, two waves per SIMD):
//  * The worker walks its contiguous share of (request, page) units in chunks
//    of 32 tokens.  A chunk (32 x 1152 B, contiguous in the page) is copied
//    from HBM straight into one slot of a 4-slot LDS ring with 16-byte
//    global-to-LDS loads, three chunks ahead of the one being computed, and
//    serves all 128 heads.
//  * Slot layout: 16-byte block x (0..71) of token t sits at position
//    32 x + (t ^ 4 (x & 3)).  Each 1 KiB load then copies a fixed per-lane
//    pattern, an MFMA operand read of 16 or 32 tokens covers whole bank rows,
//    and the column gathers of the value product fall on different banks.
//  * Scores: wave w owns heads [16w, 16w+16).  Its query slice (18 K-blocks
//    of 32) stays in registers as the B operand of v_mfma_f32_16x16x32_bf16;
//    latent rows are the A operand, so S^T [16 tokens x 16 heads] comes out
//    with each lane holding 4 tokens of one head; the two 16-token blocks of
//    a chunk are two independent MFMA chains.  Operands are read two
//    K-blocks ahead of their MFMAs.
//  * Softmax: per head a running maximum (base 2, log2(e) folded into the
//    scale) that is only raised when a chunk's maximum exceeds it by more
//    than 8, so weights stay <= 2^8 and the value rows rarely need rescaling.
//    The running sum adds the fp32 weights; only the MFMA operand is rounded
//    to bf16.  All accumulation is fp32.
//  * Values: wave w owns value dims [64w, 64w+64) of every head: O [128 x 64]
//    fp32 accumulators (v_mfma_f32_32x32x16_bf16), P [heads x 32 tokens]
//    from LDS as A, latent columns gathered from the ring as B.
//  * A piece that is a whole request writes out/lse; otherwise normalised
//    partials go to a slot that the merge kernel (merge.hip) combines.
#include <hip/hip_ext.h>

#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWaves = 8;
constexpr int kBlock = kWaves * 64;
constexpr int kRowBytes = kMlaLatent * 2;             // 1152 bytes per token in HBM
constexpr int kXB = kRowBytes / 16;                   // 72 16-byte blocks per token
constexpr int kSlotBytes = kXB * kMlaChunk * 16;      // 36864
constexpr int kSlotLoads = kSlotBytes / 1024;         // 36 wave-wide 16-byte loads
constexpr int kMaxLoadsPerWave = (kSlotLoads + kWaves - 1) / kWaves;   // 5
constexpr int kSlots = 4;
constexpr int kHG = kMlaMaxHeads;                     // heads per workgroup
constexpr int kPRow = 80;                             // bytes per head row of P (64 + 16 pad)
constexpr int kSKB = kMlaLatent / 32;                 // 18 K-blocks of the score product
constexpr int kHW = 16;                               // score heads per wave
constexpr int kDW = kMlaV / kWaves;                   // 64 value dims per wave
constexpr float kRaise = 8.0f;                        // running max moves only past this margin
constexpr int kPD = 2;                                // score operand reads in flight (K-blocks)

static_assert(kHG == kWaves * kHW, "each wave owns 16 score heads");

struct __align__(16) Smem {
    char ring[kSlots][kSlotBytes];
    char p[kHG * kPRow];
    float alpha[kHG];
    float fin_l[kHG];
    int flags[kWaves];
};

// Compute/load cursor over the chunks of a worker's share.  Wave-uniform.
struct Cursor {
    int b, p, ci;      // request, page, chunk within the page
    int len, pages;    // request length and page count
    int nch;           // chunks of page p holding live tokens
    int k;             // unit (page) index within the share
};

__device__ __forceinline__ int chunks_of_page(int len, int p, int P) {
    const int live = min(P, len - p * P);
    return (live + kMlaChunk - 1) / kMlaChunk;
}

__device__ __forceinline__ void cursor_init(Cursor& c, const WaveShare& sh, const int32_t* seq_lens, int P) {
    c.b = sh.b;
    c.p = sh.p;
    c.ci = 0;
    c.len = sload_i32(seq_lens + c.b);
    c.pages = (c.len + P - 1) / P;
    c.nch = chunks_of_page(c.len, c.p, P);
    c.k = 0;
}

// Advance one chunk.  Moving past the share's last unit leaves k == n and
// reads nothing.
__device__ __forceinline__ void cursor_next(Cursor& c, const int32_t* seq_lens, int P, int n) {
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
    c.nch = chunks_of_page(c.len, c.p, P);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Written as inline assembly so that the compiler, which cannot tell which
// LDS bytes such a load writes, does not drain every outstanding load before
// each LDS access; completion is tracked with wait_vmcnt below instead.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_addr)
                 : "memory", "m0");
}

// Wait until at most N vector memory operations of this wave are outstanding.
// Loads complete in issue order, so this makes every load issued before the
// last N complete.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only (does not wait for global loads).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Start the scalar read of *next_pid, wait until at most N vector memory
// operations of this wave are outstanding (the chunk about to be computed has
// landed), then meet the workgroup at a barrier.  The page-id read overlaps
// the wait for the chunk instead of stalling the wave on its own.
template <int N>
__device__ __forceinline__ int wait_chunk_barrier(const int32_t* next_pid) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt vmcnt(%2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                 : "=s"(v)
                 : "s"(next_pid), "n"(N)
                 : "memory");
    return v;
}

typedef short short4v __attribute__((ext_vector_type(4)));

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

// Transposing 8-byte LDS read (gfx950): see the value-operand note in the kernel.
__device__ __forceinline__ short4v ds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

__device__ __forceinline__ floatx16_t mfma32(bf16x8_t a, bf16x8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int H>
__global__ __launch_bounds__(kBlock, 1) void mla_attn_kernel(MlaArgs a) {
    constexpr int HG = H < kHG ? H : kHG;            // heads of this workgroup
    constexpr int NS = H / HG;                        // workgroups per worker
    constexpr int nhb = (HG + 31) / 32;               // 32-head blocks of the value product
    static_assert(H % 16 == 0 && H <= kMlaMaxHeads && H % HG == 0, "heads");
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int l16 = lane & 15;
    const int q4l = (lane >> 4) & 3;                  // lane group of 16
    const int w = uniform(tid >> 6);
    const int g = blockIdx.x % a.workers;             // worker
    const int hs = blockIdx.x / a.workers;            // head half
    const int h0 = hs * HG;                           // first head of this workgroup
    const int P = a.page_size;
    const char* kvb = static_cast<const char*>(a.kv);

    const WaveShare sh = plan_share(a.seq_lens, a.batch, P, 1, a.workers, g);
    if (sh.has_empty && w == 0 && hs == 0) {
        for_each_empty_request(a.seq_lens, a.batch, a.workers, g, [&](int b) {
            uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(b) * H * kMlaV;
            for (int i = lane; i < H * kMlaV; i += 64) o[i] = 0;
            if (a.lse != nullptr)
                for (int h = lane; h < H; h += 64) a.lse[static_cast<int64_t>(b) * H + h] = -__builtin_inff();
        });
    }
    const int A = sh.active;
    if (g == 0 && hs == 0 && tid == 0) *a.plan_info = make_int2(static_cast<int>(sh.W), A);
    if (g >= A) return;
    const int n = static_cast<int>(sh.c1 - sh.c0);

    // ---- LDS set-up: P rows of absent heads stay zero, their alpha one.
    for (int i = tid; i < kHG * kPRow / 4; i += kBlock) reinterpret_cast<int*>(sm.p)[i] = 0;
    for (int i = tid; i < kHG; i += kBlock) sm.alpha[i] = 1.0f;
    if (tid < kWaves) sm.flags[tid] = 0;

    // ---- chunk loader: wave w issues loads q = w + 8 i (5 loads for w < 4,
    //      4 otherwise); load q fills positions [64 q, 64 q + 64): x = 2 q +
    //      half, t' = l32, source token t = t' ^ 4 ((2 q + half) & 3), and
    //      (2 q) & 3 = 2 (w & 1) for every i.
    const int nq = (kSlotLoads - w + kWaves - 1) / kWaves;
    Cursor lc;
    cursor_init(lc, sh, a.seq_lens, P);
    int issued = 0;                                             // chunks issued so far
    auto issue_chunk = [&](int pid) {
        int ln = lane;
        asm volatile("" : "+v"(ln));      // recomputed per chunk rather than held in a register
        const int dma_off = ((ln & 31) ^ (((2 * (w & 1) + (ln >> 5)) & 3) << 2)) * kRowBytes + (ln >> 5) * 16;
        const char* src = kvb + (static_cast<int64_t>(pid) * P + lc.ci * kMlaChunk) * kRowBytes + dma_off;
        const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)sm.ring[issued % kSlots]));
#pragma unroll
        for (int i = 0; i < kMaxLoadsPerWave; ++i) {
            const int q = w + kWaves * i;
            if (i < nq) lds_dma16(src + 32 * q, lds_base + q * 1024);
        }
        ++issued;
        cursor_next(lc, a.seq_lens, P, n);
    };

    // ---- per-lane LDS offsets
    // score operand: token tb*16 + l16, block x = 4 kb + q4l (x & 3 = q4l)
    const int s_base = q4l * 512 + ((l16 ^ (q4l << 2)) << 4);
    // value operand by transposing reads (ds_read_b64_tr_b16): in each group of
    // 16 lanes, lane 4a+e receives element e of the 8-byte rows addressed by
    // lanes a, 4+a, 8+a, 12+a.  Lane s of group G therefore addresses dims
    // 16 (G & 1) + 4 (s & 3) .. +3 of token 8 (G >> 1) + (s >> 2) (+4 for the
    // second read), so that lane l ends up with tokens 8 (l / 32) + j of dim
    // l % 32, the B operand of the 32x32x16 product.
    const int tr_s = lane & 15, tr_g = lane >> 4;
    const int tr_x = 2 * (tr_g & 1) + ((tr_s >> 1) & 1);       // block within the 32 dims (x & 3)
    const int tr_t = (8 * (tr_g >> 1) + (tr_s >> 2)) ^ (4 * tr_x);   // swizzled token position
    const int tr_base = (kDW / 8) * w * 512 + tr_x * 512 + tr_t * 16 + 8 * (tr_s & 1);
    const int tr_base2 = tr_base + ((tr_x & 1) ? -64 : 64);    // tokens + 4 (position bit 2 flips)
    const int pr_base = l32 * kPRow + half * 16;                // P operand of the value product
    const int hw = w * kHW;                                     // this wave's score heads (local)
    const int pw_base = (hw + l16) * kPRow + q4l * 8;           // P row written by this lane
    const bool s_active = hw < HG;
    const int dw = w * kDW;                                     // this wave's value dims

    bf16x8_t qreg[kSKB];
    float m_run = kMaxInit, l_run = 0.0f;
    floatx16_t acc[nhb][2];

    auto load_q = [&](int b) {
        if (!s_active) return;
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(
            static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * H + h0 + hw + l16) * kMlaLatent + 8 * q4l);
#pragma unroll
        for (int kb = 0; kb < kSKB; ++kb) qreg[kb] = src[kb * 4];
        // Let the compiler see these loads complete here (this also drains the
        // chunk ring, once per piece): otherwise it would keep them pending
        // around the loop and wait on the ring's loads inside the score product.
        __builtin_amdgcn_s_waitcnt(0xF70);
    };
    auto reset = [&]() {
        m_run = kMaxInit;
        l_run = 0.0f;
#pragma unroll
        for (int hb = 0; hb < nhb; ++hb)
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[hb][db][r] = 0.0f;
    };

    Cursor cc;
    cursor_init(cc, sh, a.seq_lens, P);
    int piece_first_unit = 0;             // k of the piece's first unit
    int piece_p0 = cc.p;                  // first page of the piece within its request
    bool first_piece = true;
    int i = 0;                            // chunk index within the share

    // prologue: three chunks in flight
    auto next_pid_addr = [&]() { return a.page_table + static_cast<int64_t>(lc.b) * a.max_pages + lc.p; };
#pragma unroll
    for (int c = 0; c < kSlots - 1; ++c)
        if (lc.k < n) issue_chunk(sload_i32(next_pid_addr()));

    // Outer loop over the pieces of the share (one request each), inner loop
    // over a piece's chunks: the query slice is live only inside a piece.
    while (cc.k < n) {
        load_q(cc.b);
        reset();
        bool stream_end = false, share_end = false;
        for (;; ++i) {
            // chunk i has landed once this wave's later loads are the only ones
            // pending; B1: chunk i visible to all, chunk i-1 done by all.  The
            // page id of the next chunk to load is read meanwhile.
            const int after = issued - 1 - i;
            const int32_t* pa = next_pid_addr();                // valid even past the share's end
            int pid;
            if (after >= 2) pid = nq == 5 ? wait_chunk_barrier<10>(pa) : wait_chunk_barrier<8>(pa);
            else if (after == 1) pid = nq == 5 ? wait_chunk_barrier<5>(pa) : wait_chunk_barrier<4>(pa);
            else pid = wait_chunk_barrier<0>(pa);
            if (lc.k < n) issue_chunk(pid);                     // into the slot chunk i-1 used

            char* slot = sm.ring[i % kSlots];
            const int nvalid = min(kMlaChunk, cc.len - cc.p * P - cc.ci * kMlaChunk);
            if (nvalid < kMlaChunk) {
                // rows past the history may hold anything (NaN): zero their value
                // part so that 0-weight x row stays 0; their scores are masked
                for (int e = tid; e < (kMlaChunk - nvalid) * (kMlaV / 8); e += kBlock) {
                    const int t = nvalid + e / (kMlaV / 8);
                    const int x = e % (kMlaV / 8);
                    *reinterpret_cast<uint4*>(slot + (x * 32 + (t ^ ((x & 3) << 2))) * 16) = make_uint4(0, 0, 0, 0);
                }
            }

            // ---- scores and softmax for this wave's 16 heads
            if (s_active) {
                // operands are read kPD K-blocks ahead of their MFMAs
                floatx4_t s0 = {}, s1 = {};
                bf16x8_t c0[kPD], c1[kPD];
                const char* sp = slot + s_base;
#pragma unroll
                for (int d = 0; d < kPD; ++d) {
                    c0[d] = *reinterpret_cast<const bf16x8_t*>(sp + d * 2048);
                    c1[d] = *reinterpret_cast<const bf16x8_t*>(sp + d * 2048 + 256);
                }
#pragma unroll
                for (int kb = 0; kb < kSKB; ++kb) {
                    const bf16x8_t a0 = c0[kb % kPD], a1 = c1[kb % kPD];
                    if (kb + kPD < kSKB) {
                        c0[kb % kPD] = *reinterpret_cast<const bf16x8_t*>(sp + (kb + kPD) * 2048);
                        c1[kb % kPD] = *reinterpret_cast<const bf16x8_t*>(sp + (kb + kPD) * 2048 + 256);
                    }
                    s0 = mfma16(a0, qreg[kb], s0);
                    s1 = mfma16(a1, qreg[kb], s1);
                }
                // keep the order written above: the first reads, then per K-block
                // two MFMAs followed by the next two reads
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPD, 0);
#pragma unroll
                for (int kb = 0; kb < kSKB; ++kb) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    if (kb + kPD < kSKB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                // lane holds S^T[token tb*16 + 4 q4l + r][head hw + l16]
                float sv[8];
                float cmax = -__builtin_inff();
                const int nv_lane = nvalid - 4 * q4l;           // live tokens counted from this lane's rows
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[r] = r < nv_lane ? s0[r] * a.scale_log2 : -__builtin_inff();
                    sv[4 + r] = 16 + r < nv_lane ? s1[r] * a.scale_log2 : -__builtin_inff();
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) cmax = fmaxf(cmax, sv[r]);
                cmax = max_xor32(max_xor16(cmax));
                const float m_new = cmax > m_run + kRaise ? cmax : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                float psum = 0.0f;
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    uint32_t pk[2];
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(sv[4 * tb + r] - m_new);
                        const float p1 = __builtin_amdgcn_exp2f(sv[4 * tb + r + 1] - m_new);
                        psum += p0 + p1;
                        pk[r >> 1] = f32_to_bf16_bits(p0) | (static_cast<uint32_t>(f32_to_bf16_bits(p1)) << 16);
                    }
                    *reinterpret_cast<uint2*>(sm.p + pw_base + tb * 32) = make_uint2(pk[0], pk[1]);
                }
                psum = sum_xor32(sum_xor16(psum));
                l_run = __builtin_fmaf(l_run, alpha, psum);
                m_run = m_new;
                if (lane < 16) sm.alpha[hw + l16] = alpha;
                const bool moved = __ballot(alpha != 1.0f) != 0ull;
                if (lane == 0) sm.flags[w] = moved;
            }
            lds_barrier();                                      // B2: P, alpha and flags visible

            // ---- value update for dims [dw, dw + 64) of every head
#pragma unroll
            for (int hb = 0; hb < nhb; ++hb) {
                if ((sm.flags[2 * hb] | sm.flags[2 * hb + 1]) == 0) continue;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[hb * 32 + q4 * 8 + 4 * half]);
#pragma unroll
                    for (int db = 0; db < 2; ++db) {
                        acc[hb][db][q4 * 4 + 0] *= al.x;
                        acc[hb][db][q4 * 4 + 1] *= al.y;
                        acc[hb][db][q4 * 4 + 2] *= al.z;
                        acc[hb][db][q4 * 4 + 3] *= al.w;
                    }
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                bf16x8_t aop[nhb];
#pragma unroll
                for (int hb = 0; hb < nhb; ++hb)
                    aop[hb] = *reinterpret_cast<const bf16x8_t*>(sm.p + pr_base + hb * 32 * kPRow + kb * 32);
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    const short4v lo = ds_read_tr16(slot + tr_base + db * 2048 + kb * 256);
                    const short4v hi = ds_read_tr16(slot + tr_base2 + db * 2048 + kb * 256);
                    const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int hb = 0; hb < nhb; ++hb) acc[hb][db] = mfma32(aop[hb], bop, acc[hb][db]);
                }
            }

            const bool page_end = cc.ci == cc.nch - 1;
            stream_end = page_end && cc.p == cc.pages - 1;
            share_end = page_end && cc.k == n - 1;
            if (stream_end || share_end) break;
            cursor_next(cc, a.seq_lens, P, n);
        }
        ++i;

        // ---- end of piece: normalise and write the result or the partial
        const bool whole = stream_end && piece_p0 == 0;
        const int b = cc.b;
        const int slot_id = first_piece ? g : A + g;
        if (s_active && lane < 16) {
            sm.fin_l[hw + l16] = l_run;
            const float lse2 = m_run + __builtin_log2f(l_run);
            const int h = h0 + hw + l16;
            if (whole) {
                if (a.lse != nullptr) a.lse[static_cast<int64_t>(b) * H + h] = lse2 * kLn2;
            } else {
                a.lse_part[static_cast<int64_t>(slot_id) * H + h] = lse2;
            }
        }
        __syncthreads();
        // lane holds O[head hb*32 + 8 q4 + 4 half + r4][dim dw + 32 db + l32]; the
        // lane index is passed through an opaque move so that this rarely run
        // block's address arithmetic is not hoisted into registers of the loop
        int le = lane;
        asm volatile("" : "+v"(le));
        const int ehalf = le >> 5, el32 = le & 31;
        if (whole) {
            uint16_t* dst = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(b) * H + h0) * kMlaV + dw + el32;
#pragma unroll
            for (int hb = 0; hb < nhb; ++hb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int hl = hb * 32 + q4 * 8 + 4 * ehalf + r4;
                        if (HG % 32 != 0 && hl >= HG) continue;
                        const float inv = __builtin_amdgcn_rcpf(sm.fin_l[hl]);
#pragma unroll
                        for (int db = 0; db < 2; ++db)
                            dst[hl * kMlaV + db * 32] = f32_to_bf16_bits(acc[hb][db][q4 * 4 + r4] * inv);
                    }
        } else {
            float* dst = a.o_part + (static_cast<int64_t>(slot_id) * H + h0) * kMlaV + dw + el32;
#pragma unroll
            for (int hb = 0; hb < nhb; ++hb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int hl = hb * 32 + q4 * 8 + 4 * ehalf + r4;
                        if (HG % 32 != 0 && hl >= HG) continue;
                        const float inv = __builtin_amdgcn_rcpf(sm.fin_l[hl]);
#pragma unroll
                        for (int db = 0; db < 2; ++db) dst[hl * kMlaV + db * 32] = acc[hb][db][q4 * 4 + r4] * inv;
                    }
        }
        if (piece_p0 == 0 && hs == 0 && tid == 0) {
            // first piece of the request: record where it starts and over how
            // many workers it is split, for the merge kernel
            const int64_t start = sh.c0 + piece_first_unit;
            const int gf = first_worker_of(start, sh.W, A);
            const int gl = last_worker_of(start + cc.pages, sh.W, A);
            a.stream_info[b] = make_int2(static_cast<int>(start), gl - gf + 1);
        }
        __syncthreads();                                        // fin_l reused by the next piece
        cursor_next(cc, a.seq_lens, P, n);
        first_piece = false;
        piece_p0 = 0;
        piece_first_unit = cc.k;
    }
    (void)NS;
}

template <int H>
hipError_t launch_h(const MlaArgs& a, hipStream_t s, const KernelEvents& ev) {
    const dim3 grid(a.workers * mla_blocks_per_worker(H));
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL(mla_attn_kernel<H>, grid, dim3(kBlock), 0, s, ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL(mla_attn_kernel<H>, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaArgs& a, hipStream_t s, const KernelEvents& ev) {
    switch (a.heads) {
        case 16: return launch_h<16>(a, s, ev);
        case 32: return launch_h<32>(a, s, ev);
        case 64: return launch_h<64>(a, s, ev);
        case 128: return launch_h<128>(a, s, ev);
        default: return hipErrorInvalidValue;
    }
}

bool mla_heads_supported(int heads) { return heads == 16 || heads == 32 || heads == 64 || heads == 128; }

int mla_blocks_per_worker(int heads) { return heads > kHG ? heads / kHG : 1; }

int mla_blocks_per_cu() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mla_attn_kernel<128>, kBlock, 0) != hipSuccess)
        return 0;
    return blocks;
}

}  // namespace da
