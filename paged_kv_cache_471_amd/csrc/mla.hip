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
// App. A.2).  All 128 heads read the same latent, so per token the work is a
// dense [heads x 576] x [576] product and a [heads] x [512] update: the
// contraction runs on MFMA.
//
// Design (one 512-thread workgroup = one worker of the device partition, one
// workgroup per CU):
//  * The worker walks its contiguous share of (request, page) units in chunks
//    of 32 tokens.  A chunk (32 x 1152 B, contiguous in the page) is copied
//    from HBM straight into one slot of a 4-slot LDS ring with 16-byte
//    global-to-LDS loads, three chunks ahead of the one being computed.  Token
//    rows sit 1168 B apart in LDS (16 B of padding), so 16 consecutive rows
//    start on 16 different 16-byte bank groups and both MFMA operand reads
//    below are free of bank conflicts; every read is a per-lane base plus an
//    immediate offset.
//  * Scores: wave w owns heads [16w, 16w+16).  Its query slice stays in
//    registers as the B operand of v_mfma_f32_16x16x32_bf16; the latent rows
//    are the A operand, so S^T [32 tokens x 16 heads] comes out with each lane
//    holding 4 consecutive tokens of one head.
//  * Softmax: per head a running maximum (base 2, log2(e) folded into the
//    scale) that is only raised when a chunk's maximum exceeds it by more than
//    8, so weights stay <= 2^8 and the output rows rarely need rescaling.  The
//    running sum adds the fp32 weights; only the MFMA operand is rounded to
//    bf16.  All accumulation is fp32.
//  * Values: wave w owns value dims [64w, 64w+64) for all heads: O [128 x 64]
//    in fp32 accumulators (v_mfma_f32_32x32x16_bf16, P from LDS as A, the
//    latent columns gathered from the ring as B).
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
constexpr int kRowBlocks = kRowBytes / 16;            // 72 16-byte blocks
constexpr int kLdsRow = kRowBytes + 16;               // 1168 bytes per token in LDS
constexpr int kLdsRowBlocks = kLdsRow / 16;           // 73
constexpr int kChunkLoads = (kMlaChunk * kLdsRowBlocks + 63) / 64;   // 37 wave-wide loads
constexpr int kSlotBytes = kChunkLoads * 1024;        // 37888
constexpr int kSlots = 4;
constexpr int kMaxLoadsPerWave = 5;
constexpr int kPRow = 80;                             // bytes per head row of P (64 + 16 pad)
constexpr int kSKB = kMlaLatent / 32;                 // 18 K-blocks of the score product
constexpr float kRaise = 8.0f;                        // running max moves only past this margin

static_assert(kMlaV == kWaves * 64, "each wave owns 64 value dims");
static_assert(kMlaMaxHeads == kWaves * 16, "each wave owns 16 score heads");

struct __align__(16) Smem {
    char ring[kSlots][kSlotBytes];
    char p[kMlaMaxHeads * kPRow];
    float alpha[kMlaMaxHeads];
    float fin_l[kMlaMaxHeads];
    int flags[kWaves];
};


// Wave-uniform 32-bit read through the scalar data cache (a read; the value is
// ready when the call returns).  Used for page ids and lengths, so that they
// do not queue behind the vector loads of the chunk ring.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

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
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only (does not wait for global loads).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

template <int H>
__global__ __launch_bounds__(kBlock, 1) void mla_attn_kernel(MlaArgs a) {
    static_assert(H % 16 == 0 && H <= kMlaMaxHeads, "heads");
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int g = blockIdx.x;
    const int P = a.page_size;
    const char* kvb = static_cast<const char*>(a.kv);

    const WaveShare sh = plan_share(a.seq_lens, a.batch, P, 1, a.workers, g);
    if (sh.has_empty && w == 0) {
        for_each_empty_request(a.seq_lens, a.batch, a.workers, g, [&](int b) {
            uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(b) * H * kMlaV;
            for (int i = lane; i < H * kMlaV; i += 64) o[i] = 0;
            if (a.lse != nullptr)
                for (int h = lane; h < H; h += 64) a.lse[static_cast<int64_t>(b) * H + h] = -__builtin_inff();
        });
    }
    const int A = sh.active;
    if (g == 0 && tid == 0) *a.plan_info = make_int2(static_cast<int>(sh.W), A);
    if (g >= A) return;
    const int n = static_cast<int>(sh.c1 - sh.c0);

    // ---- LDS set-up: P rows of absent heads stay zero, their alpha one.
    for (int i = tid; i < kMlaMaxHeads * kPRow / 4; i += kBlock) reinterpret_cast<int*>(sm.p)[i] = 0;
    for (int i = tid; i < kMlaMaxHeads; i += kBlock) sm.alpha[i] = 1.0f;
    if (tid < kWaves) sm.flags[tid] = 0;

    // ---- chunk loader: wave w issues loads q = w, w + 8, ... of each chunk
    const int nq = (kChunkLoads - w + kWaves - 1) / kWaves;    // 5 for w < 5, else 4
    Cursor lc;
    cursor_init(lc, sh, a.seq_lens, P);
    int issued = 0;                                             // chunks issued so far
    auto issue_chunk = [&]() {
        const int pid = sload_i32(a.page_table + static_cast<int64_t>(lc.b) * a.max_pages + lc.p);
        const char* src = kvb + (static_cast<int64_t>(pid) * P + lc.ci * kMlaChunk) * kRowBytes;
        const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)sm.ring[issued % kSlots]));
        int ln = lane;
        asm volatile("" : "+v"(ln));      // recomputed per chunk rather than held in registers
#pragma unroll
        for (int i = 0; i < kMaxLoadsPerWave; ++i) {
            if (i < nq) {
                const int pos = (w + i * kWaves) * 64 + ln;     // 16-byte block in the slot
                const int t = pos / kLdsRowBlocks;
                const int x = pos - t * kLdsRowBlocks;
                // pad blocks and the slot's tail get a harmless copy of a live block
                const int off = (t < kMlaChunk && x < kRowBlocks) ? t * kRowBytes + x * 16
                                                                  : min(t, kMlaChunk - 1) * kRowBytes;
                lds_dma16(src + off, lds_base + (w + i * kWaves) * 1024);
            }
        }
        ++issued;
        cursor_next(lc, a.seq_lens, P, n);
    };

    // ---- per-piece state
    const int hw = w * 16;                // this wave's score heads
    const bool s_active = hw < H;
    const int hh = lane & 15;             // head within the wave's 16
    const int tq = lane >> 4;             // token quad within a 16-token block
    bf16x8_t qreg[kSKB];
    float m_run = kMaxInit, l_run = 0.0f;
    floatx16_t acc[4][2];
    constexpr int nhb = (H + 31) >> 5;    // 32-head blocks of the value product

    auto load_q = [&](int b) {
        if (!s_active) return;
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(
            static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * H + hw + hh) * kMlaLatent + 8 * tq);
#pragma unroll
        for (int kb = 0; kb < kSKB; ++kb) qreg[kb] = src[kb * 4];
        // Let the compiler see these loads complete here (this also drains the
        // chunk ring, once per piece): otherwise it would keep them pending
        // around the loop and wait on the ring's loads inside every score block.
        __builtin_amdgcn_s_waitcnt(0xF70);
    };
    auto reset = [&]() {
        m_run = kMaxInit;
        l_run = 0.0f;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
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

    load_q(cc.b);
    reset();
    // prologue: three chunks in flight
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i)
        if (lc.k < n) issue_chunk();

    const int dw = w * 64;                // this wave's value dims

    for (int i = 0; cc.k < n; ++i) {
        // chunk i has landed once this wave's later loads are the only ones pending
        const int after = issued - 1 - i;
        if (after >= 2) {
            if (nq == 5) wait_vmcnt<10>(); else wait_vmcnt<8>();
        } else if (after == 1) {
            if (nq == 5) wait_vmcnt<5>(); else wait_vmcnt<4>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();                                          // B1: chunk i visible; chunk i-1 done
        if (lc.k < n) issue_chunk();                            // into the slot chunk i-1 used

        char* slot = sm.ring[i % kSlots];
        const int nvalid = min(kMlaChunk, cc.len - cc.p * P - cc.ci * kMlaChunk);
        if (nvalid < kMlaChunk) {
            // rows past the history may hold anything (NaN): zero their value
            // part so that 0-weight x row stays 0; their scores are masked
            for (int i2 = tid; i2 < (kMlaChunk - nvalid) * (kMlaV / 8); i2 += kBlock) {
                const int t = nvalid + i2 / (kMlaV / 8);
                *reinterpret_cast<uint4*>(slot + t * kLdsRow + (i2 % (kMlaV / 8)) * 16) = make_uint4(0, 0, 0, 0);
            }
        }

        // ---- scores and softmax for this wave's 16 heads
        if (s_active) {
            floatx4_t s[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                s[tb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                // A row = token tb*16 + hh, k = 32 kb + 8 tq .. + 8
                const char* base = slot + (tb * 16 + hh) * kLdsRow + tq * 16;
#pragma unroll
                for (int kb = 0; kb < kSKB; ++kb) {
                    const bf16x8_t c = *reinterpret_cast<const bf16x8_t*>(base + kb * 64);
                    s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c, qreg[kb], s[tb], 0, 0, 0);
                }
            }
            // lane holds S^T[token tb*16 + 4*tq + r][head hh]
            float sv[2][4];
            float cmax = -__builtin_inff();
            const int nv_lane = nvalid - 4 * tq;                // live tokens from this lane's first
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = tb * 16 + r < nv_lane ? s[tb][r] * a.scale_log2 : -__builtin_inff();
                    sv[tb][r] = v;
                    cmax = fmaxf(cmax, v);
                }
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
            const float m_new = cmax > m_run + kRaise ? cmax : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float psum = 0.0f;
            char* prow = sm.p + (hw + hh) * kPRow;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                uint32_t pk[2];
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(sv[tb][r] - m_new);
                    const float p1 = __builtin_amdgcn_exp2f(sv[tb][r + 1] - m_new);
                    psum += p0 + p1;
                    pk[r >> 1] = f32_to_bf16_bits(p0) | (static_cast<uint32_t>(f32_to_bf16_bits(p1)) << 16);
                }
                *reinterpret_cast<uint2*>(prow + (tb * 16 + 4 * tq) * 2) = make_uint2(pk[0], pk[1]);
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            l_run = __builtin_fmaf(l_run, alpha, psum);
            m_run = m_new;
            if (lane < 16) sm.alpha[hw + hh] = alpha;
            const bool moved = __ballot(alpha != 1.0f) != 0ull;
            if (lane == 0) sm.flags[w] = moved;
        }
        lds_barrier();                                          // B2: P, alpha and flags visible

        // ---- value update for dims [dw, dw + 64) of every head
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            if (hb >= nhb) continue;
            if ((sm.flags[2 * hb] | sm.flags[2 * hb + 1]) == 0) continue;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[hb * 32 + q4 * 8 + 4 * (lane >> 5)]);
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    acc[hb][db][q4 * 4 + 0] *= al.x;
                    acc[hb][db][q4 * 4 + 1] *= al.y;
                    acc[hb][db][q4 * 4 + 2] *= al.z;
                    acc[hb][db][q4 * 4 + 3] *= al.w;
                }
            }
        }
        const int half = lane >> 5;
        const int dl = lane & 31;
        // B operand: latent column d of tokens kb*16 + 8*half + i2, i2 < 8
        const char* vbase = slot + 8 * half * kLdsRow + (dw + dl) * 2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8_t bop[2];
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const char* base = vbase + kb * 16 * kLdsRow + db * 64;
                uint16_t e[8];
#pragma unroll
                for (int i2 = 0; i2 < 8; ++i2) e[i2] = *reinterpret_cast<const uint16_t*>(base + i2 * kLdsRow);
                uint32_t wv[4];
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) wv[i2] = static_cast<uint32_t>(e[2 * i2]) | (static_cast<uint32_t>(e[2 * i2 + 1]) << 16);
                bop[db] = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
            }
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                if (hb >= nhb) continue;
                const bf16x8_t aop = *reinterpret_cast<const bf16x8_t*>(sm.p + (hb * 32 + dl) * kPRow + (kb * 16 + 8 * half) * 2);
#pragma unroll
                for (int db = 0; db < 2; ++db)
                    acc[hb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[db], acc[hb][db], 0, 0, 0);
            }
        }

        // ---- end of piece?
        const bool page_end = cc.ci == cc.nch - 1;
        const bool stream_end = page_end && cc.p == cc.pages - 1;
        const bool share_end = page_end && cc.k == n - 1;
        if (stream_end || share_end) {
            const bool whole = stream_end && piece_p0 == 0;
            const int b = cc.b;
            const int slot_id = first_piece ? g : A + g;
            if (s_active && lane < 16) {
                sm.fin_l[hw + hh] = l_run;
                const float lse2 = m_run + __builtin_log2f(l_run);
                if (whole) {
                    if (a.lse != nullptr) a.lse[static_cast<int64_t>(b) * H + hw + hh] = lse2 * kLn2;
                } else {
                    a.lse_part[static_cast<int64_t>(slot_id) * H + hw + hh] = lse2;
                }
            }
            __syncthreads();
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int hf = ln >> 5, dln = ln & 31;
#pragma unroll
            for (int hb = 0; hb < nhb; ++hb) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int h = hb * 32 + q4 * 8 + 4 * hf + r4;
                        if (H % 32 != 0 && h >= H) continue;
                        const float inv = 1.0f / sm.fin_l[h];
                        const int64_t row = (static_cast<int64_t>(whole ? b : slot_id) * H + h) * kMlaV + dw + dln;
#pragma unroll
                        for (int db = 0; db < 2; ++db) {
                            const float v = acc[hb][db][q4 * 4 + r4] * inv;
                            if (whole)
                                static_cast<uint16_t*>(a.out)[row + db * 32] = f32_to_bf16_bits(v);
                            else
                                a.o_part[row + db * 32] = v;
                        }
                    }
                }
            }
            if (piece_p0 == 0 && tid == 0) {
                // first piece of the request: record where it starts and over how
                // many workers it is split, for the merge kernel
                const int64_t start = sh.c0 + piece_first_unit;
                const int gf = first_worker_of(start, sh.W, A);
                const int gl = last_worker_of(start + cc.pages, sh.W, A);
                a.stream_info[b] = make_int2(static_cast<int>(start), gl - gf + 1);
            }
            __syncthreads();                                    // fin_l reused by the next piece
            reset();
        }
        const bool next_piece = stream_end && !share_end;
        cursor_next(cc, a.seq_lens, P, n);
        if (next_piece) {
            first_piece = false;
            piece_p0 = 0;
            piece_first_unit = cc.k;
            load_q(cc.b);
        }
    }

}

template <int H>
hipError_t launch_h(const MlaArgs& a, hipStream_t s, const KernelEvents& ev) {
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL(mla_attn_kernel<H>, dim3(a.workers), dim3(kBlock), 0, s, ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL(mla_attn_kernel<H>, dim3(a.workers), dim3(kBlock), 0, s, a);
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

int mla_blocks_per_cu() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mla_attn_kernel<128>, kBlock, 0) != hipSuccess)
        return 0;
    return blocks;
}

}  // namespace da
