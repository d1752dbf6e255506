// Paged absorbed-MLA decode attention for 128 query heads: one worker per
// workgroup of four wavefronts, each wave owning 32 heads outright (gfx950).
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
// App. A.2).  Per token the work is a dense [heads x 576] x [576] product and a
// [heads] x [512] update, so both products run on the matrix cores.
//
// Design (one 256-thread workgroup per CU, one wave per SIMD, 512 registers
// per lane):
//  * The worker walks its contiguous share of (request, page) units in chunks
//    of 32 tokens.  A chunk (36 KiB, contiguous in its page) is copied from HBM
//    into one slot of a 4-slot LDS ring with 16-byte global-to-LDS loads, three
//    chunks ahead of the one being computed.  Each load brings 8 tokens x one
//    whole 128-byte line of their latent rows, with the non-temporal hint
//    (every byte is read once); wave w loads tokens 8w..8w+7 of every chunk.
//    Slot layout: 16-byte block x (0..71) of token t sits at position
//        64 ((t >> 3) + 4 (x >> 3)) + 16 ((x & 7) >> 1) + ((t & 15) ^ 8 (x & 1)),
//    so that each load fills 1 KiB of consecutive positions, and the score
//    operand reads (16 tokens of one block per 16 lanes) and the transposing
//    value reads (8 tokens of two adjacent blocks per 32 lanes) each touch
//    every LDS bank once.
//  * Wave w owns heads [32 w, 32 w + 32) for the whole chunk: its query slice
//    (32 heads x 576, 144 registers) is the B operand of the score product
//    S^T[32 tokens][32 heads] on v_mfma_f32_16x16x32_bf16, with latent rows
//    read from the ring as the A operand; the lane holding S^T[token][head]
//    also runs that head's online softmax (running maximum in base 2, raised
//    only when a chunk's maximum exceeds it by more than 8, so weights stay
//    <= 2^8 and the accumulators are rarely rescaled); and its fp32
//    accumulators O[32 heads][512] (256 registers) take the value product on
//    v_mfma_f32_16x16x32_bf16 with the softmax weights straight from the score
//    registers as the A operand.  The score tile leaves lane (q, j) with tokens
//    4q..4q+3 and 16+4q..16+4q+3 of head j, which is exactly an A operand of
//    the value product once its 32 tokens are taken in that order; the value
//    operand is gathered in the same token order with transposing LDS reads.
//  * Nothing moves between waves but the latent chunk: one barrier per chunk
//    (chunk landed everywhere, previous slot free), no score exchange, no
//    softmax weights in LDS.
//  * Rows past a history's end in its last chunk may hold anything (NaN): the
//    wave that loaded each value block zeroes those rows before the barrier,
//    and their scores are masked.
//  * Every piece leaves its raw accumulators and per-head (max, sum) in a
//    slot of its own; the merge kernel at the end of this file normalises
//    each request from its pieces.  A head whose maximum moves by more than
//    kRaise (rare) folds the accumulators into the slot and restarts them from
//    zero, so no vector instruction ever reads or writes them.
#include <hip/hip_ext.h>

#include "da_mla.h"

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * 64;
constexpr int kLoadsPerWave = kMlaSlotLoads / kWaves;   // 9 of a chunk's 36 loads
static_assert(kMlaSlotLoads % kWaves == 0, "load split");
constexpr int kSlots = 4;
constexpr int kHW = 32;                      // heads per wave
constexpr int kNHB = kHW / 16;               // 16-head blocks per wave
constexpr int kHeads = kWaves * kHW;         // 128
constexpr int kKB = kMlaLatent / 32;         // 18 score K-blocks
constexpr int kVB = kMlaV / 16;              // 32 value dim blocks
constexpr float kRaise = 8.0f;               // running max moves only past this margin
constexpr int kPD = 4;                       // score operand K-blocks in flight
constexpr int kVD = 4;                       // value operand dim blocks in flight
static_assert(kKB == 2 * kLoadsPerWave, "one chunk load every second K-block");

// Row of q, out and lse that request b of the (possibly row-expanded) batch
// reads and writes (MlaArgs::row_batch, rows).
__device__ __forceinline__ int64_t io_row(const MlaArgs& a, int b) {
    return a.rows > 1 ? static_cast<int64_t>(b % a.row_batch) * a.rows + b / a.row_batch : b;
}

struct __align__(16) WaveSmem {
    char ring[kSlots][kMlaSlotBytes];
};
static_assert(sizeof(WaveSmem) <= 160 * 1024, "LDS");

// Read *next_pid through the scalar cache, then meet the workgroup.
__device__ __forceinline__ int pid_barrier(const int32_t* next_pid) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                 : "=s"(v)
                 : "s"(next_pid)
                 : "memory");
    return v;
}

// Score products in the VGPR form of v_mfma_f32_16x16x32_bf16.  The value
// accumulators fill all 256 AGPRs, so the compiler, which would give every
// matrix instruction of the kernel AGPR accumulators, is kept from placing the
// score tiles there by issuing these through inline assembly.  Dependent
// accumulation into the same registers needs no wait states; a chain starts
// from the inline constant 0 (no vector write of its accumulator precedes it),
// and score_guard() supplies the wait states a vector read of the results
// needs, which the compiler does not insert after inline assembly.
__device__ __forceinline__ floatx4_t score_mfma_first(bf16x8_t a, bf16x8_t b) {
    floatx4_t c;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    return c;
}
__device__ __forceinline__ void score_mfma(floatx4_t& c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_guard(floatx4_t& c0, floatx4_t& c1, floatx4_t& c2, floatx4_t& c3) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
}

// Value products, accumulating in AGPRs (the whole AGPR file holds a wave's
// O[32 heads][512]).  Issued through inline assembly as well, so that the
// register allocator keeps the accumulators in AGPRs across the loop; the
// wait states around them are supplied explicitly: value_guard() before the
// first one of a chunk (its weight operands and, after a rescale, its
// accumulators were just written by vector instructions) and acc_guard()
// before vector instructions read the accumulators at the end of a piece.
__device__ __forceinline__ void value_mfma(floatx4_t& c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// The first value product of a piece starts from the inline constant 0: the
// accumulators are never zeroed by vector instructions (which would build the
// zeros in VGPRs and keep them live across the query loads).
__device__ __forceinline__ floatx4_t value_mfma_first(bf16x8_t a, bf16x8_t b) {
    floatx4_t c;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&a"(c) : "v"(a), "v"(b));
    return c;
}
__device__ __forceinline__ void value_guard(bf16x8_t& p0, bf16x8_t& p1) {
    asm volatile("s_nop 4" : "+v"(p0), "+v"(p1));
}
__device__ __forceinline__ void acc_guard() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// 16 bytes of accumulator straight from AGPRs to global memory.
__device__ __forceinline__ void acc_store(float* dst, const floatx4_t& c) {
    asm volatile("global_store_dwordx4 %0, %1, off" : : "v"(dst), "a"(c) : "memory");
}
// 16 bytes from global memory, bypassing the vector L1 (a lane reads back
// what it stored moments before; see fold_into_slot).
__device__ __forceinline__ floatx4_t load_bypass(const float* src) {
    floatx4_t v;
    asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(src) : "memory");
    return v;
}

__global__ __launch_bounds__(kBlock, 1) void mla_wave_kernel(MlaArgs a) {
    constexpr int H = kHeads;
    __shared__ WaveSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int g = blockIdx.x;
    const int P = a.page_size;
    const char* kvb = static_cast<const char*>(a.kv);
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    // Lane-derived offsets used outside the chunk loop's hot path are
    // recomputed where they are used, from a lane index passed through an
    // opaque move: hoisted out of the loops, they would stay live across them
    // and push the query slice out of the register file.
    auto fresh_lane = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };

    const WaveShare sh = plan_share(a.seq_lens, a.batch, P, 1, a.workers, g);
    if (sh.has_empty && w == 0) {
        for_each_empty_request(a.seq_lens, a.batch, a.workers, g, [&](int b) {
            uint16_t* o = static_cast<uint16_t*>(a.out) + io_row(a, b) * H * kMlaV;
            for (int e = lane; e < H * kMlaV; e += 64) o[e] = 0;
            if (a.lse != nullptr)
                for (int h = lane; h < H; h += 64) a.lse[io_row(a, b) * H + h] = -__builtin_inff();
        });
    }
    const int A = sh.active;
    if (g == 0 && tid == 0) *a.plan_info = make_int2(static_cast<int>(sh.W), A);
    if (g >= A) return;
    const int n = static_cast<int>(sh.c1 - sh.c0);

    // ---- chunk loader.  Wave w issues loads q = w + 4 j (j < 9); load q fills
    //      ring positions [64 q, 64 q + 64) with tokens 8 w + (lane & 7) and
    //      blocks 8 j + x', x' = 2 (lane >> 4) + (((lane >> 3) & 1) ^ (w & 1)):
    //      the inverse of the slot layout on those positions.
    MlaCursor lc;
    mla_cursor_init(lc, sh, a.seq_lens, P);
    int issued = 0;                                              // chunks issued so far
    const int dma_off = (8 * w + (lane & 7)) * kMlaRowBytes + 16 * (2 * (lane >> 4) + (((lane >> 3) & 1) ^ (w & 1)));
    auto dma_src = [&](int pid) {
        return kvb + (static_cast<int64_t>(pid) * P + lc.ci * kMlaChunk) * kMlaRowBytes + dma_off;
    };
    auto dma_lds = [&]() {
        return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)sm.ring[issued % kSlots]));
    };
    auto dma_load = [&](const char* src, uint32_t lds_base, int j) {
        const int q = w + kWaves * j;
        mla_lds_dma16_nt(src + 128 * j, lds_base + q * 1024);
    };
    auto chunk_issued = [&]() {
        ++issued;
        mla_cursor_next(lc, a.seq_lens, P, n);
    };
    auto next_pid_addr = [&]() { return a.page_table + static_cast<int64_t>(lc.b) * a.max_pages + lc.p; };

    // ---- per-lane LDS offsets
    // score operand (A of 16x16x32): token l16 (+16: 128 positions on), K-block
    // kb: block x = 4 kb + q4, so x >> 3 = kb >> 1, (x & 7) >> 1 =
    // 2 (kb & 1) + (q4 >> 1) and x & 1 = q4 & 1
    const int s_base = 16 * (64 * (l16 >> 3) + 16 * (q4 >> 1) + (l16 ^ ((q4 & 1) << 3)));
    auto s_koff = [](int kb) { return 16 * (256 * (kb >> 1) + 32 * (kb & 1)); };
    // value operand (B of 16x16x32) by transposing reads: addressing lane
    // s = l16 of group q4 reads dims 16 db + 4 (s & 3) .. +3 of token
    // 4 q4 + (s >> 2) (16 more for the second read: 128 positions on), so that
    // lane (q4, j) ends with dim 16 db + j at tokens 4 q4 + 0..3, then
    // 16 + 4 q4 + 0..3.  Block x = 2 db + ((s & 3) >> 1): x >> 3 = db >> 2,
    // (x & 7) >> 1 = db & 3, x & 1 = (s & 3) >> 1.
    const int va = l16 & 3, vt = 4 * q4 + (l16 >> 2);
    const int v_base = 16 * (64 * (vt >> 3) + ((vt & 15) ^ (8 * (va >> 1)))) + 8 * (va & 1);
    auto v_doff = [](int db) { return 16 * (256 * (db >> 2) + 16 * (db & 3)); };

    bf16x8_t qreg[kNHB][kKB];
    float m_run[kNHB];
    float l_run[kNHB];       // this lane's part of each head's running sum (its four lanes add up to it)
    floatx4_t acc[kNHB][kVB];

    auto load_q = [&](int b) {
        const int ln = fresh_lane();
#pragma unroll
        for (int hb = 0; hb < kNHB; ++hb) {
            const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(
                static_cast<const uint16_t*>(a.q) +
                (io_row(a, b) * H + kHW * w + 16 * hb + (ln & 15)) * kMlaLatent + 8 * (ln >> 4));
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) qreg[hb][kb] = src[kb * 4];
        }
        // Let the compiler see these loads complete here (this also drains the
        // chunk ring, once per piece): otherwise it would keep them pending
        // around the loop and wait on the ring's loads inside the score product.
        __builtin_amdgcn_s_waitcnt(0xF70);
    };
    auto reset = [&]() {
#pragma unroll
        for (int hb = 0; hb < kNHB; ++hb) {
            m_run[hb] = kMaxInit;
            l_run[hb] = 0.0f;
        }
    };

    // Piece-level state of a rare restart (a head's maximum moved by more than
    // kRaise): the slot already holds an earlier part of the piece, with
    // per-head running max m_seg and sum l_seg.
    bool folded = false;
    float m_seg[kNHB], l_seg[kNHB];
    int64_t cur_slot = 0;
    // Fold the accumulators (weights relative to maxima m_a, sums l_a) into the
    // slot: store them raw; if the slot already holds part of the piece, store
    // them to this worker's scratch instead and combine both with their
    // log-sum-exp weights, tile by tile, in vector registers.
    auto fold_into_slot = [&](const float (&m_a)[kNHB], const float (&l_a)[kNHB]) {
        const int le = fresh_lane();
        float* slot_t = a.o_part + cur_slot * H * kMlaV + (2 * w) * (kVB * 256) + le * 4;
        float* tmp_t = a.o_tmp + static_cast<int64_t>(g) * H * kMlaV + (2 * w) * (kVB * 256) + le * 4;
        float* dst = folded ? tmp_t : slot_t;
        acc_guard();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 0; hb < kNHB; ++hb)
#pragma unroll
            for (int db = 0; db < kVB; ++db) acc_store(dst + (hb * kVB + db) * 256, acc[hb][db]);
        __builtin_amdgcn_sched_barrier(0);
        if (!folded) {
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) {
                m_seg[hb] = m_a[hb];
                l_seg[hb] = l_a[hb];
            }
            return;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int hb = 0; hb < kNHB; ++hb) {
            const float M = fmaxf(m_seg[hb], m_a[hb]);
            const float f1 = __builtin_amdgcn_exp2f(m_seg[hb] - M);
            const float f2 = __builtin_amdgcn_exp2f(m_a[hb] - M);
            l_seg[hb] = l_seg[hb] * f1 + l_a[hb] * f2;
            m_seg[hb] = M;
            // tile rows are heads 4 q4 + r; their factors sit in lanes 4 q4 + r
            float f1r[4], f2r[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f1r[r] = __shfl(f1, 4 * (le >> 4) + r, 64);
                f2r[r] = __shfl(f2, 4 * (le >> 4) + r, 64);
            }
#pragma unroll 1
            for (int db = 0; db < kVB; ++db) {
                float* sp = slot_t + (hb * kVB + db) * 256;
                const floatx4_t x = load_bypass(sp);
                const floatx4_t y = load_bypass(tmp_t + (hb * kVB + db) * 256);
                floatx4_t z;
#pragma unroll
                for (int r = 0; r < 4; ++r) z[r] = x[r] * f1r[r] + y[r] * f2r[r];
                *reinterpret_cast<floatx4_t*>(sp) = z;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    MlaCursor cc;
    mla_cursor_init(cc, sh, a.seq_lens, P);
    int piece_first_unit = 0;             // k of the piece's first unit
    int piece_p0 = cc.p;                  // first page of the piece within its request
    int i = 0;                            // chunk index within the share

    // prologue: three chunks in flight
#pragma unroll
    for (int c = 0; c < kSlots - 1; ++c) {
        if (lc.k < n) {
            const char* src = dma_src(sload_i32(next_pid_addr()));
            const uint32_t base = dma_lds();
#pragma unroll
            for (int j = 0; j < kLoadsPerWave; ++j) dma_load(src, base, j);
            chunk_issued();
        }
    }

    while (cc.k < n) {
        load_q(cc.b);
        reset();
        folded = false;
        cur_slot = static_cast<int64_t>(cc.b) + g;
        bool first_chunk = true;
        bool stream_end = false, share_end = false;
        for (;; ++i) {
            // ---- this wave's loads of chunk i have landed once only its later
            //      chunks' loads are pending
            const int after = issued - 1 - i;
            if (after >= 2) mla_wait_vmcnt<2 * kLoadsPerWave>();
            else if (after == 1) mla_wait_vmcnt<kLoadsPerWave>();
            else mla_wait_vmcnt<0>();
            char* slot = sm.ring[i % kSlots];
            const int nvalid = min(kMlaChunk, cc.len - cc.p * P - cc.ci * kMlaChunk);
            if (nvalid < kMlaChunk) {
                // a history's last chunk: rows past its end may hold anything
                // (NaN); zero the value part (blocks x < 64) of those among the
                // tokens this wave loaded, 8 w .. 8 w + 7, so that weight 0 times
                // the row stays 0
                const int t0 = max(8 * w, nvalid);
                const int rows = 8 * w + 8 - t0;
                for (int e = fresh_lane(); e < 64 * rows; e += 64) {
                    const int x = e & 63;
                    const int t = t0 + (e >> 6);
                    const int pos = 64 * ((t >> 3) + 4 * (x >> 3)) + 16 * ((x & 7) >> 1) + ((t & 15) ^ (8 * (x & 1)));
                    *reinterpret_cast<uint4*>(slot + pos * 16) = make_uint4(0, 0, 0, 0);
                }
            }
            // B1: chunk i visible to all, chunk i-1 done by all (its slot takes
            // chunk i+3); the page id of the next chunk to load is read meanwhile
            const int pid = pid_barrier(next_pid_addr());
            const bool more = lc.k < n;
            const char* dsrc = more ? dma_src(pid) : nullptr;
            const uint32_t dlds = dma_lds();

            // ---- scores S^T[token 16 tb + 4 q4 + r][head 16 hb + l16] over the
            //      576-wide latent; the loads of chunk i+3 are spread over it
            floatx4_t sacc[2][kNHB];
            {
                const char* sp = slot + s_base;
                bf16x8_t c0[kPD], c1[kPD];
#pragma unroll
                for (int d = 0; d < kPD; ++d) {
                    c0[d] = *reinterpret_cast<const bf16x8_t*>(sp + s_koff(d));
                    c1[d] = *reinterpret_cast<const bf16x8_t*>(sp + s_koff(d) + 2048);
                }
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb) {
                    const bf16x8_t a0 = c0[kb % kPD], a1 = c1[kb % kPD];
                    if (kb + kPD < kKB) {
                        c0[kb % kPD] = *reinterpret_cast<const bf16x8_t*>(sp + s_koff(kb + kPD));
                        c1[kb % kPD] = *reinterpret_cast<const bf16x8_t*>(sp + s_koff(kb + kPD) + 2048);
                    }
#pragma unroll
                    for (int hb = 0; hb < kNHB; ++hb) {
                        if (kb == 0) {
                            sacc[0][hb] = score_mfma_first(a0, qreg[hb][kb]);
                            sacc[1][hb] = score_mfma_first(a1, qreg[hb][kb]);
                        } else {
                            score_mfma(sacc[0][hb], a0, qreg[hb][kb]);
                            score_mfma(sacc[1][hb], a1, qreg[hb][kb]);
                        }
                    }
                    if (more && (kb & 1)) dma_load(dsrc, dlds, kb >> 1);
                }
                static_assert(kNHB == 2, "score_guard covers four tiles");
                score_guard(sacc[0][0], sacc[0][1], sacc[1][0], sacc[1][1]);
            }
            if (more) chunk_issued();

            // ---- online softmax of this wave's 32 heads, entirely in registers:
            //      head 16 hb + l16 spreads over lanes l16 + 16 q (q < 4).  The
            //      running maximum is raised only when some score exceeds it by
            //      more than kRaise, which one ballot over the lanes' own maxima
            //      detects; only then are a head's four lanes reduced to its
            //      chunk maximum.  Otherwise the weights take the running maximum
            //      as it stands, and each lane keeps its own part of the running
            //      sum, which is reduced over the four lanes when it is needed.
            bf16x8_t pop[kNHB];
            float sv[kNHB][8], lmax[kNHB];
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[hb][r] = sacc[0][hb][r] * a.scale_log2;
                    sv[hb][4 + r] = sacc[1][hb][r] * a.scale_log2;
                }
                if (nvalid < kMlaChunk) {                           // wave-uniform
                    const int nv = nvalid - 4 * (fresh_lane() >> 4);   // live tokens from this lane's rows
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (r >= nv) sv[hb][r] = -__builtin_inff();
                        if (16 + r >= nv) sv[hb][4 + r] = -__builtin_inff();
                    }
                }
                lmax[hb] = sv[hb][0];
#pragma unroll
                for (int r = 1; r < 8; ++r) lmax[hb] = fmaxf(lmax[hb], sv[hb][r]);
            }
            bool raise = false;
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) raise = raise || lmax[hb] > m_run[hb] + kRaise;
            float m_next[kNHB];
            bool restart = first_chunk;
            if (__ballot(raise) != 0ull) {                          // wave-uniform, rare after a piece's first chunk
#pragma unroll
                for (int hb = 0; hb < kNHB; ++hb) {
                    const float cmax = max_xor32(max_xor16(lmax[hb]));
                    m_next[hb] = cmax > m_run[hb] + kRaise ? cmax : m_run[hb];
                }
                restart = restart || __ballot(m_next[0] != m_run[0] || m_next[kNHB - 1] != m_run[kNHB - 1]) != 0ull;
            } else {
#pragma unroll
                for (int hb = 0; hb < kNHB; ++hb) m_next[hb] = m_run[hb];
            }
            float psum[kNHB];
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) {
                float p[8];
                psum[hb] = 0.0f;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(sv[hb][r] - m_next[hb]);
                    psum[hb] += p[r];
                }
                const uint32_t pk[4] = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                        pack_bf16x2(p[6], p[7])};
                pop[hb] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
            // A head's maximum moved (rare): rather than rescaling the
            // accumulators, which vector instructions never touch, fold them
            // (weights relative to the old maxima) into the piece's slot and
            // start a new accumulation from zero with this chunk.
            if (restart && !first_chunk) {
                float l_tot[kNHB];
#pragma unroll
                for (int hb = 0; hb < kNHB; ++hb) l_tot[hb] = sum_xor32(sum_xor16(l_run[hb]));
                fold_into_slot(m_run, l_tot);
                folded = true;
            }
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) {
                l_run[hb] = restart ? psum[hb] : l_run[hb] + psum[hb];
                m_run[hb] = m_next[hb];
            }

            // ---- values O[head][dim 16 db + l16] += P[head][32 tokens] V[32 tokens][dim]
            {
                auto vread = [&](int db) {
                    const char* vp = slot + v_base + v_doff(db);
                    const short4v lo = ds_read_tr16(vp);
                    const short4v hi = ds_read_tr16(vp + 2048);
                    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                };
                bf16x8_t vb[kVD];
#pragma unroll
                for (int d = 0; d < kVD; ++d) vb[d] = vread(d);
                static_assert(kNHB == 2, "value_guard covers two weight operands");
                value_guard(pop[0], pop[1]);
                if (restart) {
#pragma unroll
                    for (int db = 0; db < kVB; ++db) {
                        const bf16x8_t bop = vb[db % kVD];
                        if (db + kVD < kVB) vb[db % kVD] = vread(db + kVD);
#pragma unroll
                        for (int hb = 0; hb < kNHB; ++hb) acc[hb][db] = value_mfma_first(pop[hb], bop);
                    }
                } else {
#pragma unroll
                    for (int db = 0; db < kVB; ++db) {
                        const bf16x8_t bop = vb[db % kVD];
                        if (db + kVD < kVB) vb[db % kVD] = vread(db + kVD);
#pragma unroll
                        for (int hb = 0; hb < kNHB; ++hb) value_mfma(acc[hb][db], pop[hb], bop);
                    }
                }
            }

            first_chunk = false;
            const bool page_end = cc.ci == cc.nch - 1;
            stream_end = page_end && cc.p == cc.pages - 1;
            share_end = page_end && cc.k == n - 1;
            if (stream_end || share_end) break;
            mla_cursor_next(cc, a.seq_lens, P, n);
        }
        ++i;

        // ---- end of piece: every piece, a whole request or not, leaves its
        //      unnormalised accumulators (as tiles, straight from the AGPRs) and
        //      per-head (running max, sum) in its slot, b + g: the pieces of
        //      request b are held by consecutive workers gf..gl, so these slots
        //      are distinct and below batch + workers.  The merge kernel below
        //      normalises and writes out and lse.
        const int b = cc.b;
        if (!folded) {
            acc_guard();
            __builtin_amdgcn_sched_barrier(0);
            const int le = fresh_lane();
            float* tiles = a.o_part + cur_slot * H * kMlaV + (2 * w) * (kVB * 256) + le * 4;
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb)
#pragma unroll
                for (int db = 0; db < kVB; ++db) acc_store(tiles + (hb * kVB + db) * 256, acc[hb][db]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) {
                m_seg[hb] = m_run[hb];
                l_seg[hb] = sum_xor32(sum_xor16(l_run[hb]));
            }
        } else {
            float l_tot[kNHB];
#pragma unroll
            for (int hb = 0; hb < kNHB; ++hb) l_tot[hb] = sum_xor32(sum_xor16(l_run[hb]));
            fold_into_slot(m_run, l_tot);
        }
        {
            const int le = fresh_lane();
            if (le < 16) {
#pragma unroll
                for (int hb = 0; hb < kNHB; ++hb)
                    reinterpret_cast<float2*>(a.lse_part)[cur_slot * H + kHW * w + 16 * hb + le] =
                        make_float2(m_seg[hb], l_seg[hb]);
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
        mla_cursor_next(cc, a.seq_lens, P, n);
        piece_p0 = 0;
        piece_first_unit = cc.k;
    }
}

// ---- merge: one 256-thread workgroup per (request, 16-head block).  The
//      pieces of request b are the slots b + gf + k, k < n, in token order
//      (gf = first worker of the request): with running max m_k and sum l_k
//      per head and raw accumulators O_k,
//          M = max_k m_k,  Z = sum_k 2^(m_k - M) l_k,
//          out = sum_k 2^(m_k - M) O_k / Z,  lse = (M + log2 Z) ln 2,
//      the attention result over the whole history up to rounding order
//      (SPLASH, §3 "Computation").  The fold runs in a fixed order.
//      Thread t holds tile lane t % 64 of the 16-head block's tiles
//      db = t / 64 + 4 j (j < 8): heads 4 q + r (q = (t % 64) / 16), dim
//      16 db + t % 16.  Two pieces are loaded per round trip.  Normalised rows
//      are staged in LDS (fp32, rows padded to 516 values so that the stores
//      of 4 rows x 16 dims hit 64 distinct banks) and written out as 16-byte
//      pieces of the bf16 [head][512] rows.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 2;                  // pieces per round trip
constexpr int kRowPad = kMlaV + 4;

__global__ __launch_bounds__(kMergeThreads) void mla_wave_merge_kernel(MlaArgs a) {
    constexpr int H = kHeads;
    __shared__ float rows[16][kRowPad];
    const int b = blockIdx.x >> 3;
    const int hblk = blockIdx.x & 7;
    const int t = threadIdx.x;
    const int L = a.seq_lens[b];
    if (L == 0) return;                                   // written by the attention kernel
    const int2 info = a.stream_info[b];
    const int2 pi = *a.plan_info;
    const int n = info.y;
    const int gf = first_worker_of(info.x, pi.x, pi.y);
    const int lane = t & 63, q = lane >> 4, l16 = lane & 15, db0 = t >> 6;
    float M[4], Z[4];
    floatx4_t acc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        M[r] = -__builtin_inff();
        Z[r] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < n; k0 += kMergeBatch) {
        floatx4_t v[kMergeBatch][8];
        float4 s01[kMergeBatch], s23[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (k0 + u < n) {
                const int64_t slot = static_cast<int64_t>(b) + gf + k0 + u;
                const float4* st = reinterpret_cast<const float4*>(a.lse_part + (slot * H + 16 * hblk + 4 * q) * 2);
                s01[u] = st[0];
                s23[u] = st[1];
                const floatx4_t* o =
                    reinterpret_cast<const floatx4_t*>(a.o_part + slot * H * kMlaV) + hblk * kVB * 64 + lane;
#pragma unroll
                for (int j = 0; j < 8; ++j) v[u][j] = o[(db0 + 4 * j) * 64];
            }
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (k0 + u < n) {
                const float mk[4] = {s01[u].x, s01[u].z, s23[u].x, s23[u].z};
                const float lk[4] = {s01[u].y, s01[u].w, s23[u].y, s23[u].w};
                float fo[4], fn[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float mn = fmaxf(M[r], mk[r]);
                    fo[r] = __builtin_amdgcn_exp2f(M[r] - mn);    // 0 on the first piece
                    fn[r] = __builtin_amdgcn_exp2f(mk[r] - mn);
                    Z[r] = Z[r] * fo[r] + lk[r] * fn[r];
                    M[r] = mn;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[j][r] = acc[j][r] * fo[r] + v[u][j][r] * fn[r];
            }
        }
    }
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) inv[r] = 1.0f / Z[r];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) rows[4 * q + r][16 * (db0 + 4 * j) + l16] = acc[j][r] * inv[r];
    if (a.lse != nullptr && db0 == 0 && l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a.lse[io_row(a, b) * H + 16 * hblk + 4 * q + r] = (M[r] + __builtin_log2f(Z[r])) * kLn2;
    }
    __syncthreads();
    uint4* out = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (io_row(a, b) * H + 16 * hblk) * kMlaV);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = t + kMergeThreads * u;            // 16 rows x 64 pieces of 8 values
        const float4 x0 = *reinterpret_cast<const float4*>(&rows[idx >> 6][(idx & 63) * 8]);
        const float4 x1 = *reinterpret_cast<const float4*>(&rows[idx >> 6][(idx & 63) * 8 + 4]);
        out[idx] = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                              pack_bf16x2(x1.z, x1.w));
    }
}

}  // namespace

hipError_t launch_mla_wave_merge(const MlaArgs& a, hipStream_t s) {
    if (a.heads != kHeads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_wave_merge_kernel, dim3(a.batch * (kHeads / 16)), dim3(kMergeThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_mla_wave(const MlaArgs& a, hipStream_t s, const KernelEvents& ev) {
    if (a.heads != kHeads) return hipErrorInvalidValue;
    const dim3 grid(a.workers);
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL(mla_wave_kernel, grid, dim3(kBlock), 0, s, ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL(mla_wave_kernel, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

int mla_wave_blocks_per_cu() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mla_wave_kernel, kBlock, 0) != hipSuccess) return 0;
    return blocks;
}

}  // namespace da
