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
//  * Scores: waves 2j and 2j+1 share heads [32j, 32j+32) and split the
//    latent: wave w takes latent half w & 1 (9 K-blocks of 32).  Its query
//    slice (2 head blocks x 9 K-blocks) stays in registers as the B operand
//    of v_mfma_f32_16x16x32_bf16; latent rows are the A operand, so partial
//    S^T [16 tokens x 16 heads] tiles come out with each lane holding 4
//    tokens of one head.  Every latent row is thus read from LDS by four
//    waves, not eight.  Wave w keeps the tiles of heads [16w, 16w+16) and
//    hands the other head block to its partner through LDS; after one
//    barrier each wave adds the partner's half and owns its 16 heads.
//    Operands are read two K-blocks ahead of their MFMAs.
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

#include "da_mla.h"

namespace da {
namespace {

constexpr int kWaves = 8;
constexpr int kBlock = kWaves * 64;
constexpr int kLoaders = 4;                           // waves that issue the chunk loads
constexpr int kLoadsPerLoader = kMlaSlotLoads / kLoaders;   // 9
static_assert(kMlaSlotLoads % kLoaders == 0 && kLoaders % 2 == 0, "loader split");
constexpr int kSlots = 4;
constexpr int kHG = kMlaMaxHeads;                     // heads per workgroup
constexpr int kPRow = 80;                             // bytes per head row of P (64 + 16 pad)
constexpr int kSKB = kMlaLatent / 64;                 // 9 K-blocks of 32 per latent half
constexpr int kHW = 16;                               // score heads per wave
constexpr int kDW = kMlaV / kWaves;                   // 64 value dims per wave
constexpr float kRaise = 8.0f;                        // running max moves only past this margin
constexpr int kPD = 2;                                // score operand reads in flight (K-blocks)

static_assert(kHG == kWaves * kHW, "each wave owns 16 score heads");

// Per-wave area of 2 KiB, used in turn by
//  * the partner's partial scores for this wave's heads (8 floats per lane),
//    written before and read after the mid-chunk barrier, then by
//  * P rows of the wave's 16 heads (80 bytes each), their rescale factors,
//    the wave's rescale flag and, at the end of a piece, the final sums.
// Every use of one kind ends before the next chunk's first barrier.
constexpr int kArea = 2048;
constexpr int kAlphaOff = kHW * kPRow;                // 1280
constexpr int kFinOff = kAlphaOff + kHW * 4;          // 1344
constexpr int kFlagOff = kFinOff + kHW * 4;           // 1408
static_assert(kFlagOff + 4 <= kArea && 2 * 64 * 16 == kArea, "area layout");

struct __align__(16) Smem {
    char ring[kSlots][kMlaSlotBytes];
    char area[kWaves][kArea];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS");


template <int H>
__global__ __launch_bounds__(kBlock, 1) void mla_attn_kernel(MlaArgs a) {
    constexpr int HG = H < kHG ? H : kHG;            // heads of this workgroup
    constexpr int NS = H / HG;                        // workgroups per worker
    constexpr int nhb = (HG + 31) / 32;               // 32-head blocks of the value product
    static_assert(H % 16 == 0 && H <= kMlaMaxHeads && H % HG == 0, "heads");
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
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

    // ---- LDS set-up: P rows of absent heads stay zero, their alpha one, and
    //      every flag zero (areas of absent heads are never written again).
    char* const xa = &sm.area[0][0];
    for (int i = tid; i < kWaves * kArea / 4; i += kBlock) {
        const int off = (4 * i) % kArea;
        reinterpret_cast<float*>(xa)[i] = off >= kAlphaOff && off < kFinOff ? 1.0f : 0.0f;
    }

    // ---- chunk loader: waves 0-3 issue loads q = w + 4 i (9 each).  Two waves
    //      share each SIMD and the first four get ahead of the other four
    //      (they wait at the barriers), so the loads go on their side.  Load q
    //      fills positions [64 q, 64 q + 64): x = 2 q + half, t' = l32, source
    //      token t = t' ^ 4 ((2 q + half) & 3), and (2 q) & 3 = 2 (w & 1) for
    //      every i.
    const bool loader = w < kLoaders;
    MlaCursor lc;
    mla_cursor_init(lc, sh, a.seq_lens, P);
    int issued = 0;                                             // chunks issued so far
    // source of this lane's part of the next chunk to load (page pid)
    auto dma_src = [&](int pid) {
        int ln = lane;
        asm volatile("" : "+v"(ln));      // recomputed per chunk rather than held in a register
        const int dma_off = ((ln & 31) ^ (((2 * (w & 1) + (ln >> 5)) & 3) << 2)) * kMlaRowBytes + (ln >> 5) * 16;
        return kvb + (static_cast<int64_t>(pid) * P + lc.ci * kMlaChunk) * kMlaRowBytes + dma_off;
    };
    auto dma_lds = [&]() {
        return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)sm.ring[issued % kSlots]));
    };
    // load j (0..8) of this loader wave's share of the chunk
    auto dma_load = [&](const char* src, uint32_t lds_base, int j) {
        const int q = w + kLoaders * j;
        mla_lds_dma16(src + 32 * q, lds_base + q * 1024);
    };
    auto chunk_issued = [&]() {
        ++issued;
        mla_cursor_next(lc, a.seq_lens, P, n);
    };
    auto issue_chunk = [&](int pid) {
        if (loader) {
            const char* src = dma_src(pid);
            const uint32_t lds_base = dma_lds();
#pragma unroll
            for (int j = 0; j < kLoadsPerLoader; ++j) dma_load(src, lds_base, j);
        }
        chunk_issued();
    };

    // ---- per-lane LDS offsets.  They are recomputed inside the chunk loop from
    //      a lane index passed through an opaque move, so that the compiler does
    //      not keep them all in registers across the loop (registers are full
    //      with the query slice and the value accumulators).
    auto fresh_lane = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    // score operand: token tb*16 + l16, block x = 4 kb + q4l (x & 3 = q4l)
    auto s_base_of = [](int ln) {
        const int q4 = (ln >> 4) & 3;
        return q4 * 512 + (((ln & 15) ^ (q4 << 2)) << 4);
    };
    // value operand by transposing reads (ds_read_b64_tr_b16): in each group of
    // 16 lanes, lane 4a+e receives element e of the 8-byte rows addressed by
    // lanes a, 4+a, 8+a, 12+a.  Lane s of group G therefore addresses dims
    // 16 (G & 1) + 4 (s & 3) .. +3 of token 8 (G >> 1) + (s >> 2) (+4 for the
    // second read), so that lane l ends up with tokens 8 (l / 32) + j of dim
    // l % 32, the B operand of the 32x32x16 product.  Returns the first
    // read's offset; the second one's differs by +-64 (position bit 2 flips).
    auto tr_base_of = [&](int ln, int& second) {
        const int s16 = ln & 15, gg = ln >> 4;
        const int x = 2 * (gg & 1) + ((s16 >> 1) & 1);          // block within the 32 dims (x & 3)
        const int t = (8 * (gg >> 1) + (s16 >> 2)) ^ (4 * x);    // swizzled token position
        const int base = (kDW / 8) * w * 512 + x * 512 + t * 16 + 8 * (s16 & 1);
        second = base + ((x & 1) ? -64 : 64);
        return base;
    };
    // P of head h sits in area h / 16, row h % 16; operand rows hb*32 + l32
    auto pr_base_of = [](int ln) { return ((ln >> 4) & 1) * kArea + (ln & 15) * kPRow + (ln >> 5) * 16; };
    const int hw = w * kHW;                                     // this wave's softmax heads (local)
    const bool s_active = hw < HG;                              // owns live heads
    // Score head blocks by role: slot 0 = this wave's own heads [16w, 16w+16),
    // slot 1 = the partner's.  With 16 heads in all (one block), both waves of
    // pair 0 compute heads [0, 16) in slot 0 and wave 1 hands its half over.
    constexpr int NQB = HG >= 32 ? 2 : 1;                       // head blocks of a score wave
    const int hg = w >> 1;                                      // 32-head group of the pair
    const int lh = w & 1;                                       // latent half
    const bool c_active = 32 * hg < HG;                         // computes partial scores
    const bool sends = NQB == 2 || lh == 1;                     // hands a block to the partner
    const int dw = w * kDW;                                     // this wave's value dims

    bf16x8_t qreg[NQB][kSKB];
    float m_run = kMaxInit, l_run = 0.0f;
    floatx16_t acc[nhb][2];

    auto load_q = [&](int b) {
        if (!c_active) return;
        const int ln = fresh_lane();
        const int l16 = ln & 15, q4l = (ln >> 4) & 3;
#pragma unroll
        for (int hb = 0; hb < NQB; ++hb) {
            const int hq = NQB == 1 ? 0 : 16 * (hb == 0 ? w : w ^ 1);
            const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(
                static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * H + h0 + hq + l16) * kMlaLatent +
                lh * (kMlaLatent / 2) + 8 * q4l);
#pragma unroll
            for (int kb = 0; kb < kSKB; ++kb) qreg[hb][kb] = src[kb * 4];
        }
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

    MlaCursor cc;
    mla_cursor_init(cc, sh, a.seq_lens, P);
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
            if (after >= 2) pid = loader ? mla_wait_chunk_barrier<2 * kLoadsPerLoader>(pa) : mla_wait_chunk_barrier<0>(pa);
            else if (after == 1) pid = loader ? mla_wait_chunk_barrier<kLoadsPerLoader>(pa) : mla_wait_chunk_barrier<0>(pa);
            else pid = mla_wait_chunk_barrier<0>(pa);
            // The loads of chunk i+3 (into the slot chunk i-1 used) are spread
            // over the score product: a wave that issues them in one burst
            // waits while the memory pipeline takes each 1 KiB load in turn.
            const bool more = lc.k < n;
            const bool dma = loader && more;
            const char* dsrc = dma ? dma_src(pid) : nullptr;
            const uint32_t dlds = dma_lds();
            if (dma && !c_active) {
#pragma unroll
                for (int j = 0; j < kLoadsPerLoader; ++j) dma_load(dsrc, dlds, j);
            }

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

            // ---- partial scores: heads [32 hg, 32 hg + 32) (slots by role), latent half lh
            floatx4_t sacc[2][NQB];
            if (c_active) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int hb = 0; hb < NQB; ++hb) sacc[tb][hb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                // operands are read kPD K-blocks ahead of their MFMAs
                bf16x8_t c0[kPD], c1[kPD];
                const char* sp = slot + s_base_of(fresh_lane()) + lh * (kSKB * 2048);
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
#pragma unroll
                    for (int hb = 0; hb < NQB; ++hb) {
                        sacc[0][hb] = mfma16(a0, qreg[hb][kb], sacc[0][hb]);
                        sacc[1][hb] = mfma16(a1, qreg[hb][kb], sacc[1][hb]);
                    }
                    static_assert(kSKB == kLoadsPerLoader, "one chunk load per K-block");
                    if (dma) dma_load(dsrc, dlds, kb);
                }
                // keep the order written above: the first reads, then per K-block
                // the MFMAs followed by the next two reads
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPD, 0);
#pragma unroll
                for (int kb = 0; kb < kSKB; ++kb) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NQB, 0);
                    if (kb + kPD < kSKB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                // the partner's head block goes to the partner's area
                if (sends) {
                    char* dst = xa + (w ^ 1) * kArea + lane * 16;
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) *reinterpret_cast<floatx4_t*>(dst + tb * 1024) = sacc[tb][NQB - 1];
                }
            }
            if (more) chunk_issued();
            mla_lds_barrier();                                      // partial scores exchanged

            // ---- softmax for this wave's 16 heads
            if (s_active) {
                const int ln = fresh_lane();
                const int q4l = (ln >> 4) & 3, l16 = ln & 15;
                const int pw_base = w * kArea + l16 * kPRow + q4l * 8;   // P row written by this lane
                const char* src = xa + w * kArea + ln * 16;
                const floatx4_t s0 = sacc[0][0] + *reinterpret_cast<const floatx4_t*>(src);
                const floatx4_t s1 = sacc[1][0] + *reinterpret_cast<const floatx4_t*>(src + 1024);
                // lane holds S^T[token tb*16 + 4 q4l + r][head hw + l16]
                float sv[8];
                float cmax = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[r] = s0[r] * a.scale_log2;
                    sv[4 + r] = s1[r] * a.scale_log2;
                }
                if (nvalid < kMlaChunk) {                       // wave-uniform: a history's last chunk
                    const int nv_lane = nvalid - 4 * q4l;       // live tokens counted from this lane's rows
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (r >= nv_lane) sv[r] = -__builtin_inff();
                        if (16 + r >= nv_lane) sv[4 + r] = -__builtin_inff();
                    }
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
                        pk[r >> 1] = pack_bf16x2(p0, p1);
                    }
                    *reinterpret_cast<uint2*>(xa + pw_base + tb * 32) = make_uint2(pk[0], pk[1]);
                }
                psum = sum_xor32(sum_xor16(psum));
                l_run = __builtin_fmaf(l_run, alpha, psum);
                m_run = m_new;
                if (lane < 16) *reinterpret_cast<float*>(xa + w * kArea + kAlphaOff + 4 * l16) = alpha;
                const bool moved = __ballot(alpha != 1.0f) != 0ull;
                if (lane == 0) *reinterpret_cast<int*>(xa + w * kArea + kFlagOff) = moved;
            }
            mla_lds_barrier();                                      // B2: P, alpha and flags visible

            // ---- value update for dims [dw, dw + 64) of every head
            const int oln = fresh_lane();
            const int ohalf = oln >> 5;
#pragma unroll
            for (int hb = 0; hb < nhb; ++hb) {
                const int f0 = *reinterpret_cast<const int*>(xa + (2 * hb) * kArea + kFlagOff);
                const int f1 = *reinterpret_cast<const int*>(xa + (2 * hb + 1) * kArea + kFlagOff);
                if ((f0 | f1) == 0) continue;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    // heads hb*32 + 8 q4 + 4 half .. +3: area 2 hb + q4 / 2
                    const float4 al = *reinterpret_cast<const float4*>(
                        xa + (2 * hb + (q4 >> 1)) * kArea + kAlphaOff + 4 * ((q4 & 1) * 8 + 4 * ohalf));
#pragma unroll
                    for (int db = 0; db < 2; ++db) {
                        acc[hb][db][q4 * 4 + 0] *= al.x;
                        acc[hb][db][q4 * 4 + 1] *= al.y;
                        acc[hb][db][q4 * 4 + 2] *= al.z;
                        acc[hb][db][q4 * 4 + 3] *= al.w;
                    }
                }
            }
            int tr_base2;
            const int tr_base = tr_base_of(oln, tr_base2);
            const int pr_base = pr_base_of(oln);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                bf16x8_t aop[nhb];
#pragma unroll
                for (int hb = 0; hb < nhb; ++hb)
                    aop[hb] = *reinterpret_cast<const bf16x8_t*>(xa + pr_base + hb * 2 * kArea + kb * 32);
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
            mla_cursor_next(cc, a.seq_lens, P, n);
        }
        ++i;

        // ---- end of piece: normalise and write the result or the partial
        const bool whole = stream_end && piece_p0 == 0;
        const int b = cc.b;
        const int slot_id = first_piece ? g : A + g;
        if (s_active && lane < 16) {
            const int l16 = fresh_lane();
            *reinterpret_cast<float*>(xa + w * kArea + kFinOff + 4 * l16) = l_run;
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
                        const float inv = __builtin_amdgcn_rcpf(
                            *reinterpret_cast<const float*>(xa + (hl >> 4) * kArea + kFinOff + 4 * (hl & 15)));
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
                        const float inv = __builtin_amdgcn_rcpf(
                            *reinterpret_cast<const float*>(xa + (hl >> 4) * kArea + kFinOff + 4 * (hl & 15)));
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
        __syncthreads();                                        // final sums read before areas are reused
        mla_cursor_next(cc, a.seq_lens, P, n);
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
