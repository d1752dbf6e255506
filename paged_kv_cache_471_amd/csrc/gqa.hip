// Paged GQA decode attention, split-KV worker kernel (gfx950, wave64).
//
// What it computes: for one decode step each request contributes one query row
// per head and reads its whole KV history ("OpWeave: Flexible Operator
// Disaggregation for Heterogeneous LLM Serving", App. A.2); every head attends
// the complete history, and a different reduction order is the same result up
// to rounding ("SPLASH: Switching Parallel Layouts of Attention with Seamless
// Handoff for LLM Serving", §3, Computation).  Grouped-query heads share one
// KV head (SPLASH §1).  The step is bandwidth-bound: its time is the KV bytes
// read over the bandwidth ("Analytical Provisioning for Attention-FFN
// Disaggregated LLM Serving under Stochastic Workloads", §3.1 and App. B.2.1).
//
// Design (one wavefront = one worker of the device partition):
//  * The worker walks its contiguous share of (request, KV head, page) units.
//    A page of one KV head is one 16-token block of K and one of V, each
//    16 * head_dim contiguous elements.
//  * Lane l covers token rows r = l / 16 (tokens r, r+4, r+8, r+12 of the page)
//    and the dims [c*D/16, (c+1)*D/16) with c = l % 16, so every load
//    instruction of the wave reads 4 whole consecutive token rows: contiguous,
//    16-byte per lane for bf16 at D = 128.
//  * K and V of the next page are in flight (register double buffer) while the
//    current page is computed; the page id two units ahead is fetched with a
//    scalar load.
//  * q . k partial sums are combined over the 16 lanes of a row with DPP; each
//    row keeps its own online-softmax state (running max, sum, accumulator) for
//    the group's query heads, so the softmax needs no cross-row traffic until
//    the piece ends.  Scores are kept in base 2 with log2(e) folded into the
//    scale.  All accumulation is fp32; bf16 K uses the bf16 dot2 instruction
//    (exact products, fp32 sum).  fp8 caches run on the matrix-core kernel
//    (gqa_mfma.hip) whatever the group: their V blocks are stored in tiles
//    that only it reads.
//  * At the end of a piece the four rows are merged; a piece that is the whole
//    stream writes out/lse, otherwise (o, log2-sum-exp) goes to a partial slot
//    that the merge kernel (merge.hip) combines.
//  * Each wave plans its own share (da_plan.h): no planner launch precedes it.
//  * Several query rows per request (multi-token prediction, short prefill
//    chunks: "SPLASH", §4.2, a request's query rows in a step; "Analytical
//    Provisioning", App. B.1, MTP depth 1) are the last q_rows tokens of the
//    history; row i sees positions t <= len - q_rows + i.  The (row, head)
//    pairs that share a KV head form the kernel's head group, so every K/V
//    page is still read once per step; the causal limit differs between the
//    group's members only on the last page or two.
#include <hip/hip_ext.h>

#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {
namespace {

constexpr int kPage = 16;           // tokens per page this kernel is written for
constexpr int kTPL = kPage / 4;     // tokens per lane per page

template <int QT, int KV, int D, int GS>
struct Cfg {
    static constexpr int EB = ElemBytes<KV>::value;
    static constexpr int DL = D / 16;             // dims per lane
    static constexpr int NW = DL * EB / 4;        // 32-bit words per lane per token row
    static constexpr bool kDot = (KV != kF32);    // bf16 pairs + dot2 for q.k
    static constexpr int QW = kDot ? DL / 2 : DL; // q registers per head
    // page buffers (NB - 1 pages in flight): as deep as registers allow at
    // two waves per SIMD
    static constexpr int NB = (GS >= 8 ? 2 : (NW <= 2 ? 4 : (NW == 4 && GS <= 4 ? 3 : 2)));
    static_assert(NW >= 1, "lane slice must be at least one word");
};

template <int NW>
struct Words {
    uint32_t w[NW];
};

// K/V words are read once per step: non-temporal loads keep them from
// displacing reusable lines in the caches (measured 10 % faster on the bf16
// workloads than plain loads).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int NW>
__device__ __forceinline__ void load_words(Words<NW>& dst, const char* p) {
    if constexpr (NW == 1) {
        dst.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (NW == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        dst.w[0] = v.x; dst.w[1] = v.y;
    } else if constexpr (NW == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        dst.w[0] = v.x; dst.w[1] = v.y; dst.w[2] = v.z; dst.w[3] = v.w;
    } else {
        static_assert(NW == 8, "unsupported lane slice");
        const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
        dst.w[0] = v0.x; dst.w[1] = v0.y; dst.w[2] = v0.z; dst.w[3] = v0.w;
        dst.w[4] = v1.x; dst.w[5] = v1.y; dst.w[6] = v1.z; dst.w[7] = v1.w;
    }
}

template <int NW>
struct PageBuf {
    Words<NW> k[kTPL];
    Words<NW> v[kTPL];
};

// Position of the worker in its share: (request, KV head, page) and the
// request's length and page count.  All fields are wave-uniform.
struct Cursor {
    int b, j, p, len, pages;
};

__device__ __forceinline__ void cursor_next(Cursor& c, const int32_t* seq_lens, int kv_heads) {
    if (++c.p < c.pages) return;
    c.p = 0;
    if (++c.j < kv_heads) return;
    c.j = 0;
    do {
        ++c.b;
        c.len = sload_i32(seq_lens + c.b);
        c.pages = (c.len + kPage - 1) / kPage;
    } while (c.pages == 0);
}

// A KV head's group has MT = GS * SP (row, head) members; RG = log2 of the
// query heads per KV head.  MT > 2^RG means several query rows per request
// (their count is read from the arguments); MT == 2^RG is the single-row
// step, where all row arithmetic folds away at compile time.  SP waves of one
// workgroup form one worker: they walk the same share of units, each with GS
// of the members, so each holds half the softmax state (two waves per SIMD
// instead of one) while the second read of every page hits the cache.
template <int QT, int KV, int D, int GS, int RG, int SP>
__global__ __launch_bounds__(kGqaBlock) void gqa_attn_kernel(GqaArgs a) {
    using C = Cfg<QT, KV, D, GS>;
    constexpr int MT = GS * SP;               // members of a KV head's group
    constexpr bool MR = MT > (1 << RG);
    constexpr int DL = C::DL, NW = C::NW, QW = C::QW, EB = C::EB;

    const int lane = threadIdx.x & 63;
    const int row = lane >> 4;            // token row within a group of 4 tokens
    const int col = lane & 15;            // dim slice
    const int wid = uniform(blockIdx.x * (kGqaBlock / 64) + (threadIdx.x >> 6));
    const int g = SP == 1 ? wid : wid / SP;   // worker
    const int m_off = SP == 1 ? 0 : (wid % SP) * GS;   // first member of this wave
    if (g >= a.workers) return;
    const int Hkv = a.kv_heads;
    const int Hq = a.q_heads;
    const int NR = MR ? a.q_rows : 1;         // query rows per request
    constexpr int gl2 = RG;                   // log2(query heads per KV head)
    const int gmask = (1 << gl2) - 1;

    const WaveShare sh = plan_share(a.seq_lens, a.batch, kPage, Hkv, a.workers, g);
    if (sh.has_empty && m_off == 0) {
        // requests with no history: out = 0, lse = -inf
        for_each_empty_request(a.seq_lens, a.batch, a.workers, g, [&](int b) {
            const int row_elems = NR * Hq * D;
            if constexpr (QT == kF32) {
                float* o = static_cast<float*>(a.out) + static_cast<int64_t>(b) * row_elems;
                for (int i = lane; i < row_elems; i += 64) o[i] = 0.0f;
            } else {
                uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(b) * row_elems;
                for (int i = lane; i < row_elems; i += 64) o[i] = 0;
            }
            if (a.lse != nullptr)
                for (int h = lane; h < NR * Hq; h += 64) a.lse[static_cast<int64_t>(b) * NR * Hq + h] = -__builtin_inff();
        });
    }
    const int NA = sh.active;             // active workers
    if (g == 0 && lane == 0 && m_off == 0) *a.plan_info = make_int2(static_cast<int>(sh.W), NA);
    if (g >= NA) return;
    const int64_t c0 = sh.c0;
    const int n = static_cast<int>(sh.c1 - sh.c0);
    const char* kvb = static_cast<const char*>(a.kv);
    const int64_t block_elems = static_cast<int64_t>(a.page_size) * D;   // one (page, K|V, head) block
    const int tile_mask = (1 << a.tile_shift) - 1;
    const int lane_off = (row * D + col * DL) * EB;                  // bytes within a 4-row group

    Cursor cc;                                 // compute cursor
    cc.b = sh.b; cc.j = sh.j; cc.p = sh.p;
    cc.len = sload_i32(a.seq_lens + cc.b);
    cc.pages = (cc.len + kPage - 1) / kPage;
    Cursor lc = cc;                            // load cursor (one unit ahead)

    // Page ids are read through the constant address space: a wave-uniform
    // read there becomes a scalar load whose wait the compiler places at the
    // first use, one unit later, so its latency hides behind a page of work.
    const cint32_t* page_table = (const cint32_t*)a.page_table;
    auto page_id = [&](const Cursor& c) -> int {
        return page_table[static_cast<int64_t>(c.b) * a.max_pages + (c.p >> a.tile_shift)];
    };
    // the tile issued is always the load cursor's
    auto issue = [&](PageBuf<NW>& buf, int pid, int j) {
        const int slot0 = (lc.p & tile_mask) * kPage;          // first token of the tile in its page
        const char* kbase = kvb + (gqa_kv_offset(pid, 0, j, slot0, Hkv, a.page_size, D)) * EB + lane_off;
        const char* vbase = kbase + static_cast<int64_t>(Hkv) * block_elems * EB;
#pragma unroll
        for (int i = 0; i < kTPL; ++i) load_words<NW>(buf.k[i], kbase + i * 4 * D * EB);
#pragma unroll
        for (int i = 0; i < kTPL; ++i) load_words<NW>(buf.v[i], vbase + i * 4 * D * EB);
    };

    // This wave's member hh is member m = m_off + hh of the group: query row
    // m >> gl2 of the request and query head (j << gl2) + (m & gmask); members
    // past the last row pad the group and are neither loaded nor written.
    auto row_of = [&](int hh) -> int { return (m_off + hh) >> gl2; };
    auto q_index = [&](int b, int j, int hh) -> int64_t {
        return (static_cast<int64_t>(b) * NR + row_of(hh)) * Hq + (j << gl2) + ((m_off + hh) & gmask);
    };

    // query registers of the current stream's head group
    uint32_t qb[GS][QW];
    float qf[GS][QW];
    auto load_q = [&](int b, int j) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            if (row_of(hh) >= NR) {
#pragma unroll
                for (int w = 0; w < QW; ++w) { qb[hh][w] = 0u; qf[hh][w] = 0.0f; }
                continue;
            }
            const int64_t base = q_index(b, j, hh) * D + col * DL;
            if constexpr (C::kDot) {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(
                    static_cast<const uint16_t*>(a.q) + base);
#pragma unroll
                for (int w = 0; w < QW; ++w) qb[hh][w] = src[w];
            } else {
                const float* src = static_cast<const float*>(a.q) + base;
#pragma unroll
                for (int w = 0; w < QW; ++w) qf[hh][w] = src[w];
            }
        }
    };

    const float sl2 = a.scale_log2;

    // online-softmax state of this row
    float m[GS], l[GS], acc[GS][DL];
    auto reset = [&]() {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            m[hh] = kMaxInit;
            l[hh] = 0.0f;
#pragma unroll
            for (int d = 0; d < DL; ++d) acc[hh][d] = 0.0f;
        }
    };

    auto process = [&](PageBuf<NW>& buf) {
        const int nvalid = cc.len - cc.p * kPage;   // >= 1
        // the page holds a position that some row may not see
        const bool tail = nvalid - (NR - 1) < kPage;
        float s[GS][kTPL];
#pragma unroll
        for (int i = 0; i < kTPL; ++i) {
            if constexpr (KV == kF32) {
                float kf[DL];
#pragma unroll
                for (int d = 0; d < DL; ++d) kf[d] = __uint_as_float(buf.k[i].w[d]);
#pragma unroll
                for (int hh = 0; hh < GS; ++hh) {
                    float t = 0.0f;
#pragma unroll
                    for (int d = 0; d < DL; ++d) t = __builtin_fmaf(qf[hh][d], kf[d], t);
                    s[hh][i] = t;
                }
            } else {
                static_assert(KV == kBF16, "bf16 or fp32 caches on this kernel");
                uint32_t kp[QW];     // bf16 pairs of this lane's slice of the key
#pragma unroll
                for (int w = 0; w < QW; ++w) kp[w] = buf.k[i].w[w];
#pragma unroll
                for (int hh = 0; hh < GS; ++hh) {
                    float t = dot2_bf16(qb[hh][0], kp[0], 0.0f);
#pragma unroll
                    for (int w = 1; w < QW; ++w) t = dot2_bf16(qb[hh][w], kp[w], t);
                    s[hh][i] = t;
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int i = 0; i < kTPL; ++i) s[hh][i] = row16_sum(s[hh][i]) * sl2;
        if (tail) {
#pragma unroll
            for (int i = 0; i < kTPL; ++i) {
                const int t = i * 4 + row;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    if (t >= nvalid - (NR - 1) + row_of(hh)) s[hh][i] = -__builtin_inff();
                if (t >= nvalid) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) buf.v[i].w[w] = 0u;
                }
            }
        }
        // Online softmax (plain update: on these bandwidth-bound formats a lazy
        // maximum's branches would cost more in load scheduling than the
        // multiplies they save).
        float p[GS][kTPL];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            float mx = s[hh][0];
#pragma unroll
            for (int i = 1; i < kTPL; ++i) mx = fmaxf(mx, s[hh][i]);
            const float mn = fmaxf(m[hh], mx);
            const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);
#pragma unroll
            for (int i = 0; i < kTPL; ++i) p[hh][i] = __builtin_amdgcn_exp2f(s[hh][i] - mn);
            float sum = p[hh][0];
#pragma unroll
            for (int i = 1; i < kTPL; ++i) sum += p[hh][i];
            m[hh] = mn;
            l[hh] = __builtin_fmaf(l[hh], alpha, sum);
#pragma unroll
            for (int d = 0; d < DL; ++d) acc[hh][d] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < kTPL; ++i) {
            float vf[DL];
            if constexpr (KV == kF32) {
#pragma unroll
                for (int d = 0; d < DL; ++d) vf[d] = __uint_as_float(buf.v[i].w[d]);
            } else {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    vf[2 * w] = bf16_lo(buf.v[i].w[w]);
                    vf[2 * w + 1] = bf16_hi(buf.v[i].w[w]);
                }
            }
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[hh][d] = __builtin_fmaf(p[hh][i], vf[d], acc[hh][d]);
        }
    };

    // merge the four rows and write the piece's result
    auto finalize = [&](bool whole, int slot) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
#pragma unroll
            for (int x = 16; x <= 32; x <<= 1) {
                const float mo = shfl_xor_f(m[hh], x);
                const float lo = shfl_xor_f(l[hh], x);
                const float mm = fmaxf(m[hh], mo);
                const float fs = __builtin_amdgcn_exp2f(m[hh] - mm);
                const float fo = __builtin_amdgcn_exp2f(mo - mm);
                l[hh] = l[hh] * fs + lo * fo;
#pragma unroll
                for (int d = 0; d < DL; ++d) {
                    const float ao = shfl_xor_f(acc[hh][d], x);
                    acc[hh][d] = acc[hh][d] * fs + ao * fo;
                }
                m[hh] = mm;
            }
        }
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            if ((hh & 3) != row || row_of(hh) >= NR) continue;
            // a row that sees no position of this piece (only with several
            // rows): o = 0, log-sum-exp -inf
            const bool seen = l[hh] > 0.0f;
            const float inv = seen ? 1.0f / l[hh] : 0.0f;
            const float lse2 = seen ? m[hh] + __builtin_log2f(l[hh]) : -__builtin_inff();
            if (whole) {
                const int64_t qi = q_index(cc.b, cc.j, hh);
                const int64_t o = qi * D + col * DL;
                if constexpr (QT == kF32) {
                    float* dst = static_cast<float*>(a.out) + o;
#pragma unroll
                    for (int d = 0; d < DL; ++d) dst[d] = acc[hh][d] * inv;
                } else {
                    uint32_t packed[DL / 2];
#pragma unroll
                    for (int d = 0; d < DL / 2; ++d) {
                        const uint32_t lo16 = f32_to_bf16_bits(acc[hh][2 * d] * inv);
                        const uint32_t hi16 = f32_to_bf16_bits(acc[hh][2 * d + 1] * inv);
                        packed[d] = lo16 | (hi16 << 16);
                    }
                    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + o);
#pragma unroll
                    for (int d = 0; d < DL / 2; ++d) dst[d] = packed[d];
                }
                if (col == 0 && a.lse != nullptr) a.lse[qi] = lse2 * kLn2;
            } else {
                float* dst = a.o_part + (static_cast<int64_t>(slot) * MT + m_off + hh) * D + col * DL;
#pragma unroll
                for (int d = 0; d < DL; ++d) dst[d] = acc[hh][d] * inv;
                if (col == 0) a.lse_part[static_cast<int64_t>(slot) * MT + m_off + hh] = lse2;
            }
        }
    };

    // ---- prologue
    load_q(cc.b, cc.j);
    reset();
    bool first_piece = true;
    int piece_p0 = cc.p;

    // NB page buffers: NB - 1 pages of K and V in flight ahead of the one computed
    constexpr int NB = C::NB;
    PageBuf<NW> buf[NB];
    int pid = page_id(lc);
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) {
        if (u < n) {
            issue(buf[u], pid, lc.j);
            if (u + 1 < n) {
                cursor_next(lc, a.seq_lens, Hkv);
                pid = page_id(lc);
            }
        }
    }

    // The wave holding a stream's first piece records where the stream starts
    // and over how many workers it is split, for the merge kernel.
    auto record_stream = [&](int64_t start) {
        if (lane != 0 || m_off != 0) return;
        const int gf = first_worker_of(start, sh.W, NA);
        const int gl = last_worker_of(start + cc.pages, sh.W, NA);
        a.stream_info[cc.b * Hkv + cc.j] = make_int2(static_cast<int>(start), gl - gf + 1);
    };

    // after computing unit k: close the piece if the stream or the share ends
    auto end_of_unit = [&](int k) {
        const bool stream_end = (cc.p == cc.pages - 1);
        const bool share_end = (k == n - 1);
        if (stream_end || share_end) {
            const bool whole = stream_end && piece_p0 == 0;
            finalize(whole, first_piece ? g : NA + g);
            if (piece_p0 == 0) record_stream(c0 + k - cc.p);
            if (!share_end) {
                cursor_next(cc, a.seq_lens, Hkv);
                first_piece = false;
                piece_p0 = 0;
                load_q(cc.b, cc.j);
                reset();
            }
        } else {
            ++cc.p;
        }
    };

    for (int k = 0; k < n;) {
#pragma unroll
        for (int r = 0; r < NB; ++r) {          // unit k sits in buf[r] (k % NB == r)
            if (k + NB - 1 < n) {
                issue(buf[(r + NB - 1) % NB], pid, lc.j);
                if (k + NB < n) {
                    cursor_next(lc, a.seq_lens, Hkv);
                    pid = page_id(lc);
                }
            }
            process(buf[r]);
            end_of_unit(k);
            if (++k >= n) break;
        }
    }
}

template <int QT, int KV, int D, int GS, int RG, int SP>
hipError_t launch_one(const GqaArgs& a, hipStream_t s, const KernelEvents& ev) {
    const int per_block = kGqaBlock / 64;
    const int grid = (a.workers * SP + per_block - 1) / per_block;
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL((gqa_attn_kernel<QT, KV, D, GS, RG, SP>), dim3(grid), dim3(kGqaBlock), 0, s,
                              ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL((gqa_attn_kernel<QT, KV, D, GS, RG, SP>), dim3(grid), dim3(kGqaBlock), 0, s, a);
    return hipGetLastError();
}

// workers (SP waves each) of the variant that fit on one CU at once
template <int QT, int KV, int D, int GS, int RG, int SP>
int workers_one() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, gqa_attn_kernel<QT, KV, D, GS, RG, SP>, kGqaBlock,
                                                     0) != hipSuccess)
        return 0;
    return blocks * (kGqaBlock / 64) / SP;
}

// per_cu != null: report the workers per CU of the variant instead of launching it
template <int QT, int KV, int D, int GS, int RG, int SP = 1>
hipError_t run_or_size(const GqaArgs* a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    if (per_cu != nullptr) {
        *per_cu = workers_one<QT, KV, D, GS, RG, SP>();
        return hipSuccess;
    }
    return launch_one<QT, KV, D, GS, RG, SP>(*a, s, ev);
}

// (members, log2 query heads per KV head): the single-row groups 1..8 and the
// multi-row shapes that fit in 8 members; 8-member multi-row groups are split
// over two waves of 4.
template <int QT, int KV, int D>
hipError_t by_group(int members, int rg, const GqaArgs* a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    switch (members * 8 + rg) {
        case 1 * 8 + 0: return run_or_size<QT, KV, D, 1, 0>(a, s, ev, per_cu);
        case 2 * 8 + 1: return run_or_size<QT, KV, D, 2, 1>(a, s, ev, per_cu);
        case 4 * 8 + 2: return run_or_size<QT, KV, D, 4, 2>(a, s, ev, per_cu);
        case 8 * 8 + 3: return run_or_size<QT, KV, D, 8, 3>(a, s, ev, per_cu);
        case 2 * 8 + 0: return run_or_size<QT, KV, D, 2, 0>(a, s, ev, per_cu);
        case 4 * 8 + 0: return run_or_size<QT, KV, D, 4, 0>(a, s, ev, per_cu);
        case 4 * 8 + 1: return run_or_size<QT, KV, D, 4, 1>(a, s, ev, per_cu);
        case 8 * 8 + 0: return run_or_size<QT, KV, D, 4, 0, 2>(a, s, ev, per_cu);
        case 8 * 8 + 1: return run_or_size<QT, KV, D, 4, 1, 2>(a, s, ev, per_cu);
        case 8 * 8 + 2: return run_or_size<QT, KV, D, 4, 2, 2>(a, s, ev, per_cu);
        default: return hipErrorInvalidValue;
    }
}

template <int QT, int KV>
hipError_t by_dim(int dim, int members, int rg, const GqaArgs* a, hipStream_t s, const KernelEvents& ev,
                  int* waves) {
    switch (dim) {
        case 64: return by_group<QT, KV, 64>(members, rg, a, s, ev, waves);
        case 128: return by_group<QT, KV, 128>(members, rg, a, s, ev, waves);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch(int q_dtype, int kv_dtype, int dim, int members, int rg, const GqaArgs* a, hipStream_t s,
                    const KernelEvents& ev, int* waves) {
    if (q_dtype == kF32 && kv_dtype == kF32) return by_dim<kF32, kF32>(dim, members, rg, a, s, ev, waves);
    if (q_dtype == kBF16 && kv_dtype == kBF16) return by_dim<kBF16, kBF16>(dim, members, rg, a, s, ev, waves);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gqa(int q_dtype, int kv_dtype, int head_dim, int members, const GqaArgs& a, hipStream_t s,
                      const KernelEvents& ev) {
    return dispatch(q_dtype, kv_dtype, head_dim, members, a.group_log2, &a, s, ev, nullptr);
}

int gqa_workers_per_cu(int q_dtype, int kv_dtype, int head_dim, int members, int group_log2) {
    int per_cu = 0;
    if (dispatch(q_dtype, kv_dtype, head_dim, members, group_log2, nullptr, nullptr, KernelEvents{}, &per_cu) !=
        hipSuccess)
        return 0;
    return per_cu;
}

}  // namespace da
