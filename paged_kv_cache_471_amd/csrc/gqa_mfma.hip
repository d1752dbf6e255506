// Paged GQA decode attention on the matrix cores, for large head groups
// (gfx950, wave64).
//
// Same operation, planner, partial slots and merge as gqa.hip ("OpWeave",
// App. A.2; "SPLASH", §1 and §3; several query rows per request: "SPLASH",
// §4.2 and "Analytical Provisioning", App. B.1).  When many query heads share
// a KV head (8 with an fp8 cache, or rows x heads with multi-token
// prediction), the vector kernel spends ~680 VALU instructions per 16-token
// page on dot products, 16-lane sums and value FMAs and becomes bound by the
// vector ALUs instead of HBM.  Here both products run on MFMA:
//
//  * Scores: S^T[16 tokens][16 members] = K[16 tokens][D] . Q^T[D][16
//    members] with v_mfma_f32_16x16x32_bf16 (D / 32 steps).  K rows are the A
//    operand: lane (R = lane / 16, C = lane % 16) holds token C's 8 values of
//    every step; Q^T is the B operand, member C.  Products of bf16 values are
//    exact in fp32 and accumulate in fp32, as the vector kernel's dot2.
//  * The result leaves lane (R, C) with tokens 4R..4R+3 of member C: the
//    online softmax of a member runs over the four lanes of its column (two
//    row swaps), in fp32.
//  * Values: O[16 members][D] += P[16 members][16 tokens] . V[16 tokens][D]
//    with v_mfma_f32_16x16x4_f32: fp32 weights and fp32 values, in four steps
//    of four tokens.  Step i takes token 4R + i from lane row R, so each lane's
//    own weights are its A operand and V loaded as tokens 4R + i, dims
//    [C D/16, (C+1) D/16) is the B operand, with no data movement.
//  * Members are the q_rows x (q_heads / kv_heads) (row, head) pairs of a KV
//    head, up to 16; unused member columns carry zero queries and are never
//    written.  Row r of a request sees positions up to len - q_rows + r.
#include <hip/hip_ext.h>

#include "da_common.h"
#include "da_launch.h"
#include "da_gqa_mfma.h"
#include "da_plan.h"

namespace da {
namespace {

constexpr int kPage = 16;           // tokens per page (one MFMA tile)
constexpr float kRaise = 8.0f;      // the running maximum moves only past this margin (base 2)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma_s(bf16x8_t a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma_v(float a, float b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Pairwise max / sum over lanes (l, l ^ 16) and (l, l ^ 32): the four lanes
// of one column of the score tile.
__device__ __forceinline__ float col_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int KV, int D>
struct MCfg {
    static constexpr int EB = ElemBytes<KV>::value;
    static constexpr int KS = D / 32;                 // score MFMA steps
    static constexpr int KW = D * EB / 64 * 4;        // K words per lane: 4 lanes share a token row
    static constexpr int DL = D / 16;                 // value dims per lane
    static constexpr int VW = DL * EB / 4;            // V words per lane per token
    // page buffers: two pages in flight, one for bf16 at head_dim 128, so that
    // two waves fit on a SIMD (256 registers each, accumulators included)
    static constexpr int NB = (EB == 2 && D == 128) ? 2 : 3;
};

template <int N>
struct MWords {
    uint32_t w[N];
};

template <int N>
__device__ __forceinline__ void load_nt(MWords<N>& dst, const char* p) {
    if constexpr (N == 1) {
        dst.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (N == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        dst.w[0] = v.x; dst.w[1] = v.y;
    } else {
        static_assert(N % 4 == 0, "16-byte pieces");
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + q);
            dst.w[4 * q] = v.x; dst.w[4 * q + 1] = v.y; dst.w[4 * q + 2] = v.z; dst.w[4 * q + 3] = v.w;
        }
    }
}

template <int KV, int D>
struct MPage {
    MWords<MCfg<KV, D>::KW> k;          // token C, this lane's quarter of the row (see k_offset)
    MWords<MCfg<KV, D>::VW> v[4];       // tokens 4R + i, dims [C DL, C DL + DL)
};

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

// Dim of the first of the 8 K values that lane row R feeds to score step s.
// The K row of a token is read by the four lanes of a column as 16-byte
// pieces at byte 64 q + 16 R (piece q of lane row R): bf16 piece q holds dims
// [32 q + 8 R, +8) = step q; an fp8 piece holds 16 dims = steps 2q and 2q+1.
template <int KV>
__device__ __forceinline__ int k_dim(int s, int R) {
    if constexpr (KV == kBF16) return 32 * s + 8 * R;
    else return 64 * (s >> 1) + 16 * R + 8 * (s & 1);
}

// Occupancy: fp8 is bounded to three workgroups (three waves per SIMD, at
// most 168 registers each): its pages are small and the stream is bound by
// latency (106.6 against 128.5 us on the long-context workload).  bf16 keeps
// the compiler's own allocation (about 200 registers plus 32 accumulation
// registers, two waves per SIMD); a tighter bound that allows three made it
// 4-5 % slower.
template <int KV>
struct MOcc {
    static constexpr int blocks_per_cu = KV == kFP8 ? 3 : 1;
};

// RG = log2(query heads per KV head).  Members m < 16 of a KV head's group are
// (row m >> RG, head m & (2^RG - 1)); a.q_rows rows.
template <int KV, int D, int RG>
__global__ __launch_bounds__(kGqaBlock, MOcc<KV>::blocks_per_cu) void gqa_mfma_kernel(GqaArgs a) {
    using C = MCfg<KV, D>;
    constexpr int KS = C::KS, KW = C::KW, DL = C::DL, VW = C::VW, EB = C::EB, NB = C::NB;
    constexpr int G = 1 << RG;

    const int lane = threadIdx.x & 63;
    const int R = lane >> 4;
    const int Cc = lane & 15;
    const int g = uniform(blockIdx.x * (kGqaBlock / 64) + (threadIdx.x >> 6));
    if (g >= a.workers) return;
    const int Hkv = a.kv_heads;
    const int Hq = a.q_heads;
    const int NR = a.q_rows;
    int MT = 1;                                   // members per stream in the partial slots
    while (MT < (NR << RG)) MT <<= 1;

    const WaveShare sh = plan_share(a.seq_lens, a.batch, kPage, Hkv, a.workers, g);
    if (sh.has_empty) {
        for_each_empty_request(a.seq_lens, a.batch, a.workers, g, [&](int b) {
            const int n = NR * Hq * D;
            uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(b) * n;
            for (int e = lane; e < n; e += 64) o[e] = 0;
            if (a.lse != nullptr)
                for (int h = lane; h < NR * Hq; h += 64) a.lse[static_cast<int64_t>(b) * NR * Hq + h] = -__builtin_inff();
        });
    }
    const int NA = sh.active;
    if (g == 0 && lane == 0) *a.plan_info = make_int2(static_cast<int>(sh.W), NA);
    if (g >= NA) return;
    const int64_t c0 = sh.c0;
    const int n = static_cast<int>(sh.c1 - sh.c0);
    const char* kvb = static_cast<const char*>(a.kv);
    const int64_t block_bytes = static_cast<int64_t>(a.page_size) * D * EB;   // one (page, K|V, head) block
    const int tile_mask = (1 << a.tile_shift) - 1;

    // member of this lane's score column, and its row / query head offset
    const int mrow = Cc >> RG;                       // query row of member Cc
    const bool mlive = mrow < NR;                    // real member (not padding)

    Cursor cc;
    cc.b = sh.b; cc.j = sh.j; cc.p = sh.p;
    cc.len = sload_i32(a.seq_lens + cc.b);
    cc.pages = (cc.len + kPage - 1) / kPage;
    Cursor lc = cc;

    const cint32_t* page_table = (const cint32_t*)a.page_table;
    auto page_id = [&](const Cursor& c) -> int {
        return page_table[static_cast<int64_t>(c.b) * a.max_pages + (c.p >> a.tile_shift)];
    };
    const int k_lane = Cc * D * EB + 16 * R;                 // byte of piece 0 in the K block
    const int v_lane = 4 * R * D * EB + Cc * DL * EB;        // byte of token 4R, dim C DL in the V block
    // the tile issued is always the load cursor's
    auto issue = [&](MPage<KV, D>& buf, int pid, int j) {
        const int slot0 = (lc.p & tile_mask) * kPage;          // first token of the tile in its page
        const char* kbase = kvb + gqa_kv_offset(pid, 0, j, slot0, Hkv, a.page_size, D) * EB;
        const char* vbase = kbase + static_cast<int64_t>(Hkv) * block_bytes;
        if constexpr (KW == 4) {
            load_nt<4>(buf.k, kbase + k_lane);
        } else {
#pragma unroll
            for (int q = 0; q < KW / 4; ++q) {
                MWords<4> t;
                load_nt<4>(t, kbase + k_lane + 64 * q);
#pragma unroll
                for (int x = 0; x < 4; ++x) buf.k.w[4 * q + x] = t.w[x];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) load_nt<VW>(buf.v[i], vbase + v_lane + i * D * EB);
    };

    // Q^T operand: member Cc, the 8 dims k_dim(s, R) of every step
    bf16x8_t qop[KS];
    auto load_q = [&](int b, int j) {
        const int64_t row = (static_cast<int64_t>(b) * NR + mrow) * Hq + (j << RG) + (Cc & (G - 1));
        const uint16_t* src = static_cast<const uint16_t*>(a.q) + row * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (mlive) {
                qop[s] = *reinterpret_cast<const bf16x8_t*>(src + k_dim<KV>(s, R));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) qop[s][e] = static_cast<__bf16>(0.0f);
            }
        }
    };

    float sl2 = a.scale_log2;
    float vsc = 1.0f;
    auto stream_scales = [&](int j) {
        sl2 = a.scale_log2;
        vsc = 1.0f;
        if constexpr (KV == kFP8) {
            sl2 *= a.k_scale[j];
            vsc = a.v_scale[j];
        }
    };

    float m_run, l_run;                           // member Cc, replicated over the column
    floatx4_t acc[DL];                            // O[member 4R + x][dim Cc DL + t] in acc[t][x]
    auto reset = [&]() {
        m_run = kMaxInit;
        l_run = 0.0f;
#pragma unroll
        for (int t = 0; t < DL; ++t) acc[t] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };

    auto process = [&](MPage<KV, D>& buf) {
        const int nvalid = cc.len - cc.p * kPage;      // >= 1
        // ---- scores S^T[4R + x][Cc]
        floatx4_t sc = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8_t kop;
            if constexpr (KV == kBF16) {
                const uint32_t w[4] = {buf.k.w[4 * s], buf.k.w[4 * s + 1], buf.k.w[4 * s + 2], buf.k.w[4 * s + 3]};
                kop = __builtin_bit_cast(bf16x8_t, w);
            } else {
                // piece s / 2 holds steps s and s+1 (8 codes each)
                const uint32_t c0w = buf.k.w[4 * (s >> 1) + 2 * (s & 1)];
                const uint32_t c1w = buf.k.w[4 * (s >> 1) + 2 * (s & 1) + 1];
                const uint32_t w[4] = {fp8x2_to_bf16x2<false>(c0w), fp8x2_to_bf16x2<true>(c0w),
                                       fp8x2_to_bf16x2<false>(c1w), fp8x2_to_bf16x2<true>(c1w)};
                kop = __builtin_bit_cast(bf16x8_t, w);
            }
            sc = mfma_s(kop, qop[s], sc);
        }
        float sv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) sv[x] = sc[x] * sl2;
        // causal / history mask: member Cc sees tokens t < nvalid - (NR - 1) + mrow
        if (nvalid - (NR - 1) < kPage) {
            const int lim = nvalid - (NR - 1) + mrow;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (4 * R + x >= lim) sv[x] = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * R + i >= nvalid) {
#pragma unroll
                    for (int w = 0; w < VW; ++w) buf.v[i].w[w] = 0u;
                }
        }
        // ---- online softmax of member Cc over the column's 16 tokens
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = col_max(mx);
        const float mn = mx > m_run + kRaise ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        float p[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) p[x] = __builtin_amdgcn_exp2f(sv[x] - mn);
        const float psum = col_sum((p[0] + p[1]) + (p[2] + p[3]));
        l_run = __builtin_fmaf(l_run, alpha, psum);
        m_run = mn;
        if (__ballot(alpha != 1.0f) != 0ull) {
            // accumulator rows are members 4R + x: their factors sit in columns 4R + x
            float al[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) al[x] = __shfl(alpha, 4 * R + x, 64);
#pragma unroll
            for (int t = 0; t < DL; ++t)
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[t][x] *= al[x];
        }
        // ---- values: step i, token 4R + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float vf[DL];
            if constexpr (KV == kBF16) {
#pragma unroll
                for (int w = 0; w < VW; ++w) {
                    vf[2 * w] = bf16_lo(buf.v[i].w[w]);
                    vf[2 * w + 1] = bf16_hi(buf.v[i].w[w]);
                }
            } else {
#pragma unroll
                for (int w = 0; w < VW; ++w) {
                    const floatx2_t lo = fp8x2_to_f32x2<false>(buf.v[i].w[w]);
                    const floatx2_t hi = fp8x2_to_f32x2<true>(buf.v[i].w[w]);
                    vf[4 * w] = lo.x; vf[4 * w + 1] = lo.y;
                    vf[4 * w + 2] = hi.x; vf[4 * w + 3] = hi.y;
                }
            }
#pragma unroll
            for (int t = 0; t < DL; ++t) acc[t] = mfma_v(p[i], vf[t], acc[t]);
        }
    };

    // write the piece: member 4R + x, dims [Cc DL, Cc DL + DL)
    auto finalize = [&](bool whole, int slot) {
        const bool seen = l_run > 0.0f;
        const float inv_col = seen ? vsc / l_run : 0.0f;
        const float lse2 = seen ? m_run + __builtin_log2f(l_run) : -__builtin_inff();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int mem = 4 * R + x;
            const float inv = __shfl(inv_col, mem, 64);
            if ((mem >> RG) >= NR) continue;
            if (whole) {
                const int64_t row = (static_cast<int64_t>(cc.b) * NR + (mem >> RG)) * Hq + (cc.j << RG) + (mem & (G - 1));
                uint16_t* dst = static_cast<uint16_t*>(a.out) + row * D + Cc * DL;
                uint32_t packed[DL / 2];
#pragma unroll
                for (int t = 0; t < DL / 2; ++t)
                    packed[t] = f32_to_bf16_bits(acc[2 * t][x] * inv) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * t + 1][x] * inv)) << 16);
#pragma unroll
                for (int t = 0; t < DL / 2; ++t) reinterpret_cast<uint32_t*>(dst)[t] = packed[t];
            } else {
                float* dst = a.o_part + (static_cast<int64_t>(slot) * MT + mem) * D + Cc * DL;
#pragma unroll
                for (int t = 0; t < DL; ++t) dst[t] = acc[t][x] * inv;
            }
        }
        if (R == 0 && mlive) {
            if (whole) {
                if (a.lse != nullptr) {
                    const int64_t row = (static_cast<int64_t>(cc.b) * NR + mrow) * Hq + (cc.j << RG) + (Cc & (G - 1));
                    a.lse[row] = lse2 * kLn2;
                }
            } else {
                a.lse_part[static_cast<int64_t>(slot) * MT + Cc] = lse2;
            }
        }
    };

    // ---- prologue
    load_q(cc.b, cc.j);
    stream_scales(cc.j);
    reset();
    bool first_piece = true;
    int piece_p0 = cc.p;

    MPage<KV, D> buf[NB];
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

    auto record_stream = [&](int64_t start) {
        if (lane != 0) return;
        const int gf = first_worker_of(start, sh.W, NA);
        const int gl = last_worker_of(start + cc.pages, sh.W, NA);
        a.stream_info[cc.b * Hkv + cc.j] = make_int2(static_cast<int>(start), gl - gf + 1);
    };

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
                stream_scales(cc.j);
                reset();
            }
        } else {
            ++cc.p;
        }
    };

    for (int k = 0; k < n;) {
#pragma unroll
        for (int r = 0; r < NB; ++r) {
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

template <int KV, int D, int RG>
hipError_t launch_m(const GqaArgs& a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    if (per_cu != nullptr) {
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, gqa_mfma_kernel<KV, D, RG>, kGqaBlock, 0) !=
            hipSuccess)
            return hipErrorInvalidValue;
        *per_cu = blocks * (kGqaBlock / 64);
        return hipSuccess;
    }
    const int per_block = kGqaBlock / 64;
    const int grid = (a.workers + per_block - 1) / per_block;
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL((gqa_mfma_kernel<KV, D, RG>), dim3(grid), dim3(kGqaBlock), 0, s, ev.start, ev.stop,
                              0, a);
    else
        hipLaunchKernelGGL((gqa_mfma_kernel<KV, D, RG>), dim3(grid), dim3(kGqaBlock), 0, s, a);
    return hipGetLastError();
}

template <int KV, int D>
hipError_t by_rg(int rg, const GqaArgs* a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    const GqaArgs dummy{};
    const GqaArgs& args = a ? *a : dummy;
    switch (rg) {
        case 0: return launch_m<KV, D, 0>(args, s, ev, per_cu);
        case 1: return launch_m<KV, D, 1>(args, s, ev, per_cu);
        case 2: return launch_m<KV, D, 2>(args, s, ev, per_cu);
        case 3: return launch_m<KV, D, 3>(args, s, ev, per_cu);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch_m(int kv_dtype, int dim, int rg, const GqaArgs* a, hipStream_t s, const KernelEvents& ev,
                      int* per_cu) {
    if (kv_dtype == kBF16 && dim == 128) return by_rg<kBF16, 128>(rg, a, s, ev, per_cu);
    if (kv_dtype == kBF16 && dim == 64) return by_rg<kBF16, 64>(rg, a, s, ev, per_cu);
    if (kv_dtype == kFP8 && dim == 128) return by_rg<kFP8, 128>(rg, a, s, ev, per_cu);
    if (kv_dtype == kFP8 && dim == 64) return by_rg<kFP8, 64>(rg, a, s, ev, per_cu);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gqa_mfma(int kv_dtype, int head_dim, const GqaArgs& a, hipStream_t s, const KernelEvents& ev) {
    return dispatch_m(kv_dtype, head_dim, a.group_log2, &a, s, ev, nullptr);
}

int gqa_mfma_workers_per_cu(int kv_dtype, int head_dim, int group_log2) {
    int per_cu = 0;
    if (dispatch_m(kv_dtype, head_dim, group_log2, nullptr, nullptr, KernelEvents{}, &per_cu) != hipSuccess) return 0;
    return per_cu;
}

}  // namespace da
