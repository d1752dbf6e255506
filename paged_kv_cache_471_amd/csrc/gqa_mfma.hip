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
//  * Values: O^T[D][16 members] += V^T[D][16 tokens] . P^T[16 tokens][16
//    members] with v_mfma_f32_16x16x16_bf16, D / 16 dim blocks.  Each fp32
//    weight is split into two bf16 terms, hi = bf16(p) and lo = bf16(p - hi),
//    so hi + lo equals p to within 2^-17 relative; both terms meet the same
//    values (bf16 as stored; fp8 codes convert to bf16 exactly) in two
//    products, exact in fp32 and accumulated in fp32.  The B operand of lane
//    (R, C) is tokens 4R..4R+3 of member C: exactly the weights that lane
//    holds after the softmax.  The A operand of dim block b is, for those four
//    tokens, the value of dim C D/16 + b.  bf16: the lane loads tokens 4R + i
//    (i < 4), dims [C D/16, (C+1) D/16) as whole-row pieces, so block b takes
//    one 16-bit half of word b / 2 of each of its four token rows (two
//    register-local packs).  fp8: the cache keeps V blocks in 16-token tiles
//    (fp8_v_byte in da_common.h) so that word b of the lane's 16-byte pieces
//    is exactly those four codes.  Row C of block b is thus dim C D/16 + b,
//    and lane (R, C) ends holding member C's dims [4R D/16, 4R D/16 + 4 D/16):
//    per page, D/16 pairs of 8-cycle bf16 steps (an fp32 product on
//    v_mfma_f32_16x16x4_f32 would take D/16 x 4 steps of 32 cycles).
//  * Members are the q_rows x (q_heads / kv_heads) (row, head) pairs of a KV
//    head, up to 16; unused member columns carry zero queries and are never
//    written.  Row r of a request sees positions up to len - q_rows + r.
#include <hip/hip_ext.h>

#include <type_traits>
#include <utility>

#include "da_common.h"
#include "da_launch.h"
#include "da_gqa_mfma.h"
#include "da_plan.h"

namespace da {
namespace {

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kPage = 16;           // tokens per page (one MFMA tile)
constexpr float kRaise = 8.0f;      // the running maximum moves only past this margin (base 2)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma_s(bf16x8_t a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx4_t mfma_v16(short4_t a, short4_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ short4_t as_short4(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(short4_t, u32x2{lo, hi});
}
// two fp32 values -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_t));
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
    // page buffers (NB - 1 pages in flight while one is computed): bf16 at
    // head dim 128 keeps one in flight (two measured equal or slower on the
    // llama8b batch, at 198 against 166 vector registers)
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
    // bf16: v[i] = token 4R + i, dims [C DL, C DL + DL); fp8: word b of
    // v[b / VW] = dim C DL + b for tokens 4R..4R+3 (one code per byte)
    MWords<MCfg<KV, D>::VW> v[4];
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

// Occupancy: fp8 is compiled for three workgroups per CU (three waves per
// SIMD, at most 168 registers each; the compiler's own allocation, one
// workgroup, made the long-context workload 128.5 against 106.6 us) but runs
// two per CU by default: with 16-byte value loads two waves per SIMD keep the
// stream busy, and a third only adds pieces to the merge (long-context
// workload 96.0-96.8 against 102.7-103.2 us per step; every fp8 shape
// measured was equal or faster).  bf16 keeps the compiler's own allocation
// (166 vector and 32 accumulation registers at head dim 128, two waves per
// SIMD); a tighter bound that allows three made it 4-5 % slower.
template <int KV>
struct MOcc {
    static constexpr int blocks_per_cu = KV == kFP8 ? 3 : 1;
    static constexpr int run_per_cu = KV == kFP8 ? 2 : 0;    // 0: as many as fit
};

// With gs = q_heads / kv_heads query heads per KV head (any count up to 16),
// member m < 16 of a KV head's group is (row m / gs, head m % gs); a.q_rows
// rows; members from q_rows * gs up only pad the tile.
template <int KV, int D>
__global__ __launch_bounds__(kGqaBlock, MOcc<KV>::blocks_per_cu) void gqa_mfma_kernel(GqaArgs a) {
    using C = MCfg<KV, D>;
    constexpr int KS = C::KS, KW = C::KW, DL = C::DL, VW = C::VW, EB = C::EB, NB = C::NB;

    const int lane = threadIdx.x & 63;
    const int R = lane >> 4;
    const int Cc = lane & 15;
    const int g = uniform(blockIdx.x * (kGqaBlock / 64) + (threadIdx.x >> 6));
    if (g >= a.workers) return;
    const int Hkv = a.kv_heads;
    const int Hq = a.q_heads;
    const int NR = a.q_rows;
    const int gs = Hq / Hkv;                      // query heads per KV head
    int MT = 1;                                   // members per stream in the partial slots
    while (MT < NR * gs) MT <<= 1;

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
    const int mrow = Cc / gs;                        // query row of member Cc
    const int mhead = Cc - mrow * gs;                // its query head within the KV head's group
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
        if constexpr (KV == kFP8) {
            // tiled fp8 V block: 16-byte piece p of lane (R, Cc) at 1024 p + 16 (16 R + Cc)
#pragma unroll
            for (int p = 0; p < DL / 4; ++p) {
                MWords<4> t;
                load_nt<4>(t, vbase + 1024 * p + 16 * lane);
#pragma unroll
                for (int x = 0; x < 4; ++x) buf.v[(4 * p + x) / VW].w[(4 * p + x) % VW] = t.w[x];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) load_nt<VW>(buf.v[i], vbase + v_lane + i * D * EB);
        }
    };

    // Q^T operand: member Cc, the 8 dims k_dim(s, R) of every step
    bf16x8_t qop[KS];
    auto load_q = [&](int b, int j) {
        const int64_t row = (static_cast<int64_t>(b) * NR + mrow) * Hq + j * gs + mhead;
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
    floatx4_t acc[DL];                            // O[member Cc][dim 4R DL + DL x + t] in acc[t][x]
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
            if constexpr (KV == kFP8) {
                // byte i of every word is token 4R + i
                const int vr = nvalid - 4 * R;
                const uint32_t keep = vr >= 4 ? ~0u : (vr <= 0 ? 0u : (1u << (8 * vr)) - 1u);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int w = 0; w < VW; ++w) buf.v[i].w[w] &= keep;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * R + i >= nvalid) {
#pragma unroll
                        for (int w = 0; w < VW; ++w) buf.v[i].w[w] = 0u;
                    }
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
            // accumulator columns are members: this lane's own factor
#pragma unroll
            for (int t = 0; t < DL; ++t)
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[t][x] *= alpha;
        }
        // ---- values: weights as bf16 hi + lo, the B operand (tokens 4R..4R+3 of member Cc)
        const uint32_t h01 = bf16x2_rne(p[0], p[1]);
        const uint32_t h23 = bf16x2_rne(p[2], p[3]);
        const uint32_t l01 = bf16x2_rne(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
        const uint32_t l23 = bf16x2_rne(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
        const short4_t bh = as_short4(h01, h23);
        const short4_t bl = as_short4(l01, l23);
        auto block = [&](auto KB) {
            constexpr int db = decltype(KB)::value;
            short4_t av;                                             // dim Cc DL + db, tokens 4R..4R+3
            if constexpr (KV == kFP8) {
                const uint32_t codes = buf.v[db / VW].w[db % VW];
                av = as_short4(fp8x2_to_bf16x2<false>(codes), fp8x2_to_bf16x2<true>(codes));
            } else {
                // word db / 2 of token 4R + i holds dims Cc DL + 2 (db / 2) + {0, 1} in its
                // low and high halves: gather this dim's half of the four tokens
                constexpr int w = db / 2;
                if constexpr ((db & 1) == 0)
                    av = as_short4((buf.v[0].w[w] & 0xffffu) | (buf.v[1].w[w] << 16),
                                   (buf.v[2].w[w] & 0xffffu) | (buf.v[3].w[w] << 16));
                else
                    av = as_short4((buf.v[0].w[w] >> 16) | (buf.v[1].w[w] & 0xffff0000u),
                                   (buf.v[2].w[w] >> 16) | (buf.v[3].w[w] & 0xffff0000u));
            }
            acc[db] = mfma_v16(av, bh, acc[db]);
            acc[db] = mfma_v16(av, bl, acc[db]);
        };
        static_for<DL>(block);
    };

    // write the piece: member Cc, dims [4R DL, 4R DL + 4 DL) (dim 4R DL + DL x + t in acc[t][x])
    auto finalize = [&](bool whole, int slot) {
        const bool seen = l_run > 0.0f;
        const float inv_col = seen ? vsc / l_run : 0.0f;
        const float lse2 = seen ? m_run + __builtin_log2f(l_run) : -__builtin_inff();
        if (mlive) {
            {
                const int d0 = 4 * R * DL;
                if (whole) {
                    const int64_t row = (static_cast<int64_t>(cc.b) * NR + mrow) * Hq + cc.j * gs + mhead;
                    uint16_t* dst = static_cast<uint16_t*>(a.out) + row * D + d0;
                    uint32_t packed[2 * DL];
#pragma unroll
                    for (int e = 0; e < 2 * DL; ++e)
                        packed[e] = bf16x2_rne(acc[(2 * e) % DL][(2 * e) / DL] * inv_col,
                                               acc[(2 * e + 1) % DL][(2 * e + 1) / DL] * inv_col);
#pragma unroll
                    for (int e = 0; e < DL / 2; ++e)
                        reinterpret_cast<u32x4*>(dst)[e] = u32x4{packed[4 * e], packed[4 * e + 1], packed[4 * e + 2],
                                                                packed[4 * e + 3]};
                } else {
                    float* dst = a.o_part + (static_cast<int64_t>(slot) * MT + Cc) * D + d0;
#pragma unroll
                    for (int e = 0; e < DL; ++e)
                        reinterpret_cast<floatx4_t*>(dst)[e] = floatx4_t{
                            acc[(4 * e) % DL][(4 * e) / DL] * inv_col, acc[(4 * e + 1) % DL][(4 * e + 1) / DL] * inv_col,
                            acc[(4 * e + 2) % DL][(4 * e + 2) / DL] * inv_col,
                            acc[(4 * e + 3) % DL][(4 * e + 3) / DL] * inv_col};
                }
            }
        }
        if (R == 0 && mlive) {
            if (whole) {
                if (a.lse != nullptr) {
                    const int64_t row = (static_cast<int64_t>(cc.b) * NR + mrow) * Hq + cc.j * gs + mhead;
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

template <int KV, int D>
hipError_t launch_m(const GqaArgs* a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    if (per_cu != nullptr) {
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, gqa_mfma_kernel<KV, D>, kGqaBlock, 0) != hipSuccess)
            return hipErrorInvalidValue;
        if (MOcc<KV>::run_per_cu > 0 && blocks > MOcc<KV>::run_per_cu) blocks = MOcc<KV>::run_per_cu;
        *per_cu = blocks * (kGqaBlock / 64);
        return hipSuccess;
    }
    const int per_block = kGqaBlock / 64;
    const int grid = (a->workers + per_block - 1) / per_block;
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL((gqa_mfma_kernel<KV, D>), dim3(grid), dim3(kGqaBlock), 0, s, ev.start, ev.stop, 0, *a);
    else
        hipLaunchKernelGGL((gqa_mfma_kernel<KV, D>), dim3(grid), dim3(kGqaBlock), 0, s, *a);
    return hipGetLastError();
}

hipError_t dispatch_m(int kv_dtype, int dim, const GqaArgs* a, hipStream_t s, const KernelEvents& ev, int* per_cu) {
    if (kv_dtype == kBF16 && dim == 128) return launch_m<kBF16, 128>(a, s, ev, per_cu);
    if (kv_dtype == kBF16 && dim == 64) return launch_m<kBF16, 64>(a, s, ev, per_cu);
    if (kv_dtype == kFP8 && dim == 128) return launch_m<kFP8, 128>(a, s, ev, per_cu);
    if (kv_dtype == kFP8 && dim == 64) return launch_m<kFP8, 64>(a, s, ev, per_cu);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gqa_mfma(int kv_dtype, int head_dim, const GqaArgs& a, hipStream_t s, const KernelEvents& ev) {
    return dispatch_m(kv_dtype, head_dim, &a, s, ev, nullptr);
}

int gqa_mfma_workers_per_cu(int kv_dtype, int head_dim) {
    int per_cu = 0;
    if (dispatch_m(kv_dtype, head_dim, nullptr, nullptr, KernelEvents{}, &per_cu) != hipSuccess) return 0;
    return per_cu;
}

}  // namespace da
