// Log-sum-exp merge of split streams (second launch of a decode step).
//
// A history cut into disjoint token ranges is recombined exactly: with
// per-piece normalised outputs o_i and base-2 log-sum-exps l_i,
//     M = max_i l_i,  Z = sum_i 2^(l_i - M),
//     o = sum_i 2^(l_i - M) o_i / Z,   lse = (M + log2 Z) * ln 2,
// the same attention result up to rounding order ("SPLASH: Switching Parallel
// Layouts of Attention with Seamless Handoff for LLM Serving", §3,
// Computation; §6 on context-parallel attention that splits one context).
//
// One 128-thread workgroup per (stream, group of heads, chunk of their float4
// columns).  Work spreads over the whole GPU, so a stream split over many
// workers (a long request on few streams) is merged with many loads in
// flight rather than by one worker: narrower column chunks leave more of a
// workgroup's threads to the pieces, each folding a few of them.
// Every reduction runs in a fixed order, so results are deterministic.
// With several query rows per request a piece can hold no position that a row
// sees; such a piece carries log-sum-exp -inf and weighs nothing, and a row
// that no piece saw gets out = 0, lse = -inf.  The running maximum is kept at
// or above kFloor, far below any real log-sum-exp, so that an empty piece
// folds in with weight 2^-inf = 0 and never as -inf - (-inf): the fold has no
// branch, and the loads of several pieces stay in flight together.
#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {
namespace {

constexpr int kThreads = 128;
constexpr float kFloor = -3.0e38f;

// NC float4 columns per thread (t, t + kThreads, ...; MLA's 512-value heads):
// the pieces of all NC columns are loaded in one pass, so the partials cost
// one round trip to memory rather than NC.  Same arithmetic and piece order
// as the general path below.
template <int NC>
__device__ __forceinline__ void fold_columns(const MergeArgs& a, int t, int b, int j, int h0, int n, int gf,
                                             int64_t start, int64_t W, int A, int heads, int d4_log2) {
    const int D = a.dim;
    const int G = a.group;
    int hh[NC], ccol[NC];
    int64_t orow[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
        const int c = t + u * kThreads;
        hh[u] = c >> d4_log2;
        ccol[u] = c - (hh[u] << d4_log2);
        const int slot_h = h0 + hh[u];
        const int r = slot_h / a.heads_per_unit;
        orow[u] = (static_cast<int64_t>(b) * a.rows + r) * heads + j * a.heads_per_unit + (slot_h - r * a.heads_per_unit);
    }
    float m[NC], z[NC];
    float4 acc[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
        m[u] = -__builtin_inff();
        z[u] = 0.0f;
        acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll 2
    for (int i = 0; i < n; ++i) {
        const int64_t sl = slot_of(gf + i, start, W, A);
        float l[NC];
        float4 o[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            l[u] = a.lse_part[sl * G + h0 + hh[u]];
            o[u] = reinterpret_cast<const float4*>(a.o_part + (sl * G + h0) * D)[t + u * kThreads];
        }
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const float mn = fmaxf(fmaxf(m[u], l[u]), kFloor);
            const float fo = __builtin_amdgcn_exp2f(m[u] - mn);   // 0 on the first piece
            const float fn = __builtin_amdgcn_exp2f(l[u] - mn);
            z[u] = z[u] * fo + fn;
            acc[u].x = acc[u].x * fo + fn * o[u].x;
            acc[u].y = acc[u].y * fo + fn * o[u].y;
            acc[u].z = acc[u].z * fo + fn * o[u].z;
            acc[u].w = acc[u].w * fo + fn * o[u].w;
            m[u] = mn;
        }
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
        if ((h0 + hh[u]) / a.heads_per_unit >= a.rows) continue;
        const float inv = z[u] > 0.0f ? 1.0f / z[u] : 0.0f;
        if (a.out_is_bf16) {
            const uint32_t lo = f32_to_bf16_bits(acc[u].x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[u].y * inv)) << 16);
            const uint32_t hi = f32_to_bf16_bits(acc[u].z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[u].w * inv)) << 16);
            reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow[u] * D)[ccol[u]] = make_uint2(lo, hi);
        } else {
            reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow[u] * D)[ccol[u]] =
                make_float4(acc[u].x * inv, acc[u].y * inv, acc[u].z * inv, acc[u].w * inv);
        }
        if (a.lse != nullptr && ccol[u] == 0)
            a.lse[orow[u]] = z[u] > 0.0f ? (m[u] + __builtin_log2f(z[u])) * kLn2 : -__builtin_inff();
    }
}

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    __shared__ float4 part[kThreads];
    __shared__ float pm[kThreads], pz[kThreads];
    const int t = threadIdx.x;
    const int nh = a.heads_per_block;
    const int per_stream = a.group / nh;
    const int chunk = blockIdx.x % a.col_chunks;
    const int blk = blockIdx.x / a.col_chunks;
    const int s = blk / per_stream;
    const int h0 = (blk % per_stream) * nh;
    if (h0 / a.heads_per_unit >= a.rows) return;         // members that only pad the group
    const int b = s / a.units;
    const int j = s % a.units;
    // independent loads first: length, stream record, plan summary
    const int L = a.seq_lens[b];
    const int2 info = a.stream_info[s];
    const int2 pi = *a.plan_info;
    if (L == 0 || info.y <= 1) return;
    const int n = info.y;
    const int64_t W = pi.x;
    const int A = pi.y;
    const int64_t start = info.x;
    const int gf = first_worker_of(start, W, A);
    const int D = a.dim;
    const int G = a.group;

    // Thread (q, c): float4 column c of [nh][D], pieces i = q, q + PL, ...  Each
    // thread folds its pieces with a running maximum, then the PL piece lanes
    // of a column are folded in a fixed order; one round trip to memory.
    const int C4 = nh * D / 4 / a.col_chunks;             // float4 columns of this workgroup
    const int cbase = chunk * C4;
    const int cols = C4 < kThreads ? C4 : kThreads;       // columns handled at once
    const int PL = kThreads / cols;                       // piece lanes per column
    const int q = t / cols;
    const int heads = a.units * a.heads_per_unit;        // query heads per row
    const int d4_log2 = __builtin_ctz(static_cast<unsigned>(D)) - 2;   // D is a power of two
    if (C4 == 4 * kThreads && a.col_chunks == 1) {
        fold_columns<4>(a, t, b, j, h0, n, gf, start, W, A, heads, d4_log2);
        return;
    }
    if (C4 == 2 * kThreads && a.col_chunks == 1) {
        fold_columns<2>(a, t, b, j, h0, n, gf, start, W, A, heads, d4_log2);
        return;
    }
    for (int c0 = 0; c0 < C4; c0 += cols) {
        const int c = cbase + c0 + t % cols;
        const int h = c >> d4_log2;
        const int cc = c - (h << d4_log2);                // float4 column within the head
        const int slot_h = h0 + h;                        // (row, head) slot of the stream
        const int r = slot_h / a.heads_per_unit;
        const int64_t out_row =
            (static_cast<int64_t>(b) * a.rows + r) * heads + j * a.heads_per_unit + (slot_h - r * a.heads_per_unit);
        float m = -__builtin_inff(), z = 0.0f;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
        for (int i = q; i < n; i += PL) {
            const int64_t sl = slot_of(gf + i, start, W, A);
            const float l = a.lse_part[sl * G + h0 + h];
            const float4 o = reinterpret_cast<const float4*>(a.o_part + (sl * G + h0) * D)[c];
            const float mn = fmaxf(fmaxf(m, l), kFloor);
            const float fo = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first piece
            const float fn = __builtin_amdgcn_exp2f(l - mn);
            z = z * fo + fn;
            acc.x = acc.x * fo + fn * o.x;
            acc.y = acc.y * fo + fn * o.y;
            acc.z = acc.z * fo + fn * o.z;
            acc.w = acc.w * fo + fn * o.w;
            m = mn;
        }
        if (PL > 1) {
            // pairwise tree over the piece lanes: in each round lane q < half
            // folds lane q + half, in a fixed order
            part[t] = acc;
            pm[t] = m;
            pz[t] = z;
            __syncthreads();
            for (int half = PL / 2; half >= 1; half >>= 1) {
                if (q < half) {
                    const int u = t + half * cols;
                    const float mo = pm[u];
                    const float mn = fmaxf(fmaxf(m, mo), kFloor);
                    const float fs = __builtin_amdgcn_exp2f(m - mn);
                    const float fo = __builtin_amdgcn_exp2f(mo - mn);
                    const float4 o = part[u];
                    z = z * fs + pz[u] * fo;
                    acc.x = acc.x * fs + o.x * fo;
                    acc.y = acc.y * fs + o.y * fo;
                    acc.z = acc.z * fs + o.z * fo;
                    acc.w = acc.w * fs + o.w * fo;
                    m = mn;
                    part[t] = acc;
                    pm[t] = m;
                    pz[t] = z;
                }
                __syncthreads();
            }
        }
        if (q == 0 && r < a.rows) {
            const float inv = z > 0.0f ? 1.0f / z : 0.0f;
            if (a.out_is_bf16) {
                const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
                const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
                reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + out_row * D)[cc] = make_uint2(lo, hi);
            } else {
                reinterpret_cast<float4*>(static_cast<float*>(a.out) + out_row * D)[cc] =
                    make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
            }
            if (a.lse != nullptr && cc == 0)
                a.lse[out_row] = z > 0.0f ? (m + __builtin_log2f(z)) * kLn2 : -__builtin_inff();
        }
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int streams, hipStream_t s) {
    const int grid = streams * (a.group / a.heads_per_block) * a.col_chunks;
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
