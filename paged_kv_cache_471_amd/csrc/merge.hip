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
// One 256-thread workgroup per (stream, group of heads).  Work spreads over
// the whole GPU, so a stream split over many workers (a long request on few
// streams) is merged with many loads in flight rather than by one worker.
// Every reduction runs in a fixed order, so results are deterministic.
#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) v = fmaxf(v, __shfl_xor(v, x, 64));
    return v;
}

// Reduce v over aligned segments of `seg` consecutive threads (seg a power of
// two, 1..256) with op; every thread of a segment gets the segment's result.
template <bool MAX>
__device__ __forceinline__ float segment_reduce(float v, int seg, float* red) {
    const int t = threadIdx.x;
    red[t] = v;
    __syncthreads();
    for (int off = seg >> 1; off >= 1; off >>= 1) {
        if ((t & (seg - 1)) < off) red[t] = MAX ? fmaxf(red[t], red[t + off]) : red[t] + red[t + off];
        __syncthreads();
    }
    const float r = red[t & ~(seg - 1)];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    __shared__ float red[kThreads];
    __shared__ float4 part[kThreads];
    __shared__ float sM[8], sZ[8];
    const int t = threadIdx.x;
    const int nh = a.heads_per_block;
    const int per_stream = a.group / nh;
    const int s = blockIdx.x / per_stream;
    const int h0 = (blockIdx.x % per_stream) * nh;
    const int b = s / a.units;
    const int j = s % a.units;
    if (a.seq_lens[b] == 0) return;
    const int2 info = a.stream_info[s];
    const int n = info.y;
    if (n <= 1) return;
    const int2 pi = *a.plan_info;
    const int64_t W = pi.x;
    const int A = pi.y;
    const int64_t start = info.x;
    const int gf = first_worker_of(start, W, A);
    const int D = a.dim;
    const int G = a.group;

    // per-head maximum and sum of the pieces' log2-sum-exps
    const int tph = kThreads / nh;              // threads per head
    const int hh = t / tph, pl = t % tph;
    float m = -__builtin_inff();
    for (int i = pl; i < n; i += tph)
        m = fmaxf(m, a.lse_part[static_cast<int64_t>(slot_of(gf + i, start, W, A)) * G + h0 + hh]);
    m = segment_reduce<true>(m, tph, red);
    float z = 0.0f;
    for (int i = pl; i < n; i += tph)
        z += __builtin_amdgcn_exp2f(a.lse_part[static_cast<int64_t>(slot_of(gf + i, start, W, A)) * G + h0 + hh] - m);
    z = segment_reduce<false>(z, tph, red);
    if (pl == 0) {
        sM[hh] = m;
        sZ[hh] = z;
        if (a.lse != nullptr)
            a.lse[static_cast<int64_t>(b) * a.units * G + j * G + h0 + hh] = (m + __builtin_log2f(z)) * kLn2;
    }
    __syncthreads();

    // weighted sum of the pieces' outputs, float4 columns of [nh][D]
    const int C4 = nh * D / 4;
    const int PL = C4 >= kThreads ? 1 : kThreads / C4;    // piece lanes per column
    const int q = t / (kThreads / PL) ;                   // this thread's piece lane
    const int64_t out_base = (static_cast<int64_t>(b) * a.units * G + j * G + h0) * D;
    for (int c0 = 0; c0 < C4; c0 += kThreads / PL) {
        const int c = c0 + t % (kThreads / PL);
        const int h = (4 * c) / D;
        const float M = sM[h];
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
        for (int i = q; i < n; i += PL) {
            const int64_t sl = slot_of(gf + i, start, W, A);
            const float w = __builtin_amdgcn_exp2f(a.lse_part[sl * G + h0 + h] - M);
            const float4 o = reinterpret_cast<const float4*>(a.o_part + (sl * G + h0) * D)[c];
            acc.x = __builtin_fmaf(w, o.x, acc.x);
            acc.y = __builtin_fmaf(w, o.y, acc.y);
            acc.z = __builtin_fmaf(w, o.z, acc.z);
            acc.w = __builtin_fmaf(w, o.w, acc.w);
        }
        if (PL > 1) {
            part[t] = acc;
            __syncthreads();
            if (q == 0) {
                for (int r = 1; r < PL; ++r) {
                    const float4 o = part[t + r * (kThreads / PL)];
                    acc.x += o.x;
                    acc.y += o.y;
                    acc.z += o.z;
                    acc.w += o.w;
                }
            }
            __syncthreads();
        }
        if (q == 0) {
            const float inv = 1.0f / sZ[h];
            if (a.out_is_bf16) {
                const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
                const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
                reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + out_base)[c] = make_uint2(lo, hi);
            } else {
                reinterpret_cast<float4*>(static_cast<float*>(a.out) + out_base)[c] =
                    make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
            }
        }
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int streams, hipStream_t s) {
    const int grid = streams * (a.group / a.heads_per_block);
    hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
