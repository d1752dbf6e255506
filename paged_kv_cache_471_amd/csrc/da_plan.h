// Wave-level split-KV planner, run inside the attention kernels.
//
// The step ends when its slowest worker ends, so the quantity to minimise is
// the largest per-worker load ("Analytical Provisioning for Attention-FFN
// Disaggregated LLM Serving under Stochastic Workloads", §3.3, barrier load),
// and attention time is linear in the token load (same paper, §3.1).  The rule
// cuts the step's total page work into equal contiguous shares:
//
//   streams (b, j), b-major, j < U; stream (b, j) owns pages_b = ceil(L_b / P)
//   units.  cp = exclusive prefix sum of pages_b; stream (b, j) covers units
//   [U*cp[b] + j*pages_b, + pages_b); W = U * cp[B].  A = min(G, W) workers are
//   active; worker g < A takes units [c_g, c_{g+1}) with c_g = floor(g*W/A).
//
// Every worker derives its own share from seq_lens (one pass over the batch,
// a wave-wide prefix sum, one search), so no planner launch precedes the
// attention kernel.  The pieces of a stream come from consecutive workers
// whose indices follow in closed form from the stream's unit range.
#pragma once

#include "da_common.h"

namespace da {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

struct WaveShare {
    int64_t W;       // total units
    int active;      // A = min(G, W)
    int64_t c0, c1;  // this worker's unit range (valid when g < active)
    int b, j, p;     // cursor of unit c0
    int has_empty;   // some request has L = 0
};

__device__ __forceinline__ int pages_of(int len, int P) { return (len + P - 1) / P; }

// Share of worker g out of G.  All lanes of the wave call it; every output is
// wave-uniform.  Lane l scans requests [l*nb, (l+1)*nb), nb = ceil(B/64).
__device__ __forceinline__ WaveShare plan_share(const int32_t* __restrict__ seq_lens, int B, int P, int U, int G,
                                                int g) {
    const int lane = threadIdx.x & 63;
    const int nb = (B + 63) >> 6;
    const int b0 = min(B, lane * nb), b1 = min(B, b0 + nb);
    int local = 0, empty = 0;
    for (int b = b0; b < b1; ++b) {
        const int L = seq_lens[b];
        local += pages_of(L, P);
        empty |= (L == 0);
    }
    const int incl = wave_incl_scan(local);
    const int excl = incl - local;
    const int total = __builtin_amdgcn_readlane(incl, 63);
    WaveShare s;
    s.W = static_cast<int64_t>(U) * total;
    s.active = static_cast<int>(min(static_cast<int64_t>(G), s.W));
    s.has_empty = __ballot(empty) != 0ull;
    s.c0 = s.c1 = 0;
    s.b = B;
    s.j = s.p = 0;
    if (g >= s.active) return s;
    s.c0 = (static_cast<int64_t>(g) * s.W) / s.active;
    s.c1 = (static_cast<int64_t>(g + 1) * s.W) / s.active;
    // the lane whose requests contain unit c0 walks them
    const bool mine = static_cast<int64_t>(U) * excl <= s.c0 && s.c0 < static_cast<int64_t>(U) * incl;
    const uint64_t m = __ballot(mine);
    const int src = __builtin_ctzll(m);
    int rb = 0, rj = 0, rp = 0;
    if (lane == src) {
        int cp = excl;
        for (int b = b0; b < b1; ++b) {
            const int pages = pages_of(seq_lens[b], P);
            if (static_cast<int64_t>(U) * (cp + pages) > s.c0) {
                const int off = static_cast<int>(s.c0 - static_cast<int64_t>(U) * cp);
                rb = b;
                rj = off / pages;
                rp = off % pages;
                break;
            }
            cp += pages;
        }
    }
    s.b = __builtin_amdgcn_readlane(rb, src);
    s.j = __builtin_amdgcn_readlane(rj, src);
    s.p = __builtin_amdgcn_readlane(rp, src);
    return s;
}

// Workers holding the pieces of the stream with unit range [start, end):
// first = largest g with c_g <= start, last = largest g with c_g < end.
__device__ __forceinline__ int first_worker_of(int64_t start, int64_t W, int A) {
    const int64_t g = ((start + 1) * A - 1) / W;
    return static_cast<int>(g < A - 1 ? g : A - 1);
}
__device__ __forceinline__ int last_worker_of(int64_t end, int64_t W, int A) {
    const int64_t g = (end * A - 1) / W;
    return static_cast<int>(g < A - 1 ? g : A - 1);
}
__device__ __forceinline__ int64_t cut_of(int g, int64_t W, int A) {
    return (static_cast<int64_t>(g) * W) / A;
}
// Partial slot of worker g's piece of the stream starting at unit `start`.
__device__ __forceinline__ int slot_of(int g, int64_t start, int64_t W, int A) {
    return cut_of(g, W, A) >= start ? g : A + g;
}

// Calls fn(b) once for every request with L_b == 0 assigned to worker g of G
// (requests are dealt round-robin).  Wave-uniform loop; all lanes call it.
template <class Fn>
__device__ __forceinline__ void for_each_empty_request(const int32_t* __restrict__ seq_lens, int B, int G, int g,
                                                       Fn&& fn) {
    const int lane = threadIdx.x & 63;
    const int nb = (B + 63) >> 6;
    for (int i = 0; i < nb; ++i) {
        const int b = lane * nb + i;
        const bool e = b < B && seq_lens[b] == 0;
        uint64_t m = __ballot(e);
        while (m) {
            const int src = __builtin_ctzll(m);
            m &= m - 1;
            const int bb = src * nb + i;
            if (bb % G == g) fn(bb);
        }
    }
}

}  // namespace da
