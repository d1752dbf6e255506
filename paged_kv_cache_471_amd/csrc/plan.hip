// Device planner: the split-KV partition of one decode step.
//
// The step ends when its slowest worker ends, so the quantity to minimise is
// the largest per-worker load ("Analytical Provisioning for Attention-FFN
// Disaggregated LLM Serving under Stochastic Workloads", §3.3, barrier load),
// and attention time is linear in the token load (same paper, §3.1).  The
// rule used here cuts the step's total page work into equal contiguous shares:
//
//   streams (b, j), b-major, j < units; stream (b, j) owns pages_b =
//   ceil(L_b / P) units.  cp = exclusive prefix sum of pages_b; stream (b, j)
//   covers units [units*cp[b] + j*pages_b, + pages_b); W = units * cp[B].
//   cut_g = floor(g * W / G), g = 0..G.  With snap > 0 a cut strictly inside a
//   stream moves to the stream's start when it is no farther from it than from
//   the end and within snap units, else to the end when within snap units.
//   Worker g takes units [cut_g, cut_{g+1}).
//
// One workgroup of 1024 threads; cp and the cuts live in LDS.
#include "da_common.h"
#include "da_launch.h"

namespace da {
namespace {

constexpr int kPlanThreads = 1024;

// Exclusive scan of one int per thread over the block; returns the thread's
// prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* scratch /*[kPlanThreads]*/, int* total) {
    const int t = threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int add = (t >= off) ? scratch[t - off] : 0;
        __syncthreads();
        scratch[t] += add;
        __syncthreads();
    }
    int incl = scratch[t];
    *total = scratch[kPlanThreads - 1];
    __syncthreads();
    return incl - v;
}

// largest b in [0, B] with units * cp[b] <= c   (cp[0] = 0 <= c)
__device__ int stream_request(const int* cp, int B, int units, int64_t c) {
    int lo = 0, hi = B;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(units) * cp[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// largest g in [0, G] with cuts[g] <= x
__device__ int last_cut_at_or_before(const int* cuts, int G, int x) {
    int lo = 0, hi = G;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cuts[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
    extern __shared__ int lds[];
    const int B = a.batch, G = a.workers, U = a.units, P = a.page_size;
    int* cp = lds;                  // [B + 1]
    int* cuts = cp + (B + 1);       // [G + 1]
    int* scratch = cuts + (G + 1);  // [kPlanThreads]
    const int t = threadIdx.x;

    // 1. pages per request and their exclusive prefix sum
    const int chunk = (B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(B, t * chunk), b1 = min(B, b0 + chunk);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int L = a.seq_lens[b];
        local += (L + P - 1) / P;
    }
    int total;
    int run = block_exclusive_scan(local, scratch, &total);
    for (int b = b0; b < b1; ++b) {
        cp[b] = run;
        run += (a.seq_lens[b] + P - 1) / P;
    }
    if (t == 0) cp[B] = total;
    __syncthreads();
    const int64_t W = static_cast<int64_t>(U) * total;

    // 2. cut points
    for (int g = t; g <= G; g += kPlanThreads) {
        int64_t c = (static_cast<int64_t>(g) * W) / G;
        if (a.snap > 0 && g > 0 && g < G && c < W) {
            int b = stream_request(cp, B, U, c);
            int pages = cp[b + 1] - cp[b];
            int64_t off = c - static_cast<int64_t>(U) * cp[b];
            int64_t start = static_cast<int64_t>(U) * cp[b] + (off / pages) * pages;
            int64_t end = start + pages;
            int64_t dlo = c - start, dhi = end - c;
            if (dlo > 0) {
                if (dlo <= dhi && dlo <= a.snap) c = start;
                else if (dhi < dlo && dhi <= a.snap) c = end;
            }
        }
        cuts[g] = static_cast<int>(c);
    }
    __syncthreads();

    // 3. cuts and cursors out
    for (int g = t; g <= G; g += kPlanThreads) {
        int c = cuts[g];
        a.cuts[g] = c;
        int4 cur = make_int4(B, 0, 0, 0);
        if (c < W) {
            int b = stream_request(cp, B, U, c);
            int pages = cp[b + 1] - cp[b];
            int off = c - U * cp[b];
            cur = make_int4(b, off / pages, off % pages, 0);
        }
        a.cursors[g] = cur;
    }
    for (int b = t; b <= B; b += kPlanThreads) a.cp[b] = cp[b];

    // 4. first worker of each stream
    for (int s = t; s < B * U; s += kPlanThreads) {
        int b = s / U, j = s % U;
        int pages = cp[b + 1] - cp[b];
        int fw = -1;
        if (pages > 0) fw = last_cut_at_or_before(cuts, G, U * cp[b] + j * pages);
        a.first_worker[s] = fw;
    }

    // 5. streams cut into several pieces: the stream of every cut strictly inside
    //    a stream whose previous cut lies at or before that stream's start.
    const int gchunk = (G + kPlanThreads - 1) / kPlanThreads;
    const int g0 = min(G, t * gchunk), g1 = min(G, g0 + gchunk);
    auto split_stream_of = [&](int g) -> int {
        if (g <= 0 || g >= G) return -1;
        int c = cuts[g];
        if (c >= W) return -1;
        int b = stream_request(cp, B, U, c);
        int pages = cp[b + 1] - cp[b];
        int off = c - U * cp[b];
        int j = off / pages, p = off % pages;
        if (p == 0) return -1;
        int start = U * cp[b] + j * pages;
        if (cuts[g - 1] > start) return -1;
        return b * U + j;
    };
    int nflag = 0;
    for (int g = g0; g < g1; ++g) nflag += (split_stream_of(g) >= 0);
    int nsplit;
    int pos = block_exclusive_scan(nflag, scratch, &nsplit);
    for (int g = g0; g < g1; ++g) {
        int s = split_stream_of(g);
        if (s >= 0) a.split_list[pos++] = s;
    }
    if (t == 0) *a.split_count = nsplit;

    // 6. empty requests: out = 0, lse = -inf
    if (a.out != nullptr) {
        const int row = a.heads * a.out_dim;
        for (int b = 0; b < B; ++b) {
            if (cp[b + 1] != cp[b]) continue;     // pages_b == 0 exactly when L_b == 0
            if (a.out_elem_bytes == 4) {
                float* o = static_cast<float*>(a.out) + static_cast<int64_t>(b) * row;
                for (int i = t; i < row; i += kPlanThreads) o[i] = 0.0f;
            } else {
                uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(b) * row;
                for (int i = t; i < row; i += kPlanThreads) o[i] = 0;
            }
            if (a.lse != nullptr)
                for (int h = t; h < a.heads; h += kPlanThreads)
                    a.lse[static_cast<int64_t>(b) * a.heads + h] = -__builtin_inff();
        }
    }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
    size_t lds = sizeof(int) * (static_cast<size_t>(a.batch) + 1 + a.workers + 1 + kPlanThreads);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace da
