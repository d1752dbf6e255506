// Debug run of the wave planner that the attention kernels execute in-kernel
// (da_plan.h): worker g writes its cut and cursor, and the per-stream
// first worker and piece count follow from the same closed forms the merge
// uses, so tests can compare them bit for bit with the integer specification.
#include "da_common.h"
#include "da_launch.h"
#include "da_plan.h"

namespace da {
namespace {

constexpr int kPlanBlock = 256;

__global__ __launch_bounds__(kPlanBlock) void plan_debug_kernel(PlanArgs a) {
    const int lane = threadIdx.x & 63;
    const int g = uniform(blockIdx.x * (kPlanBlock / 64) + (threadIdx.x >> 6));
    if (g >= a.workers) return;
    const WaveShare sh = plan_share(a.seq_lens, a.batch, a.page_size, a.units, a.workers, g);
    const int A = sh.active;
    if (lane == 0) {
        if (g < A) {
            a.cuts[g] = static_cast<int32_t>(sh.c0);
            a.cursors[g] = make_int4(sh.b, sh.j, sh.p, 0);
        } else {
            a.cuts[g] = static_cast<int32_t>(sh.W);
            a.cursors[g] = make_int4(a.batch, 0, 0, 0);
        }
        if (g == 0) {
            a.active[0] = A;
            a.cuts[a.workers] = static_cast<int32_t>(sh.W);
            a.cursors[a.workers] = make_int4(a.batch, 0, 0, 0);
        }
    }
    if (g != 0) return;
    // worker 0 also lists every stream: lane l walks requests [l*nb, (l+1)*nb)
    const int B = a.batch, U = a.units, P = a.page_size;
    const int nb = (B + 63) >> 6;
    const int b0 = min(B, lane * nb), b1 = min(B, b0 + nb);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += pages_of(a.seq_lens[b], P);
    int cp = wave_incl_scan(local) - local;
    for (int b = b0; b < b1; ++b) {
        const int pages = pages_of(a.seq_lens[b], P);
        for (int j = 0; j < U; ++j) {
            int fw = -1, count = 0;
            if (pages > 0) {
                const int64_t start = static_cast<int64_t>(U) * cp + static_cast<int64_t>(j) * pages;
                fw = first_worker_of(start, sh.W, A);
                count = last_worker_of(start + pages, sh.W, A) - fw + 1;
            }
            a.first_worker[b * U + j] = fw;
            a.piece_count[b * U + j] = count;
        }
        cp += pages;
    }
}

}  // namespace

hipError_t launch_plan_debug(const PlanArgs& a, hipStream_t s) {
    const int grid = (a.workers + kPlanBlock / 64 - 1) / (kPlanBlock / 64);
    hipLaunchKernelGGL(plan_debug_kernel, dim3(grid), dim3(kPlanBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
