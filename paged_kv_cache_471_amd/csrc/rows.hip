// Several query rows per request on the absorbed MLA path.
//
// A request's query rows in a step are one in plain decode, two with
// multi-token prediction of depth 1 ("SPLASH", §4.2, the rows q_i of each
// request; "Analytical Provisioning", App. B.1, the DeepSeek-V3 configuration
// with MTP depth 1).  The rows are the last ones of the history and row i sees
// positions up to its own, so each row is a decode query over a history cut
// at its own length.  This kernel writes, for each row, that length and a copy
// of the request's page-table entries the row reads; the MLA attention and
// merge kernels then run over batch * rows requests.  In the request-major
// order (b * rows + i) the queries and outputs [batch][rows][heads][...]
// already sit in that order; in the row-major order (i * batch + b, taken by
// the 128-head kernel) that kernel maps each request to its q / out row, and
// the workers that hold one request's rows end up G / rows apart in the
// plan, where they stream the same latent pages at about the same time.
#include "da_common.h"
#include "da_rows.h"

namespace da {
namespace {

constexpr int kRowsBlock = 128;

__global__ __launch_bounds__(kRowsBlock) void rows_expand_kernel(RowsArgs a) {
    const int r = blockIdx.x;                   // expanded request (see RowsArgs::row_major)
    const int nb = a.rows / a.block;            // expanded requests per request
    const int b = a.row_major ? r % a.batch : r / nb;
    const int k = a.row_major ? r / a.batch : r - b * nb;
    const int L = a.seq_lens[b];
    // the block's last row, k block + block - 1, sees positions up to
    // L - rows + k block + block - 1
    const int len = max(0, L - a.rows + (k + 1) * a.block);
    if (threadIdx.x == 0) a.lens_out[r] = len;
    const int pages = (len + a.page_size - 1) / a.page_size;
    const int32_t* src = a.page_table + static_cast<int64_t>(b) * a.max_pages;
    int32_t* dst = a.table_out + static_cast<int64_t>(r) * a.max_pages;
    for (int p = threadIdx.x; p < pages; p += kRowsBlock) dst[p] = src[p];
}

}  // namespace

hipError_t launch_rows_expand(const RowsArgs& a, hipStream_t s) {
    if (a.block < 1 || a.rows % a.block != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rows_expand_kernel, dim3(a.batch * (a.rows / a.block)), dim3(kRowsBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace da
