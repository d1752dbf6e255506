// Host/device interface of the multi-row expansion for the MLA path (rows.hip).
#pragma once

#include "da_launch.h"

namespace da {

// Request b with `rows` query rows becomes the requests b * rows + i,
// i < rows, of lengths max(0, L_b - rows + 1 + i), all over request b's pages:
// the causal mask among a request's new rows is then a plain history length.
struct RowsArgs {
    const int32_t* seq_lens;    // [batch]
    const int32_t* page_table;  // [batch][max_pages]
    int32_t* lens_out;          // [batch * rows]
    int32_t* table_out;         // [batch * rows][max_pages]; entries past a row's pages untouched
    int batch, rows, page_size, max_pages;
    // rows per expanded request: request (b, k) holds rows [k block,
    // (k + 1) block) of request b; 1 = every row a request of its own
    int block;
    // 0: expanded request b * rows + i is row i of request b; 1: it is
    // i * batch + b (row-major over the rows, so that the same row of every
    // request forms one contiguous half, third, ... of the expanded batch)
    int row_major;
};

hipError_t launch_rows_expand(const RowsArgs& a, hipStream_t s);

}  // namespace da
