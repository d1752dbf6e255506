/*
 * decode_attn.h - paged decode attention on AMD MI355X (gfx950), C ABI.
 *
 * One call computes one decode step of one attention layer for a batch of
 * variable-length requests.  Each request brings a single query row per head
 * and attends over its whole cached history, which lives in fixed-size pages
 * reached through a per-request page table.
 *
 * Sources for the operation (titles of the pages it is defined from):
 *  - one query token per request, the full KV cache of its context read, a
 *    memory-bound operator: "OpWeave: Flexible Operator Disaggregation for
 *    Heterogeneous LLM Serving", App. A.2 (Execution-regime assumptions);
 *  - every query head attends the complete history, the result defined up to
 *    floating-point reduction order: "SPLASH: Switching Parallel Layouts of
 *    Attention with Seamless Handoff for LLM Serving", §3 (Computation);
 *    a query reads its complete causal prefix, one query row per request in
 *    decode: SPLASH §4.1 (Handoff) and §4.2;
 *  - grouped-query heads and the head-shared MLA latent: SPLASH §1 and §2;
 *    latent width 512 + 64 = 576: "Analytical Provisioning for Attention-FFN
 *    Disaggregated LLM Serving under Stochastic Workloads", App. B.1;
 *  - the KV history grows by one appended token per step and is read whole:
 *    Analytical Provisioning §2 and Fig. 1; paged KV-cache management:
 *    OpWeave §8; FP8 E4M3 KV with scales: SPLASH App. C.1 and App. B.1.
 *
 * Semantics (for request b, query head h, L = seq_lens[b]):
 *     j = h / (Hq / Hkv)                        (GQA: contiguous head groups)
 *     s_t = scale * <q[b][h], k_t>,  t < L      (k_t: KV head j's key of token t)
 *     out[b][h] = sum_t exp(s_t) v_t / sum_t exp(s_t)
 *     lse[b][h] = ln sum_t exp(s_t)             (natural log, fp32)
 *     L == 0  ->  out = 0, lse = -inf
 * Token t lives in physical page page_table[b][t / P], slot t % P.  Slots at
 * or past L in the last page are never read into the result (they may hold
 * NaN); page_table entries at or past ceil(L / P) are never read.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers of the current HIP device,
 *    dense and row-major as documented; descriptors are HOST pointers.
 *  - The caller owns every buffer; the library never frees or keeps them.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t, NULL for
 *    the null stream).  Nothing reads device data on the host; there is no
 *    host synchronisation on the path.
 *  - Every host-detectable error returns a negative status BEFORE any HIP
 *    call is made; a HIP launch failure returns DA_ERR_HIP.  Data-dependent
 *    preconditions (page ids < num_pages, L <= max_pages_per_seq * P,
 *    L >= 0) are the caller's: the kernels do not check them.
 *  - Results are bitwise deterministic for identical inputs on one device.
 *  - The library keeps one workspace per (device, stream), grown with
 *    hipMalloc the first time a shape needs more; growing synchronises the
 *    device.  Calls on one stream are ordered; calls on different streams
 *    use different workspaces.  The _ws entry points take a workspace the
 *    caller owns instead and allocate nothing.
 *  - Once a stream's workspace is large enough (after one call of that size
 *    on it), a call only enqueues kernel launches on the stream: it can be
 *    captured into a HIP graph and replayed (the graph keeps the workspace's
 *    address, so no larger call may run on that stream meanwhile).
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DA_OK               0
#define DA_ERR_NULL        -1   /* a required pointer is NULL */
#define DA_ERR_SHAPE       -2   /* sizes inconsistent or out of range */
#define DA_ERR_DTYPE       -3   /* unknown dtype tag, or q/kv combination not offered */
#define DA_ERR_UNSUPPORTED -4   /* valid request outside what the kernels implement */
#define DA_ERR_WORKSPACE   -5   /* workspace could not be allocated */
#define DA_ERR_HIP         -6   /* a HIP call failed; see decode_attn_last_hip_error() */
#define DA_ERR_DATA        -7   /* decode_attn_validate_inputs: device data breaks a precondition */
#define DA_ERR_SCRATCH     -8   /* decode_attn_paged_noalloc: the call needs more than its static scratch */

/* storage dtype tags */
#define DA_F32       0          /* IEEE binary32 */
#define DA_BF16      1          /* bfloat16, stored as 16-bit patterns */
#define DA_FP8_E4M3  2          /* OCP fp8 E4M3FN (bias 7, max 448, no inf) */

/*
 * Paged GQA / MQA / MHA cache description.
 *
 * kv_pages layout: [num_pages][2][num_kv_heads][page_size][head_dim] of
 * kv_dtype; index 0 of the second axis holds keys, 1 values.  Each
 * (page, K|V, head) block is page_size * head_dim contiguous elements,
 * row-major [slot][dim], except the V blocks of an fp8 cache: those are kept
 * in tiles of 16 slots (16 * head_dim bytes each, in slot order), and within
 * a tile, with DL = head_dim / 16, the code of slot s (0..15) and dim d sits
 * at byte 1024 * ((d % DL) / 4) + 256 * (s / 4) + 16 * (d / DL) + 4 * (d % 4)
 * + s % 4, so that the codes of four consecutive slots for one dim are
 * adjacent (the layout the matrix-core kernel reads with 16-byte loads).
 * decode_kv_append writes and paged_kv_gather reads this layout.
 * q: [batch][num_q_heads][head_dim] of q_dtype; out: same shape and dtype.
 * lse: [batch][num_q_heads] fp32.  page_table: int32 [batch][max_pages_per_seq].
 * seq_lens: int32 [batch].
 *
 * Offered: head_dim in {64, 128}; page_size 16, 32, 64, 128 or 256 (the
 * kernels walk 16-token tiles of a page); num_q_heads / num_kv_heads from
 * 1 to 16 (a kernel takes at most 16 (row, head) pairs per KV head on the
 * matrix cores and 8 on the vector ALUs; more query rows than that run in
 * row blocks, see decode_attn_paged_rows); group sizes that are not a power
 * of two, and groups of 16, need bf16 queries (matrix cores); (q_dtype, kv_dtype) in
 * {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3)}.  For fp8, k_scale and v_scale are device fp32
 * [num_kv_heads]; a stored code x of KV head j means e4m3(x) * scale[j].
 *
 * Kernels: bf16 queries with 2 to 16 query heads (or, with several query
 * rows, row x head pairs) per KV head run on the matrix cores (scores and
 * values as MFMA products, softmax weights computed in fp32 and split into
 * two bf16 terms for the value product); fp8 caches run there for every
 * group size, and so do groups that are not a power of two; fp32 queries
 * and a single bf16 query head per KV head on the vector ALUs.  Both
 * give the same semantics and the same tolerances; kv_pages must be 16-byte
 * aligned on the matrix-core path.
 *
 * workers: number of workers, 0 selects the library default (one per resident
 * wavefront; for fp8 caches two workgroups of four wavefronts per CU, fewer
 * than fit, which measured faster).  A worker is one wavefront that
 * processes one contiguous share
 * of all (request, KV head, page) units; see decode_attn_plan for the rule.
 * Limits: batch <= 8192, workers <= 16384.
 */
typedef struct da_paged_desc {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages_per_seq;
    int32_t q_dtype;
    int32_t kv_dtype;
    int32_t workers;
    const float* k_scale;
    const float* v_scale;
} da_paged_desc;

/*
 * Absorbed MLA cache description: one head-shared bf16 latent of latent_dim
 * values per token (576 = 512 + 64); every head's key is the whole latent and
 * its value the first v_dim (512) values.
 * kv_pages: bf16 [num_pages][page_size][latent_dim]; q: bf16
 * [batch][num_heads][latent_dim] (already absorbed and roped); out: bf16
 * [batch][num_heads][v_dim]; lse: fp32 [batch][num_heads].
 * Offered: latent_dim 576, v_dim 512, page_size a multiple of 32 up to 256,
 * num_heads in {16, 32, 64, 128}.  workers: number of workgroups (0 = one per
 * compute unit); each processes one contiguous share of all (request, page)
 * units.  Limits: batch <= 8192, workers <= 2048.
 */
typedef struct da_mla_desc {
    int32_t batch;
    int32_t num_heads;
    int32_t latent_dim;
    int32_t v_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages_per_seq;
    int32_t workers;
} da_mla_desc;

/*
 * decode_attn_paged - one decode step of paged grouped-query attention.
 *   desc        host; shapes and dtypes as above.
 *   q           device, [B][Hq][D] q_dtype.
 *   kv_pages    device, [num_pages][2][Hkv][P][D] kv_dtype.
 *   page_table  device, int32 [B][max_pages_per_seq].
 *   seq_lens    device, int32 [B]; history length including this step's token.
 *   scale       multiplies q.k before the (natural) softmax.
 *   out         device, [B][Hq][D] q_dtype (written).
 *   lse         device, fp32 [B][Hq] (written), or NULL to skip it.
 *   stream      hipStream_t.
 * Returns DA_OK or a negative status.
 */
int decode_attn_paged(const da_paged_desc* desc, const void* q, const void* kv_pages,
                      const int32_t* page_table, const int32_t* seq_lens, float scale,
                      void* out, float* lse, void* stream);

/*
 * decode_attn_paged_rows - decode_attn_paged with q_rows query rows per
 * request: a request's query rows in a step are one in plain decode and more
 * with multi-token prediction (MTP depth 1 gives 2) or a short prefill chunk
 * ("SPLASH", §4.2 Transition-aware scheduling, the rows q_i of each request;
 * "Analytical Provisioning", App. B.1).  The rows are the last q_rows tokens
 * of each history, already appended: row i sees positions
 * t <= seq_lens[b] - q_rows + i (causal among the new rows, older history
 * whole).  A row that sees no position (seq_lens[b] < q_rows - i) gets
 * out = 0 and lse = -inf.
 *   q_rows      1 .. 16.  When q_rows * (Hq / Hkv) exceeds a kernel's tile
 *               (16 pairs on the matrix cores, 8 on the vector ALUs), the
 *               rows run in blocks of the largest divisor of q_rows that
 *               fits, each block a request of its own over the same pages
 *               (the pages are then read once per block, and batch *
 *               blocks must stay within the batch limit; the workspace holds
 *               the blocks' lengths and page tables).
 *   q           device, [B][q_rows][Hq][D] q_dtype.
 *   out         device, [B][q_rows][Hq][D] q_dtype (written).
 *   lse         device, fp32 [B][q_rows][Hq] (written), or NULL.
 * Other arguments, layouts and errors as decode_attn_paged; each K/V page is
 * read once for all rows of a block.
 */
int decode_attn_paged_rows(const da_paged_desc* desc, int32_t q_rows, const void* q, const void* kv_pages,
                           const int32_t* page_table, const int32_t* seq_lens, float scale,
                           void* out, float* lse, void* stream);

/*
 * decode_attn_mla - one decode step of absorbed MLA attention over the
 * head-shared latent.  Arguments as decode_attn_paged with the MLA layouts.
 */
int decode_attn_mla(const da_mla_desc* desc, const void* q, const void* kv_pages,
                    const int32_t* page_table, const int32_t* seq_lens, float scale,
                    void* out, float* lse, void* stream);

/*
 * decode_attn_mla_rows - decode_attn_mla with q_rows query rows per request
 * (the DeepSeek-V3 configuration decodes with multi-token prediction of depth
 * 1, two rows per request: "Analytical Provisioning", App. B.1; a request's
 * query rows q_i: "SPLASH", §4.2).  Row i of request b sees latent positions
 * t <= seq_lens[b] - q_rows + i; a row that sees none gets out = 0, lse = -inf.
 *   q_rows      >= 1, with batch * q_rows <= 8192.
 *   q           device, bf16 [B][q_rows][heads][576].
 *   out         device, bf16 [B][q_rows][heads][512] (written).
 *   lse         device, fp32 [B][q_rows][heads] (written), or NULL.
 * Each row runs as a request of its own over request b's pages (a small
 * kernel writes the rows' lengths and page tables into the library's
 * workspace first), so the latent is read once per row.  Other arguments and
 * errors as decode_attn_mla.
 */
int decode_attn_mla_rows(const da_mla_desc* desc, int32_t q_rows, const void* q, const void* kv_pages,
                         const int32_t* page_table, const int32_t* seq_lens, float scale,
                         void* out, float* lse, void* stream);
/*
 * decode_kv_append - write this step's new token into each request's paged
 * history (the history grows by one token per decode step and is then read
 * whole: Analytical Provisioning §2 and Fig. 1; paged KV-cache management:
 * OpWeave §8; FP8 E4M3 KV with scales: SPLASH App. C.1 and App. B.1).
 *   desc        host; the same description as decode_attn_paged; q_dtype is
 *               the dtype of k_new and v_new.
 *   k_new       device, [B][Hkv][D] q_dtype (16-byte aligned for fp32, 8 for bf16).
 *   v_new       device, [B][Hkv][D] q_dtype.
 *   kv_pages    device, [num_pages][2][Hkv][P][D] kv_dtype; for each request
 *               with positions[b] = t >= 0 and each KV head j, the slot of
 *               token t (page page_table[b][t / P], slot t % P) is written;
 *               nothing else is touched.
 *   page_table  device, int32 [B][max_pages_per_seq].
 *   positions   device, int32 [B]: the token index of the new token (the
 *               history length before this step); negative: no append.
 *   stream      hipStream_t.
 * Values: same dtype as the cache -> copied bit for bit.  bf16 into an fp8
 * cache -> y = x / scale[j] computed in fp32, stored as the e4m3fn code
 * nearest to y (ties to the even code), |y| > 448 saturating to +-448 and
 * NaN stored as 0x7F (k_scale for K, v_scale for V).
 * Data-dependent preconditions (t < max_pages_per_seq * P, the page ids
 * read valid, no two requests writing one slot) are the caller's.
 * Returns DA_OK or a negative status.
 */
int decode_kv_append(const da_paged_desc* desc, const void* k_new, const void* v_new, void* kv_pages,
                     const int32_t* page_table, const int32_t* positions, void* stream);
/*
 * decode_kv_append_mla - the same for the absorbed-MLA cache: latent_new
 * device bf16 [B][latent_dim] (16-byte aligned) is copied into slot t % P of
 * page page_table[b][t / P] of kv_pages bf16 [num_pages][P][latent_dim].
 */
int decode_kv_append_mla(const da_mla_desc* desc, const void* latent_new, void* kv_pages,
                         const int32_t* page_table, const int32_t* positions, void* stream);

/*
 * decode_attn_plan - run the split-KV planner that the attention kernels
 * execute in-kernel, alone, and write what it decides (for tests and tools).
 * The rule: stream (b, j), j < units, owns ceil(seq_lens[b] / page_size) page
 * units (the GQA kernels plan in 16-token tiles whatever their cache's page
 * size, with units = num_kv_heads: pass page_size 16 to reproduce their
 * plan; the MLA kernel plans in its pages, with units = 1); streams are
 * ordered b-major; W is the total; A = min(workers, W)
 * workers are active and worker g < A takes units [floor(g*W/A),
 * floor((g+1)*W/A)).  The step ends with its slowest worker, so the largest
 * share is what the rule minimises ("Analytical Provisioning for Attention-FFN
 * Disaggregated LLM Serving under Stochastic Workloads", §3.3).
 *   units        number of KV heads (GQA) or 1 (MLA).
 *   active       device int32 [1]: A.
 *   cuts         device int32 [workers + 1]: the first unit of each worker,
 *                W for g >= A.
 *   cursors      device int32 [workers + 1][4]: (request, unit, page, 0) of
 *                each cut, (batch, 0, 0, 0) where the cut is W.
 *   first_worker device int32 [batch * units]: worker holding the first piece
 *                of each stream, -1 for empty streams.
 *   piece_count  device int32 [batch * units]: number of workers the stream
 *                is split over (0 for empty streams).
 * Asynchronous on `stream`.  Returns DA_ERR_NULL / DA_ERR_SHAPE /
 * DA_ERR_UNSUPPORTED (batch > 8192, workers > 16384) before any launch.
 */
int decode_attn_plan(int32_t batch, const int32_t* seq_lens, int32_t page_size, int32_t units,
                     int32_t workers, int32_t* active, int32_t* cuts, int32_t* cursors,
                     int32_t* first_worker, int32_t* piece_count, void* stream);

/*
 * paged_kv_gather - copy every live token of the paged cache, through the same
 * address function the attention kernels use, into a dense array (a bitwise
 * copy, no arithmetic).  GQA (mla == 0): dense is
 * [batch][max_pages_per_seq*page_size][2][Hkv][D] of kv_dtype; MLA (mla == 1,
 * desc fields: num_kv_heads = 1, head_dim = latent_dim): dense is
 * [batch][max_pages_per_seq*page_size][latent_dim].  Rows t >= L are left
 * untouched.  Asynchronous on `stream`.
 */
int paged_kv_gather(const da_paged_desc* desc, int32_t mla, const void* kv_pages,
                    const int32_t* page_table, const int32_t* seq_lens, void* dense, void* stream);

/*
 * Caller-owned workspace (for callers that allocate up front: stream or graph
 * capture, several streams sharing no library state).
 *
 * decode_attn_workspace_size: bytes of device workspace one call of the GQA
 * path (gqa non-NULL) or the MLA path (mla non-NULL; exactly one of them)
 * with q_rows query rows per request needs on the current device, for these
 * descriptor values (batch, heads, dims, page size, max_pages_per_seq and
 * workers; a workers value of 0 takes the device default).  Host query, no
 * device work; 0 bytes for batch 0.  Returns the descriptor's own errors
 * (DA_ERR_SHAPE / DA_ERR_DTYPE / DA_ERR_UNSUPPORTED) or DA_ERR_NULL.
 *
 * decode_attn_paged_ws / decode_attn_mla_ws: decode_attn_paged_rows /
 * decode_attn_mla_rows (q_rows = 1 is the single-row call, bitwise the same
 * result) with the workspace passed in: a device buffer of workspace_bytes,
 * 256-byte aligned, owned by the caller and not kept by the library.  The
 * library makes no allocation on this path.  Errors before any launch:
 * DA_ERR_NULL (workspace NULL while batch > 0), DA_ERR_SHAPE (misaligned),
 * DA_ERR_WORKSPACE (workspace_bytes below decode_attn_workspace_size), and
 * those of the allocating entry points.  The workspace needs no initial
 * value (each call writes what it later reads); it is in use until the call
 * completes on `stream`, so calls that may overlap need distinct workspaces.
 */
int decode_attn_workspace_size(const da_paged_desc* gqa_or_null, const da_mla_desc* mla_or_null, int32_t q_rows,
                               size_t* bytes);
int decode_attn_paged_ws(const da_paged_desc* desc, int32_t q_rows, const void* q, const void* kv_pages,
                         const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);
int decode_attn_mla_ws(const da_mla_desc* desc, int32_t q_rows, const void* q, const void* kv_pages,
                       const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attn_paged_noalloc - for callers that cannot allocate device memory
 * and cannot hand in a workspace either (code under stream or graph capture,
 * tight serving loops, harnesses that forbid allocation): decode_attn_paged_rows
 * (q_rows = 1 is decode_attn_paged) whose workspace is a fixed scratch array
 * the library holds in device memory, DA_NOALLOC_SCRATCH_BYTES per device.
 * Each device that runs the library keeps its own copy from the moment the
 * library's code is loaded onto it until the process ends.
 *   Arguments, layouts and results as decode_attn_paged_rows; the results are
 *   bitwise those of decode_attn_paged_ws with the same descriptor (workers
 *   included).
 *   Makes no hipMalloc / hipFree and calls no allocating library routine.
 *   Errors: those of decode_attn_paged_rows, plus DA_ERR_SCRATCH when
 *   decode_attn_workspace_size for this call exceeds DA_NOALLOC_SCRATCH_BYTES
 *   (before any launch; smaller batches or fewer workers fit), and DA_ERR_HIP
 *   if the scratch address cannot be obtained on the current device.
 * Every call on one device shares that device's scratch: calls that may
 * overlap in time on one device (different streams, or host threads without
 * ordering) race and give wrong results; order them on one stream.  Nothing
 * in the scratch needs an initial value (each call writes what it later
 * reads), so leftovers of an earlier call do no harm.
 */
#define DA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int decode_attn_paged_noalloc(const da_paged_desc* desc, int32_t q_rows, const void* q, const void* kv_pages,
                              const int32_t* page_table, const int32_t* seq_lens, float scale, void* out,
                              float* lse, void* stream);

/*
 * decode_attn_validate_inputs - debug check of the data-dependent
 * preconditions the kernels do not check: for every request b,
 * 0 <= seq_lens[b] <= max_pages_per_seq * page_size, and every page-table
 * entry the history uses (the first ceil(seq_lens[b] / page_size) of row b)
 * lies in [0, num_pages).  Exactly one of gqa / mla is non-NULL and gives
 * the sizes.  Copies seq_lens and page_table to the host and SYNCHRONISES
 * `stream`; not for the hot path.  Returns DA_OK, DA_ERR_DATA on the first
 * violation, or the descriptor / pointer errors.
 */
int decode_attn_validate_inputs(const da_paged_desc* gqa_or_null, const da_mla_desc* mla_or_null,
                                const int32_t* page_table, const int32_t* seq_lens, void* stream);

/*
 * decode_attn_kernel_name - the attention kernel a call with this descriptor
 * and q_rows query rows runs ("gqa_mfma_kernel", "gqa_attn_kernel",
 * "mla_wave_kernel" or "mla_attn_kernel"), as the same host checks and
 * choice decide it; NULL when the call would be refused.  Exactly one of
 * gqa / mla is non-NULL.  Host only: no device call, no allocation; the
 * string is static.
 */
const char* decode_attn_kernel_name(const da_paged_desc* gqa_or_null, const da_mla_desc* mla_or_null,
                                    int32_t q_rows);

/* default number of workers for each path on the current device (host query). */
int decode_attn_default_workers(const da_paged_desc* gqa_or_null, const da_mla_desc* mla_or_null,
                                int32_t* workers);

/*
 * Kernel timer (profiling aid).  decode_attn_timer_begin creates max_launches
 * start/stop event pairs for the calling thread on the current device; until
 * decode_attn_timer_end, each decode_attn_* call launches its main attention
 * kernel with hipExtLaunchKernel and the next pair, so the dispatch itself
 * records when that kernel starts and ends (no extra packets on the stream).
 * Calls beyond max_launches are not timed.  decode_attn_timer_end waits for
 * the recorded events, returns the summed kernel time in milliseconds and the
 * number of timed launches, and releases the events.
 */
/*
 * Kernel choice for profiling: with DA_GQA_VECTOR=1 in the environment when
 * the library first runs a GQA call, every group of up to 8 (row, head)
 * members takes the vector kernel, including the 4 to 8 member bf16 groups
 * that otherwise run on the matrix cores (fp8 caches always run on the
 * matrix cores).  Results stay within the same bounds; not for production
 * use.
 */
int decode_attn_timer_begin(int32_t max_launches);
int decode_attn_timer_end(double* total_ms, int32_t* launches);

/* human-readable text of a status code (static storage). */
const char* decode_attn_status_str(int status);

/* the last HIP error code seen by the library on this thread (0 if none). */
int decode_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DECODE_ATTN_H */
