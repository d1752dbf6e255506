// C-ABI layer: argument validation, workspace, kernel dispatch.
//
// Every check that can be made on the host runs before the first HIP call, so
// a bad call returns its status without touching the device.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/decode_attn.h"
#include "da_append.h"
#include "da_gqa_mfma.h"
#include "da_rows.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return DA_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

namespace da {
// Lets other translation units of the library record a failed HIP call for
// decode_attn_last_hip_error().
int hip_failure(hipError_t e) { return hip_fail(e); }
}  // namespace da

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace

// One buffer per (device, stream), carved into: the plan summary (W, active
// workers), the per-stream (first unit, pieces) records, and the partial slots
// of split streams: 2 * workers slots of [heads][dim] fp32 values and [heads]
// log2-sum-exps.  Nothing in it needs an initial value: every call writes what
// it later reads.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Returns a device buffer of at least `bytes` for (current device, stream).
int get_workspace(hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[{dev, stream}];
    if (ws.bytes < bytes) {
        size_t want = round_up(bytes + bytes / 4, 1 << 20);
        if (ws.ptr != nullptr) {
            // earlier calls on any stream may still read the old buffer
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return hip_fail(e);
            e = hipFree(ws.ptr);
            if (e != hipSuccess) return hip_fail(e);
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        e = hipMalloc(&ws.ptr, want);
        if (e != hipSuccess) {
            g_last_hip_error = static_cast<int>(e);
            ws.ptr = nullptr;
            return DA_ERR_WORKSPACE;
        }
        ws.bytes = want;
    }
    *out = ws.ptr;
    return DA_OK;
}

struct SplitBuffers {
    int2* plan_info;
    int2* stream_info;
    float* o_part;
    float* lse_part;
    int32_t* extra;         // extra_ints int32 values for the caller (multi-row expansion)
};

size_t split_layout(int streams, int G, int heads, int dim, char* base, SplitBuffers* sb, size_t extra_ints = 0) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* p = base ? base + off : nullptr;
        off = round_up(off + bytes, 256);
        return p;
    };
    SplitBuffers t;
    t.plan_info = reinterpret_cast<int2*>(take(sizeof(int2)));
    t.stream_info = reinterpret_cast<int2*>(take(sizeof(int2) * static_cast<size_t>(streams)));
    t.o_part = reinterpret_cast<float*>(take(sizeof(float) * 2 * static_cast<size_t>(G) * heads * dim));
    t.lse_part = reinterpret_cast<float*>(take(sizeof(float) * 2 * static_cast<size_t>(G) * heads));
    t.extra = extra_ints ? reinterpret_cast<int32_t*>(take(sizeof(int32_t) * extra_ints)) : nullptr;
    if (sb) *sb = t;
    return off;
}

// The 128-head MLA kernel keeps one slot per piece (index request + worker,
// below batch + workers) of raw [128][512] fp32 accumulators and [128] (max,
// sum) pairs, plus a [128][512] scratch area per worker.
size_t mla_wave_layout(int batch, int G, char* base, SplitBuffers* sb, float** tmp, size_t extra_ints = 0) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* p = base ? base + off : nullptr;
        off = round_up(off + bytes, 256);
        return p;
    };
    const size_t slots = static_cast<size_t>(batch) + G;
    const size_t tile = static_cast<size_t>(da::kMlaWaveHeads) * da::kMlaV;
    SplitBuffers t;
    t.plan_info = reinterpret_cast<int2*>(take(sizeof(int2)));
    t.stream_info = reinterpret_cast<int2*>(take(sizeof(int2) * static_cast<size_t>(batch)));
    t.o_part = reinterpret_cast<float*>(take(sizeof(float) * slots * tile));
    t.lse_part = reinterpret_cast<float*>(take(sizeof(float) * 2 * slots * da::kMlaWaveHeads));
    float* tp = reinterpret_cast<float*>(take(sizeof(float) * static_cast<size_t>(G) * tile));
    t.extra = extra_ints ? reinterpret_cast<int32_t*>(take(sizeof(int32_t) * extra_ints)) : nullptr;
    if (sb) *sb = t;
    if (tmp) *tmp = tp;
    return off;
}

// A workspace the caller owns (the _ws entry points): used as given, never
// grown; the library allocates nothing on that path.
struct CallerWorkspace {
    void* ptr;
    size_t bytes;
};

// Carves the buffers of one call out of the caller's workspace or the
// library's: `layout(base)` returns the bytes needed (base null) or fills the
// pointers.
template <class Layout>
int get_buffers(hipStream_t s, const CallerWorkspace* cws, Layout&& layout) {
    const size_t need = layout(nullptr);
    void* base = nullptr;
    if (cws != nullptr) {
        if (cws->ptr == nullptr) return DA_ERR_NULL;
        if (!aligned(cws->ptr, 256)) return DA_ERR_SHAPE;
        if (cws->bytes < need) return DA_ERR_WORKSPACE;
        base = cws->ptr;
    } else {
        int st = get_workspace(s, need, &base);
        if (st != DA_OK) return st;
    }
    layout(static_cast<char*>(base));
    return DA_OK;
}

int get_split_buffers(hipStream_t s, int streams, int G, int heads, int dim, SplitBuffers* sb,
                      size_t extra_ints = 0, const CallerWorkspace* cws = nullptr) {
    const size_t need = split_layout(streams, G, heads, dim, nullptr, nullptr, extra_ints);
    void* base = nullptr;
    if (cws != nullptr) {
        if (cws->ptr == nullptr) return DA_ERR_NULL;
        if (!aligned(cws->ptr, 256)) return DA_ERR_SHAPE;
        if (cws->bytes < need) return DA_ERR_WORKSPACE;
        base = cws->ptr;
    } else {
        int st = get_workspace(s, need, &base);
        if (st != DA_OK) return st;
    }
    split_layout(streams, G, heads, dim, static_cast<char*>(base), sb, extra_ints);
    return DA_OK;
}

// ---------------------------------------------------------------- kernel timer

struct Timer {
    bool on = false;
    size_t next = 0;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};
thread_local Timer g_timer;

// Events for the next main-kernel launch of this thread (none if the timer is off or full).
da::KernelEvents next_kernel_events() {
    da::KernelEvents k;
    if (g_timer.on && g_timer.next < g_timer.ev.size()) {
        k.start = g_timer.ev[g_timer.next].first;
        k.stop = g_timer.ev[g_timer.next].second;
        ++g_timer.next;
    }
    return k;
}

void timer_release() {
    for (auto& p : g_timer.ev) {
        (void)hipEventDestroy(p.first);
        (void)hipEventDestroy(p.second);
    }
    g_timer.ev.clear();
    g_timer.next = 0;
    g_timer.on = false;
}

// ---------------------------------------------------------------- device facts

struct DeviceInfo {
    int num_cus = 0;
    // workers per CU of each kernel variant (occupancy queries), by variant key
    std::map<uint32_t, int> per_cu;
};
std::mutex g_dev_mutex;
std::map<int, DeviceInfo> g_dev;

int device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceInfo& d = g_dev[dev];
    if (d.num_cus == 0) {
        e = hipDeviceGetAttribute(&d.num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e);
    }
    *cus = d.num_cus;
    return DA_OK;
}

// Compute units of the current device and the workers per CU of the variant
// named by `key`, which `query` reports (0 = no such variant).  Both are
// fixed for a device and a build, so each is asked once per process and
// device; a failed query (0) is not kept.
template <typename Query>
int device_workers(uint32_t key, Query query, int* cus, int* per_cu) {
    int st = device_cus(cus);
    if (st != DA_OK) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    {
        std::lock_guard<std::mutex> lock(g_dev_mutex);
        auto& m = g_dev[dev].per_cu;
        auto it = m.find(key);
        if (it != m.end()) {
            *per_cu = it->second;
            return DA_OK;
        }
    }
    const int v = query();
    if (v > 0) {
        std::lock_guard<std::mutex> lock(g_dev_mutex);
        g_dev[dev].per_cu[key] = v;
    }
    *per_cu = v;
    return DA_OK;
}

// ---------------------------------------------------------------- validation

int check_paged(const da_paged_desc* d) {
    if (d == nullptr) return DA_ERR_NULL;
    if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->page_size < 1 ||
        d->num_pages < 1 || d->max_pages_per_seq < 1 || d->workers < 0)
        return DA_ERR_SHAPE;
    if (d->num_q_heads % d->num_kv_heads != 0) return DA_ERR_SHAPE;
    const bool qok = d->q_dtype == DA_F32 || d->q_dtype == DA_BF16;
    const bool kok = d->kv_dtype == DA_F32 || d->kv_dtype == DA_BF16 || d->kv_dtype == DA_FP8_E4M3;
    if (!qok || !kok) return DA_ERR_DTYPE;
    const bool combo = (d->q_dtype == DA_F32 && d->kv_dtype == DA_F32) ||
                       (d->q_dtype == DA_BF16 && d->kv_dtype == DA_BF16) ||
                       (d->q_dtype == DA_BF16 && d->kv_dtype == DA_FP8_E4M3);
    if (!combo) return DA_ERR_DTYPE;
    const int group = d->num_q_heads / d->num_kv_heads;
    if (d->head_dim != 64 && d->head_dim != 128) return DA_ERR_UNSUPPORTED;
    // pages of 16 << k tokens: the kernels walk 16-token tiles
    if (d->page_size < 16 || d->page_size > 256 || (d->page_size & (d->page_size - 1)) != 0)
        return DA_ERR_UNSUPPORTED;
    // any group up to 16 query heads per KV head; groups that are not a power
    // of two run on the matrix-core kernel only, so they need bf16 queries
    if (group > 16) return DA_ERR_UNSUPPORTED;
    if ((group & (group - 1)) != 0 && d->q_dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
    if (d->batch > da::kMaxBatch || d->workers > da::kMaxWorkers) return DA_ERR_UNSUPPORTED;
    const int64_t units_bound =
        static_cast<int64_t>(d->num_kv_heads) * d->batch * d->max_pages_per_seq * (d->page_size / 16);
    if (units_bound >= (int64_t(1) << 31)) return DA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(d->max_pages_per_seq) * d->page_size >= (int64_t(1) << 31)) return DA_ERR_SHAPE;
    if (d->kv_dtype == DA_FP8_E4M3 && (d->k_scale == nullptr || d->v_scale == nullptr)) return DA_ERR_NULL;
    return DA_OK;
}

// Groups of 2 to 16 (row, head) members with bf16 queries run on the
// matrix-core kernel (gqa_mfma.hip): from 8 query heads per K/V page up the
// vector kernel is bound by its ALUs, and at 4 and 2 the matrix-core kernel
// measured 4 % faster (less vector work beside the loads; llama8b lengths,
// 8 KV heads: 127.8 against 132.6 us at 4, 125.6 against 130.5 us at 2).  A
// single member (one-row MHA) and fp32 queries run on the vector kernel
// (gqa.hip), equal or 0.6 % faster there; fp8 caches run on the matrix-core
// kernel for every group size.
//
// Profiling aid: DA_GQA_VECTOR=1 in the environment (read once per process)
// sends every group the vector kernel can take (up to 8 members) to it, so
// that both kernels can be measured on the same workload.
bool vector_forced() {
    static const bool forced = [] {
        const char* e = std::getenv("DA_GQA_VECTOR");
        return e != nullptr && e[0] == '1' && e[1] == '\0';
    }();
    return forced;
}

bool gqa_uses_mfma(const da_paged_desc* d, int q_rows) {
    const int want = q_rows * (d->num_q_heads / d->num_kv_heads);
    // fp8 caches keep their V blocks in tiles that only the matrix-core
    // kernel reads: every group size runs there
    if (d->kv_dtype == DA_FP8_E4M3) return d->q_dtype == DA_BF16 && want <= 16;
    // the vector kernel maps members to heads with shifts: powers of two only
    const int group = d->num_q_heads / d->num_kv_heads;
    if ((group & (group - 1)) != 0) return d->q_dtype == DA_BF16 && want <= 16;
    if (want <= 8 && vector_forced()) return false;
    return d->q_dtype == DA_BF16 && d->kv_dtype == DA_BF16 && want >= 2 && want <= 16;
}

// (row, head) members of one KV head's group in the GQA kernels: q_rows times
// the query heads per KV head, padded to a power of two; 0 when no kernel has
// that many (16 on the matrix-core kernel, 8 on the vector one).
int gqa_members(const da_paged_desc* d, int q_rows) {
    const int want = q_rows * (d->num_q_heads / d->num_kv_heads);
    int gs = 1;
    while (gs < want) gs <<= 1;
    return gs <= (gqa_uses_mfma(d, q_rows) ? 16 : 8) ? gs : 0;
}

int resolve_gqa_workers(const da_paged_desc* d, int members, bool mfma, int* G) {
    if (d->workers > 0) {
        *G = d->workers;
        return DA_OK;
    }
    const int group_log2 = __builtin_ctz(static_cast<unsigned>(d->num_q_heads / d->num_kv_heads));
    // variant key: kernel family, dtypes, head dim, members, group
    const uint32_t key = (mfma ? 1u : 0u) | (static_cast<uint32_t>(d->q_dtype) << 1) |
                         (static_cast<uint32_t>(d->kv_dtype) << 4) | (static_cast<uint32_t>(d->head_dim) << 7) |
                         (static_cast<uint32_t>(members) << 16) | (static_cast<uint32_t>(group_log2) << 24);
    int cus = 0, per_cu = 0;
    int st = device_workers(
        key,
        [&] {
            return mfma ? da::gqa_mfma_workers_per_cu(d->kv_dtype, d->head_dim)
                        : da::gqa_workers_per_cu(d->q_dtype, d->kv_dtype, d->head_dim, members, group_log2);
        },
        &cus, &per_cu);
    if (st != DA_OK) return st;
    if (per_cu <= 0) return DA_ERR_UNSUPPORTED;
    int g = cus * per_cu;
    if (g > da::kMaxWorkers) g = da::kMaxWorkers;
    *G = g;
    return DA_OK;
}

int check_mla(const da_mla_desc* d) {
    if (d == nullptr) return DA_ERR_NULL;
    if (d->batch < 0 || d->num_heads < 1 || d->latent_dim < 1 || d->v_dim < 1 || d->page_size < 1 ||
        d->num_pages < 1 || d->max_pages_per_seq < 1 || d->workers < 0)
        return DA_ERR_SHAPE;
    if (d->v_dim > d->latent_dim) return DA_ERR_SHAPE;
    if (d->latent_dim != da::kMlaLatent || d->v_dim != da::kMlaV) return DA_ERR_UNSUPPORTED;
    if (d->page_size % da::kMlaChunk != 0 || d->page_size > 256) return DA_ERR_UNSUPPORTED;
    if (!da::mla_heads_supported(d->num_heads)) return DA_ERR_UNSUPPORTED;
    if (d->batch > da::kMaxBatch || d->workers > da::kMlaMaxWorkers) return DA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(d->batch) * d->max_pages_per_seq >= (int64_t(1) << 31)) return DA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(d->max_pages_per_seq) * d->page_size >= (int64_t(1) << 31)) return DA_ERR_SHAPE;
    return DA_OK;
}

int resolve_mla_workers(const da_mla_desc* d, int* G) {
    if (d->workers > 0) {
        *G = d->workers;
        return DA_OK;
    }
    const bool wave = d->num_heads == da::kMlaWaveHeads;
    // variant keys above every GQA key (bit 31): the two MLA kernels
    const uint32_t key = (1u << 31) | (wave ? 1u : 0u);
    int cus = 0, per_cu = 0;
    int st = device_workers(
        key, [&] { return wave ? da::mla_wave_blocks_per_cu() : da::mla_blocks_per_cu(); }, &cus, &per_cu);
    if (st != DA_OK) return st;
    int g = wave ? cus * per_cu : cus * per_cu / da::mla_blocks_per_worker(d->num_heads);
    if (g <= 0) return DA_ERR_UNSUPPORTED;
    if (g > da::kMlaMaxWorkers) g = da::kMlaMaxWorkers;
    *G = g;
    return DA_OK;
}

// Query rows per attention call of a GQA step with q_rows rows: all of them
// when their (row, head) pairs fit a kernel's member tile, else the largest
// divisor of q_rows that does.  A step whose rows are split runs as
// batch * (q_rows / block) requests of block rows each, request-major
// (b * blocks + k holds rows [k block, (k + 1) block) of request b), so the
// q, out and lse rows of the expanded requests are those of [batch][q_rows]
// in place and the kernels need no mapping; each expanded request's history
// is cut where its last row's view ends.  0 when no block fits.
int gqa_row_block(const da_paged_desc* d, int q_rows) {
    for (int r = q_rows; r >= 1; --r)
        if (q_rows % r == 0 && gqa_members(d, r) != 0) return r;
    return 0;
}

// The descriptor of the attention calls of a GQA step (batch expanded when
// its rows run in blocks) and their rows per request; DA_OK or a status.
int gqa_call_shape(const da_paged_desc* d, int q_rows, da_paged_desc* call, int* block) {
    *block = gqa_row_block(d, q_rows);
    if (*block == 0) return DA_ERR_UNSUPPORTED;
    *call = *d;
    if (*block < q_rows) {
        const int64_t expanded = static_cast<int64_t>(d->batch) * (q_rows / *block);
        if (expanded > da::kMaxBatch) return DA_ERR_UNSUPPORTED;
        call->batch = static_cast<int32_t>(expanded);
        const int64_t units_bound =
            static_cast<int64_t>(call->num_kv_heads) * call->batch * call->max_pages_per_seq * (call->page_size / 16);
        if (units_bound >= (int64_t(1) << 31)) return DA_ERR_UNSUPPORTED;
    }
    return DA_OK;
}

// Workspace bytes of one call: the same checks, worker count and layout as
// gqa_step / mla_step, so that a buffer of this size is always enough.
int gqa_workspace_bytes(const da_paged_desc* d, int q_rows, size_t* bytes) {
    int st = check_paged(d);
    if (st != DA_OK) return st;
    if (q_rows < 1 || q_rows > 16) return q_rows < 1 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
    da_paged_desc cd;
    int block = 0;
    st = gqa_call_shape(d, q_rows, &cd, &block);
    if (st != DA_OK) return st;
    const int members = gqa_members(&cd, block);
    *bytes = 0;
    if (cd.batch == 0) return DA_OK;
    int G = 0;
    st = resolve_gqa_workers(&cd, members, gqa_uses_mfma(&cd, block), &G);
    if (st != DA_OK) return st;
    const size_t extra = block < q_rows ? static_cast<size_t>(cd.batch) * (1 + cd.max_pages_per_seq) : 0;
    *bytes = split_layout(cd.batch * cd.num_kv_heads, G, members, cd.head_dim, nullptr, nullptr, extra);
    return DA_OK;
}

int mla_workspace_bytes(const da_mla_desc* dd, int q_rows, size_t* bytes) {
    int st = check_mla(dd);
    if (st != DA_OK) return st;
    if (q_rows < 1) return DA_ERR_SHAPE;
    // rows run as batch * q_rows requests: form the product in 64 bits so that
    // no q_rows can wrap it into a small, valid-looking batch
    const int64_t expanded = static_cast<int64_t>(dd->batch) * q_rows;
    if (expanded > da::kMaxBatch) return DA_ERR_UNSUPPORTED;
    da_mla_desc rd = *dd;
    rd.batch = static_cast<int32_t>(expanded);
    if (static_cast<int64_t>(rd.batch) * rd.max_pages_per_seq >= (int64_t(1) << 31)) return DA_ERR_UNSUPPORTED;
    *bytes = 0;
    if (rd.batch == 0) return DA_OK;
    int G = 0;
    st = resolve_mla_workers(&rd, &G);
    if (st != DA_OK) return st;
    const size_t extra = q_rows > 1 ? static_cast<size_t>(rd.batch) * (1 + rd.max_pages_per_seq) : 0;
    *bytes = rd.num_heads == da::kMlaWaveHeads ? mla_wave_layout(rd.batch, G, nullptr, nullptr, nullptr, extra)
                                               : split_layout(rd.batch, G, rd.num_heads, rd.v_dim, nullptr, nullptr, extra);
    return DA_OK;
}

int gqa_step(const da_paged_desc* dd, int rows_total, const void* q, const void* kv_pages,
             const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse, void* stream,
             const CallerWorkspace* cws = nullptr) {
    int st = check_paged(dd);
    if (st != DA_OK) return st;
    if (rows_total < 1 || rows_total > 16) return rows_total < 1 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
    da_paged_desc cd;
    int q_rows = 0;                                   // rows per request of the attention call
    st = gqa_call_shape(dd, rows_total, &cd, &q_rows);
    if (st != DA_OK) return st;
    const da_paged_desc* d = &cd;
    const bool blocked = q_rows < rows_total;
    const int members = gqa_members(d, q_rows);
    const bool mfma = gqa_uses_mfma(d, q_rows);
    if (q == nullptr || kv_pages == nullptr || page_table == nullptr || seq_lens == nullptr || out == nullptr)
        return DA_ERR_NULL;
    const int elem_kv = d->kv_dtype == DA_F32 ? 4 : (d->kv_dtype == DA_BF16 ? 2 : 1);
    const size_t lane_bytes = static_cast<size_t>(d->head_dim / 16) * elem_kv;
    if (!aligned(kv_pages, lane_bytes < 16 && !mfma ? lane_bytes : 16) || !aligned(q, 16) || !aligned(out, 16) ||
        !aligned(lse, 4) || !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return DA_ERR_SHAPE;
    if (!(scale == scale)) return DA_ERR_SHAPE;
    if (d->batch == 0) return DA_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    int G = 0;
    st = resolve_gqa_workers(d, members, mfma, &G);
    if (st != DA_OK) return st;
    const int group = d->num_q_heads / d->num_kv_heads;
    const int group_log2 = __builtin_ctz(static_cast<unsigned>(group));
    const int streams = d->batch * d->num_kv_heads;
    SplitBuffers sb;
    const size_t extra = blocked ? static_cast<size_t>(d->batch) * (1 + d->max_pages_per_seq) : 0;
    st = get_split_buffers(s, streams, G, members, d->head_dim, &sb, extra, cws);
    if (st != DA_OK) return st;
    if (blocked) {
        da::RowsArgs ra{};
        ra.seq_lens = seq_lens;
        ra.page_table = page_table;
        ra.lens_out = sb.extra;
        ra.table_out = sb.extra + d->batch;
        ra.batch = dd->batch;
        ra.rows = rows_total;
        ra.block = q_rows;
        ra.page_size = d->page_size;
        ra.max_pages = d->max_pages_per_seq;
        ra.row_major = 0;
        hipError_t e = da::launch_rows_expand(ra, s);
        if (e != hipSuccess) return hip_fail(e);
        seq_lens = ra.lens_out;
        page_table = ra.table_out;
    }

    da::GqaArgs ga{};
    ga.q = q;
    ga.kv = kv_pages;
    ga.page_table = page_table;
    ga.seq_lens = seq_lens;
    ga.k_scale = d->k_scale;
    ga.v_scale = d->v_scale;
    ga.scale_log2 = scale * 1.4426950408889634f;
    ga.batch = d->batch;
    ga.q_heads = d->num_q_heads;
    ga.kv_heads = d->num_kv_heads;
    ga.page_size = d->page_size;
    ga.tile_shift = __builtin_ctz(static_cast<unsigned>(d->page_size)) - 4;
    ga.max_pages = d->max_pages_per_seq;
    ga.workers = G;
    ga.q_rows = q_rows;
    ga.group_log2 = group_log2;
    ga.plan_info = sb.plan_info;
    ga.stream_info = sb.stream_info;
    ga.out = out;
    ga.lse = lse;
    ga.o_part = sb.o_part;
    ga.lse_part = sb.lse_part;
    hipError_t e = mfma ? da::launch_gqa_mfma(d->kv_dtype, d->head_dim, ga, s, next_kernel_events())
                        : da::launch_gqa(d->q_dtype, d->kv_dtype, d->head_dim, members, ga, s, next_kernel_events());
    if (e != hipSuccess) return hip_fail(e);

    da::MergeArgs ma{};
    ma.seq_lens = seq_lens;
    ma.plan_info = sb.plan_info;
    ma.stream_info = sb.stream_info;
    ma.o_part = sb.o_part;
    ma.lse_part = sb.lse_part;
    ma.out = out;
    ma.lse = lse;
    ma.units = d->num_kv_heads;
    ma.group = members;
    ma.dim = d->head_dim;
    ma.rows = q_rows;
    ma.heads_per_unit = group;
    // Streams split into about two pieces or fewer are merged by one
    // workgroup for all the heads of their group (fewer, fuller workgroups;
    // most of them return at once); more deeply split streams by one
    // workgroup per head, so that their pieces spread over more lanes, and
    // streams of more than 16 pieces (few long requests) also by column
    // chunks, down to 4 float4 columns per workgroup, so that each of a
    // workgroup's threads folds about four pieces.  Full 16-member groups
    // split in up to 16 pieces merge two heads per workgroup (llama8b lengths
    // at 128/8 heads: 142.0 against 145.5 us per step with one head; at 4 and
    // 8 members one head measured best).
    const int pieces = ga.workers / (streams > 0 ? streams : 1);
    ma.heads_per_block = pieces <= 2 && members * d->head_dim <= 4 * 128 ? members : (members >= 16 && pieces <= 16 ? 2 : 1);
    ma.col_chunks = 1;
    if (ma.heads_per_block == 1 && pieces > 16) {
        const int c4 = d->head_dim / 4;
        while (ma.col_chunks * 4 < c4 && (c4 / ma.col_chunks) * pieces > 4 * 128) ma.col_chunks *= 2;
    }
    ma.out_is_bf16 = d->q_dtype == DA_BF16;
    e = da::launch_merge(ma, streams, s);
    if (e != hipSuccess) return hip_fail(e);
    return DA_OK;
}

// One MLA step with q_rows query rows per request.  Several rows run as
// batch * q_rows requests (rows.hip writes their lengths and page tables into
// the workspace); q, out and lse [batch][q_rows][heads][...] are already laid
// out as those requests.
int mla_step(const da_mla_desc* dd, int q_rows, const void* q, const void* kv_pages, const int32_t* page_table,
             const int32_t* seq_lens, float scale, void* out, float* lse, void* stream,
             const CallerWorkspace* cws = nullptr) {
    int st = check_mla(dd);
    if (st != DA_OK) return st;
    if (q_rows < 1) return DA_ERR_SHAPE;
    // rows run as batch * q_rows requests: form the product in 64 bits so that
    // no q_rows can wrap it into a small, valid-looking batch
    const int64_t expanded = static_cast<int64_t>(dd->batch) * q_rows;
    if (expanded > da::kMaxBatch) return DA_ERR_UNSUPPORTED;
    da_mla_desc rd = *dd;
    rd.batch = static_cast<int32_t>(expanded);
    if (static_cast<int64_t>(rd.batch) * rd.max_pages_per_seq >= (int64_t(1) << 31)) return DA_ERR_UNSUPPORTED;
    const da_mla_desc* d = &rd;
    if (q == nullptr || kv_pages == nullptr || page_table == nullptr || seq_lens == nullptr || out == nullptr)
        return DA_ERR_NULL;
    if (!aligned(kv_pages, 16) || !aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
        !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return DA_ERR_SHAPE;
    if (!(scale == scale)) return DA_ERR_SHAPE;
    if (d->batch == 0) return DA_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    int G = 0;
    st = resolve_mla_workers(d, &G);
    if (st != DA_OK) return st;
    SplitBuffers sb;
    float* tmp = nullptr;
    const bool wave = d->num_heads == da::kMlaWaveHeads;
    const size_t extra = q_rows > 1 ? static_cast<size_t>(d->batch) * (1 + d->max_pages_per_seq) : 0;
    if (wave)
        st = get_buffers(s, cws, [&](char* base) { return mla_wave_layout(d->batch, G, base, &sb, &tmp, extra); });
    else
        st = get_split_buffers(s, d->batch, G, d->num_heads, d->v_dim, &sb, extra, cws);
    if (st != DA_OK) return st;
    if (q_rows > 1) {
        da::RowsArgs ra{};
        ra.seq_lens = seq_lens;
        ra.page_table = page_table;
        ra.lens_out = sb.extra;
        ra.table_out = sb.extra + d->batch;
        ra.batch = dd->batch;
        ra.rows = q_rows;
        ra.block = 1;
        ra.page_size = d->page_size;
        ra.max_pages = d->max_pages_per_seq;
        // the 128-head kernel takes the rows row-major: the workers that run
        // a request's rows then sit G / q_rows apart, on the same XCD when
        // that distance is a multiple of 8, and stream the same latent pages
        // at about the same time (the second read meets the caches)
        ra.row_major = wave ? 1 : 0;
        hipError_t e = da::launch_rows_expand(ra, s);
        if (e != hipSuccess) return hip_fail(e);
        seq_lens = ra.lens_out;
        page_table = ra.table_out;
    }

    da::MlaArgs ma{};
    ma.q = q;
    ma.kv = kv_pages;
    ma.page_table = page_table;
    ma.seq_lens = seq_lens;
    ma.scale_log2 = scale * 1.4426950408889634f;
    ma.batch = d->batch;
    ma.heads = d->num_heads;
    ma.page_size = d->page_size;
    ma.max_pages = d->max_pages_per_seq;
    ma.workers = G;
    ma.plan_info = sb.plan_info;
    ma.stream_info = sb.stream_info;
    ma.out = out;
    ma.lse = lse;
    ma.o_part = sb.o_part;
    ma.lse_part = sb.lse_part;
    ma.o_tmp = tmp;
    ma.row_batch = dd->batch;
    ma.rows = wave ? q_rows : 1;
    if (wave) {
        hipError_t e = da::launch_mla_wave(ma, s, next_kernel_events());
        if (e != hipSuccess) return hip_fail(e);
        e = da::launch_mla_wave_merge(ma, s);
        if (e != hipSuccess) return hip_fail(e);
        return DA_OK;
    }
    hipError_t e = da::launch_mla(ma, s, next_kernel_events());
    if (e != hipSuccess) return hip_fail(e);

    da::MergeArgs mg{};
    mg.seq_lens = seq_lens;
    mg.plan_info = sb.plan_info;
    mg.stream_info = sb.stream_info;
    mg.o_part = sb.o_part;
    mg.lse_part = sb.lse_part;
    mg.out = out;
    mg.lse = lse;
    mg.units = 1;
    mg.group = d->num_heads;
    mg.dim = d->v_dim;
    mg.rows = 1;
    mg.heads_per_unit = d->num_heads;
    // four heads per merge workgroup: two float4 columns of [4][512] per
    // thread, both loaded in one pass (measured: 20.4 us against 20.8 with
    // eight heads and four columns per thread)
    mg.heads_per_block = d->num_heads >= 4 ? 4 : d->num_heads;
    mg.col_chunks = 1;
    mg.out_is_bf16 = 1;
    e = da::launch_merge(mg, d->batch, s);
    if (e != hipSuccess) return hip_fail(e);
    return DA_OK;
}

}  // namespace

extern "C" {

const char* decode_attn_status_str(int status) {
    switch (status) {
        case DA_OK: return "ok";
        case DA_ERR_NULL: return "a required pointer is NULL";
        case DA_ERR_SHAPE: return "sizes inconsistent or out of range";
        case DA_ERR_DTYPE: return "unknown dtype or dtype combination not offered";
        case DA_ERR_UNSUPPORTED: return "valid request outside what the kernels implement";
        case DA_ERR_WORKSPACE: return "workspace allocation failed";
        case DA_ERR_HIP: return "a HIP call failed";
        case DA_ERR_DATA: return "device data violates a precondition (length or page id out of range)";
        case DA_ERR_SCRATCH: return "the call needs more workspace than the no-allocation entry point's static scratch holds";
        default: return "unknown status";
    }
}

int decode_attn_last_hip_error(void) { return g_last_hip_error; }

int decode_attn_timer_begin(int32_t max_launches) {
    if (max_launches < 1 || max_launches > 1000000) return DA_ERR_SHAPE;
    timer_release();
    g_timer.ev.reserve(static_cast<size_t>(max_launches));
    for (int i = 0; i < max_launches; ++i) {
        hipEvent_t a = nullptr, b = nullptr;
        hipError_t e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        if (e != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            timer_release();
            return hip_fail(e);
        }
        g_timer.ev.emplace_back(a, b);
    }
    g_timer.on = true;
    return DA_OK;
}

int decode_attn_timer_end(double* total_ms, int32_t* launches) {
    if (total_ms == nullptr || launches == nullptr) return DA_ERR_NULL;
    double sum = 0.0;
    int st = DA_OK;
    for (size_t i = 0; i < g_timer.next; ++i) {
        hipError_t e = hipEventSynchronize(g_timer.ev[i].second);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timer.ev[i].first, g_timer.ev[i].second);
        if (e != hipSuccess) {
            st = hip_fail(e);
            break;
        }
        sum += ms;
    }
    *total_ms = sum;
    *launches = static_cast<int32_t>(g_timer.next);
    timer_release();
    return st;
}

int decode_attn_paged(const da_paged_desc* d, const void* q, const void* kv_pages, const int32_t* page_table,
                      const int32_t* seq_lens, float scale, void* out, float* lse, void* stream) {
    return gqa_step(d, 1, q, kv_pages, page_table, seq_lens, scale, out, lse, stream);
}

int decode_attn_paged_rows(const da_paged_desc* d, int32_t q_rows, const void* q, const void* kv_pages,
                           const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                           void* stream) {
    return gqa_step(d, q_rows, q, kv_pages, page_table, seq_lens, scale, out, lse, stream);
}

int decode_attn_mla(const da_mla_desc* d, const void* q, const void* kv_pages, const int32_t* page_table,
                    const int32_t* seq_lens, float scale, void* out, float* lse, void* stream) {
    return mla_step(d, 1, q, kv_pages, page_table, seq_lens, scale, out, lse, stream);
}

int decode_attn_mla_rows(const da_mla_desc* d, int32_t q_rows, const void* q, const void* kv_pages,
                         const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                         void* stream) {
    return mla_step(d, q_rows, q, kv_pages, page_table, seq_lens, scale, out, lse, stream);
}

int decode_attn_workspace_size(const da_paged_desc* gqa, const da_mla_desc* mla, int32_t q_rows, size_t* bytes) {
    if (bytes == nullptr || (gqa == nullptr) == (mla == nullptr)) return DA_ERR_NULL;
    return gqa != nullptr ? gqa_workspace_bytes(gqa, q_rows, bytes) : mla_workspace_bytes(mla, q_rows, bytes);
}

int decode_attn_paged_ws(const da_paged_desc* d, int32_t q_rows, const void* q, const void* kv_pages,
                         const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
    const CallerWorkspace cws{workspace, workspace_bytes};
    return gqa_step(d, q_rows, q, kv_pages, page_table, seq_lens, scale, out, lse, stream, &cws);
}

int decode_attn_mla_ws(const da_mla_desc* d, int32_t q_rows, const void* q, const void* kv_pages,
                       const int32_t* page_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
    const CallerWorkspace cws{workspace, workspace_bytes};
    return mla_step(d, q_rows, q, kv_pages, page_table, seq_lens, scale, out, lse, stream, &cws);
}

int decode_attn_validate_inputs(const da_paged_desc* gqa, const da_mla_desc* mla, const int32_t* page_table,
                                const int32_t* seq_lens, void* stream) {
    if ((gqa == nullptr) == (mla == nullptr) || page_table == nullptr || seq_lens == nullptr) return DA_ERR_NULL;
    int st = gqa != nullptr ? check_paged(gqa) : check_mla(mla);
    if (st != DA_OK) return st;
    const int B = gqa != nullptr ? gqa->batch : mla->batch;
    const int P = gqa != nullptr ? gqa->page_size : mla->page_size;
    const int max_pages = gqa != nullptr ? gqa->max_pages_per_seq : mla->max_pages_per_seq;
    const int num_pages = gqa != nullptr ? gqa->num_pages : mla->num_pages;
    if (B == 0) return DA_OK;
    std::vector<int32_t> lens(static_cast<size_t>(B));
    std::vector<int32_t> table(static_cast<size_t>(B) * max_pages);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(lens.data(), seq_lens, lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(table.data(), page_table, table.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
    for (int b = 0; b < B; ++b) {
        const int64_t L = lens[static_cast<size_t>(b)];
        if (L < 0 || L > static_cast<int64_t>(max_pages) * P) return DA_ERR_DATA;
        const int64_t used = (L + P - 1) / P;
        for (int64_t p = 0; p < used; ++p) {
            const int32_t id = table[static_cast<size_t>(b) * max_pages + p];
            if (id < 0 || id >= num_pages) return DA_ERR_DATA;
        }
    }
    return DA_OK;
}

int decode_kv_append(const da_paged_desc* d, const void* k_new, const void* v_new, void* kv_pages,
                     const int32_t* page_table, const int32_t* positions, void* stream) {
    int st = check_paged(d);
    if (st != DA_OK) return st;
    if (k_new == nullptr || v_new == nullptr || kv_pages == nullptr || page_table == nullptr || positions == nullptr)
        return DA_ERR_NULL;
    const size_t in_align = d->q_dtype == DA_F32 ? 16 : 8;
    if (!aligned(k_new, in_align) || !aligned(v_new, in_align) || !aligned(kv_pages, 16) ||
        !aligned(page_table, 4) || !aligned(positions, 4))
        return DA_ERR_SHAPE;
    if (d->batch == 0) return DA_OK;
    da::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.kv = kv_pages;
    a.page_table = page_table;
    a.positions = positions;
    a.k_scale = d->k_scale;
    a.v_scale = d->v_scale;
    a.batch = d->batch;
    a.kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.page_size = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.in_dtype = d->q_dtype;
    a.kv_dtype = d->kv_dtype;
    hipError_t e = da::launch_kv_append(a, static_cast<hipStream_t>(stream), next_kernel_events());
    return e == hipSuccess ? DA_OK : hip_fail(e);
}

int decode_kv_append_mla(const da_mla_desc* d, const void* latent_new, void* kv_pages, const int32_t* page_table,
                         const int32_t* positions, void* stream) {
    int st = check_mla(d);
    if (st != DA_OK) return st;
    if (latent_new == nullptr || kv_pages == nullptr || page_table == nullptr || positions == nullptr)
        return DA_ERR_NULL;
    if (!aligned(latent_new, 16) || !aligned(kv_pages, 16) || !aligned(page_table, 4) || !aligned(positions, 4))
        return DA_ERR_SHAPE;
    if (d->batch == 0) return DA_OK;
    da::AppendArgs a{};
    a.k_new = latent_new;
    a.kv = kv_pages;
    a.page_table = page_table;
    a.positions = positions;
    a.batch = d->batch;
    a.page_size = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.in_dtype = DA_BF16;
    a.kv_dtype = DA_BF16;
    hipError_t e = da::launch_kv_append_mla(a, static_cast<hipStream_t>(stream), next_kernel_events());
    return e == hipSuccess ? DA_OK : hip_fail(e);
}

int decode_attn_plan(int32_t batch, const int32_t* seq_lens, int32_t page_size, int32_t units, int32_t workers,
                     int32_t* active, int32_t* cuts, int32_t* cursors, int32_t* first_worker, int32_t* piece_count,
                     void* stream) {
    if (seq_lens == nullptr || active == nullptr || cuts == nullptr || cursors == nullptr ||
        first_worker == nullptr || piece_count == nullptr)
        return DA_ERR_NULL;
    if (batch < 1 || page_size < 1 || units < 1 || workers < 1) return DA_ERR_SHAPE;
    if (batch > da::kMaxBatch || workers > da::kMaxWorkers) return DA_ERR_UNSUPPORTED;
    if (!aligned(cursors, 16)) return DA_ERR_SHAPE;
    da::PlanArgs pa{};
    pa.seq_lens = seq_lens;
    pa.batch = batch;
    pa.page_size = page_size;
    pa.units = units;
    pa.workers = workers;
    pa.active = active;
    pa.cuts = cuts;
    pa.cursors = reinterpret_cast<int4*>(cursors);
    pa.first_worker = first_worker;
    pa.piece_count = piece_count;
    hipError_t e = da::launch_plan_debug(pa, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return DA_OK;
}

int paged_kv_gather(const da_paged_desc* d, int32_t mla, const void* kv_pages, const int32_t* page_table,
                    const int32_t* seq_lens, void* dense, void* stream) {
    if (d == nullptr || kv_pages == nullptr || page_table == nullptr || seq_lens == nullptr || dense == nullptr)
        return DA_ERR_NULL;
    if (d->batch < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->page_size < 1 || d->max_pages_per_seq < 1)
        return DA_ERR_SHAPE;
    if (mla != 0 && mla != 1) return DA_ERR_SHAPE;
    if (mla && d->num_kv_heads != 1) return DA_ERR_SHAPE;
    const int eb = d->kv_dtype == DA_F32 ? 4 : (d->kv_dtype == DA_BF16 ? 2 : (d->kv_dtype == DA_FP8_E4M3 ? 1 : 0));
    if (eb == 0) return DA_ERR_DTYPE;
    if ((d->head_dim * eb) % 4 != 0) return DA_ERR_UNSUPPORTED;
    if (!aligned(kv_pages, 4) || !aligned(dense, 4)) return DA_ERR_SHAPE;
    if (d->max_pages_per_seq > 65535 || d->batch > 65535) return DA_ERR_UNSUPPORTED;
    da::GatherArgs ga{};
    ga.kv = kv_pages;
    ga.page_table = page_table;
    ga.seq_lens = seq_lens;
    ga.dense = dense;
    ga.batch = d->batch;
    ga.kv_heads = d->num_kv_heads;
    ga.head_dim = d->head_dim;
    ga.page_size = d->page_size;
    ga.max_pages = d->max_pages_per_seq;
    ga.elem_bytes = eb;
    ga.mla = mla;
    hipError_t e = da::launch_gather(ga, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return DA_OK;
}

const char* decode_attn_kernel_name(const da_paged_desc* gqa, const da_mla_desc* mla, int32_t q_rows) {
    if ((gqa == nullptr) == (mla == nullptr) || q_rows < 1 || q_rows > 16) return nullptr;
    if (gqa != nullptr) {
        // the same checks and choice as gqa_step
        da_paged_desc cd;
        int block = 0;
        if (check_paged(gqa) != DA_OK || gqa_call_shape(gqa, q_rows, &cd, &block) != DA_OK) return nullptr;
        return gqa_uses_mfma(&cd, block) ? "gqa_mfma_kernel" : "gqa_attn_kernel";
    }
    if (check_mla(mla) != DA_OK) return nullptr;
    // the same limit as mla_step: rows run as batch * q_rows requests
    if (static_cast<int64_t>(mla->batch) * q_rows > da::kMaxBatch) return nullptr;
    return mla->num_heads == da::kMlaWaveHeads ? "mla_wave_kernel" : "mla_attn_kernel";
}

int decode_attn_default_workers(const da_paged_desc* gqa, const da_mla_desc* mla, int32_t* workers) {
    if (workers == nullptr || (gqa == nullptr) == (mla == nullptr)) return DA_ERR_NULL;
    int G = 0;
    int st = DA_OK;
    if (gqa != nullptr) {
        st = check_paged(gqa);
        if (st != DA_OK) return st;
        da_paged_desc dd = *gqa;
        dd.workers = 0;
        st = resolve_gqa_workers(&dd, gqa_members(&dd, 1), gqa_uses_mfma(&dd, 1), &G);
    } else {
        st = check_mla(mla);
        if (st != DA_OK) return st;
        da_mla_desc dd = *mla;
        dd.workers = 0;
        st = resolve_mla_workers(&dd, &G);
    }
    if (st != DA_OK) return st;
    *workers = G;
    return DA_OK;
}

}  // extern "C"
