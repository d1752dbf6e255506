/*
 * A native caller of libdecode_attn.so: plain C99 and the HIP runtime's C
 * API, no Python and no torch.  It reads one decode batch from a directory,
 * runs it through the C ABI twice on a stream of its own -- the allocating
 * entry point (decode_attn_paged / decode_attn_mla) and the workspace entry
 * point (decode_attn_paged_ws / decode_attn_mla_ws, with a buffer of
 * decode_attn_workspace_size bytes from hipMalloc) -- and writes both results
 * back for the test to check.
 *
 *   decode_caller DIR
 *
 * DIR/meta.txt, one line:
 *   gqa B Hq Hkv D P num_pages max_pages q_dtype kv_dtype scale
 *   mla B H latent_dim v_dim P num_pages max_pages scale
 * and the raw arrays, in the layouts decode_attn.h states: q.bin, kv.bin,
 * page_table.bin, seq_lens.bin (+ k_scale.bin, v_scale.bin for an fp8 cache).
 * Written: out.bin, lse.bin (first call), out_ws.bin, lse_ws.bin (second).
 * Exit status 0 on success, 1 on a HIP or I/O error, 2 when the library
 * returns an error status (its text is printed).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "decode_attn.h"

#define HIP_OK(call)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));               \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)

static void lib_ok(int status, const char* what) {
    if (status != DA_OK) {
        fprintf(stderr, "%s: status %d (%s)\n", what, status, decode_attn_status_str(status));
        exit(2);
    }
}

static char* path_of(const char* dir, const char* name) {
    size_t n = strlen(dir) + strlen(name) + 2;
    char* p = (char*)malloc(n);
    if (p == NULL) exit(1);
    snprintf(p, n, "%s/%s", dir, name);
    return p;
}

/* the whole file, which must hold exactly `want` bytes */
static void* read_exact(const char* dir, const char* name, size_t want) {
    char* p = path_of(dir, name);
    FILE* f = fopen(p, "rb");
    if (f == NULL) {
        fprintf(stderr, "cannot open %s\n", p);
        exit(1);
    }
    void* buf = malloc(want ? want : 1);
    size_t got = fread(buf, 1, want, f);
    int extra = fgetc(f);
    fclose(f);
    if (got != want || extra != EOF) {
        fprintf(stderr, "%s: expected %zu bytes\n", p, want);
        exit(1);
    }
    free(p);
    return buf;
}

static void write_all(const char* dir, const char* name, const void* buf, size_t n) {
    char* p = path_of(dir, name);
    FILE* f = fopen(p, "wb");
    if (f == NULL || fwrite(buf, 1, n, f) != n || fclose(f) != 0) {
        fprintf(stderr, "cannot write %s\n", p);
        exit(1);
    }
    free(p);
}

/* a device copy of DIR/name (`bytes` long) */
static void* upload(const char* dir, const char* name, size_t bytes) {
    void* h = read_exact(dir, name, bytes);
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return d;
}

static void download(const char* dir, const char* name, const void* d, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    write_all(dir, name, h, bytes);
    free(h);
}

static size_t dtype_bytes(int32_t t) { return t == DA_F32 ? 4 : t == DA_BF16 ? 2 : 1; }

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 1;
    }
    const char* dir = argv[1];
    char* mp = path_of(dir, "meta.txt");
    FILE* mf = fopen(mp, "r");
    if (mf == NULL) {
        fprintf(stderr, "cannot open %s\n", mp);
        return 1;
    }
    char kind[8] = {0};
    if (fscanf(mf, "%7s", kind) != 1) return 1;

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int is_mla = strcmp(kind, "mla") == 0;
    da_paged_desc g;
    da_mla_desc m;
    size_t q_bytes, kv_bytes, out_bytes, lse_bytes, pt_bytes, sl_bytes;
    float scale = 0.0f;
    void *k_scale = NULL, *v_scale = NULL;
    memset(&g, 0, sizeof g);
    memset(&m, 0, sizeof m);
    if (is_mla) {
        if (fscanf(mf, "%d %d %d %d %d %d %d %f", &m.batch, &m.num_heads, &m.latent_dim, &m.v_dim, &m.page_size,
                   &m.num_pages, &m.max_pages_per_seq, &scale) != 8)
            return 1;
        q_bytes = (size_t)m.batch * m.num_heads * m.latent_dim * 2;
        kv_bytes = (size_t)m.num_pages * m.page_size * m.latent_dim * 2;
        out_bytes = (size_t)m.batch * m.num_heads * m.v_dim * 2;
        lse_bytes = (size_t)m.batch * m.num_heads * 4;
        pt_bytes = (size_t)m.batch * m.max_pages_per_seq * 4;
        sl_bytes = (size_t)m.batch * 4;
    } else if (strcmp(kind, "gqa") == 0) {
        if (fscanf(mf, "%d %d %d %d %d %d %d %d %d %f", &g.batch, &g.num_q_heads, &g.num_kv_heads, &g.head_dim,
                   &g.page_size, &g.num_pages, &g.max_pages_per_seq, &g.q_dtype, &g.kv_dtype, &scale) != 10)
            return 1;
        q_bytes = (size_t)g.batch * g.num_q_heads * g.head_dim * dtype_bytes(g.q_dtype);
        kv_bytes = (size_t)g.num_pages * 2 * g.num_kv_heads * g.page_size * g.head_dim * dtype_bytes(g.kv_dtype);
        out_bytes = q_bytes;
        lse_bytes = (size_t)g.batch * g.num_q_heads * 4;
        pt_bytes = (size_t)g.batch * g.max_pages_per_seq * 4;
        sl_bytes = (size_t)g.batch * 4;
        if (g.kv_dtype == DA_FP8_E4M3) {
            k_scale = upload(dir, "k_scale.bin", (size_t)g.num_kv_heads * 4);
            v_scale = upload(dir, "v_scale.bin", (size_t)g.num_kv_heads * 4);
            g.k_scale = (const float*)k_scale;
            g.v_scale = (const float*)v_scale;
        }
    } else {
        fprintf(stderr, "unknown kind %s\n", kind);
        return 1;
    }
    fclose(mf);
    free(mp);

    void* q = upload(dir, "q.bin", q_bytes);
    void* kv = upload(dir, "kv.bin", kv_bytes);
    void* pt = upload(dir, "page_table.bin", pt_bytes);
    void* sl = upload(dir, "seq_lens.bin", sl_bytes);
    void *out = NULL, *lse = NULL, *out_ws = NULL, *lse_ws = NULL, *ws = NULL;
    HIP_OK(hipMalloc(&out, out_bytes));
    HIP_OK(hipMalloc(&lse, lse_bytes));
    HIP_OK(hipMalloc(&out_ws, out_bytes));
    HIP_OK(hipMalloc(&lse_ws, lse_bytes));

    size_t ws_bytes = 0;
    if (is_mla) {
        lib_ok(decode_attn_mla(&m, q, kv, (const int32_t*)pt, (const int32_t*)sl, scale, out, (float*)lse, stream),
               "decode_attn_mla");
        lib_ok(decode_attn_workspace_size(NULL, &m, 1, &ws_bytes), "decode_attn_workspace_size");
        HIP_OK(hipMalloc(&ws, ws_bytes));
        lib_ok(decode_attn_mla_ws(&m, 1, q, kv, (const int32_t*)pt, (const int32_t*)sl, scale, out_ws,
                                  (float*)lse_ws, ws, ws_bytes, stream),
               "decode_attn_mla_ws");
    } else {
        lib_ok(decode_attn_paged(&g, q, kv, (const int32_t*)pt, (const int32_t*)sl, scale, out, (float*)lse,
                                 stream),
               "decode_attn_paged");
        lib_ok(decode_attn_workspace_size(&g, NULL, 1, &ws_bytes), "decode_attn_workspace_size");
        HIP_OK(hipMalloc(&ws, ws_bytes));
        lib_ok(decode_attn_paged_ws(&g, 1, q, kv, (const int32_t*)pt, (const int32_t*)sl, scale, out_ws,
                                    (float*)lse_ws, ws, ws_bytes, stream),
               "decode_attn_paged_ws");
    }
    HIP_OK(hipStreamSynchronize(stream));

    download(dir, "out.bin", out, out_bytes);
    download(dir, "lse.bin", lse, lse_bytes);
    download(dir, "out_ws.bin", out_ws, out_bytes);
    download(dir, "lse_ws.bin", lse_ws, lse_bytes);
    printf("%s batch %d: ok, workspace %zu bytes\n", kind, is_mla ? m.batch : g.batch, ws_bytes);

    void* bufs[] = {q, kv, pt, sl, out, lse, out_ws, lse_ws, ws, k_scale, v_scale};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i] != NULL) HIP_OK(hipFree(bufs[i]));
    HIP_OK(hipStreamDestroy(stream));
    return 0;
}
