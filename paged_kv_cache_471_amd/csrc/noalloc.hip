// Paged GQA decode for callers that cannot allocate device memory: the
// workspace of decode_attn_paged_ws comes from a fixed scratch array that the
// library's code object carries, one copy per device.
//
// The array is a device symbol: on the host its name is only a stand-in, so
// host code never passes it to a kernel or a copy.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and every launch uses that address.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/decode_attn.h"

namespace da {
int hip_failure(hipError_t e);
}

namespace {

constexpr size_t kScratchBytes = DA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch is a whole number of 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on first use.
int scratch_address(void** addr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return da::hip_failure(e);
    if (dev < 0 || dev >= kMaxDevices) return DA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return da::hip_failure(e);
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return DA_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return DA_OK;
}

}  // namespace

extern "C" int decode_attn_paged_noalloc(const da_paged_desc* desc, int32_t q_rows, const void* q,
                                         const void* kv_pages, const int32_t* page_table, const int32_t* seq_lens,
                                         float scale, void* out, float* lse, void* stream) {
    // the size query runs every host check of the call and resolves the
    // worker count exactly as the launch will
    size_t need = 0;
    int st = decode_attn_workspace_size(desc, nullptr, q_rows, &need);
    if (st != DA_OK) return st;
    if (need > kScratchBytes) return DA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != DA_OK) return st;
    return decode_attn_paged_ws(desc, q_rows, q, kv_pages, page_table, seq_lens, scale, out, lse, ws, kScratchBytes,
                                stream);
}
