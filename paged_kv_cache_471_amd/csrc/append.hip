// Paged KV append (gfx950): each decode step writes the new token's K/V (GQA)
// or latent (MLA) into its page slot before the history is read whole
// ("Analytical Provisioning for Attention-FFN Disaggregated LLM Serving under
// Stochastic Workloads", §2 and Fig. 1; "OpWeave: Flexible Operator
// Disaggregation for Heterogeneous LLM Serving", §8 paged KV-cache
// management).  An fp8 cache stores e4m3 codes with one scale per KV head
// (SPLASH, App. C.1 and App. B.1).
//
// Token t of request b sits in page page_table[b][t / P], slot t % P; a
// negative position skips the request.  GQA: one workgroup per (request, K|V)
// writes Hkv * D values, four per thread (16-byte stores for fp32, 8 for
// bf16, 4 for fp8 K; fp8 V blocks are tiled, fp8_v_byte in da_common.h, so
// the four codes of an fp8 V row go to their own bytes).  MLA: one workgroup
// per request copies its 1152-byte latent with 16-byte stores.
#include <hip/hip_ext.h>

#include "da_common.h"
#include "da_append.h"

namespace da {
namespace {

constexpr int kAppendBlock = 256;

// fp32 -> OCP e4m3fn code: the nearest value with ties to the even code;
// |y| >= 448 (infinity included) gives the largest finite magnitude with y's
// sign, NaN the code 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;                      // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;              // |y| >= 448
    uint32_t c;
    if (a < 0x3c800000u) {
        // |y| < 2^-6: the codes are m * 2^-9, m = 0..7 (m = 8 is 2^-6, code 8)
        c = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    } else {
        // keep 3 mantissa bits, rounding the 20 dropped ones to nearest even;
        // a carry moves into the exponent field, as it should
        const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        c = (r >> 20) - (120u << 3);                        // ((e - 127 + 7) << 3) | m
    }
    return sign | c;
}

// Four consecutive input elements of one thread, as loaded.
template <int IN> struct Quad;
template <> struct Quad<kF32> { using T = float4; };
template <> struct Quad<kBF16> { using T = uint2; };

template <int IN>
__device__ __forceinline__ typename Quad<IN>::T load_quad(const void* src, int64_t i) {
    using T = typename Quad<IN>::T;
    constexpr int kElem = IN == kF32 ? 4 : 2;
    return *reinterpret_cast<const T*>(static_cast<const char*>(src) + i * kElem);
}

template <int IN, int OUT>
__device__ __forceinline__ void store_quad(const AppendArgs& a, int which, int j, int r, int d, int64_t di,
                                           typename Quad<IN>::T w) {
    if constexpr (IN == kF32 && OUT == kF32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.kv) + di) = w;
    } else if constexpr (IN == kBF16 && OUT == kBF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.kv) + di) = w;
    } else {
        static_assert(IN == kBF16 && OUT == kFP8, "append combination");
        const float s = (which ? a.v_scale : a.k_scale)[j];
        const uint32_t c0 = f32_to_e4m3(bf16_lo(w.x) / s);
        const uint32_t c1 = f32_to_e4m3(bf16_hi(w.x) / s);
        const uint32_t c2 = f32_to_e4m3(bf16_lo(w.y) / s);
        const uint32_t c3 = f32_to_e4m3(bf16_hi(w.y) / s);
        uint8_t* kv = static_cast<uint8_t*>(a.kv);
        if (which == 0) {
            *reinterpret_cast<uint32_t*>(kv + di) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        } else {
            // the V block of (page, head) starts at di - r D - d
            uint8_t* block = kv + (di - static_cast<int64_t>(r) * a.head_dim - d);
            block[fp8_v_byte(r, d, a.head_dim)] = static_cast<uint8_t>(c0);
            block[fp8_v_byte(r, d + 1, a.head_dim)] = static_cast<uint8_t>(c1);
            block[fp8_v_byte(r, d + 2, a.head_dim)] = static_cast<uint8_t>(c2);
            block[fp8_v_byte(r, d + 3, a.head_dim)] = static_cast<uint8_t>(c3);
        }
    }
}

template <int IN, int OUT>
__global__ __launch_bounds__(kAppendBlock) void kv_append_kernel(AppendArgs a) {
    const int b = blockIdx.x >> 1;
    const int which = blockIdx.x & 1;                       // 0: K, 1: V
    const int D = a.head_dim;
    const int HD = a.kv_heads * D;
    const void* src = which ? a.v_new : a.k_new;
    const int64_t s0 = static_cast<int64_t>(b) * HD;
    const int t = a.positions[b];
    if (t < 0) return;
    const int pg = a.page_table[static_cast<int64_t>(b) * a.max_pages + t / a.page_size];
    const int r = t % a.page_size;
    for (int e = 4 * threadIdx.x; e < HD; e += 4 * kAppendBlock) {
        const int j = e / D;
        const int d = e % D;
        const int64_t di = (((static_cast<int64_t>(pg) * 2 + which) * a.kv_heads + j) * a.page_size + r) * D + d;
        store_quad<IN, OUT>(a, which, j, r, d, di, load_quad<IN>(src, s0 + e));
    }
}

__global__ __launch_bounds__(128) void mla_append_kernel(AppendArgs a) {
    const int b = blockIdx.x;
    const int t = a.positions[b];
    if (t < 0 || threadIdx.x >= kMlaLatent / 8) return;
    const uint4 w = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) +
                                                   static_cast<int64_t>(b) * kMlaLatent)[threadIdx.x];
    const int pg = a.page_table[static_cast<int64_t>(b) * a.max_pages + t / a.page_size];
    const int r = t % a.page_size;
    reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.kv) +
                             (static_cast<int64_t>(pg) * a.page_size + r) * kMlaLatent)[threadIdx.x] = w;
}

template <typename K>
hipError_t launch(K kernel, int grid, int block, hipStream_t s, const KernelEvents& ev, const AppendArgs& a) {
    if (ev.start != nullptr)
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s, const KernelEvents& ev) {
    const int grid = 2 * a.batch;
    if (a.in_dtype == kF32 && a.kv_dtype == kF32) return launch(kv_append_kernel<kF32, kF32>, grid, kAppendBlock, s, ev, a);
    if (a.in_dtype == kBF16 && a.kv_dtype == kBF16) return launch(kv_append_kernel<kBF16, kBF16>, grid, kAppendBlock, s, ev, a);
    if (a.in_dtype == kBF16 && a.kv_dtype == kFP8) return launch(kv_append_kernel<kBF16, kFP8>, grid, kAppendBlock, s, ev, a);
    return hipErrorInvalidValue;
}

hipError_t launch_kv_append_mla(const AppendArgs& a, hipStream_t s, const KernelEvents& ev) {
    return launch(mla_append_kernel, a.batch, 128, s, ev, a);
}

}  // namespace da
