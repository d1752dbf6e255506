// Device helpers shared by the decode-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kFP8 = 2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// initial running max: finite, far below any real score, so that
// exp2(init - m) is exactly 0 and exp2(init - init) is 1 (no inf - inf).
constexpr float kMaxInit = -1.0e30f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

template <int DT> struct ElemBytes;
template <> struct ElemBytes<kF32> { static constexpr int value = 4; };
template <> struct ElemBytes<kBF16> { static constexpr int value = 2; };
template <> struct ElemBytes<kFP8> { static constexpr int value = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, b);
}

// a.x*b.x + a.y*b.y + c with bf16 pairs and fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// a.x*b.x + a.y*b.y (the same operation with a zero addend).  The compiler
// emits the accumulate-in-place encoding for dot2_bf16, which needs a move of
// 0.0 into the destination first; the three-operand encoding takes the zero
// as an inline constant.
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// two OCP e4m3 codes (bytes 0,1 or 2,3 of w) -> packed bf16 pair (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// two OCP e4m3 codes -> two fp32 values (exact).
template <bool HI>
__device__ __forceinline__ floatx2_t fp8x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
}

// Data-parallel-primitive move within a row of 16 lanes.
// (old value 0 with bound_ctrl lets the compiler fold the move into the add)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the
// bitwise-identical total (each step adds a commutative pair).
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror: quad q <-> quad q^1 within 8
    x += dpp_mov<0x140>(x);  // row_mirror: half 0 <-> half 1
    return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only kernel data (page tables, lengths) seen through the constant
// address space; wave-uniform reads of it compile to scalar loads.
typedef const __attribute__((address_space(4))) int32_t cint32_t;

// Wave-uniform 32-bit read through the scalar data cache (a read; the value is
// ready when the call returns).  Used for page ids and lengths, so that they
// do not queue behind the vector loads of the KV stream.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

// Byte of (slot, dim d) within the V block [P][D] of one (page, KV head) of
// an fp8 cache: the block is kept in 16-token tiles (16 D bytes each), and
// within a tile, with DL = D / 16 (D = 64 or 128), the code of token s and dim
// d sits at 1024 ((d mod DL) / 4) + 256 (s / 4) + 16 (d / DL) + 4 (d mod 4) +
// (s mod 4): lane (R, C) of a wavefront reading 16-byte pieces at 1024 p +
// 16 (16 R + C) receives, for tokens 4R..4R+3, the codes of dims C DL + 4p ..
// C DL + 4p + 3, one dim per 32-bit word.
__device__ __forceinline__ int fp8_v_byte(int slot, int d, int head_dim) {
    const int DL = head_dim >> 4;
    const int s = slot & 15;
    return (slot >> 4) * 16 * head_dim + 1024 * ((d & (DL - 1)) >> 2) + 256 * (s >> 2) + 16 * (d / DL) +
           4 * (d & 3) + (s & 3);
}

// Address function of the paged GQA cache [num_pages][2][Hkv][P][D]:
// element offset of (page, sel = 0 key / 1 value, kv head, slot, dim 0).
__device__ __forceinline__ int64_t gqa_kv_offset(int page, int sel, int head, int slot, int num_kv_heads,
                                                 int page_size, int head_dim) {
    return ((static_cast<int64_t>(page) * 2 + sel) * num_kv_heads + head) *
               static_cast<int64_t>(page_size * head_dim) +
           static_cast<int64_t>(slot) * head_dim;
}

// Address function of the paged MLA latent cache [num_pages][P][Dk].
__device__ __forceinline__ int64_t mla_kv_offset(int page, int slot, int page_size, int latent_dim) {
    return (static_cast<int64_t>(page) * page_size + slot) * latent_dim;
}

}  // namespace da
