// Device helpers shared by the gfx950 kernels of the qlin library.
// Storage conversions, vector types and wave64 cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

enum DType { F16 = 0, BF16 = 1, F32 = 2, I32 = 3 };

// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, num_records
// in bytes, dword 3 = data format 32 (raw byte addressing).
__device__ __forceinline__ v4i make_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const int64_t n = bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF;
    return v4i{static_cast<int>(a & 0xFFFFFFFFu), static_cast<int>((a >> 32) & 0xFFFFu),
               static_cast<int>(n), 0x00020000};
}

// ---- scalar storage conversions ------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // v_cvt_pk_bf16_f32
}

// Two floats rounded to bfloat16 (RNE) by one conversion: a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// float -> fp16 bits, round half to even, of the fp32 value f as given: the
// empty asm keeps the compiler from folding the multiply that produced f into
// the conversion (v_fma_mix rounds the unrounded product once, which can
// differ from rounding the fp32 product).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    asm("" : "+v"(f));
    _Float16 h = static_cast<_Float16>(f);  // v_cvt_f16_f32
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Eight consecutive elements of a row, widened to fp32.  p must be 16-byte
// aligned (32-byte rows of f32 are read as two 16-byte loads).
template <int DT>
__device__ __forceinline__ void load8(const void* p, float f[8]);

template <>
__device__ __forceinline__ void load8<F16>(const void* p, float f[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = f16_bits_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
        f[2 * i + 1] = f16_bits_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
}

template <>
__device__ __forceinline__ void load8<BF16>(const void* p, float f[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<F32>(const void* p, float f[8]) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// fp32 product rounded on its own, never fused into a following add.  The
// fold multiply feeds the first Hadamard butterfly; left to the compiler, it
// becomes fma(x0, m0, x1 * m1) in some kernels and not in others, and
// kernels that must produce the same codes would then round differently.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

// max(m, |a|, |b|) in one instruction.  Written as fmaxf, values that come
// out of inline assembly (the DPP butterflies) are first quieted one by one
// (v_max x, |x|, |x|) because the compiler cannot prove them canonical: an
// extra instruction per value.  For finite and quiet-NaN inputs the result is
// the fmaxf one (a quiet NaN operand is ignored).
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
    float r;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}

// ---- wave64 cross-lane helpers -------------------------------------------

// Value held by lane (lane ^ mask).  For mask < 32 this is ds_swizzle in
// bit-mask mode (and 0x1F, xor mask), which needs no LDS allocation.
template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
    if constexpr (MASK < 32) {
        constexpr int pattern = (MASK << 10) | 0x1F;
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), pattern));
    } else {
        return __shfl_xor(v, MASK, 64);
    }
}

// Value a DPP move brings in (no LDS round trip); 0 from a disabled lane.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max(float v, int width) {
    // width is a power of two <= 64; reduce within aligned groups of `width`.
    // Within a 16-lane row by DPP: the two quad swaps leave every quad
    // holding its maximum, so the half-row mirror (lane i <- 7 - i) then
    // meets the other quad and the row mirror (i <- 15 - i) the other half.
    // Inputs are magnitudes (>= 0), for which a disabled lane's 0 is neutral.
    if (width >= 2) v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
    if (width >= 4) v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
    if (width >= 8) v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
    if (width >= 16) v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
    if (width >= 32) v = fmaxf(v, lane_xor<16>(v));
    if (width >= 64) v = fmaxf(v, lane_xor<32>(v));
    return v;
}

// Exact GeLU, t * (1 + erf(t / sqrt 2)) / 2, in fp32 (device-library erff).
__device__ __forceinline__ float gelu_erf(float t) {
    return 0.5f * t * (1.0f + erff(t * 0.70710678118654752440f));
}

}  // namespace qlin
