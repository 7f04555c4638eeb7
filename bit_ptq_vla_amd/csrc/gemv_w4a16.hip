// Weight-only int4 projection for small batches (W4A16, group-128 fp16
// scales), for gfx950.  The LoopQ abstract places this case at batch 1 in
// the memory-bound action expert; the packed weights dominate the traffic, so
// the kernel streams them from HBM once with 16-byte coalesced loads.
//
//   y[m][n] = fp16( sum_g s16[n][g] * sum_{k in g} x[m][k] * code[n][k] )
//
// A wave owns one output row n; lane l walks the row's 16-byte chunks
// (32 codes, k = 32c .. 32c+31) c = l, l+64, ...  A chunk lies inside one
// 128-wide group, so its partial dot product is scaled once by the group's
// fp16 scale.  Decoding a byte (codes 2j, 2j+1): bias both nibbles by 8 (xor
// 0x88888888 on the dword, giving 0..15), byte-permute the byte into both
// 16-bit halves, keep the low nibble in bits 0-3 and the high one in bits
// 20-23, and or in the fp16 exponent of 1024: the halves read 1024 + u_lo and
// 1024 + 16 u_hi.  One packed fp16 FMA with (1, 1/16) and (-1032, -72)
// returns the two codes exactly.  v_dot2_f32_f16 then multiplies them with
// the matching pair of x values and accumulates in fp32.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

// Codes of one packed dword (8 codes) as four fp16 pairs in k order.
__device__ __forceinline__ void decode8(uint32_t w, h2 out[4]) {
    const uint32_t u = w ^ 0x88888888u;
    const h2 mul = {static_cast<_Float16>(1.0f), static_cast<_Float16>(0.0625f)};
    const h2 add = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-72.0f)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // byte j of u into bytes 0 and 2 (selector bytes pick from {u, u})
        const uint32_t sel = (static_cast<uint32_t>(j) << 16) | static_cast<uint32_t>(j) | 0x0C000C00u;
        const uint32_t t = __builtin_amdgcn_perm(u, u, sel);
        const uint32_t bits = (t & 0x00F0000Fu) | 0x64006400u;
        const h2 hv = __builtin_bit_cast(h2, bits);
        out[j] = hv * mul + add;  // v_pk_fma_f16, exact on these integers
    }
}

template <int MT>
__global__ __launch_bounds__(256) void gemv_w4a16_kernel(const _Float16* __restrict__ x,
                                                         const uint8_t* __restrict__ wq,
                                                         const _Float16* __restrict__ ws,
                                                         int64_t m, int64_t n, int64_t k,
                                                         _Float16* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * MT;
    const int64_t chunks = k / 32;
    const uint4* wrow = reinterpret_cast<const uint4*>(wq + row * (k / 2));
    const _Float16* srow = ws + row * (k / 128);

    float acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = 0.f;

    for (int64_t c = lane; c < chunks; c += 64) {
        const uint4 wv = wrow[c];
        const float s = static_cast<float>(srow[c >> 2]);
        h2 codes[16];
        decode8(wv.x, codes);
        decode8(wv.y, codes + 4);
        decode8(wv.z, codes + 8);
        decode8(wv.w, codes + 12);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (m0 + i < m) {
                const uint4* xp = reinterpret_cast<const uint4*>(x + (m0 + i) * k + c * 32);
                float part = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 xv = xp[q];
                    part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv.x), codes[4 * q + 0], part, false);
                    part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv.y), codes[4 * q + 1], part, false);
                    part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv.z), codes[4 * q + 2], part, false);
                    part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv.w), codes[4 * q + 3], part, false);
                }
                acc[i] += part * s;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0 && m0 + i < m) y[(m0 + i) * n + row] = static_cast<_Float16>(v);
    }
}

template <int MT>
hipError_t launch_mt(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                     void* y, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((n + 3) / 4), static_cast<unsigned>((m + MT - 1) / MT));
    hipLaunchKernelGGL((gemv_w4a16_kernel<MT>), grid, dim3(256), 0, st,
                       static_cast<const _Float16*>(x), static_cast<const uint8_t*>(wq),
                       static_cast<const _Float16*>(ws), m, n, k, static_cast<_Float16*>(y));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                             int64_t n, int64_t k, int group, void* y, hipStream_t st) {
    (void)group;  // 128, checked by the caller
    if (m <= 1) return launch_mt<1>(x, wq, w_scale, m, n, k, y, st);
    if (m <= 2) return launch_mt<2>(x, wq, w_scale, m, n, k, y, st);
    if (m <= 4) return launch_mt<4>(x, wq, w_scale, m, n, k, y, st);
    return launch_mt<8>(x, wq, w_scale, m, n, k, y, st);
}

}  // namespace qlin
