// Weight-only int4 projection for small batches (W4A16, group-128 fp16
// scales), for gfx950.  The LoopQ abstract places this case at batch 1 in
// the memory-bound action expert; the packed weights dominate the traffic, so
// the kernel streams them from HBM once with 16-byte coalesced loads and keeps
// as many of them in flight as the registers allow.
//
//   y[m][n] = fp16( sum_g s16[n][g] * sum_{k in g} x[m][k] * code[n][k] )
//
// A wave owns R output rows; lane l walks the rows' 16-byte chunks (32 codes,
// k = 32c .. 32c+31) c = l, l+64, ...  Every weight load of the wave's rows is
// issued before any is decoded (non-temporal: the weights are read once).  A
// chunk lies inside one 128-wide group, so its partial dot product is scaled
// once by the group's fp16 scale.  Decoding a byte (codes 2j, 2j+1): bias
// both nibbles by 8 (xor 0x88888888 on the dword, giving 0..15), byte-permute
// the byte into both 16-bit halves, keep the low nibble in bits 0-3 and the
// high one in bits 20-23, and or in the fp16 exponent of 1024: the halves read
// 1024 + u_lo and 1024 + 16 u_hi.  One packed fp16 FMA with (1, 1/16) and
// (-1032, -72) returns the two codes exactly.  v_dot2_f32_f16 multiplies them
// with the matching pair of x values and accumulates in fp32.

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

// Dot product of 32 codes (one 16-byte chunk) with 32 fp16 x values.
__device__ __forceinline__ float chunk_dot(const uint4 wv, const uint4 (&xv)[4]) {
    h2 codes[16];
    decode8(wv.x, codes);
    decode8(wv.y, codes + 4);
    decode8(wv.z, codes + 8);
    decode8(wv.w, codes + 12);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv[q].x), codes[4 * q + 0], part, false);
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv[q].y), codes[4 * q + 1], part, false);
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv[q].z), codes[4 * q + 2], part, false);
        part = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, xv[q].w), codes[4 * q + 3], part, false);
    }
    return part;
}

// R rows per wave, CH chunk slots per lane per row (CH * 64 >= k / 32), MT
// token rows of x per pass (blockIdx.y selects the pass).
template <int R, int CH, int MT>
__global__ __launch_bounds__(256) void gemv_w4a16_kernel(const _Float16* __restrict__ x,
                                                         const uint8_t* __restrict__ wq,
                                                         const _Float16* __restrict__ ws,
                                                         int64_t m, int64_t n, int64_t k,
                                                         _Float16* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * R;
    if (row0 >= n) return;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * MT;
    const int chunks = static_cast<int>(k / 32);

    // all weight chunks (and their group scales) of the wave's rows first
    uint4 wv[R][CH];
    float sc[R][CH];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        const uint4* wrow = reinterpret_cast<const uint4*>(wq + (row < n ? row : 0) * (k / 2));
        const _Float16* srow = ws + (row < n ? row : 0) * (k / 128);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + 64 * j;
            const bool ok = row < n && c < chunks;
            wv[r][j] = ok ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + c)))
                          : make_uint4(0, 0, 0, 0);
            sc[r][j] = ok ? static_cast<float>(srow[c >> 2]) : 0.f;
        }
    }

    float acc[MT][R];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + 64 * j;
        if (c >= chunks) break;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (m0 + i >= m) break;
            const uint4* xp = reinterpret_cast<const uint4*>(x + (m0 + i) * k + static_cast<int64_t>(c) * 32);
            const uint4 xv[4] = {xp[0], xp[1], xp[2], xp[3]};
#pragma unroll
            for (int r = 0; r < R; ++r) acc[i][r] += chunk_dot(wv[r][j], xv) * sc[r][j];
        }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum(acc[i][r]);
            if (lane == 0 && m0 + i < m && row0 + r < n) y[(m0 + i) * n + row0 + r] = static_cast<_Float16>(v);
        }
    }
}

template <int R, int CH, int MT>
hipError_t launch_g(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                    void* y, hipStream_t st) {
    const int64_t waves = (n + R - 1) / R;
    dim3 grid(static_cast<unsigned>((waves + 3) / 4), static_cast<unsigned>((m + MT - 1) / MT));
    hipLaunchKernelGGL((gemv_w4a16_kernel<R, CH, MT>), grid, dim3(256), 0, st,
                       static_cast<const _Float16*>(x), static_cast<const uint8_t*>(wq),
                       static_cast<const _Float16*>(ws), m, n, k, static_cast<_Float16*>(y));
    return hipGetLastError();
}

template <int CH>
hipError_t launch_ch(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                     void* y, hipStream_t st) {
    // R = 4 rows per wave keeps 4 * CH 16-byte weight loads per lane in flight
    constexpr int R = CH <= 4 ? 4 : 2;
    if (m <= 1) return launch_g<R, CH, 1>(x, wq, ws, m, n, k, y, st);
    if (m <= 2) return launch_g<R, CH, 2>(x, wq, ws, m, n, k, y, st);
    if (m <= 4) return launch_g<R, CH, 4>(x, wq, ws, m, n, k, y, st);
    return launch_g<R, CH, 8>(x, wq, ws, m, n, k, y, st);
}

}  // namespace

hipError_t launch_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                             int64_t n, int64_t k, int group, void* y, hipStream_t st) {
    (void)group;  // 128, checked by the caller
    const int64_t chunks = k / 32;
    const int64_t ch = (chunks + 63) / 64;   // chunk slots per lane
    if (ch <= 1) return launch_ch<1>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 2) return launch_ch<2>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 4) return launch_ch<4>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 8) return launch_ch<8>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 16) return launch_ch<16>(x, wq, w_scale, m, n, k, y, st);
    return hipErrorInvalidValue;
}

}  // namespace qlin
