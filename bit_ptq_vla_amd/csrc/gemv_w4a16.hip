// Weight-only int4 projection for one to three token rows (W4A16, group-128
// fp16 scales), for gfx950; more rows go to the matrix-core kernel.  The
// LoopQ abstract places this case at batch 1 in the memory-bound action
// expert; the packed weights dominate the traffic, so the kernel streams them
// from HBM once with 16-byte coalesced loads and has every load of a wave in
// flight at once.
//
//   y[m][n] = fp16( sum_g s16[n][g] * sum_{k in g} x[m][k] * code[n][k] )
//
// Work split: a block of four waves shares MT token rows of x, staged once in
// LDS; a wave owns R output rows; lane l takes the rows' 16-byte chunks
// (32 codes, k = 32c .. 32c+31) c = l, l+64, ... (CH slots).  A chunk lies
// inside one 128-wide group, so its partial dot product is scaled once by the
// group's fp16 scale.  blockIdx.y walks the token rows MT at a time.
//
// Latency is the cost at these sizes (one pass over a few MB), so no load
// sits behind a branch: out-of-range rows and chunks read a clamped, valid
// address and contribute through a zero scale, and the weight loads of the
// whole wave are issued before anything waits.
//
// Decoding, 8 codes (one dword w, code j in nibble j) in 5 instructions:
// u = w ^ 0x88888888 biases every nibble to code + 8 (0..15).  Masking u and
// u >> 8 with 0x000F000F or 0x00F000F0 and or-ing in 0x6400 (fp16 1024) puts
// two codes into the mantissas of an fp16 pair: h = 1024 + (code + 8) for the
// even codes (pairs k0,k4 and k2,k6) and h = 1024 + 16 (code + 8) for the odd
// ones (k1,k5 and k3,k7).  v_dot2_f32_f16 multiplies such a pair with the
// matching pair of x values, which the LDS staging stores in that order, and
// accumulates in fp32 (one accumulator for even, one for odd codes).  Then
//   sum_k x_k code_k = acc_even + acc_odd / 16 - (1032 Sx_even + 72 Sx_odd),
// where the x sums of the chunk are formed once, at staging, for all rows.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

// LDS of a block: x pieces (MT k 2 bytes), chunk terms (MT k / 8 bytes) and a
// 4 KB slot that takes the fp16 scales of its 4R rows (one 16-byte word per
// thread; 4R k / 64 <= 4096 since R * CH <= 32).
constexpr int64_t kGemvLdsBytes = 65536 + 4096 + 8192;
constexpr int64_t gemv_lds_bytes(int64_t mt, int64_t /*r*/, int64_t k) {
    return mt * (k * 2 + k / 8) + 4096;
}

// fp16 pair held in a dword.  Taken by value: a bit cast applied directly to a
// component of an ext_vector lvalue (v.y) reads component 0 with this
// compiler, so components are copied out first.
__device__ __forceinline__ h2 as_h2(int v) { return __builtin_bit_cast(h2, v); }

// sum_k x_k code_k over one chunk (32 codes in wv) plus the chunk's bias
// term, which the caller subtracts; x pieces in the staged pair order.
__device__ __forceinline__ float chunk_dot(const v4i wv, const v4i (&xv)[4]) {
    float even = 0.f, odd = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // (w & mask) ^ (bias | magic) == ((w ^ 0x88888888) & mask) | magic: one v_bitop3 each
        const uint32_t u = static_cast<uint32_t>(wv[q]);
        const uint32_t us = u >> 8;
        const int e0 = static_cast<int>((u & 0x000F000Fu) ^ 0x64086408u);   // k0, k4
        const int o0 = static_cast<int>((u & 0x00F000F0u) ^ 0x64806480u);   // k1, k5
        const int e1 = static_cast<int>((us & 0x000F000Fu) ^ 0x64086408u);  // k2, k6
        const int o1 = static_cast<int>((us & 0x00F000F0u) ^ 0x64806480u);  // k3, k7
        const v4i xq = xv[q];
        even = __builtin_amdgcn_fdot2(as_h2(xq.x), as_h2(e0), even, false);
        even = __builtin_amdgcn_fdot2(as_h2(xq.y), as_h2(e1), even, false);
        odd = __builtin_amdgcn_fdot2(as_h2(xq.z), as_h2(o0), odd, false);
        odd = __builtin_amdgcn_fdot2(as_h2(xq.w), as_h2(o1), odd, false);
    }
    return __builtin_fmaf(odd, 0.0625f, even);
}

// v + the value of another lane chosen by a DPP control (rows outside
// ROW_MASK add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wave, complete in lane 63: pairs and quads
// (quad_perm), half rows (row_half_mirror), rows (row_mirror), then the row
// broadcasts of lanes 15 and 31.
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v = add_dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = add_dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = add_dpp<0x141, 0xF>(v);  // row_half_mirror
    v = add_dpp<0x140, 0xF>(v);  // row_mirror
    v = add_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = add_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// LDS layout: token row i, 16-byte piece q (0..3) of chunk c at v4i index
// (i * 4 + q) * chunks + c, so the 64 lanes of a wave (consecutive chunks)
// read consecutive 16-byte words.  A piece holds x_0..x_7 of its 8 codes as
// the pairs (x0,x4), (x2,x6), (x1,x5), (x3,x7).  After the pieces, float
// bias[i][c] = 1032 Sx_even + 72 Sx_odd of the chunk, then the fp16 scales of
// the block's rows as stored in w_scale.
template <int R, int CH, int MT>
__global__ __launch_bounds__(256) void gemv_w4a16_kernel(const _Float16* __restrict__ x,
                                                         const uint8_t* __restrict__ wq,
                                                         const _Float16* __restrict__ ws,
                                                         int64_t m, int64_t n, int64_t k,
                                                         _Float16* __restrict__ y) {
    static_assert(R * CH <= 32, "the block's scales must fit one 16-byte word per thread");
    extern __shared__ v4i xs[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * R;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * MT;
    const int chunks = static_cast<int>(k / 32);
    const int groups = static_cast<int>(k / 128);
    const int kv = static_cast<int>(k / 8);  // 16-byte words per token row; CH * 256 >= kv

    // 1. x rows m0 .. m0+MT-1 (clamped to m-1), first: waiting for them then
    //    leaves the weight loads in flight (the load counter drains in order)
    v4i xr[MT][CH];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t tok = m0 + i < m ? m0 + i : m - 1;
        const v4i* xrow = reinterpret_cast<const v4i*>(x + tok * k);
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const int e = tid + 256 * t < kv ? tid + 256 * t : kv - 1;
            xr[i][t] = xrow[e];
        }
    }
    // 2. the group scales of the block's 4R rows (contiguous, at most 16 bytes
    //    per thread; the buffer descriptor returns zeros past the last row)
    const int64_t rb0 = static_cast<int64_t>(blockIdx.x) * 4 * R;
    const int sbytes = static_cast<int>((n - rb0 < 4 * R ? n - rb0 : 4 * R) * groups * 2);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16*>(ws + rb0 * groups), 0, sbytes, 0x00020000);
    const v4i sraw = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_s, tid * 16, 0, 0));
    __builtin_amdgcn_sched_barrier(0);  // issued ahead of the weights: its wait leaves them in flight

    // 3. weight chunks of the wave's rows (clamped, no branch)
    v4i wv[R][CH];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r < n ? row0 + r : n - 1;
        const v4i* wrow = reinterpret_cast<const v4i*>(wq + row * (k / 2));
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + 64 * j < chunks ? lane + 64 * j : chunks - 1;
            wv[r][j] = __builtin_nontemporal_load(wrow + c);
        }
    }

    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the LDS stores wait
    // 4. stage x in pair order, the chunk terms 1032 Sx_even + 72 Sx_odd and the scales
    float* xbias = reinterpret_cast<float*>(xs + MT * 4 * chunks);
    v4i* sc_lds = reinterpret_cast<v4i*>(xbias + MT * chunks);
    sc_lds[tid] = sraw;  // unconditional: a conditional store lets the compiler sink the load
    const h2 k_even = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 k_odd = {static_cast<_Float16>(72.0f), static_cast<_Float16>(72.0f)};
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            // a clamped index rewrites the last word with its own value
            const int e0 = tid + 256 * t;
            const int e = e0 < kv ? e0 : kv - 1;  // = 4 c + q
            const v4i d = xr[i][t];
            v4i o;
            o.x = static_cast<int>(__builtin_amdgcn_perm(d.z, d.x, 0x05040100u));  // x0, x4
            o.y = static_cast<int>(__builtin_amdgcn_perm(d.w, d.y, 0x05040100u));  // x2, x6
            o.z = static_cast<int>(__builtin_amdgcn_perm(d.z, d.x, 0x07060302u));  // x1, x5
            o.w = static_cast<int>(__builtin_amdgcn_perm(d.w, d.y, 0x07060302u));  // x3, x7
            xs[(i * 4 + (e & 3)) * chunks + (e >> 2)] = o;
            // products with 1032 and 72 are exact; the four pieces of a chunk sit in four
            // consecutive lanes (a DPP quad)
            float b = __builtin_amdgcn_fdot2(as_h2(o.x), k_even, 0.f, false);
            b = __builtin_amdgcn_fdot2(as_h2(o.y), k_even, b, false);
            b = __builtin_amdgcn_fdot2(as_h2(o.z), k_odd, b, false);
            b = __builtin_amdgcn_fdot2(as_h2(o.w), k_odd, b, false);
            b = add_dpp<0xB1, 0xF>(b);
            b = add_dpp<0x4E, 0xF>(b);
            if (e0 < kv && (e & 3) == 0) xbias[i * chunks + (e >> 2)] = b;
        }
    }
    __syncthreads();

    // 5. dot products; invalid chunks and rows carry a zero scale
    const _Float16* sc16 = reinterpret_cast<const _Float16*>(sc_lds) + wave * R * groups;
    _Float16 sh[R][CH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + 64 * j < chunks ? lane + 64 * j : chunks - 1;
            sh[r][j] = sc16[r * groups + (c >> 2)];
        }
    __builtin_amdgcn_sched_barrier(0);  // the LDS reads above go out back to back
    float sc[R][CH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < CH; ++j)
            sc[r][j] = (row0 + r < n && lane + 64 * j < chunks) ? static_cast<float>(sh[r][j]) : 0.f;

    float acc[MT][R];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + 64 * j < chunks ? lane + 64 * j : chunks - 1;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const v4i* xp = xs + i * 4 * chunks + c;
            v4i xv[4];
            xv[0] = xp[0];
            xv[1] = xp[chunks];
            xv[2] = xp[2 * chunks];
            xv[3] = xp[3 * chunks];
            const float bias = xbias[i * chunks + c];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[i][r] = __builtin_fmaf(chunk_dot(wv[r][j], xv) - bias, sc[r][j], acc[i][r]);
        }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum_lane63(acc[i][r]);
            if (lane == 63 && m0 + i < m && row0 + r < n) y[(m0 + i) * n + row0 + r] = static_cast<_Float16>(v);
        }
    }
}

template <int R, int CH, int MT>
hipError_t launch_g(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                    void* y, hipStream_t st) {
    const int64_t waves = (n + R - 1) / R;
    const int64_t lds = gemv_lds_bytes(MT, R, k);
    if (lds > kGemvLdsBytes) return hipErrorInvalidValue;
    dim3 grid(static_cast<unsigned>((waves + 3) / 4), static_cast<unsigned>((m + MT - 1) / MT));
    hipLaunchKernelGGL((gemv_w4a16_kernel<R, CH, MT>), grid, dim3(256), static_cast<size_t>(lds), st,
                       static_cast<const _Float16*>(x), static_cast<const uint8_t*>(wq),
                       static_cast<const _Float16*>(ws), m, n, k, static_cast<_Float16*>(y));
    return hipGetLastError();
}

template <int R, int CH>
hipError_t launch_mt(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                     void* y, hipStream_t st) {
    // token rows per pass: as many as m (at most 3 here) needs, at most 4, with MT * k * 2
    // within the LDS budget (k > (CH / 2) * 2048 bounds MT from above, so larger MT are
    // never built)
    constexpr int kMaxMt = CH <= 4 ? 4 : CH <= 8 ? 2 : 1;
    int mt = 1;
    while (mt < kMaxMt && mt < m && gemv_lds_bytes(2 * mt, R, k) <= kGemvLdsBytes) mt *= 2;
    if constexpr (kMaxMt >= 4) {
        if (mt == 4) return launch_g<R, CH, 4>(x, wq, ws, m, n, k, y, st);
    }
    if constexpr (kMaxMt >= 2) {
        if (mt == 2) return launch_g<R, CH, 2>(x, wq, ws, m, n, k, y, st);
    }
    return launch_g<R, CH, 1>(x, wq, ws, m, n, k, y, st);
}

template <int CH>
hipError_t launch_ch(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                     void* y, hipStream_t st) {
    // R * CH 16-byte weight loads per lane stay in flight; R = 4 only where
    // n still gives >= 256 blocks of four waves (one per CU)
    if constexpr (CH <= 4) {
        if (n >= 4 * 4 * 256) return launch_mt<4, CH>(x, wq, ws, m, n, k, y, st);
    }
    return launch_mt<2, CH>(x, wq, ws, m, n, k, y, st);
}

}  // namespace

namespace {

// Streaming-read reference: every byte of src read once with 16-byte loads,
// UNR loads in flight per lane, xor-folded into one word per block (so the
// loads are not dead).  bytes is a multiple of 16.
constexpr int kReadUnroll = 4;
__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* src, int64_t words16, uint32_t* sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < words16; i += kReadUnroll * stride) {
        v4i v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= static_cast<uint32_t>(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    for (; i < words16; i += stride) {
        const v4i v = __builtin_nontemporal_load(src + i);
        acc ^= static_cast<uint32_t>(v.x ^ v.y ^ v.z ^ v.w);
    }
    __shared__ uint32_t red[4];
    for (int o = 32; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, hipStream_t st) {
    const int64_t words16 = bytes / 16;
    int64_t blocks = (words16 + 256 * kReadUnroll - 1) / (256 * kReadUnroll);
    const int64_t cap = static_cast<int64_t>(device_cus()) * 8;
    if (blocks > cap) blocks = cap;
    if (blocks > sink_words) blocks = sink_words;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<const v4i*>(src), words16, sink);
    return hipGetLastError();
}

hipError_t launch_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                             int64_t n, int64_t k, int group, void* y, hipStream_t st) {
    (void)group;  // 128, checked by the caller
    // from four token rows on, the matrix-core kernel (each weight decoded once
    // for all rows) is faster than the vector dot products here (measured at
    // n, k = 1024 and 4096)
    if (m > 3) return launch_skinny_w4a16(x, wq, w_scale, m, n, k, y, st);
    const int64_t chunks = k / 32;
    const int64_t ch = (chunks + 63) / 64;   // chunk slots per lane
    if (ch <= 1) return launch_ch<1>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 2) return launch_ch<2>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 4) return launch_ch<4>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 6) return launch_ch<6>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 8) return launch_ch<8>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 12) return launch_ch<12>(x, wq, w_scale, m, n, k, y, st);
    if (ch <= 16) return launch_ch<16>(x, wq, w_scale, m, n, k, y, st);
    return hipErrorInvalidValue;
}

}  // namespace qlin
