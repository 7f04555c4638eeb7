// Integer projection for up to 64 token rows on the gfx950 matrix cores: the
// GEMM with int32 accumulation and the dequantizing epilogue of the W4A4,
// W8A8 and W4A8 schemes (FoldQuantVLA abstract: W4A4 projections in the
// iterative action expert, W8A8 for the projections kept at eight bits;
// QuantVLA summary: W4A8), for the small row counts of the action expert.
//
//   y[m][n] = out( float(acc) * s_x[m] * s_w[n] ),  acc = sum_k qx[m][k] * qw[n][k]
//
// The large-tile GEMM puts at most 50 of its 128 tile rows to use at these
// sizes and has few tiles to spread; here a block owns 16 output columns and
// 16 MW token rows, and its eight waves take contiguous slices of k.  int32
// partial tiles add exactly, so the slice order does not matter and results
// equal the large-tile GEMM's bit for bit (same epilogue arithmetic).
//
// Operands.  v_mfma_i32_16x16x64_i8: lane l = c + 16 q feeds row (A) or
// column (B) c with 16 k values.  A piece of 128 k (64 for W8A8) gives lane
// quarter q the k range [32 q, 32 q + 32) (W8A8: [16 q, 16 q + 16)), split in
// two MFMA steps of 16.  int4 codes are unpacked to int8 with the nibble in
// the high half (16 * code: k order 0 2 4 6 8 .. 14 1 3 .. 15 per 16 codes),
// so W4A4 accumulates 256 * acc and W4A8 16 * acc (its int8 activations are
// put into the same k order); the epilogue folds 2^-8 / 2^-4 into s_w exactly.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

enum Scheme { W4A4 = 0, W8A8 = 1, W4A8 = 2 };

// 16 int4 codes (two dwords, code j in nibble j) as int8 16 * code, k order
// 0 2 4 6 | 8 10 12 14 | 1 3 5 7 | 9 11 13 15.
__device__ __forceinline__ v4i unpack16(int w0, int w1) {
    const uint32_t a = static_cast<uint32_t>(w0), b = static_cast<uint32_t>(w1);
    return v4i{static_cast<int>((a << 4) & 0xF0F0F0F0u), static_cast<int>((b << 4) & 0xF0F0F0F0u),
               static_cast<int>(a & 0xF0F0F0F0u), static_cast<int>(b & 0xF0F0F0F0u)};
}

// 16 int8 values in natural k order, put into the order of unpack16.
__device__ __forceinline__ v4i reorder16(v4i d) {
    return v4i{static_cast<int>(__builtin_amdgcn_perm(d.y, d.x, 0x06040200u)),
               static_cast<int>(__builtin_amdgcn_perm(d.w, d.z, 0x06040200u)),
               static_cast<int>(__builtin_amdgcn_perm(d.y, d.x, 0x07050301u)),
               static_cast<int>(__builtin_amdgcn_perm(d.w, d.z, 0x07050301u))};
}

template <int S>
struct Cfg {
    static constexpr bool A4 = (S == W4A4);
    static constexpr bool B4 = (S != W8A8);
    static constexpr int PK = (S == W8A8) ? 64 : 128;       // k per piece
    static constexpr int STEPS = PK / 64;                   // MFMA steps per piece
    static constexpr int AW = A4 ? 1 : STEPS;               // 16-byte A words per lane and piece
    static constexpr int BW = B4 ? 1 : STEPS;
    static constexpr int ASH = (S == W4A4) ? 8 : (S == W4A8) ? 4 : 0;
};

template <int S, int MW>
struct Piece {
    v4i a[MW][Cfg<S>::AW];
    v4i b[Cfg<S>::BW];
};

// Piece p of the lane's rows; ok == false (the lane's word lies past k in a
// half-full last W4A4 piece) reads piece 0 instead and keeps zeros.
template <int S, int MW>
__device__ __forceinline__ void load_piece(Piece<S, MW>& f, const v4i* const (&xp)[MW], const v4i* wp, int p,
                                           bool ok) {
    using C = Cfg<S>;
    const int pa = ok ? p : 0;
    const v4i zero = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < C::BW; ++j) {
        const v4i v = __builtin_nontemporal_load(wp + pa * (C::B4 ? 4 : C::STEPS * 4) + j);
        f.b[j] = ok ? v : zero;
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int j = 0; j < C::AW; ++j) {
            const v4i v = xp[mt][pa * (C::A4 ? 4 : C::STEPS * 4) + j];
            f.a[mt][j] = ok ? v : zero;
        }
}

template <int S, int MW>
__device__ __forceinline__ void mma_piece(const Piece<S, MW>& f, v4i (&acc)[MW]) {
    using C = Cfg<S>;
#pragma unroll
    for (int s = 0; s < C::STEPS; ++s) {
        v4i bv;
        if constexpr (C::B4) bv = unpack16(f.b[0][2 * s], f.b[0][2 * s + 1]);
        else bv = f.b[s];
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            v4i av;
            if constexpr (C::A4) av = unpack16(f.a[mt][0][2 * s], f.a[mt][0][2 * s + 1]);
            else if constexpr (S == W4A8) av = reorder16(f.a[mt][s]);
            else av = f.a[mt][s];
            acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[mt], 0, 0, 0);
        }
    }
}

template <int S, int MW, int WK>
__global__ __launch_bounds__(64 * WK) void skinny_int_kernel(const uint8_t* __restrict__ xq,
                                                             const float* __restrict__ sx,
                                                             const uint8_t* __restrict__ wq,
                                                             const float* __restrict__ sw, int64_t m,
                                                             int64_t n, int64_t k, void* __restrict__ y,
                                                             int y_dtype) {
    using C = Cfg<S>;
    constexpr int T = MW * 256;  // int32 of one wave's partial tile
    __shared__ int32_t red[WK * T];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q = lane >> 4;
    // W4A4 takes k % 128 == 64: a last piece of 64 codes, whose lane
    // quarters 2 and 3 (bytes 32 .. 63 of the piece) hold no codes
    const int pieces = static_cast<int>((k + C::PK - 1) / C::PK);
    const int p0 = wave * pieces / WK, p1 = (wave + 1) * pieces / WK;
    const int64_t col0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MW);
    const int64_t ka = C::A4 ? k / 2 : k, kb = C::B4 ? k / 2 : k;
    // lane (c, q): 16 bytes per operand word at byte offset (W8A8: 16 q, else
    // 16 q for int4 / 32 q for int8 operands) within a piece's row bytes
    const int qa = C::A4 ? 16 * q : (C::STEPS == 2 ? 32 * q : 16 * q);
    const int qb = C::B4 ? 16 * q : (C::STEPS == 2 ? 32 * q : 16 * q);

    // rows past m and columns past n read clamped, valid addresses; neither is stored
    const v4i* xp[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
        const int64_t r = row0 + 16 * mt + c16;
        xp[mt] = reinterpret_cast<const v4i*>(xq + (r < m ? r : m - 1) * ka + qa);
    }
    const int64_t cl = col0 + c16;
    const v4i* wp = reinterpret_cast<const v4i*>(wq + (cl < n ? cl : n - 1) * kb + qb);

    v4i acc[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) acc[mt] = v4i{0, 0, 0, 0};

    // two pieces per trip, both loaded before either is multiplied (a lone
    // last piece reloads itself: branch-free, every wait count static)
    const int64_t kbytes_row = C::A4 ? k / 2 : k;   // W4A4: bytes of a row
    for (int p = p0; p < p1; p += 2) {
        Piece<S, MW> f0, f1;
        const int p1st = p + 1 < p1 ? p + 1 : p;
        const bool ok0 = !C::A4 || static_cast<int64_t>(p) * 64 + 16 * q < kbytes_row;
        const bool ok1 = !C::A4 || static_cast<int64_t>(p1st) * 64 + 16 * q < kbytes_row;
        load_piece<S, MW>(f0, xp, wp, p, ok0);
        load_piece<S, MW>(f1, xp, wp, p1st, ok1);
        mma_piece<S, MW>(f0, acc);
        if (p + 1 < p1) mma_piece<S, MW>(f1, acc);
    }

    // partial tiles: [wave][mt][j][lane]; integer sums are exact in any order
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave * T + (mt * 4 + j) * 64 + lane] = acc[mt][j];
    __syncthreads();

    for (int o = tid; o < T; o += 64 * WK) {
        uint32_t u = 0;  // (modular adds: the exact total fits int32 for k < 2^17)
#pragma unroll
        for (int w = 0; w < WK; ++w) u += static_cast<uint32_t>(red[w * T + o]);
        const int32_t v = static_cast<int32_t>(u);
        const int ln = o & 63, j = (o >> 6) & 3, mt = o >> 8;
        const int64_t row = row0 + 16 * mt + 4 * (ln >> 4) + j;
        const int64_t col = col0 + (ln & 15);
        if (row >= m || col >= n) continue;
        const int64_t idx = row * n + col;
        if (y_dtype == I32) {
            static_cast<int32_t*>(y)[idx] = v >> C::ASH;
        } else {
            // the large-tile GEMM's epilogue: 2^-ASH joins the column scale exactly
            const float swc = sw[col] * (1.0f / static_cast<float>(1 << C::ASH));
            const float f = static_cast<float>(v) * sx[row] * swc;
            if (y_dtype == BF16) static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(f);
            else if (y_dtype == F16) static_cast<uint16_t*>(y)[idx] = f32_to_f16_bits(f);
            else static_cast<float*>(y)[idx] = f;
        }
    }
}

template <int S, int MW>
hipError_t launch_sm(const void* xq, const float* sx, const void* wq, const float* sw, int64_t m, int64_t n,
                     int64_t k, void* y, int y_dtype, hipStream_t st) {
    constexpr int WK = 8;
    dim3 grid(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>((m + 16 * MW - 1) / (16 * MW)));
    hipLaunchKernelGGL((skinny_int_kernel<S, MW, WK>), grid, dim3(64 * WK), 0, st,
                       static_cast<const uint8_t*>(xq), sx, static_cast<const uint8_t*>(wq), sw, m, n, k, y,
                       y_dtype);
    return hipGetLastError();
}

template <int S>
hipError_t launch_ss(const void* xq, const float* sx, const void* wq, const float* sw, int64_t m, int64_t n,
                     int64_t k, void* y, int y_dtype, hipStream_t st) {
    const int64_t tiles = (m + 15) / 16;
    if (tiles <= 1) return launch_sm<S, 1>(xq, sx, wq, sw, m, n, k, y, y_dtype, st);
    if (tiles <= 2) return launch_sm<S, 2>(xq, sx, wq, sw, m, n, k, y, y_dtype, st);
    if (tiles <= 3) return launch_sm<S, 3>(xq, sx, wq, sw, m, n, k, y, y_dtype, st);
    return launch_sm<S, 4>(xq, sx, wq, sw, m, n, k, y, y_dtype, st);
}

}  // namespace

hipError_t launch_skinny_int(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                             int64_t m, int64_t n, int64_t k, bool int4, bool a8, void* y, int y_dtype,
                             hipStream_t st) {
    if (int4 && !a8) return launch_ss<W4A4>(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, st);
    if (int4) return launch_ss<W4A8>(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, st);
    return launch_ss<W8A8>(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, st);
}

}  // namespace qlin
