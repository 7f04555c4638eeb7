// Integer GEMM with int32 accumulation and a fused dequantizing epilogue,
// for gfx950 (FoldQuantVLA abstract: W4A4 / W8A8 native integer execution of
// the projections).
//
//   acc[m][n] = sum_k A[m][k] * B[n][k]      A = activation codes, B = weight codes
//   y[m][n]   = round(fp32(acc) * x_scale[m] * w_scale[n])
//
// Both operands are k-contiguous ("NT"), which is the operand layout of the
// MFMA: a lane supplies 16 consecutive bytes of one row.  The contraction
// runs on v_mfma_i32_32x32x32_i8 (32x32 output tile, 32-deep k per issue).
// A and B are fed with the same lane -> k mapping, so the order in which the
// instruction walks k inside one issue does not matter for the exact sum.
//
// int4 operands: a packed byte holds element 2j (low nibble) and 2j+1 (high
// nibble).  (w << 4) & 0xF0F0F0F0 puts every low nibble in the high half of
// its byte and w & 0xF0F0F0F0 does the same for the high nibbles: each byte
// then reads as the signed int8 16*code.  Unpacking A and B alike keeps the
// pairing of k, the MFMA accumulates 256 * acc exactly (|256 * acc| <= 256 *
// k * 49 < 2^31 for k < 171196), and an arithmetic shift by 8 restores acc.
//
// Tiling: a 256-lane block (4 waves, 2 x 2) owns a BM x BN output tile; each
// wave owns (BM/2) x (BN/2) as (BM/64) x (BN/64) MFMA tiles held in
// accumulator registers.  K advances in stages of 64 bytes per row (64 int8
// or 128 int4 codes): 16-byte global loads into registers for stage s+1 are
// in flight while stage s is read from LDS (double buffer, rows padded to 80
// bytes so that 16-byte LDS reads of 8 consecutive rows hit distinct banks).
// Block indices are remapped so that each XCD (dispatch is round-robin over
// the 8 XCDs) works on a contiguous range of tiles with M fastest, which
// keeps a weight tile in one XCD's L2 while it is reused.
// Split-K writes int32 partial tiles; a second kernel sums them in a fixed
// order (integer addition: bit-exact) and applies the epilogue.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int STAGE_BYTES = 64;   // bytes of one row per pipeline stage
constexpr int LDS_PITCH = 80;     // padded LDS row pitch in bytes

struct GemmParams {
    const int8_t* a;      // [m][kbytes]
    const int8_t* b;      // [n][kbytes]
    const float* sx;      // [m]
    const float* sw;      // [n]
    void* y;              // [m][n]
    int32_t* ws;          // split-K partials [splits][m][n]
    int64_t m, n;
    int64_t kbytes;       // bytes per row of A and B
    int stages;           // ceil(kbytes / 64)
    int stages_per_split;
    int tiles_m, tiles_n, splits;
    int y_dtype;
};

__device__ __forceinline__ v4i unpack_lo(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    (void)w2; (void)w3;
    return v4i{static_cast<int>((w0 << 4) & 0xF0F0F0F0u), static_cast<int>((w1 << 4) & 0xF0F0F0F0u),
               static_cast<int>(w0 & 0xF0F0F0F0u), static_cast<int>(w1 & 0xF0F0F0F0u)};
}

__device__ __forceinline__ void store_out(void* y, int64_t idx, int dt, float v) {
    if (dt == BF16) {
        static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
    } else if (dt == F16) {
        static_cast<uint16_t*>(y)[idx] = f32_to_f16_bits(v);
    } else {
        static_cast<float*>(y)[idx] = v;
    }
}

// Stores one wave's accumulator tiles.  OUT = -1 writes raw int32 partials
// (split-K), I32 raw accumulators, else the dequantized value in that dtype.
// Accumulator r of a 32x32 MFMA tile sits at column lane%32 and row
// 8*(r/4) + 4*(lane/32) + r%4.
template <int TM, int TN, bool INT4, int OUT>
__device__ __forceinline__ void write_tile(const v16i (&acc)[TM][TN], const GemmParams& p,
                                           int64_t row_base, int64_t col_base, int lane, void* dst) {
    const int col_in = lane & 31;
    const int row_in = (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t col = col_base + j * 32 + col_in;
        const bool col_ok = col < p.n;
        float swv = 0.f;
        if constexpr (OUT == BF16 || OUT == F16 || OUT == F32) swv = col_ok ? p.sw[col] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row_base + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                int32_t a = acc[i][j][r];
                if constexpr (INT4) a >>= 8;
                if (col_ok && row < p.m) {
                    const int64_t idx = row * p.n + col;
                    if constexpr (OUT == -1 || OUT == I32) {
                        static_cast<int32_t*>(dst)[idx] = a;
                    } else {
                        const float v = static_cast<float>(a) * p.sx[row] * swv;
                        if constexpr (OUT == BF16) static_cast<uint16_t*>(dst)[idx] = f32_to_bf16_rne(v);
                        else if constexpr (OUT == F16) static_cast<uint16_t*>(dst)[idx] = f32_to_f16_bits(v);
                        else static_cast<float*>(dst)[idx] = v;
                    }
                }
            }
            // keep the scheduler from hoisting every accumulator read at once
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int BM, int BN, bool INT4, int OUT>
__global__ __launch_bounds__(256) void gemm_i8_kernel(GemmParams p) {
    constexpr int TM = BM / 64;            // MFMA tiles per wave along M
    constexpr int TN = BN / 64;            // ... along N
    constexpr int ALD = BM * 4 / 256;      // 16-byte loads per lane per stage (A)
    constexpr int BLD = BN * 4 / 256;
    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * LDS_PITCH];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][BN * LDS_PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware remap of the linear block index.
    const int nblocks = gridDim.x;
    int bid = blockIdx.x;
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    const int tiles_mn = p.tiles_m * p.tiles_n;
    const int split = bid / tiles_mn;
    const int t_mn = bid - split * tiles_mn;
    const int tile_n = t_mn / p.tiles_m;
    const int tile_m = t_mn - tile_n * p.tiles_m;
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
    const int s_begin = split * p.stages_per_split;
    int s_end = s_begin + p.stages_per_split;
    if (s_end > p.stages) s_end = p.stages;

    // Global loads go through buffer resources based at the tile's first
    // row: rows past the end of the matrix fall outside num_records and read
    // as zero, so ragged M / N tails need no clamping.  Lane tid loads row
    // tid/4 (+64 per extra load) at byte (tid%4)*16 of the stage.
    const int ld_row = tid >> 2;
    const int ld_col = (tid & 3) * 16;
    const int64_t a_rem = (p.m - m0) * p.kbytes;
    const int64_t b_rem = (p.n - n0) * p.kbytes;
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(p.a + m0 * p.kbytes), 0,
        static_cast<int>(a_rem < 0x7FFFFFFF ? a_rem : 0x7FFFFFFF), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(p.b + n0 * p.kbytes), 0,
        static_cast<int>(b_rem < 0x7FFFFFFF ? b_rem : 0x7FFFFFFF), 0x00020000);
    const int a_voff = ld_row * static_cast<int>(p.kbytes) + ld_col;
    const int row64 = 64 * static_cast<int>(p.kbytes);
    const int lds_wr = ld_row * LDS_PITCH + ld_col;

    uint4 ra[ALD], rb[BLD];
    auto gload = [&](int s) {
        const int kb = s * STAGE_BYTES;
        // A short last stage (int4 with k % 128 == 64) must not read into the
        // next row: its upper half gets offset 2^31, beyond every num_records.
        const bool kin = kb + ld_col < p.kbytes;
        const int off = a_voff + kb;
#pragma unroll
        for (int i = 0; i < ALD; ++i)
            ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rsrc_a, kin ? off + i * row64 : static_cast<int>(0x80000000u), 0, 0));
#pragma unroll
        for (int i = 0; i < BLD; ++i)
            rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rsrc_b, kin ? off + i * row64 : static_cast<int>(0x80000000u), 0, 0));
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ALD; ++i)
            *reinterpret_cast<uint4*>(&lds_a[buf][lds_wr + i * 64 * LDS_PITCH]) = ra[i];
#pragma unroll
        for (int i = 0; i < BLD; ++i)
            *reinterpret_cast<uint4*>(&lds_b[buf][lds_wr + i * 64 * LDS_PITCH]) = rb[i];
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // lane's LDS read offsets: row lane%32 of each 32-row tile, 16 bytes at
    // byte (lane/32)*16 of each 32-byte k-slice
    const int rd_row = lane & 31;
    const int rd_col = (lane >> 5) * 16;
    const int a_rd = (wm * (BM / 2) + rd_row) * LDS_PITCH + rd_col;
    const int b_rd = (wn * (BN / 2) + rd_row) * LDS_PITCH + rd_col;

    if (s_begin < s_end) {
        gload(s_begin);
        sstore(0);
    }
    __syncthreads();

    for (int s = s_begin; s < s_end; ++s) {
        const int buf = (s - s_begin) & 1;
        if (s + 1 < s_end) gload(s + 1);
        const int8_t* la = lds_a[buf];
        const int8_t* lb = lds_b[buf];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {   // two 32-byte slices per stage
            uint4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const uint4*>(la + a_rd + i * 32 * LDS_PITCH + ks * 32);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = *reinterpret_cast<const uint4*>(lb + b_rd + j * 32 * LDS_PITCH + ks * 32);
            if constexpr (INT4) {
                // 16 bytes = 32 codes per lane -> two MFMA operands
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v4i oa[TM], ob[TN];
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        oa[i] = h == 0 ? unpack_lo(fa[i].x, fa[i].y, 0, 0) : unpack_lo(fa[i].z, fa[i].w, 0, 0);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        ob[j] = h == 0 ? unpack_lo(fb[j].x, fb[j].y, 0, 0) : unpack_lo(fb[j].z, fb[j].w, 0, 0);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oa[i], ob[j], acc[i][j], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        v4i oa = {static_cast<int>(fa[i].x), static_cast<int>(fa[i].y),
                                  static_cast<int>(fa[i].z), static_cast<int>(fa[i].w)};
                        v4i ob = {static_cast<int>(fb[j].x), static_cast<int>(fb[j].y),
                                  static_cast<int>(fb[j].z), static_cast<int>(fb[j].w)};
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oa, ob, acc[i][j], 0, 0, 0);
                    }
            }
        }
        if (s + 1 < s_end) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    void* dst = (OUT == -1) ? static_cast<void*>(p.ws + static_cast<int64_t>(split) * p.m * p.n) : p.y;
    write_tile<TM, TN, INT4, OUT>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane, dst);
}

// Sum of split-K partials in split order, then the epilogue.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int32_t* ws, int splits, int64_t m,
                                                            int64_t n, const float* sx,
                                                            const float* sw, void* y, int y_dtype) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = m * n;
    if (i >= total) return;
    int32_t a = 0;
    for (int s = 0; s < splits; ++s) a += ws[static_cast<int64_t>(s) * total + i];
    if (y_dtype == I32) {
        static_cast<int32_t*>(y)[i] = a;
        return;
    }
    const int64_t row = i / n, col = i - row * n;
    store_out(y, i, y_dtype, static_cast<float>(a) * sx[row] * sw[col]);
}

template <int BM, int BN, bool INT4, int OUT>
hipError_t launch_tile(const GemmParams& p, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(p.tiles_m * p.tiles_n * p.splits));
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, INT4, OUT>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int BM, int BN, bool INT4>
hipError_t launch_out(const GemmParams& p, hipStream_t st) {
    if (p.splits > 1) return launch_tile<BM, BN, INT4, -1>(p, st);
    switch (p.y_dtype) {
        case BF16: return launch_tile<BM, BN, INT4, BF16>(p, st);
        case F16: return launch_tile<BM, BN, INT4, F16>(p, st);
        case F32: return launch_tile<BM, BN, INT4, F32>(p, st);
        case I32: return launch_tile<BM, BN, INT4, I32>(p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, bool int4) {
    GemmPlan g;
    g.bm = (m > 128) ? 256 : 128;
    g.bn = 256;
    const int64_t tiles = ((m + g.bm - 1) / g.bm) * ((n + g.bn - 1) / g.bn);
    const int64_t kbytes = int4 ? k / 2 : k;
    const int64_t stages = (kbytes + STAGE_BYTES - 1) / STAGE_BYTES;
    int splits = 1;
    // fill the 256 CUs when the tile grid is small, keeping >= 8 stages per split
    while (tiles * splits < 256 && stages / (splits * 2) >= 8) splits *= 2;
    g.splits = splits;
    g.ws_bytes = (splits > 1) ? static_cast<int64_t>(splits) * m * n * 4 : 0;
    return g;
}

hipError_t launch_gemm(const GemmPlan& plan, const void* xq, const float* x_scale, const void* wq,
                       const float* w_scale, int64_t m, int64_t n, int64_t k, bool int4, void* y,
                       int y_dtype, int32_t* ws, hipStream_t st) {
    GemmParams p;
    p.a = static_cast<const int8_t*>(xq);
    p.b = static_cast<const int8_t*>(wq);
    p.sx = x_scale; p.sw = w_scale; p.y = y; p.ws = ws;
    p.m = m; p.n = n;
    p.kbytes = int4 ? k / 2 : k;
    p.stages = static_cast<int>((p.kbytes + STAGE_BYTES - 1) / STAGE_BYTES);
    p.splits = plan.splits;
    p.stages_per_split = (p.stages + plan.splits - 1) / plan.splits;
    p.tiles_m = static_cast<int>((m + plan.bm - 1) / plan.bm);
    p.tiles_n = static_cast<int>((n + plan.bn - 1) / plan.bn);
    p.y_dtype = y_dtype;
    hipError_t e;
    if (plan.bm == 256) e = int4 ? launch_out<256, 256, true>(p, st) : launch_out<256, 256, false>(p, st);
    else e = int4 ? launch_out<128, 256, true>(p, st) : launch_out<128, 256, false>(p, st);
    if (e != hipSuccess) return e;
    if (plan.splits > 1) {
        const int64_t total = m * n;
        dim3 grid(static_cast<unsigned>((total + 255) / 256));
        hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, ws, plan.splits, m, n,
                           x_scale, w_scale, y, y_dtype);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace qlin
