// Weight-only int4 projection for 9..64 token rows (W4A16, group-128 fp16
// scales) on the gfx950 matrix cores.  The iterative action expert (FoldQuantVLA
// abstract; memory-bound per the LoopQ abstract) runs its projections on a
// small set of action tokens at every denoising step: too many rows for the
// vector GEMV (its dot products grow with m), too few for the large-tile
// GEMMs.  Here the packed weights are decoded to exact fp16 integers in
// registers and multiplied with the fp16 activations by v_mfma_f32_16x16x32_f16.
//
//   y[m][n] = fp16( sum_g s16[n][g] * sum_{k in g} x[m][k] * code[n][k] )
//
// Each group's inner sum is accumulated on its own (fp32, products exact),
// then scaled and added, so the order of operations is the definition's.
//
// Work split.  A block owns a strip of 16 output columns and 16 MW token rows
// (blockIdx.y walks the rows); its WK waves take contiguous slices of the k
// groups.  A wave accumulates its slice in registers; the WK partial tiles are
// added in LDS in a fixed order, so results do not depend on timing.
//
// Staging.  The MFMA operand layout gives each load instruction 16 rows and
// 32 cache lines if x is read straight into registers, and the L1 then runs
// at about half its byte rate.  So a wave copies its group of x rows into LDS
// with LDS-DMA loads that each cover four whole rows (eight lines), swizzled
// so that the fragment reads below hit every LDS bank once.
//
// MFMA k slots.  Lane l = c + 16 q (c = l % 16, q = l / 16) feeds row (A) or
// column (B) c, eight k values per step.  Within a group, step s (0..3) gives
// lane quarter q the codes k = 128 g + 32 q + 8 s + e, e = 0..7: over a group
// a lane then reads one 16-byte word of packed weights (32 codes) and 64
// contiguous bytes of each of its x rows.  A and B use the same assignment,
// which is all the contraction needs.
//
// Decoding.  Byte b of a weight dword holds codes 2b (low nibble) and 2b+1
// (high nibble).  v_perm places that byte under an fp16 exponent byte 0x64 in
// both halves of a dword; a mask keeps the low nibble in the low half and the
// high nibble in the high half and an xor adds 8 to each (two's complement ->
// offset binary), giving the fp16 values 1024 + (c + 8) and 1024 + 16 (c + 8).
// One packed fp16 fma with (1, 1/16) and (-1032, -72) leaves c in both halves
// exactly.  Four such pairs give the eight codes of a step in k order.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ h2 decode_pair(uint32_t t, uint32_t sel) {
    uint32_t p = __builtin_amdgcn_perm(0x64646464u, t, sel);
    p = (p & 0xFFF0FF0Fu) ^ 0x00800008u;
    const h2 mul = {static_cast<_Float16>(1.0f), static_cast<_Float16>(0.0625f)};
    const h2 add = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-72.0f)};
    return __builtin_elementwise_fma(__builtin_bit_cast(h2, p), mul, add);
}

// Codes 0..7 of a dword as exact fp16 values, in k order.
__device__ __forceinline__ h8 decode8(int w) {
    const uint32_t t = static_cast<uint32_t>(w);
    const h2 p0 = decode_pair(t, 0x04000400u);
    const h2 p1 = decode_pair(t, 0x04010401u);
    const h2 p2 = decode_pair(t, 0x04020402u);
    const h2 p3 = decode_pair(t, 0x04030403u);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Waits until at most N of this wave's vector-memory operations are
// outstanding.  Every vector-memory load in the main loop is one of the DMA
// loads below, so the counts are exact.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte load of every lane from rsrc + voff straight into LDS at
// lds_addr + 16 * lane (LDS DMA through M0); offsets at or past the
// descriptor's size fetch nothing.  Inline assembly, so that the compiler adds
// no waits of its own behind it; the kernel orders it with wait_vm.  No
// register result: the address operand is read at issue.
__device__ __forceinline__ void dma_lds16(v4i rsrc, int voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory", "m0");
}

// LDS of one staged group: the x rows of the block's row tile (16 MW rows of
// 256 bytes = 128 fp16; the sixteen 16-byte pieces of row r sit at slots
// piece ^ (r & 15)), then the strip's packed weights as the lanes load them.
template <int MW>
struct Stage {
    static constexpr int XB = MW * 16 * 256;
    static constexpr int BYTES = XB + 1024;
};

// Issues the DMA loads of group g into the stage at lds_addr: up to 4 MW
// loads of four x rows each (the group's 256 bytes of a row are two whole
// cache lines), then one of the weights (lane c + 16 q: column c, bytes
// 16 q .. 16 q + 15 of the group's 64).  Rows past m and columns past n lie
// beyond the descriptors (rows = m - first row of the tile, wave-uniform).
// The stage's rows past m keep stale values: they only reach output rows
// that are not stored.
template <int MW>
__device__ __forceinline__ void stage_group(const v4i& rs_x, const v4i& rs_w, int g, int kb2, int kb,
                                            int lane, uint32_t lds_addr, int rows) {
    const int rl = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < 4 * MW; ++i) {
        const int r = 4 * i + rl;
        if (4 * i < rows)  // (loads of four rows all past m are not issued)
            dma_lds16(rs_x, r * kb2 + g * 256 + 16 * (p ^ (r & 15)), lds_addr + i * 1024);
    }
    dma_lds16(rs_w, p * kb + g * 64 + 16 * rl, lds_addr + Stage<MW>::XB);
}

// The products of one staged group, scaled by the group's scale and added to
// acc.  Lane (c, q) reads row 16 mt + c, piece 4 q + s of the x slice and its
// own 16 bytes of weights.
template <int MW>
__device__ __forceinline__ void mma_stage(const uint8_t* st, int lane, float scale, f4 (&acc)[MW]) {
    const int c = lane & 15, q = lane >> 4;
    const v4i bw = *reinterpret_cast<const v4i*>(st + Stage<MW>::XB + 16 * lane);
    v4i a[MW][4];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            a[mt][s] = *reinterpret_cast<const v4i*>(st + (16 * mt + c) * 256 + 16 * ((4 * q + s) ^ c));
    f4 part[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) part[mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const h8 bv = decode8(bw[s]);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            part[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a[mt][s]), bv, part[mt], 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][j] = __builtin_fmaf(scale, part[mt][j], acc[mt][j]);
}

// Block: one strip of 16 output columns, 16 MW token rows (blockIdx.y), WK
// waves each taking a contiguous slice of the k groups.  A wave stages one
// group at a time; with two waves per SIMD the other wave's products run
// while one waits for its loads.
template <int MW, int WK>
__global__ __launch_bounds__(64 * WK) void skinny_w4a16_kernel(const _Float16* __restrict__ x,
                                                               const uint8_t* __restrict__ wq,
                                                               const _Float16* __restrict__ ws,
                                                               int64_t m, int64_t n, int64_t k,
                                                               _Float16* __restrict__ y) {
    constexpr int SB = Stage<MW>::BYTES;
    constexpr int T = MW * 256;              // floats of one wave's partial tile
    constexpr int STAGING = WK * SB;
    constexpr int RED = WK * T * 4;
    __shared__ __align__(16) uint8_t lds[STAGING > RED ? STAGING : RED];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int groups = static_cast<int>(k / 128);
    const int g0 = wave * groups / WK, g1 = (wave + 1) * groups / WK;
    const int64_t col0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t row0 = static_cast<int64_t>(blockIdx.y) * (16 * MW);
    const int rows = __builtin_amdgcn_readfirstlane(static_cast<int>(m - row0 < 16 * MW ? m - row0 : 16 * MW));
    const int kb = static_cast<int>(k / 2), kb2 = static_cast<int>(k * 2);
    const v4i rs_x = make_rsrc(x + row0 * k, (m - row0) * k * 2);
    const v4i rs_w = make_rsrc(wq + col0 * (k / 2), (n - col0) * (k / 2));
    const int64_t col = col0 + (lane & 15);
    const _Float16* srow = ws + (col < n ? col : n - 1) * groups;
    const float ok = col < n ? 1.f : 0.f;
    uint8_t* mine = lds + wave * SB;
    const uint32_t mine_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(mine));

    f4 acc[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};

    if (g0 < g1) {
        // Scales are converted where they are needed anyway (the empty asm pins
        // the conversion, and with it the compiler's wait for the load, there:
        // placed later, that wait would also cover DMA loads in flight).  The
        // first group's scale load goes out behind its DMA, so both travel together.
        stage_group<MW>(rs_x, rs_w, g0, kb2, kb, lane, mine_addr, rows);
        float sc = static_cast<float>(srow[g0]) * ok;
        asm volatile("" : "+v"(sc));
        for (int g = g0; g < g1; ++g) {
            const bool more = g + 1 < g1;
            const _Float16 sh = srow[more ? g + 1 : g];
            wait_vm<0>();  // the stage and the scale load are complete
            float sn = static_cast<float>(sh) * ok;
            asm volatile("" : "+v"(sn));
            mma_stage<MW>(mine, lane, sc, acc);
            if (more) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every read of the stage is back
                stage_group<MW>(rs_x, rs_w, g + 1, kb2, kb, lane, mine_addr, rows);
            }
            sc = sn;
        }
    }
    __syncthreads();  // every stage read: the LDS now takes the partial tiles

    // partial tiles: [wave][mt][j][lane], 64 consecutive floats per store
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave * T + (mt * 4 + j) * 64 + lane] = acc[mt][j];
    __syncthreads();

    // each output: the WK partials added in slice order
    for (int o = tid; o < T; o += 64 * WK) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WK; ++w) v += red[w * T + o];
        const int ln = o & 63, j = (o >> 6) & 3, mt = o >> 8;
        const int64_t row = row0 + 16 * mt + 4 * (ln >> 4) + j;
        const int64_t cl = col0 + (ln & 15);
        if (row < m && cl < n) y[row * n + cl] = static_cast<_Float16>(v);
    }
}

template <int MW>
hipError_t launch_mw(const void* x, const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                     void* y, hipStream_t st) {
    constexpr int WK = 8;  // slices of the k groups (waves per block)
    dim3 grid(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>((m + 16 * MW - 1) / (16 * MW)));
    hipLaunchKernelGGL((skinny_w4a16_kernel<MW, WK>), grid, dim3(64 * WK), 0, st,
                       static_cast<const _Float16*>(x), static_cast<const uint8_t*>(wq),
                       static_cast<const _Float16*>(ws), m, n, k, static_cast<_Float16*>(y));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                               int64_t n, int64_t k, void* y, hipStream_t st) {
    const int64_t tiles = (m + 15) / 16;
    if (tiles <= 1) return launch_mw<1>(x, wq, w_scale, m, n, k, y, st);
    if (tiles <= 2) return launch_mw<2>(x, wq, w_scale, m, n, k, y, st);
    if (tiles <= 3) return launch_mw<3>(x, wq, w_scale, m, n, k, y, st);
    return launch_mw<4>(x, wq, w_scale, m, n, k, y, st);
}

}  // namespace qlin
