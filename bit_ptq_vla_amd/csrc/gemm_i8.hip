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
// or 128 int4 codes).  Stages land in a ring of NS LDS buffers by LDS DMA
// (buffer_load ... lds, 16 bytes per lane, no register round trip), issued
// NS-1 stages ahead; one s_waitcnt + s_barrier per stage publishes a stage
// and retires the buffer the next DMA overwrites.  Within a stage buffer the
// four 16-byte chunks of a row are XOR-swizzled so that the MFMA operand
// reads (ds_read_b128, 32 rows x one chunk) are bank-conflict free.
// Block indices are remapped so that each XCD (dispatch is round-robin over
// the 8 XCDs) works on a contiguous range of tiles with M fastest, which
// keeps a weight tile in one XCD's L2 while it is reused.
// The epilogue stages each wave's tile through LDS and writes 16-byte rows.
// Split-K writes int32 partial tiles; a second kernel sums them in a fixed
// order (integer addition: bit-exact) and applies the epilogue.

#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

constexpr int STAGE_BYTES = 64;   // bytes of one row per pipeline stage
constexpr int OOB_OFFSET = 0x7FFFFFF0;   // a buffer offset past every range: the hardware returns zeros

// f(std::integral_constant<int, Q>) for Q = B .. E-1 in order: loop bodies whose
// indices must be compile-time constants (register arrays, instruction order).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

struct GemmParams {
    const int8_t* a;      // [m][kbytes]
    const int8_t* b;      // [n][kbytes]
    const float* sx;      // [m]
    const float* sw;      // [n]
    void* y;              // [m][n]
    int32_t* ws;          // split-K partials [splits][m][n]
    int64_t m, n;
    int64_t kbytes;       // bytes per row of B (and of A, except W4A8)
    int64_t kbytes_a;     // bytes per row of A
    int stages;           // ceil(kbytes / 64)
    int stages_per_split;
    int tiles_m, tiles_n, splits;
    int group_m;          // tile order: 0 = rows fastest over the whole grid, else groups of group_m tile rows
    int y_dtype;
};

// OUT codes of the epilogue: -1 raw int32 split-K partials, a dtype (F16,
// BF16, F32, I32), or OUT_GEGLU + dtype for the fused GeGLU output.
constexpr int OUT_GEGLU = 16;

// 16 packed int4 codes (two dwords) -> one MFMA operand of 16 int8 values 16 * code:
// the even codes of both dwords, then the odd codes.
__device__ __forceinline__ v4i unpack_int4(uint32_t w0, uint32_t w1) {
    return v4i{static_cast<int>((w0 << 4) & 0xF0F0F0F0u), static_cast<int>((w1 << 4) & 0xF0F0F0F0u),
               static_cast<int>(w0 & 0xF0F0F0F0u), static_cast<int>(w1 & 0xF0F0F0F0u)};
}

// 16 int8 values k0..k15 (W4A8 activations) in the k order of unpack_int4:
// k 0 2 4 6 | 8 10 12 14 | 1 3 5 7 | 9 11 13 15 (v_perm_b32 byte selects).
__device__ __forceinline__ v4i order_int8_as_int4(uint4 d) {
    return v4i{static_cast<int>(__builtin_amdgcn_perm(d.y, d.x, 0x06040200u)),
               static_cast<int>(__builtin_amdgcn_perm(d.w, d.z, 0x06040200u)),
               static_cast<int>(__builtin_amdgcn_perm(d.y, d.x, 0x07050301u)),
               static_cast<int>(__builtin_amdgcn_perm(d.w, d.z, 0x07050301u))};
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

// LDS layout of one pipeline stage: row r of a tile holds 64 bytes as four
// 16-byte chunks; chunk c is stored at chunk slot c ^ swz(r).  The MFMA
// operand read (ds_read_b128: lane l reads chunk c (+1 for l >= 32) of row
// l % 32) is free of bank conflicts with this choice of swz on gfx950, by
// counter measurement (SQ_LDS_BANK_CONFLICT zero, against two-way conflicts
// for ((r >> 1) ^ (r >> 3)) & 3 and four-way without a swizzle).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
// The same for 128-byte rows (eight chunks, W4A8's A operand), also measured
// conflict-free: (r >> 1) & 7.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Waits until at most N of this wave's vector-memory operations (here: the
// DMA loads into LDS) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most `after` groups of L loads are outstanding, for a
// runtime after <= A (compile-time counts: one s_waitcnt per branch).
template <int L, int A>
__device__ __forceinline__ void wait_groups(int after) {
    if constexpr (A <= 0) {
        wait_vmcnt<0>();
    } else {
        if (after >= A) wait_vmcnt<A * L>();
        else wait_groups<L, A - 1>(after);
    }
}

// 16-byte load of every lane from rsrc + voff straight into LDS at
// lds_addr + 16 * lane (LDS DMA through M0).  Offsets at or past num_records
// fetch nothing.  Written as inline assembly so that the compiler does not
// add its own conservative waits on LDS reads behind it: the caller orders
// the DMA with explicit s_waitcnt vmcnt + s_barrier.  The instruction has no
// register result; its address operand is read at issue.
__device__ __forceinline__ void dma16(v4i rsrc, int voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_addr)
        : "memory", "m0");
}

// ---- GeLU for the fused GeGLU epilogue -------------------------------------

// max(g, 0) for the bfloat16 g in the low half of w, in one instruction.
// fmaxf on the bit-cast value first quiets it (v_max x, x, x), since the
// compiler cannot tell that a value produced by v_cvt_pk_bf16_f32 is never a
// signalling NaN; for every other input the result is fmaxf's.
__device__ __forceinline__ float relu_bf16_word(uint32_t w) {
    float r;
    asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(__uint_as_float(w << 16)));
    return r;
}
// T(x) = x * Phi(-x) = -gelu(-x) for the bfloat16 values 2^-12 <= x < 16
// (16 exponents x 128 mantissas, 8 KB), evaluated in float64 through erfc
// and rounded to fp32.  Then gelu(g) = -T(|g|) for g < 0 and g - T(g) for
// g > 0: both within about one fp32 rounding of the exact value (T is the
// small part of gelu(g) = g - T for g > 0, so the subtraction loses nothing).
// |g| < 2^-12: g/2 + g^2/sqrt(2 pi) (the next term is 2^-36 relative);
// |g| >= 16: g or 0 (T(16) ~ 1e-56).
constexpr int GTAB_EF0 = 127 - 12;
constexpr int GTAB_N = 16 * 128;
constexpr int GTAB_BYTES = GTAB_N * 4;

__device__ float g_gelu_neg_tab[GTAB_N];

__global__ void gelu_neg_tab_init_kernel() {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= GTAB_N) return;
    const double x = static_cast<double>(__uint_as_float(static_cast<uint32_t>(i + (GTAB_EF0 << 7)) << 16));
    g_gelu_neg_tab[i] = static_cast<float>(0.5 * x * erfc(x * 0.70710678118654752440));
}

// gelu of a bfloat16 value (bits) that the table does not cover
__device__ __forceinline__ float gelu_outside_tab(uint32_t bits) {
    const float g = __uint_as_float(bits << 16);
    const float tiny = fmaf(g * g, 0.39894228040143267794f, 0.5f * g);
    const float big = g > 0.f ? g : (g == g ? 0.f : g);
    return (((bits & 0x7FFFu) >> 7) < static_cast<uint32_t>(GTAB_EF0)) ? tiny : big;
}

// GeGLU epilogue of a wave's (BM/2) x (BN/2) tile whose columns are gate and
// up rows of W interleaved in blocks of 32: MFMA column tiles 2q (gate) and
// 2q+1 (up) hold the same output channels, so a lane has g and u of one
// element in registers.  g and u are dequantized in fp32 and rounded to
// bfloat16 (as the unfused chain stores them), gelu(g) is formed from the
// T table kept in LDS (16 table reads in flight per group, one branch per
// group for values outside it), h = gelu(g) * u is rounded to the output
// dtype and staged through LDS for 16-byte row stores of the (BM/2) x (BN/4)
// h tile.  V: v16i (int32 accumulators) or v16f (fp32 accumulators holding
// exact integers).
template <int BM, int BN, int ASH, int ODT, int STAGE, typename V>
__device__ __forceinline__ void store_tile_geglu(const V (&acc)[BM / 64][BN / 64], const GemmParams& p,
                                                 int64_t row0, int64_t col0, int lane, const float* tab,
                                                 int8_t* region) {
    constexpr int TM = BM / 64, TN = BN / 64;
    static_assert(TN % 2 == 0, "gate/up column tiles come in pairs");
    constexpr int WM = BM / 2, WH = BN / 4;              // wave tile rows, h columns
    constexpr int E = (ODT == BF16 || ODT == F16) ? 2 : 4;
    constexpr int ROWB = WH * E;
    constexpr int PITCH = ROWB + (E == 2 ? 16 : 32);
    constexpr int RP = (WM * PITCH <= STAGE) ? WM : (WM / 2 * PITCH <= STAGE) ? WM / 2 : 16;
    static_assert(RP >= 16 && WM % RP == 0 && RP * PITCH <= STAGE, "staging does not fit");
    constexpr int CPR = ROWB / 16;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t nh = p.n / 2;                          // h columns
    const int64_t hcol0 = col0 / 2;

    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sx), 0, static_cast<int>(p.m * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sw), 0, static_cast<int>(p.n * 4), 0x00020000);
    float swg[TN / 2], swu[TN / 2];
#pragma unroll
    for (int q = 0; q < TN / 2; ++q) {
        swg[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rs_w, static_cast<int>((col0 + 64 * q + l32) * 4), 0, 0));
        swu[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rs_w, static_cast<int>((col0 + 64 * q + 32 + l32) * 4), 0, 0));
        if constexpr (ASH > 0) {   // the accumulator holds 2^ASH * acc; the power of two is exact
            swg[q] *= 1.0f / static_cast<float>(1 << ASH);
            swu[q] *= 1.0f / static_cast<float>(1 << ASH);
        }
    }
    const bool vec_ok = ((nh * E) & 15) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;

#pragma unroll
    for (int pass = 0; pass < WM / RP; ++pass) {
#pragma unroll
        for (int rr = 0; rr < RP; rr += 32) {
            const int i = (pass * RP + rr) / 32;
            f4 sxv[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                sxv[g4] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                    rs_x, static_cast<int>((row0 + i * 32 + 8 * g4 + 4 * half) * 4), 0, 0));
#pragma unroll
            for (int q = 0; q < TN / 2; ++q) {
                // The 16 values of a lane: g and u rounded to bfloat16 by one
                // conversion (g low half, u high half), the table byte offset of
                // |g| formed from that word, all table reads in flight together.
                // toff = 4 * (|g| bits - first tabulated) keeps bits 13..16 clear
                // exactly when the table covers |g| (a borrow or an overflow sets
                // them); one branch per group for values outside the table.
                uint32_t pk[16], toff[16];
                uint32_t any = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sx = sxv[r >> 2][r & 3];
                    const float g = static_cast<float>(acc[i][2 * q][r]) * sx * swg[q];
                    const float u = static_cast<float>(acc[i][2 * q + 1][r]) * sx * swu[q];
                    pk[r] = pk_bf16(g, u);
                    toff[r] = (pk[r] << 2) - static_cast<uint32_t>(GTAB_EF0 << 9);
                    any |= toff[r];
                }
                float gl[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float t = *reinterpret_cast<const float*>(reinterpret_cast<const int8_t*>(tab) +
                                                                    (toff[r] & 0x1FFCu));
                    gl[r] = relu_bf16_word(pk[r]) - t;   // relu(g) - T(|g|)
                }
                if (any & 0x1E000u) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (toff[r] & 0x1E000u) gl[r] = gelu_outside_tab(pk[r] & 0xFFFFu);
                }
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int rl = rr + 8 * (r >> 2) + 4 * half + (r & 3);   // rows rl, rl + 1
                    if (RP < 32 && rl >= RP) continue;
                    const float h0 = gl[r] * __uint_as_float(pk[r] & 0xFFFF0000u);
                    const float h1 = gl[r + 1] * __uint_as_float(pk[r + 1] & 0xFFFF0000u);
                    int8_t* at = region + rl * PITCH + (q * 32 + l32) * E;
                    if constexpr (ODT == BF16) {
                        const uint32_t hp = pk_bf16(h0, h1);
                        *reinterpret_cast<uint16_t*>(at) = static_cast<uint16_t>(hp);
                        *reinterpret_cast<uint16_t*>(at + PITCH) = static_cast<uint16_t>(hp >> 16);
                    } else if constexpr (ODT == F16) {
                        *reinterpret_cast<uint16_t*>(at) = f32_to_f16_bits(h0);
                        *reinterpret_cast<uint16_t*>(at + PITCH) = f32_to_f16_bits(h1);
                    } else {
                        *reinterpret_cast<float*>(at) = h0;
                        *reinterpret_cast<float*>(at + PITCH) = h1;
                    }
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
#pragma unroll 4
        for (int c = lane; c < RP * CPR; c += 64) {
            const int rl = c / CPR, cc = c - rl * CPR;
            const uint4 v = *reinterpret_cast<const uint4*>(region + rl * PITCH + cc * 16);
            const int64_t gr = row0 + pass * RP + rl;
            const int64_t gc = hcol0 + cc * (16 / E);
            if (gr < p.m) {
                char* out = static_cast<char*>(p.y) + (gr * nh + gc) * E;
                if (vec_ok && gc + 16 / E <= nh) {
                    __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(out));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 16 / E; ++e) {
                        if (gc + e < nh) {
                            if constexpr (E == 2)
                                reinterpret_cast<uint16_t*>(out)[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
                            else
                                reinterpret_cast<uint32_t*>(out)[e] = w[e];
                        }
                    }
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    }
}

// Stores a wave's (BM/2) x (BN/2) accumulator tile through LDS so that the
// global writes are 16-byte, row-contiguous stores.  The wave owns one LDS
// ring buffer (STAGE bytes) after the main loop.  Rows are staged RP at a
// time; the staged row pitch is padded (16 B for 2-byte, 32 B for 4-byte
// elements) so that the two half-waves, which write rows 4 apart, hit
// different banks.  OUT: -1 raw int32 partial, I32 raw accumulators, else
// the dequantized value acc * x_scale[row] * w_scale[col] rounded to OUT.
template <int BM, int BN, int ASH, int OUT, int STAGE, typename V>
__device__ __forceinline__ void store_tile_lds(const V (&acc)[BM / 64][BN / 64], const GemmParams& p,
                                               int64_t row0, int64_t col0, int lane, int8_t* region,
                                               void* dst) {
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr bool FLOAT_OUT = (OUT == BF16 || OUT == F16 || OUT == F32);
    constexpr int E = (OUT == BF16 || OUT == F16) ? 2 : 4;
    constexpr int ROWB = WN * E;
    constexpr int PITCH = ROWB + (E == 2 ? 16 : 32);
    // staged rows per pass: the largest WM / 2^j that fits the buffer
    constexpr int RP = (WM * PITCH <= STAGE) ? WM : (WM / 2 * PITCH <= STAGE) ? WM / 2
                     : (WM / 4 * PITCH <= STAGE) ? WM / 4 : 32;
    static_assert(RP >= 32 && WM % RP == 0, "staging does not fit");
    constexpr int TPP = RP / 32;                        // MFMA row tiles per pass
    constexpr int CPR = ROWB / 16;                      // 16-byte chunks per row
    const int l32 = lane & 31, half = lane >> 5;

    // scales through buffer loads: out-of-range rows / columns read as 0
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sx), 0, static_cast<int>(FLOAT_OUT ? p.m * 4 : 0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sw), 0, static_cast<int>(FLOAT_OUT ? p.n * 4 : 0), 0x00020000);
    float swv[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        swv[j] = 0.f;
        if constexpr (FLOAT_OUT)
            swv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rs_w, static_cast<int>((col0 + j * 32 + l32) * 4), 0, 0));
        // int4 operands: the accumulator holds 2^ASH * acc; scaling by a power of
        // two commutes with fp32 rounding, so 2^-ASH joins the column scale exactly
        if constexpr (FLOAT_OUT && ASH > 0) swv[j] *= 1.0f / static_cast<float>(1 << ASH);
    }
    const int64_t ldy = p.n;
    const bool vec_ok = ((p.n * E) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;

#pragma unroll
    for (int pass = 0; pass < WM / RP; ++pass) {
        // ---- accumulators -> LDS (MFMA layout: column lane%32, row 8(r/4) + 4(lane/32) + r%4)
#pragma unroll
        for (int ti = 0; ti < TPP; ++ti) {
            const int i = pass * TPP + ti;
            f4 sxv[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                sxv[g] = f4{0.f, 0.f, 0.f, 0.f};
                if constexpr (FLOAT_OUT)
                    sxv[g] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                        rs_x, static_cast<int>((row0 + i * 32 + 8 * g + 4 * half) * 4), 0, 0));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    // rows rl and rl + 1 of this lane's column
                    const int rl = ti * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    int8_t* at = region + rl * PITCH + (j * 32 + l32) * E;
                    // (an fp32 accumulator holds an exact integer)
                    int32_t a0 = static_cast<int32_t>(acc[i][j][r]), a1 = static_cast<int32_t>(acc[i][j][r + 1]);
                    if constexpr (FLOAT_OUT) {
                        const float v0 = static_cast<float>(a0) * sxv[r >> 2][r & 3] * swv[j];
                        const float v1 = static_cast<float>(a1) * sxv[r >> 2][(r & 3) + 1] * swv[j];
                        if constexpr (OUT == BF16) {
                            const uint32_t vp = pk_bf16(v0, v1);
                            *reinterpret_cast<uint16_t*>(at) = static_cast<uint16_t>(vp);
                            *reinterpret_cast<uint16_t*>(at + PITCH) = static_cast<uint16_t>(vp >> 16);
                        } else if constexpr (OUT == F16) {
                            *reinterpret_cast<uint16_t*>(at) = f32_to_f16_bits(v0);
                            *reinterpret_cast<uint16_t*>(at + PITCH) = f32_to_f16_bits(v1);
                        } else {
                            *reinterpret_cast<float*>(at) = v0;
                            *reinterpret_cast<float*>(at + PITCH) = v1;
                        }
                    } else {
                        if constexpr (ASH > 0) { a0 >>= ASH; a1 >>= ASH; }
                        *reinterpret_cast<int32_t*>(at) = a0;
                        *reinterpret_cast<int32_t*>(at + PITCH) = a1;
                    }
                }
            }
        }
        // the wave's own LDS writes complete before it reads them back
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        // ---- LDS -> global, 16 bytes per lane
#pragma unroll 4
        for (int c = lane; c < RP * CPR; c += 64) {
            const int rl = c / CPR, cc = c - rl * CPR;
            const uint4 v = *reinterpret_cast<const uint4*>(region + rl * PITCH + cc * 16);
            const int64_t gr = row0 + pass * RP + rl;
            const int64_t gc = col0 + cc * (16 / E);
            if (gr < p.m) {
                char* out = static_cast<char*>(dst) + (gr * ldy + gc) * E;
                if (vec_ok && gc + 16 / E <= p.n) {
                    __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(out));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 16 / E; ++e) {
                        if (gc + e < p.n) {
                            if constexpr (E == 2)
                                reinterpret_cast<uint16_t*>(out)[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
                            else
                                reinterpret_cast<uint32_t*>(out)[e] = w[e];
                        }
                    }
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    }
}

// INT4: B (weights) is packed int4.  A8 (with INT4): A (activations) is
// int8 while B is int4 (W4A8); a stage then holds 128 k: 128 bytes of an A
// row and 64 bytes of a B row.
template <int BM, int BN, int MINB, int NS, bool INT4, int OUT, bool A8 = false>
__global__ __launch_bounds__(256, MINB) void gemm_i8_kernel(GemmParams p) {
    static_assert(!A8 || INT4, "W4A8 takes int4 weights");
    // NS: pipeline stages (ring of LDS buffers)
    constexpr int TM = BM / 64;                  // MFMA tiles per wave along M
    constexpr int TN = BN / 64;                  // ... along N
    constexpr int SA = A8 ? 2 * STAGE_BYTES : STAGE_BYTES;   // A bytes per row per stage
    constexpr int A_INSTR = BM * SA / 4096;      // 16-byte DMA loads per lane per stage (A)
    constexpr int B_INSTR = BN / 64;
    constexpr int LOADS = A_INSTR + B_INSTR;     // per lane per stage
    constexpr int STAGE = BM * SA + BN * STAGE_BYTES;
    constexpr int ASH = A8 ? 4 : (INT4 ? 8 : 0);   // accumulator = 2^ASH * acc
    // The DMA is issued through inline assembly, invisible to the compiler,
    // so one array serves the whole ring (and the epilogue staging after it).
    // The fused GeGLU epilogue keeps its GeLU table at LDS offset 0 (table reads
    // then take no base address) from the start; the ring follows it.
    constexpr bool GEGLU = OUT >= OUT_GEGLU;
    constexpr int RING0 = GEGLU ? GTAB_BYTES : 0;
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING0 + NS * STAGE];
    int8_t* const ring = lds + RING0;

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
    int tile_m, tile_n;
    if (p.group_m > 0) {
        // Groups of group_m tile rows, rows fastest inside a group: the tiles an
        // XCD runs at once form a group_m x (CUs / group_m) patch, so each A
        // panel is shared by the patch's columns and each B panel by its rows
        // while they stream through that XCD's L2 (long k: the panels do not
        // fit, only their current k-slabs do).
        const int per_group = p.group_m * p.tiles_n;
        const int g = t_mn / per_group;
        const int first = g * p.group_m;
        const int rows = (p.tiles_m - first) < p.group_m ? (p.tiles_m - first) : p.group_m;
        const int r = t_mn - g * per_group;
        tile_n = r / rows;
        tile_m = first + (r - tile_n * rows);
    } else {
        tile_n = t_mn / p.tiles_m;
        tile_m = t_mn - tile_n * p.tiles_m;
    }
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
    const int s_begin = split * p.stages_per_split;
    int s_end = s_begin + p.stages_per_split;
    if (s_end > p.stages) s_end = p.stages;
    const int nst = s_end > s_begin ? s_end - s_begin : 0;

    // Buffer resources based at the tile's first row: rows past the matrix
    // are out of range (the hardware returns zeros, nothing is fetched).
    const int64_t a_rem = (p.m - m0) * p.kbytes_a;
    const int64_t b_rem = (p.n - n0) * p.kbytes;
    const v4i rsrc_a = make_rsrc(p.a + m0 * p.kbytes_a, a_rem);
    const v4i rsrc_b = make_rsrc(p.b + n0 * p.kbytes, b_rem);

    // DMA mapping: load instruction i of wave w fills LDS chunk slots
    // [(4i + w) * 64, +64) of its operand, i.e. 16 rows; lane l fills slot
    // P = (4i + w) * 64 + l = row (P >> 2), slot (P & 3), so it fetches the
    // row's chunk (P & 3) ^ swz(row).
    // W4A8's 128-byte A rows: eight chunks, 8 rows per instruction and wave,
    // slot P -> row P >> 3, chunk (P & 7) ^ swz8(row).
    const int dma_row0 = wave * 16 + (lane >> 2);            // + 64 * i
    const int dma_chunk = (lane & 3) ^ swz(dma_row0);        // swz(row + 64 i) == swz(row)
    const int dma_voff = dma_row0 * static_cast<int>(p.kbytes) + dma_chunk * 16;
    const int row64 = 64 * static_cast<int>(p.kbytes);
    const int dma_row0_a = A8 ? wave * 8 + (lane >> 3) : dma_row0;   // + 32 * i (A8)
    const int dma_chunk_a = A8 ? (lane & 7) ^ swz8(dma_row0_a) : dma_chunk;   // swz8(row + 32 i) == swz8(row)
    const int dma_voff_a = dma_row0_a * static_cast<int>(p.kbytes_a) + dma_chunk_a * 16;
    const int rowstep_a = (A8 ? 32 : 64) * static_cast<int>(p.kbytes_a);

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // W4A4 with k % 128 == 64: the last stage holds 32 bytes of each row; the
    // lanes of its other two chunks take an offset past the buffer range, so
    // those LDS chunks receive zeros (which add nothing) instead of the next
    // row's bytes.  Both operands share the lane's chunk.
    const int kbytes_i = static_cast<int>(p.kbytes);
    auto issue = [&](int st, int8_t* buf) {
        const int kb = (s_begin + st) * STAGE_BYTES;
        const int ka = (s_begin + st) * SA;
        const uint32_t a_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf)) + wave_u * 1024;
        const uint32_t b_dst = a_dst + BM * SA;
        bool live = true;
        if constexpr (INT4 && !A8) live = kb + dma_chunk * 16 < kbytes_i;
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i)
            dma16(rsrc_a, live ? dma_voff_a + ka + i * rowstep_a : OOB_OFFSET, a_dst + i * 4096);
#pragma unroll
        for (int i = 0; i < B_INSTR; ++i) dma16(rsrc_b, live ? dma_voff + kb + i * row64 : OOB_OFFSET, b_dst + i * 4096);
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // MFMA operand reads: lane reads row (lane % 32) of each 32-row tile,
    // chunk 2*ks + lane/32 of the stage's 64 bytes.
    const int l32 = lane & 31;
    const int hsel = lane >> 5;
    const int sw = swz(l32);  // tile bases are multiples of 32: swz(base + l32) == swz(l32)
    const int a_rd0 = (wm * (BM / 2) + l32) * SA + ((0 + hsel) ^ sw) * 16;
    const int a_rd1 = (wm * (BM / 2) + l32) * SA + ((2 + hsel) ^ sw) * 16;
    const int b_rd0 = BM * SA + (wn * (BN / 2) + l32) * STAGE_BYTES + ((0 + hsel) ^ sw) * 16;
    const int b_rd1 = BM * SA + (wn * (BN / 2) + l32) * STAGE_BYTES + ((2 + hsel) ^ sw) * 16;
    // W4A8: the int8 A values of B chunk c = 2 ks + hsel, k-slice h, are A
    // chunk 2 c + h of the 128-byte A row
    const int sw8 = swz8(l32);
    const int a8_row = (wm * (BM / 2) + l32) * SA;

    // Pipeline unit: what one 16-byte LDS read per operand fragment feeds.
    // int4: one chunk (two MFMA k-slices once unpacked), two units per stage;
    // int8: the whole stage (two chunks, one k-slice each), one unit per stage.
    // The reads of unit u+1 are in flight while unit u's MFMAs run, and for
    // int4 the unpacking of the next k-slice runs under the current MFMAs.
    constexpr int UPS = INT4 ? 2 : 1;
    constexpr int FR = INT4 ? 1 : 2;
    constexpr int FRA = A8 ? 2 : FR;   // A reads per unit and row tile
    struct Unit {
        uint4 a[FRA][TM];
        uint4 b[FR][TN];
    };
    auto read_unit = [&](const int8_t* st, int ks0, Unit& u) {
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const int ar = (ks0 + f) == 0 ? a_rd0 : a_rd1;
            const int br = (ks0 + f) == 0 ? b_rd0 : b_rd1;
            if constexpr (!A8) {
#pragma unroll
                for (int i = 0; i < TM; ++i) u.a[f][i] = *reinterpret_cast<const uint4*>(st + ar + i * 32 * SA);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) u.b[f][j] = *reinterpret_cast<const uint4*>(st + br + j * 32 * STAGE_BYTES);
        }
        if constexpr (A8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ch = (2 * (2 * ks0 + hsel) + h) ^ sw8;
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    u.a[h][i] = *reinterpret_cast<const uint4*>(st + a8_row + ch * 16 + i * 32 * SA);
            }
        }
    };
    // int4 k-slice h (0: dwords x,y; 1: z,w) of a unit as MFMA operands; the
    // int8 A of W4A8 is put into the same k order as the unpacked nibbles
    auto unpack = [&](const Unit& u, int h, v4i (&oa)[TM], v4i (&ob)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (A8)
                oa[i] = order_int8_as_int4(u.a[h][i]);
            else
                oa[i] = h == 0 ? unpack_int4(u.a[0][i].x, u.a[0][i].y) : unpack_int4(u.a[0][i].z, u.a[0][i].w);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
            ob[j] = h == 0 ? unpack_int4(u.b[0][j].x, u.b[0][j].y) : unpack_int4(u.b[0][j].z, u.b[0][j].w);
    };
    auto mfma_slice = [&](const v4i (&oa)[TM], const v4i (&ob)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oa[i], ob[j], acc[i][j], 0, 0, 0);
    };

    // GeGLU: the table's DMA goes first, so the prologue's wait for stage 0
    // (loads complete in issue order) covers it, and its barrier publishes it.
    if constexpr (GEGLU) {
        static_assert(GTAB_BYTES == 2 * 4 * 1024, "two 16-byte loads per lane");
        const v4i rsrc_t = make_rsrc(reinterpret_cast<const int8_t*>(g_gelu_neg_tab), GTAB_BYTES);
        const uint32_t t_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave_u * 1024;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(rsrc_t, (i * 4 + wave) * 1024 + lane * 16, t_dst + i * 4096);
    }

    // prologue: NS stages in flight, stage 0 published, its first unit read
    {
        const int pro = nst < NS ? nst : NS;
#pragma unroll
        for (int pst = 0; pst < NS; ++pst)
            if (pst < pro) issue(pst, ring + pst * STAGE);
        // stage 0 has landed once at most pro - 1 stages are outstanding
        wait_groups<LOADS, NS - 1>(pro - 1);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    // A wave whose rows all lie past m (the lower half of a ragged last M tile)
    // still takes part in the DMA and the barriers, but reads no fragments and
    // issues no MFMA: its SIMD's MFMA time goes to the co-resident block.
    const bool wave_active = m0 + wm * (BM / 2) < p.m;

    Unit cur;
    v4i op_a[TM], op_b[TN];   // int4: unpacked k-slice 0 of `cur`
    if (wave_active) {
        read_unit(ring, 0, cur);
        if constexpr (INT4) unpack(cur, 0, op_a, op_b);
    }

    // One stage: its units in turn.  Before the last unit's MFMAs the next
    // stage is published (this wave's DMA for it landed + barrier, after every
    // read of this stage's buffer has completed), the buffer of this stage
    // takes the DMA of stage it + NS, and the next stage's first unit is read.
    auto stage_step = [&](auto mf, int it, int8_t* buf, int8_t* nbuf) {
        constexpr bool MF = decltype(mf)::value;   // this wave computes
#pragma unroll
        for (int ks = 0; ks < UPS; ++ks) {
            const bool last = ks == UPS - 1;
            Unit nxt;
            if (!last) {
                if constexpr (MF) read_unit(buf, ks + 1, nxt);
            } else {
                if (it + 1 < nst) {
                    // stage it+1 has landed once at most min(NS-2, nst-2-it) later stages are outstanding
                    const int after = (nst - 2 - it) < (NS - 2) ? (nst - 2 - it) : (NS - 2);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wait_groups<LOADS, NS - 2>(after);
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    if (it + NS < nst) issue(it + NS, buf);
                }
                // after the final stage this reads stale LDS that nothing uses
                if constexpr (MF) read_unit(nbuf, 0, nxt);
            }
            if constexpr (!MF) {
                // no fragments, no MFMA
            } else if constexpr (INT4) {
                v4i o1a[TM], o1b[TN];
                unpack(cur, 1, o1a, o1b);
                mfma_slice(op_a, op_b);
                unpack(nxt, 0, op_a, op_b);   // unused after the last unit (no branch: one schedule)
                mfma_slice(o1a, o1b);
                // scheduling: next unit's reads first, then each MFMA with ~4 VALU of unpacking
                __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
                for (int g = 0; g < 2 * TM * TN; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            } else {
                v4i a0[TM], b0[TN], a1[TM], b1[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) { a0[i] = __builtin_bit_cast(v4i, cur.a[0][i]); a1[i] = __builtin_bit_cast(v4i, cur.a[1][i]); }
#pragma unroll
                for (int j = 0; j < TN; ++j) { b0[j] = __builtin_bit_cast(v4i, cur.b[0][j]); b1[j] = __builtin_bit_cast(v4i, cur.b[1][j]); }
                mfma_slice(a0, b0);
                mfma_slice(a1, b1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * TM * TN, 0);
            }
            if constexpr (MF) cur = nxt;
        }
    };

    // Whole groups of NS stages: the ring positions are compile-time constants.
    auto main_loop = [&](auto mf) {
        const int nfull = nst - nst % NS;
        for (int it0 = 0; it0 < nfull; it0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) stage_step(mf, it0 + u, ring + u * STAGE, ring + ((u + 1) % NS) * STAGE);
        }
        for (int it = nfull; it < nst; ++it) {
            const int u = it - nfull;
            stage_step(mf, it, ring + u * STAGE, ring + ((u + 1) % NS) * STAGE);
        }
    };
    if (wave_active) main_loop(std::true_type{});
    else main_loop(std::false_type{});

    // ---- epilogue: every wave is done with the ring; each takes one buffer
    __syncthreads();
    if (!wave_active) return;   // no output rows (no block-wide barrier follows)
    if constexpr (GEGLU) {
        constexpr int REGION = NS * STAGE / 4 / 16 * 16;  // per-wave staging bytes
        store_tile_geglu<BM, BN, ASH, OUT - OUT_GEGLU, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2),
                                                                lane, reinterpret_cast<const float*>(lds),
                                                                ring + wave * REGION);
    } else {
        void* dst = (OUT == -1) ? static_cast<void*>(p.ws + static_cast<int64_t>(split) * p.m * p.n) : p.y;
        constexpr int REGION = NS * STAGE / 4 / 16 * 16;  // per-wave staging bytes
        store_tile_lds<BM, BN, ASH, OUT, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                                  ring + wave * REGION, dst);
    }
}

// ---- 256 x 256 tiles, one block per CU ------------------------------------
//
// For grids with at least one 256 x 256 tile per CU.  Four waves, one per
// SIMD, each owning a 128 x 128 accumulator tile (4 x 4 MFMA tiles, 256
// accumulator registers): half the LDS bytes per MFMA of a 64 x 128 wave tile.
// With one wave per SIMD nothing else hides a stall of that wave, so each
// stage's instruction order is fixed by hand (sched_barrier between groups):
//   - a few MFMAs of the stage first, issued before the stage's
//     synchronisation (own DMA of the next stage landed, s_barrier), so the
//     matrix pipe stays busy while the four waves meet;
//   - then the remaining MFMAs, one at a time, each followed by one of the
//     stage's memory instructions: the DMA of stage it + NS into the buffer
//     this stage's fragments came from (free after the barrier), and the
//     LDS reads of the next stage's fragments (published by the barrier);
//   - int4 operands: the nibble unpack of the next k-slice runs under the
//     current k-slice's MFMAs (3 VALU per MFMA).
// Stages hold 64 bytes of a B row (int8: 2 k-slices of 32; int4: 4 k-slices;
// W4A8: 4 k-slices, 128 bytes of an A row).  The ring, the swizzle, the
// operand order, the epilogue and the tile order are those of gemm_i8_kernel.
template <bool INT4, int OUT, bool A8>
__global__ __launch_bounds__(256, 1) void gemm256_kernel(GemmParams p) {
    static_assert(!A8 || INT4, "W4A8 takes int4 weights");
    constexpr int BM = 256, BN = 256, TM = 4, TN = 4;
    constexpr int NS = A8 ? 3 : 4;
    constexpr int SA = A8 ? 2 * STAGE_BYTES : STAGE_BYTES;
    constexpr int A_INSTR = BM * SA / 4096;      // 16-byte DMA loads per lane per stage (A)
    constexpr int B_INSTR = BN / 64;
    constexpr int LOADS = A_INSTR + B_INSTR;
    constexpr int STAGE = BM * SA + BN * STAGE_BYTES;
    constexpr int ASH = A8 ? 4 : (INT4 ? 8 : 0);
    constexpr bool GEGLU = OUT >= OUT_GEGLU;
    constexpr int RING0 = GEGLU ? GTAB_BYTES : 0;
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING0 + NS * STAGE];
    int8_t* const ring = lds + RING0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int nblocks = gridDim.x;
    int bid = blockIdx.x;
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    int tile_m, tile_n;
    {
        const int t_mn = bid;   // no split-K on this path
        if (p.group_m > 0) {
            const int per_group = p.group_m * p.tiles_n;
            const int g = t_mn / per_group;
            const int first = g * p.group_m;
            const int rows = (p.tiles_m - first) < p.group_m ? (p.tiles_m - first) : p.group_m;
            const int r = t_mn - g * per_group;
            tile_n = r / rows;
            tile_m = first + (r - tile_n * rows);
        } else {
            tile_n = t_mn / p.tiles_m;
            tile_m = t_mn - tile_n * p.tiles_m;
        }
    }
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
    const int nst = p.stages;
    // The loop runs a multiple of NS stages with the same instructions in every
    // stage (no branch between MFMAs, so the accumulators stay in place): the
    // DMA of a stage past the end takes an offset past the buffer's range, and
    // the hardware fills zeros (no memory access), which add nothing.
    constexpr int STEP = (NS % 2 == 0 || INT4) ? NS : 2 * NS;   // int8 also alternates register sets
    const int nstp = (nst + STEP - 1) / STEP * STEP;
    constexpr int OOB = 0x7FFFFFF0;

    const v4i rsrc_a = make_rsrc(p.a + m0 * p.kbytes_a, (p.m - m0) * p.kbytes_a);
    const v4i rsrc_b = make_rsrc(p.b + n0 * p.kbytes, (p.n - n0) * p.kbytes);

    // DMA mapping (as gemm_i8_kernel): load i of wave w fills 16 rows
    const int dma_row0 = wave * 16 + (lane >> 2);
    const int dma_chunk = (lane & 3) ^ swz(dma_row0);
    const int dma_voff = dma_row0 * static_cast<int>(p.kbytes) + dma_chunk * 16;
    const int row64 = 64 * static_cast<int>(p.kbytes);
    const int dma_row0_a = A8 ? wave * 8 + (lane >> 3) : dma_row0;
    const int dma_chunk_a = A8 ? (lane & 7) ^ swz8(dma_row0_a) : dma_chunk;
    const int dma_voff_a = dma_row0_a * static_cast<int>(p.kbytes_a) + dma_chunk_a * 16;
    const int rowstep_a = (A8 ? 32 : 64) * static_cast<int>(p.kbytes_a);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // DMA load q (0 .. LOADS-1) of stage st into buffer buf (zeros past the last stage)
    auto dma_one = [&](int st, int8_t* buf, int q) __attribute__((always_inline)) {
        const uint32_t a_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf)) + wave_u * 1024;
        const bool live = st < nst;
        if (q < A_INSTR)
            dma16(rsrc_a, live ? dma_voff_a + st * SA + q * rowstep_a : OOB, a_dst + q * 4096);
        else
            dma16(rsrc_b, live ? dma_voff + st * STAGE_BYTES + (q - A_INSTR) * row64 : OOB,
                  a_dst + BM * SA + (q - A_INSTR) * 4096);
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int l32 = lane & 31;
    const int hsel = lane >> 5;
    const int sw = swz(l32);
    const int a_row = (wm * (BM / 2) + l32) * SA;
    const int b_row = BM * SA + (wn * (BN / 2) + l32) * STAGE_BYTES;
    const int sw8 = swz8(l32);
    // the 16-byte operand read of row tile i (A) / column tile j (B) for chunk pair c (0 or 1)
    auto rd_a = [&](const int8_t* st, int c, int i) __attribute__((always_inline)) -> uint4 {
        return *reinterpret_cast<const uint4*>(st + a_row + ((2 * c + hsel) ^ sw) * 16 + i * 32 * SA);
    };
    auto rd_b = [&](const int8_t* st, int c, int j) __attribute__((always_inline)) -> uint4 {
        return *reinterpret_cast<const uint4*>(st + b_row + ((2 * c + hsel) ^ sw) * 16 + j * 32 * STAGE_BYTES);
    };
    // W4A8: the int8 A values of B chunk (2c + hsel) are A chunks 2 (2c + hsel) + h
    auto rd_a8 = [&](const int8_t* st, int c, int h, int i) __attribute__((always_inline)) -> uint4 {
        return *reinterpret_cast<const uint4*>(st + a_row + ((2 * (2 * c + hsel) + h) ^ sw8) * 16 + i * 32 * SA);
    };
    // MFMA q (0 .. 15) of a k-slice: row tile q / 4, column tile q % 4 (q a compile-time constant)
    auto mfma_one = [&](const v4i (&oa)[TM], const v4i (&ob)[TN], auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oa[q >> 2], ob[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
    };
    // published: stage it + 1 landed for every wave (every stage issues the
    // same LOADS DMAs, so NS - 2 later stages are in flight), buffer of stage it free
    auto sync_next = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<(NS - 2) * LOADS>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if constexpr (GEGLU) {
        static_assert(GTAB_BYTES == 2 * 4 * 1024, "two 16-byte loads per lane");
        const v4i rsrc_t = make_rsrc(reinterpret_cast<const int8_t*>(g_gelu_neg_tab), GTAB_BYTES);
        const uint32_t t_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave_u * 1024;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(rsrc_t, (i * 4 + wave) * 1024 + lane * 16, t_dst + i * 4096);
    }
    {
#pragma unroll
        for (int pst = 0; pst < NS; ++pst)
#pragma unroll
            for (int q = 0; q < LOADS; ++q) dma_one(pst, ring + pst * STAGE, q);
        wait_vmcnt<(NS - 1) * LOADS>();   // stage 0 (and the GeLU table, issued first) landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }

    if constexpr (!INT4) {
        // ---- int8 x int8: 2 k-slices per stage; fragments double-buffered
        struct Frag {
            uint4 a[2][TM];
            uint4 b[2][TN];
        };
        Frag f[2];
        auto read_frag = [&](const int8_t* st, Frag& fr) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fr.a[c][i] = rd_a(st, c, i);
#pragma unroll
                for (int j = 0; j < TN; ++j) fr.b[c][j] = rd_b(st, c, j);
            }
        };
        read_frag(ring, f[0]);
        auto stage = [&](auto par, int it, int8_t* buf, int8_t* nbuf) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;
            Frag& cur = f[P];
            Frag& nxt = f[P ^ 1];
            v4i a0[TM], b0[TN], a1[TM], b1[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) { a0[i] = __builtin_bit_cast(v4i, cur.a[0][i]); a1[i] = __builtin_bit_cast(v4i, cur.a[1][i]); }
#pragma unroll
            for (int j = 0; j < TN; ++j) { b0[j] = __builtin_bit_cast(v4i, cur.b[0][j]); b1[j] = __builtin_bit_cast(v4i, cur.b[1][j]); }
            // 4 MFMAs cover the synchronisation
            static_for<0, 4>([&](auto qc) __attribute__((always_inline)) { mfma_one(a0, b0, qc); });
            __builtin_amdgcn_sched_barrier(0);
            sync_next();
            // 28 MFMAs, each followed by one memory instruction: 8 DMA, 16 LDS reads
            static_for<4, 32>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                if constexpr (q < 16) mfma_one(a0, b0, qc);
                else mfma_one(a1, b1, std::integral_constant<int, q - 16>{});
                constexpr int mi = q - 4;
                if constexpr (mi < LOADS) {
                    dma_one(it + NS, buf, mi);
                } else if constexpr (mi < LOADS + 16) {
                    constexpr int r = mi - LOADS, c = r >> 3, t = r & 7;
                    if constexpr (t < TM) nxt.a[c][t] = rd_a(nbuf, c, t);
                    else nxt.b[c][t - TM] = rd_b(nbuf, c, t - TM);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int it = 0; it < nstp; it += 4) {
            stage(std::integral_constant<int, 0>{}, it, ring, ring + STAGE);
            stage(std::integral_constant<int, 1>{}, it + 1, ring + STAGE, ring + 2 * STAGE);
            stage(std::integral_constant<int, 0>{}, it + 2, ring + 2 * STAGE, ring + 3 * STAGE);
            stage(std::integral_constant<int, 1>{}, it + 3, ring + 3 * STAGE, ring);
        }
    } else {
        // ---- int4 weights (W4A4, W4A8): 4 k-slices per stage in two units of
        // one 16-byte read per fragment (A8: two A reads per row tile)
        constexpr int FRA = A8 ? 2 : 1;
        struct Unit {
            uint4 a[FRA][TM];
            uint4 b[TN];
        };
        auto read_unit = [&](const int8_t* st, int c, Unit& u) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (A8) {
                    u.a[0][i] = rd_a8(st, c, 0, i);
                    u.a[1][i] = rd_a8(st, c, 1, i);
                } else {
                    u.a[0][i] = rd_a(st, c, i);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) u.b[j] = rd_b(st, c, j);
        };
        // number of 16-byte reads of a unit, and the r-th of them (r a compile-time constant)
        constexpr int UREADS = FRA * TM + TN;
        auto read_one = [&](const int8_t* st, int c, Unit& u, auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            if constexpr (r < FRA * TM) {
                if constexpr (A8) u.a[r / TM][r % TM] = rd_a8(st, c, r / TM, r % TM);
                else u.a[0][r] = rd_a(st, c, r);
            } else {
                u.b[r - FRA * TM] = rd_b(st, c, r - FRA * TM);
            }
        };
        // k-slice h (0: dwords x,y; 1: z,w) of a unit as MFMA operands
        auto unpack_a = [&](const Unit& u, int h, int i) __attribute__((always_inline)) -> v4i {
            if constexpr (A8) return order_int8_as_int4(u.a[h][i]);
            else return h == 0 ? unpack_int4(u.a[0][i].x, u.a[0][i].y) : unpack_int4(u.a[0][i].z, u.a[0][i].w);
        };
        auto unpack_b = [&](const Unit& u, int h, int j) __attribute__((always_inline)) -> v4i {
            return h == 0 ? unpack_int4(u.b[j].x, u.b[j].y) : unpack_int4(u.b[j].z, u.b[j].w);
        };
        Unit u0, u1;
        v4i oa[TM], ob[TN], pa[TM], pb[TN];
        read_unit(ring, 0, u0);
#pragma unroll
        for (int i = 0; i < TM; ++i) oa[i] = unpack_a(u0, 0, i);
#pragma unroll
        for (int j = 0; j < TN; ++j) ob[j] = unpack_b(u0, 0, j);
        // one MFMA, then operand f (0..7: row tiles then column tiles) of the
        // next k-slice unpacked into (na, nb)
        auto mfma_unpack = [&](const v4i (&ca)[TM], const v4i (&cb)[TN], auto qc, const Unit& src, int h,
                               v4i (&na)[TM], v4i (&nb)[TN]) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            mfma_one(ca, cb, qc);
            if constexpr (q < TM) na[q] = unpack_a(src, h, q);
            else if constexpr (q < TM + TN) nb[q - TM] = unpack_b(src, h, q - TM);
        };
        auto stage = [&](int it, int8_t* buf, int8_t* nbuf) __attribute__((always_inline)) {
            // slice 0 (oa, ob): MFMAs with unit 1 read from this stage and slice 1 unpacked
            static_for<0, 16>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                mfma_unpack(oa, ob, qc, u0, 1, pa, pb);
                if constexpr (q < UREADS) read_one(buf, 1, u1, qc);
                __builtin_amdgcn_sched_barrier(0);
            });
            // slice 1 (pa, pb): 4 MFMAs, synchronisation, then MFMAs with the DMA of
            // stage it + NS and slice 2 (unit 1, k-slice 0) unpacked
            static_for<0, 4>([&](auto qc) __attribute__((always_inline)) { mfma_one(pa, pb, qc); });
            __builtin_amdgcn_sched_barrier(0);
            sync_next();
            static_for<4, 16>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                mfma_one(pa, pb, qc);
                constexpr int f = q - 4;   // 0 .. 11
                if constexpr (f < TM) oa[f] = unpack_a(u1, 0, f);
                else if constexpr (f < TM + TN) ob[f - TM] = unpack_b(u1, 0, f - TM);
                if constexpr (f < LOADS) dma_one(it + NS, buf, f);
                __builtin_amdgcn_sched_barrier(0);
            });
            // slice 2 (oa, ob): MFMAs with the rest of the DMA, the next stage's unit 0
            // read, and slice 3 (unit 1, k-slice 1) unpacked
            static_for<0, 16>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                mfma_unpack(oa, ob, qc, u1, 1, pa, pb);
                constexpr int f = q + 12;
                if constexpr (f < LOADS) dma_one(it + NS, buf, f);
                if constexpr (q >= 4 && q - 4 < UREADS) read_one(nbuf, 0, u0, std::integral_constant<int, q - 4>{});
                __builtin_amdgcn_sched_barrier(0);
            });
            // slice 3 (pa, pb): MFMAs with the next stage's slice 0 unpacked
            static_for<0, 16>([&](auto qc) __attribute__((always_inline)) {
                mfma_unpack(pa, pb, qc, u0, 0, oa, ob);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int it = 0; it < nstp; it += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) stage(it + u, ring + u * STAGE, ring + ((u + 1) % NS) * STAGE);
        }
    }

    // ---- epilogue: the zero-fill DMAs past the last stage have landed and every
    // wave is done with the ring; each wave takes one buffer's worth
    wait_vmcnt<0>();
    __syncthreads();
    if (m0 + wm * (BM / 2) >= p.m) return;   // no output rows in this wave
    constexpr int REGION = NS * STAGE / 4 / 16 * 16;
    if constexpr (GEGLU) {
        store_tile_geglu<BM, BN, ASH, OUT - OUT_GEGLU, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2),
                                                                lane, reinterpret_cast<const float*>(lds),
                                                                ring + wave * REGION);
    } else {
        store_tile_lds<BM, BN, ASH, OUT, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                                  ring + wave * REGION, p.y);
    }
}

// ---- E2M3 operands: W4A4 codes on the FP6 matrix cores ---------------------
//
// The int4-grid codes (-7 .. 7) stored as FP6 E2M3 fields, 32 per 24 bytes,
// code j of a row at bits 6j .. 6j+5, feed v_mfma_scale_f32_32x32x64_f8f6f4
// with both operands E2M3 and unit block scales (E8M0 127).  Every grid value
// is exact in E2M3, a product of two is exact in fp32, and every partial sum
// is an integer of magnitude below 49 k < 2^24, so the fp32 accumulator holds
// exactly the int32 accumulator of the integer kernels.  The instruction does
// 32 x 32 x 64 in the cycles the int8 one takes for 32 x 32 x 32.
//
// A lane supplies 32 fields (six dwords) of one row per issue.  A stage holds
// 128 k of a row: 96 bytes, six 16-byte chunks.  Lane half h reads chunks
// 3h .. 3h+2 with three ds_read_b128; the first 24 bytes feed the stage's
// first k-step and the last 24 its second.  A and B fragments are read the
// same way, so each issue pairs equal k.  In LDS, chunk c of row r sits at
// chunk slot c ^ ((r >> 3) & 1): with a 96-byte pitch rows r and r + 8 start
// on the same banks, and the swizzle gives them slots of opposite parity
// (16 lanes of a ds_read_b128 then reach 16 distinct 16-byte bank groups).
// The ring is three stages deep; buffers are addressed at run time, so the
// branch-free loop body covers two stages (the fragment register parity) and
// K pads to an even stage count at most.  Tiles: 256 x 256 (one block per CU,
// waves 128 x 128) for grids that fill the chip, else 128 x 128 (two blocks
// per CU, waves 64 x 64).
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v12i_t __attribute__((ext_vector_type(12)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

template <int BM, int BN, int MINB, int OUT>
__global__ __launch_bounds__(256, MINB) void gemm_f6_kernel(GemmParams p) {
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int NS = 3;
    constexpr int SB = 96;                          // bytes of a row per stage (128 codes)
    constexpr int STAGE = (BM + BN) * SB;
    constexpr int LOADS = (BM + BN) * SB / 4096;    // 16-byte DMA loads per lane per stage
    constexpr int LA = BM * SB / 4096;              // ... of them for A
    static_assert(LA * 4096 == BM * SB && LOADS * 4096 == STAGE, "whole 1 KB loads per wave");
    constexpr int MF = 2 * TM * TN;                 // MFMAs per stage
    constexpr int READS = 3 * (TM + TN);            // 16-byte fragment reads per stage
    constexpr int OPS = LOADS + READS;
    constexpr bool GEGLU = OUT >= OUT_GEGLU;
    constexpr int RING0 = GEGLU ? GTAB_BYTES : 0;
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING0 + NS * STAGE];
    int8_t* const ring = lds + RING0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int nblocks = gridDim.x;
    int bid = blockIdx.x;
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    int tile_m, tile_n;
    if (p.group_m > 0) {
        const int per_group = p.group_m * p.tiles_n;
        const int g = bid / per_group;
        const int first = g * p.group_m;
        const int rows = (p.tiles_m - first) < p.group_m ? (p.tiles_m - first) : p.group_m;
        const int r = bid - g * per_group;
        tile_n = r / rows;
        tile_m = first + (r - tile_n * rows);
    } else {
        tile_n = bid / p.tiles_m;
        tile_m = bid - tile_n * p.tiles_m;
    }
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
    const int nst = p.stages;
    const int nstp = (nst + 1) & ~1;
    constexpr int OOB = 0x7FFFFFF0;
    const int kb = static_cast<int>(p.kbytes);

    const v4i rsrc_a = make_rsrc(p.a + m0 * p.kbytes, (p.m - m0) * p.kbytes);
    const v4i rsrc_b = make_rsrc(p.b + n0 * p.kbytes, (p.n - n0) * p.kbytes);

    // DMA: load q of wave w fills the 64 chunk slots at stage offset (4q + w) KB
    // (A rows first, then B rows); the lane's slot holds chunk pos ^ swizzle of its row
    int dvoff[LOADS];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int slot = (4 * q + wave) * 64 + lane;
        const int s2 = q < LA ? slot : slot - BM * 6;
        const int r = s2 / 6, pos = s2 - r * 6;
        dvoff[q] = r * kb + (pos ^ ((r >> 3) & 1)) * 16;
    }
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
    auto dma_one = [&](int st, uint32_t buf_addr, int q) __attribute__((always_inline)) {
        const int off = st < nst ? dvoff[q] + st * SB : OOB;
        dma16(q < LA ? rsrc_a : rsrc_b, off, buf_addr + wave_u * 1024 + q * 4096);
    };

    v16f_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // the three chunks this lane reads of a row (lane half h: chunks 3h .. 3h+2)
    const int l32 = lane & 31;
    const int hsel = lane >> 5;
    const int sw = (l32 >> 3) & 1;
    const int a_row = (wm * (BM / 2) + l32) * SB;
    const int b_row = BM * SB + (wn * (BN / 2) + l32) * SB;
    int coff[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) coff[t] = ((3 * hsel + t) ^ sw) * 16;

    // a fragment: the 48 bytes (12 dwords) of one row for the stage's two k-steps,
    // held as one 12-dword vector so that each k-step's six dwords are a
    // contiguous register range of it
    struct Frag {
        v12i_t a[TM];
        v12i_t b[TN];
    };
    Frag f[2];
    // read r (0 .. READS-1) of a fragment set from the stage buffer at st
    auto read_one = [&](const int8_t* st, Frag& fr, auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        constexpr int which = r / 3, t = r % 3;
        const v4i d = (which < TM)
                          ? *reinterpret_cast<const v4i*>(st + a_row + coff[t] + which * 32 * SB)
                          : *reinterpret_cast<const v4i*>(st + b_row + coff[t] + (which - TM) * 32 * SB);
        v12i_t& v = (which < TM) ? fr.a[which < TM ? which : 0] : fr.b[which < TM ? 0 : which - TM];
        v[4 * t + 0] = d.x;
        v[4 * t + 1] = d.y;
        v[4 * t + 2] = d.z;
        v[4 * t + 3] = d.w;
    };
    // the six dwords of k-step ks (0, 1) of a fragment
    auto operand = [](const v12i_t& c, auto kc) __attribute__((always_inline)) -> v8i_t {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks == 0)
            return __builtin_shufflevector(c, c, 0, 1, 2, 3, 4, 5, -1, -1);
        else
            return __builtin_shufflevector(c, c, 6, 7, 8, 9, 10, 11, -1, -1);
    };
    // MFMA q (0 .. MF-1) of a stage: k-step q / (TM TN), row tile (q % (TM TN)) / TN, column tile q % TN
    auto mfma_one = [&](const Frag& fr, auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        constexpr int ks = q / (TM * TN), i = (q % (TM * TN)) / TN, j = q % TN;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            operand(fr.a[i], std::integral_constant<int, ks>{}), operand(fr.b[j], std::integral_constant<int, ks>{}),
            acc[i][j], 2, 2, 0, 127, 0, 127);
    };
    auto sync_next = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<(NS - 2) * LOADS>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if constexpr (GEGLU) {
        static_assert(GTAB_BYTES == 2 * 4 * 1024, "two 16-byte loads per lane");
        const v4i rsrc_t = make_rsrc(reinterpret_cast<const int8_t*>(g_gelu_neg_tab), GTAB_BYTES);
        const uint32_t t_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave_u * 1024;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(rsrc_t, (i * 4 + wave) * 1024 + lane * 16, t_dst + i * 4096);
    }
#pragma unroll
    for (int pst = 0; pst < NS; ++pst)
#pragma unroll
        for (int q = 0; q < LOADS; ++q) dma_one(pst, ring_addr + pst * STAGE, q);
    wait_vmcnt<(NS - 1) * LOADS>();   // stage 0 (and the GeLU table, issued first) landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    static_for<0, READS>([&](auto rc) __attribute__((always_inline)) { read_one(ring, f[0], rc); });

    // one stage: 4 MFMAs, the synchronisation, then the remaining MFMAs with the
    // DMA of stage it + NS into this stage's buffer and the next stage's
    // fragment reads spread over them
    auto stage = [&](auto par, int it, int bi) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        const Frag& cur = f[P];
        Frag& nxt = f[P ^ 1];
        const int nbi = bi == NS - 1 ? 0 : bi + 1;
        const uint32_t buf_addr = ring_addr + bi * STAGE;
        const int8_t* nbuf = ring + nbi * STAGE;
        static_for<0, 4>([&](auto qc) __attribute__((always_inline)) { mfma_one(cur, qc); });
        __builtin_amdgcn_sched_barrier(0);
        sync_next();
        static_for<4, MF>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            mfma_one(cur, qc);
            // the memory operations o with 4 + o (MF - 4) / OPS == q
            static_for<0, OPS>([&](auto oc) __attribute__((always_inline)) {
                constexpr int o = decltype(oc)::value;
                if constexpr (4 + o * (MF - 4) / OPS == q) {
                    if constexpr (o < LOADS) dma_one(it + NS, buf_addr, o);
                    else read_one(nbuf, nxt, std::integral_constant<int, o - LOADS>{});
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int bi = 0;
    for (int it = 0; it < nstp; it += 2) {
        stage(std::integral_constant<int, 0>{}, it, bi);
        bi = bi == NS - 1 ? 0 : bi + 1;
        stage(std::integral_constant<int, 1>{}, it + 1, bi);
        bi = bi == NS - 1 ? 0 : bi + 1;
    }

    // ---- epilogue (as gemm256_kernel): the ring is free once every wave is past it
    wait_vmcnt<0>();
    __syncthreads();
    if (m0 + wm * (BM / 2) >= p.m) return;
    constexpr int REGION = NS * STAGE / 4 / 16 * 16;
    if constexpr (GEGLU) {
        store_tile_geglu<BM, BN, 0, OUT - OUT_GEGLU, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                                             reinterpret_cast<const float*>(lds),
                                                             ring + wave * REGION);
    } else {
        store_tile_lds<BM, BN, 0, OUT, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                               ring + wave * REGION, p.y);
    }
}

// ---- E2M3 with two blocks per CU --------------------------------------------
//
// The fused GeGLU GEMM on grids that fill the chip: 128 x 256 tiles, four
// waves of 64 x 128, so that one block's epilogue (the GeLU work) runs under
// the co-resident block's main loop, as for the int4 tiles (52224 x 32768 x
// 2048: 3.10 ms against 3.64 ms with 256 x 256 tiles, one block per CU).  Two
// blocks fit a CU with a two-stage ring (2 x 36 KB + the 8 KB GeLU table) and
// fragments held per k-step rather than per stage: a k-step's operand of a
// row is 24 bytes, a 16-byte and an 8-byte LDS read (k-step 0: chunk 3h and
// the low half of chunk 3h+1; k-step 1: the high half of chunk 3h+1 and chunk
// 3h+2).  Per stage: the k-step-0 MFMAs with the k-step-1 reads under them;
// the synchronisation (next stage landed, every wave past this stage's
// reads); the k-step-1 MFMAs with the DMA of stage it + 2 into this stage's
// buffer and the next stage's k-step-0 reads under them.
typedef int v2i_t __attribute__((ext_vector_type(2)));
template <int OUT>
__global__ __launch_bounds__(256, 2) void gemm_f6w_kernel(GemmParams p) {
    constexpr int BM = 128, BN = 256, TM = 2, TN = 4, NS = 2, SB = 96;
    constexpr int STAGE = (BM + BN) * SB;
    constexpr int LOADS = STAGE / 4096;
    constexpr int LA = BM * SB / 4096;
    static_assert(LA * 4096 == BM * SB && LOADS * 4096 == STAGE, "whole 1 KB loads per wave");
    constexpr int KM = TM * TN;                 // MFMAs per k-step
    constexpr int KR = 2 * (TM + TN);           // LDS reads per k-step
    constexpr bool GEGLU = OUT >= OUT_GEGLU;
    constexpr int RING0 = GEGLU ? GTAB_BYTES : 0;
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING0 + NS * STAGE];
    int8_t* const ring = lds + RING0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int nblocks = gridDim.x;
    int bid = blockIdx.x;
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    int tile_m, tile_n;
    if (p.group_m > 0) {
        const int per_group = p.group_m * p.tiles_n;
        const int g = bid / per_group;
        const int first = g * p.group_m;
        const int rows = (p.tiles_m - first) < p.group_m ? (p.tiles_m - first) : p.group_m;
        const int r = bid - g * per_group;
        tile_n = r / rows;
        tile_m = first + (r - tile_n * rows);
    } else {
        tile_n = bid / p.tiles_m;
        tile_m = bid - tile_n * p.tiles_m;
    }
    const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
    const int nst = p.stages;
    const int nstp = (nst + 1) & ~1;
    constexpr int OOB = 0x7FFFFFF0;
    const int kb = static_cast<int>(p.kbytes);

    const v4i rsrc_a = make_rsrc(p.a + m0 * p.kbytes, (p.m - m0) * p.kbytes);
    const v4i rsrc_b = make_rsrc(p.b + n0 * p.kbytes, (p.n - n0) * p.kbytes);

    int dvoff[LOADS];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int slot = (4 * q + wave) * 64 + lane;
        const int s2 = q < LA ? slot : slot - BM * 6;
        const int r = s2 / 6, pos = s2 - r * 6;
        dvoff[q] = r * kb + (pos ^ ((r >> 3) & 1)) * 16;
    }
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
    auto dma_one = [&](int st, uint32_t buf_addr, int q) __attribute__((always_inline)) {
        const int off = st < nst ? dvoff[q] + st * SB : OOB;
        dma16(q < LA ? rsrc_a : rsrc_b, off, buf_addr + wave_u * 1024 + q * 4096);
    };

    v16f_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int l32 = lane & 31;
    const int hsel = lane >> 5;
    const int sw = (l32 >> 3) & 1;
    const int a_row = (wm * (BM / 2) + l32) * SB;
    const int b_row = BM * SB + (wn * (BN / 2) + l32) * SB;
    const int c0 = ((3 * hsel + 0) ^ sw) * 16, c1 = ((3 * hsel + 1) ^ sw) * 16, c2 = ((3 * hsel + 2) ^ sw) * 16;

    struct KF {
        v8i_t a[TM];
        v8i_t b[TN];
    };
    KF f[2];
    // read r (0 .. KR-1) of k-step KS of a fragment set from the stage buffer st
    auto read_one = [&](const int8_t* st, KF& fr, auto kc, auto rc) __attribute__((always_inline)) {
        constexpr int KS = decltype(kc)::value;
        constexpr int r = decltype(rc)::value;
        constexpr int which = r / 2, t = r % 2;
        const int8_t* row = (which < TM) ? st + a_row + which * 32 * SB : st + b_row + (which - TM) * 32 * SB;
        v8i_t& v = (which < TM) ? fr.a[which < TM ? which : 0] : fr.b[which < TM ? 0 : which - TM];
        if constexpr (KS == 0) {
            if constexpr (t == 0) {
                const v4i d = *reinterpret_cast<const v4i*>(row + c0);
                v[0] = d.x; v[1] = d.y; v[2] = d.z; v[3] = d.w;
            } else {
                const v2i_t e = *reinterpret_cast<const v2i_t*>(row + c1);
                v[4] = e.x; v[5] = e.y;
            }
        } else {
            if constexpr (t == 0) {
                const v2i_t e = *reinterpret_cast<const v2i_t*>(row + c1 + 8);
                v[0] = e.x; v[1] = e.y;
            } else {
                const v4i d = *reinterpret_cast<const v4i*>(row + c2);
                v[2] = d.x; v[3] = d.y; v[4] = d.z; v[5] = d.w;
            }
        }
    };
    auto mfma_one = [&](const KF& fr, auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        constexpr int i = q / TN, j = q % TN;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr.a[i], fr.b[j], acc[i][j], 2, 2, 0, 127, 0,
                                                                      127);
    };

    if constexpr (GEGLU) {
        static_assert(GTAB_BYTES == 2 * 4 * 1024, "two 16-byte loads per lane");
        const v4i rsrc_t = make_rsrc(reinterpret_cast<const int8_t*>(g_gelu_neg_tab), GTAB_BYTES);
        const uint32_t t_dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave_u * 1024;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(rsrc_t, (i * 4 + wave) * 1024 + lane * 16, t_dst + i * 4096);
    }
#pragma unroll
    for (int pst = 0; pst < NS; ++pst)
#pragma unroll
        for (int q = 0; q < LOADS; ++q) dma_one(pst, ring_addr + pst * STAGE, q);
    wait_vmcnt<LOADS>();   // stage 0 (and the GeLU table, issued first) landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    static_for<0, KR>([&](auto rc) __attribute__((always_inline)) {
        read_one(ring, f[0], std::integral_constant<int, 0>{}, rc);
    });

    auto stage = [&](auto par, int it) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;   // buffer of this stage
        const int8_t* buf = ring + P * STAGE;
        const int8_t* nbuf = ring + (P ^ 1) * STAGE;
        const uint32_t buf_addr = ring_addr + P * STAGE;
        // k-step 0: its MFMAs, the k-step-1 reads of this stage under them
        static_for<0, KM>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            mfma_one(f[0], qc);
            static_for<0, KR>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;
                if constexpr (r * KM / KR == q) read_one(buf, f[1], std::integral_constant<int, 1>{}, rc);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // next stage landed (the only DMA in flight), every wave past this stage's reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // k-step 1: its MFMAs, the DMA of stage it + 2 and the next stage's k-step-0 reads under them
        static_for<0, KM>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            mfma_one(f[1], qc);
            static_for<0, LOADS + KR>([&](auto oc) __attribute__((always_inline)) {
                constexpr int o = decltype(oc)::value;
                if constexpr (o * KM / (LOADS + KR) == q) {
                    if constexpr (o < LOADS) dma_one(it + NS, buf_addr, o);
                    else read_one(nbuf, f[0], std::integral_constant<int, 0>{}, std::integral_constant<int, o - LOADS>{});
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int it = 0; it < nstp; it += 2) {
        stage(std::integral_constant<int, 0>{}, it);
        stage(std::integral_constant<int, 1>{}, it + 1);
    }

    wait_vmcnt<0>();
    __syncthreads();
    if (m0 + wm * (BM / 2) >= p.m) return;
    constexpr int REGION = NS * STAGE / 4 / 16 * 16;
    if constexpr (GEGLU) {
        store_tile_geglu<BM, BN, 0, OUT - OUT_GEGLU, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                                             reinterpret_cast<const float*>(lds),
                                                             ring + wave * REGION);
    } else {
        store_tile_lds<BM, BN, 0, OUT, REGION>(acc, p, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                                               ring + wave * REGION, p.y);
    }
}

template <int OUT>
hipError_t launch_f6w(const GemmParams& p, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(p.tiles_m * p.tiles_n));
    hipLaunchKernelGGL((gemm_f6w_kernel<OUT>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int ODT>
hipError_t launch_f6w_geglu(const GemmParams& p, hipStream_t st) {
    return launch_f6w<OUT_GEGLU + ODT>(p, st);
}

// Sum of split-K partials in split order (integer: bit-exact), then the
// epilogue; four consecutive outputs per lane (n % 4 == 0), else one.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int32_t* ws, int splits, int64_t m,
                                                            int64_t n, const float* sx,
                                                            const float* sw, void* y, int y_dtype) {
    const int64_t total = m * n;
    const bool vec = (n & 3) == 0;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * (vec ? 4 : 1);
    if (i0 >= total) return;
    const int cnt = vec ? 4 : 1;
    int32_t a[4] = {0, 0, 0, 0};
    for (int s = 0; s < splits; ++s) {
        const int32_t* src = ws + static_cast<int64_t>(s) * total + i0;
        if (vec) {
            const int4 v = *reinterpret_cast<const int4*>(src);
            a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
        } else {
            a[0] += src[0];
        }
    }
    const int64_t row = i0 / n;
    for (int e = 0; e < cnt; ++e) {
        const int64_t i = i0 + e, col = i - row * n;
        if (y_dtype == I32) static_cast<int32_t*>(y)[i] = a[e];
        else store_out(y, i, y_dtype, static_cast<float>(a[e]) * sx[row] * sw[col]);
    }
}

// The same for n % 8 == 0: eight consecutive outputs per lane, 32-byte
// partial reads, one 16-byte (or two) output store.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(const int32_t* ws, int splits, int64_t m,
                                                             int64_t n, const float* sx,
                                                             const float* sw, void* y) {
    const int64_t total = m * n;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
    if (i0 >= total) return;
    v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
    for (int s = 0; s < splits; ++s) {
        const v4i* src = reinterpret_cast<const v4i*>(ws + static_cast<int64_t>(s) * total + i0);
        a0 += __builtin_nontemporal_load(src);
        a1 += __builtin_nontemporal_load(src + 1);
    }
    const int32_t a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    if constexpr (DT == I32) {
        reinterpret_cast<v4i*>(y)[i0 / 4] = a0;
        reinterpret_cast<v4i*>(y)[i0 / 4 + 1] = a1;
    } else {
        const int64_t row = i0 / n, col = i0 - row * n;
        const float sxr = sx[row];
        const f4 w0 = *reinterpret_cast<const f4*>(sw + col);
        const f4 w1 = *reinterpret_cast<const f4*>(sw + col + 4);
        const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(a[e]) * sxr * wv[e];
        if constexpr (DT == BF16) {
            const v4i o = {static_cast<int>(pk_bf16(v[0], v[1])), static_cast<int>(pk_bf16(v[2], v[3])),
                           static_cast<int>(pk_bf16(v[4], v[5])), static_cast<int>(pk_bf16(v[6], v[7]))};
            reinterpret_cast<v4i*>(y)[i0 / 8] = o;
        } else if constexpr (DT == F16) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = f32_to_f16_bits(v[2 * e]) | (static_cast<uint32_t>(f32_to_f16_bits(v[2 * e + 1])) << 16);
            reinterpret_cast<v4i*>(y)[i0 / 8] = v4i{static_cast<int>(o[0]), static_cast<int>(o[1]),
                                                    static_cast<int>(o[2]), static_cast<int>(o[3])};
        } else {
            reinterpret_cast<f4*>(y)[i0 / 4] = f4{v[0], v[1], v[2], v[3]};
            reinterpret_cast<f4*>(y)[i0 / 4 + 1] = f4{v[4], v[5], v[6], v[7]};
        }
    }
}

template <int BM, int BN, int MINB, int NS, bool INT4, int OUT, bool A8 = false>
hipError_t launch_tile(const GemmParams& p, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(p.tiles_m * p.tiles_n * p.splits));
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, MINB, NS, INT4, OUT, A8>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <bool INT4, int OUT, bool A8>
hipError_t launch_256(const GemmParams& p, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(p.tiles_m * p.tiles_n));
    hipLaunchKernelGGL((gemm256_kernel<INT4, OUT, A8>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <bool INT4, bool A8>
hipError_t launch_256_out(const GemmParams& p, hipStream_t st) {
    switch (p.y_dtype) {
        case BF16: return launch_256<INT4, BF16, A8>(p, st);
        case F16: return launch_256<INT4, F16, A8>(p, st);
        case F32: return launch_256<INT4, F32, A8>(p, st);
        case I32: return launch_256<INT4, I32, A8>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int MINB, int NS, bool INT4, bool A8 = false>
hipError_t launch_out(const GemmParams& p, hipStream_t st) {
    if (p.splits > 1) return launch_tile<BM, BN, MINB, NS, INT4, -1, A8>(p, st);
    switch (p.y_dtype) {
        case BF16: return launch_tile<BM, BN, MINB, NS, INT4, BF16, A8>(p, st);
        case F16: return launch_tile<BM, BN, MINB, NS, INT4, F16, A8>(p, st);
        case F32: return launch_tile<BM, BN, MINB, NS, INT4, F32, A8>(p, st);
        case I32: return launch_tile<BM, BN, MINB, NS, INT4, I32, A8>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int MINB, int NS, bool INT4>
hipError_t launch_geglu_out(const GemmParams& p, hipStream_t st) {
    switch (p.y_dtype) {
        case BF16: return launch_tile<BM, BN, MINB, NS, INT4, OUT_GEGLU + BF16>(p, st);
        case F16: return launch_tile<BM, BN, MINB, NS, INT4, OUT_GEGLU + F16>(p, st);
        case F32: return launch_tile<BM, BN, MINB, NS, INT4, OUT_GEGLU + F32>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int MINB, int OUT>
hipError_t launch_f6(const GemmParams& p, hipStream_t st) {
    dim3 grid(static_cast<unsigned>(p.tiles_m * p.tiles_n));
    hipLaunchKernelGGL((gemm_f6_kernel<BM, BN, MINB, OUT>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int BM, int BN, int MINB>
hipError_t launch_f6_out(const GemmParams& p, bool geglu, hipStream_t st) {
    if (geglu) {
        switch (p.y_dtype) {
            case BF16: return launch_f6<BM, BN, MINB, OUT_GEGLU + BF16>(p, st);
            case F16: return launch_f6<BM, BN, MINB, OUT_GEGLU + F16>(p, st);
            case F32: return launch_f6<BM, BN, MINB, OUT_GEGLU + F32>(p, st);
        }
        return hipErrorInvalidValue;
    }
    switch (p.y_dtype) {
        case BF16: return launch_f6<BM, BN, MINB, BF16>(p, st);
        case F16: return launch_f6<BM, BN, MINB, F16>(p, st);
        case F32: return launch_f6<BM, BN, MINB, F32>(p, st);
        case I32: return launch_f6<BM, BN, MINB, I32>(p, st);
    }
    return hipErrorInvalidValue;
}

OncePerDevice g_gtab_once;

hipError_t fill_gelu_neg_tab(hipStream_t st) {
    hipLaunchKernelGGL(gelu_neg_tab_init_kernel, dim3((GTAB_N + 255) / 256), dim3(256), 0, st);
    return hipGetLastError();
}

// The fused epilogue's GeLU table of this device, filled before first use.
hipError_t ensure_gelu_neg_tab(hipStream_t st) { return fill_once_per_device(g_gtab_once, st, fill_gelu_neg_tab); }

}  // namespace

// Split-K scratch of the entry point for callers that cannot allocate: one
// file-scope device array, held by every GPU the library runs on until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up
// once per device and kept in g_scratch_dev.
static __device__ __align__(256) int32_t scratch[kStaticScratchBytes / 4];

namespace {
std::mutex g_scratch_mu;
int32_t* g_scratch_dev[64] = {nullptr};
}  // namespace

hipError_t static_scratch(int32_t** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = static_cast<int32_t*>(p);
    }
    *ptr = g_scratch_dev[dev];
    return hipSuccess;
}

hipError_t launch_gemm(const GemmPlan& plan, const void* xq, const float* x_scale, const void* wq,
                       const float* w_scale, int64_t m, int64_t n, int64_t k, bool int4, bool a8, void* y,
                       int y_dtype, int32_t* ws, hipStream_t st) {
    if (plan.bm == 256 && plan.m_tail > 0 && plan.m_tail < m) {
        // the full rounds of 256 x 256 tiles, then the last rows as 128 x 128
        // tiles (two blocks per CU): the same per-element arithmetic
        GemmPlan head = plan;
        head.m_tail = 0;
        const int64_t mh = m - plan.m_tail;
        hipError_t e = launch_gemm(head, xq, x_scale, wq, w_scale, mh, n, k, int4, a8, y, y_dtype, ws, st);
        if (e != hipSuccess) return e;
        GemmPlan tail;
        tail.bm = tail.bn = 128;
        tail.splits = 1;
        tail.deep = false;
        tail.group_m = 0;
        tail.ws_bytes = 0;
        tail.m_tail = 0;
        const int64_t a_row = (int4 && !a8) ? k / 2 : k;
        const int64_t y_elem = (y_dtype == BF16 || y_dtype == F16) ? 2 : 4;
        return launch_gemm(tail, static_cast<const int8_t*>(xq) + mh * a_row, x_scale ? x_scale + mh : nullptr, wq,
                           w_scale, plan.m_tail, n, k, int4, a8, static_cast<char*>(y) + mh * n * y_elem, y_dtype,
                           ws, st);
    }
    GemmParams p;
    p.a = static_cast<const int8_t*>(xq);
    p.b = static_cast<const int8_t*>(wq);
    p.sx = x_scale; p.sw = w_scale; p.y = y; p.ws = ws;
    p.m = m; p.n = n;
    p.kbytes = int4 ? k / 2 : k;
    p.kbytes_a = (int4 && !a8) ? k / 2 : k;
    p.stages = static_cast<int>((p.kbytes + STAGE_BYTES - 1) / STAGE_BYTES);
    p.splits = plan.splits;
    p.stages_per_split = (p.stages + plan.splits - 1) / plan.splits;
    p.tiles_m = static_cast<int>((m + plan.bm - 1) / plan.bm);
    p.tiles_n = static_cast<int>((n + plan.bn - 1) / plan.bn);
    p.group_m = plan.group_m;
    p.y_dtype = y_dtype;
    hipError_t e;
    if (plan.bm == 256) {
        if (plan.splits != 1) return hipErrorInvalidValue;
        if (a8) e = launch_256_out<true, true>(p, st);
        else if (int4) e = launch_256_out<true, false>(p, st);
        else e = launch_256_out<false, false>(p, st);
    } else if (a8) {
        if (!int4 || plan.bn != 128) return hipErrorInvalidValue;
        e = plan.deep ? launch_out<128, 128, 1, 6, true, true>(p, st) : launch_out<128, 128, 2, 3, true, true>(p, st);
    } else if (plan.bn == 256) {
        if (!int4) return hipErrorInvalidValue;
        e = plan.deep ? launch_out<128, 256, 1, 6, true>(p, st) : launch_out<128, 256, 2, 3, true>(p, st);
    } else if (plan.bm == 64) {
        if (int4 || a8 || !plan.deep || plan.splits != 1) return hipErrorInvalidValue;
        e = launch_out<64, 64, 1, 8, false>(p, st);
    } else if (plan.deep) {
        e = int4 ? launch_out<128, 128, 1, 8, true>(p, st) : launch_out<128, 128, 1, 8, false>(p, st);
    } else {
        e = int4 ? launch_out<128, 128, 2, 4, true>(p, st) : launch_out<128, 128, 2, 4, false>(p, st);
    }
    if (e != hipSuccess) return e;
    if (plan.splits > 1) {
        const int64_t total = m * n;
        const bool v8 = n % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(w_scale) & 15) == 0;
        if (v8) {
            dim3 grid(static_cast<unsigned>((total / 8 + 255) / 256));
            switch (y_dtype) {
                case BF16: hipLaunchKernelGGL(splitk_reduce8_kernel<BF16>, grid, dim3(256), 0, st, ws, plan.splits, m, n, x_scale, w_scale, y); break;
                case F16: hipLaunchKernelGGL(splitk_reduce8_kernel<F16>, grid, dim3(256), 0, st, ws, plan.splits, m, n, x_scale, w_scale, y); break;
                case F32: hipLaunchKernelGGL(splitk_reduce8_kernel<F32>, grid, dim3(256), 0, st, ws, plan.splits, m, n, x_scale, w_scale, y); break;
                default: hipLaunchKernelGGL(splitk_reduce8_kernel<I32>, grid, dim3(256), 0, st, ws, plan.splits, m, n, x_scale, w_scale, y); break;
            }
        } else {
            const int64_t per = (n % 4 == 0) ? 4 : 1;
            dim3 grid(static_cast<unsigned>((total / per + 255) / 256));
            hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, ws, plan.splits, m, n,
                               x_scale, w_scale, y, y_dtype);
        }
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_gemm_f6(const GemmPlan& plan, const void* xq, const float* x_scale, const void* wq,
                          const float* w_scale, int64_t m, int64_t n, int64_t k, void* y, int y_dtype, bool geglu,
                          hipStream_t st) {
    if (plan.splits != 1) return hipErrorInvalidValue;
    if (geglu) {
        hipError_t e = ensure_gelu_neg_tab(st);
        if (e != hipSuccess) return e;
    }
    GemmParams p;
    p.a = static_cast<const int8_t*>(xq);
    p.b = static_cast<const int8_t*>(wq);
    p.sx = x_scale; p.sw = w_scale; p.y = y; p.ws = nullptr;
    p.m = m; p.n = n;
    p.kbytes = k / 4 * 3;
    p.kbytes_a = p.kbytes;
    p.stages = static_cast<int>(k / 128);
    p.splits = 1;
    p.stages_per_split = p.stages;
    p.tiles_m = static_cast<int>((m + plan.bm - 1) / plan.bm);
    p.tiles_n = static_cast<int>((n + plan.bn - 1) / plan.bn);
    p.group_m = plan.group_m;
    p.y_dtype = y_dtype;
    if (plan.bm == 128 && plan.bn == 256) {   // the two-blocks-per-CU GeGLU kernel
        if (!geglu) return hipErrorInvalidValue;
        switch (p.y_dtype) {
            case BF16: return launch_f6w_geglu<BF16>(p, st);
            case F16: return launch_f6w_geglu<F16>(p, st);
            case F32: return launch_f6w_geglu<F32>(p, st);
        }
        return hipErrorInvalidValue;
    }
    if (plan.bm == 256) return launch_f6_out<256, 256, 1>(p, geglu, st);
    if (plan.bm == 128 && plan.bn == 128) return launch_f6_out<128, 128, 2>(p, geglu, st);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_geglu(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                             int64_t m, int64_t n, int64_t k, bool int4, void* y, int y_dtype,
                             hipStream_t st) {
    if (!int4) return hipErrorInvalidValue;   // the gate|up projections run at W4A4
    hipError_t e = ensure_gelu_neg_tab(st);
    if (e != hipSuccess) return e;
    const GemmPlan plan = plan_gemm(m, n, k, int4, false, false);   // tile shape; the fused epilogue takes no split
    GemmParams p;
    p.a = static_cast<const int8_t*>(xq);
    p.b = static_cast<const int8_t*>(wq);
    p.sx = x_scale; p.sw = w_scale; p.y = y; p.ws = nullptr;
    p.m = m; p.n = n;
    p.kbytes = int4 ? k / 2 : k;
    p.kbytes_a = p.kbytes;
    p.stages = static_cast<int>((p.kbytes + STAGE_BYTES - 1) / STAGE_BYTES);
    p.splits = 1;
    p.stages_per_split = p.stages;
    p.tiles_m = static_cast<int>((m + plan.bm - 1) / plan.bm);
    p.tiles_n = static_cast<int>((n + plan.bn - 1) / plan.bn);
    p.group_m = plan.group_m;
    p.y_dtype = y_dtype;
    if (plan.bm == 256) {
        switch (p.y_dtype) {
            case BF16: return launch_256<true, OUT_GEGLU + BF16, false>(p, st);
            case F16: return launch_256<true, OUT_GEGLU + F16, false>(p, st);
            case F32: return launch_256<true, OUT_GEGLU + F32, false>(p, st);
        }
        return hipErrorInvalidValue;
    }
    if (plan.bn == 256)
        return plan.deep ? launch_geglu_out<128, 256, 1, 6, true>(p, st) : launch_geglu_out<128, 256, 2, 3, true>(p, st);
    return plan.deep ? launch_geglu_out<128, 128, 1, 8, true>(p, st) : launch_geglu_out<128, 128, 2, 4, true>(p, st);
}

}  // namespace qlin
