// Fold -> block Hadamard -> per-row symmetric quantization, for gfx950.
//
// One kernel serves both the online activation stage (multiplier = 1/s,
// FoldQuantVLA abstract: channel scaling, block Hadamard, dynamic per-token
// quantization) and the offline per-output-channel weight stage (multiplier
// = s, the same rotation, round-to-nearest).  A row of k values is held by a
// group of G lanes (G a power of two, 8..256); lane t holds, for chunk pass
// c, the 8 contiguous values starting at c*8G + 8t, loaded with one 16-byte
// load.  The Hadamard block b (a power of two <= 256, Sylvester order) is
// applied as an unnormalised fast Walsh-Hadamard transform: log2(min(b,8))
// butterfly stages inside the lane's registers, then log2(b/8) stages across
// lanes (lane ^ 1, 2, ... via ds_swizzle).  The 1/sqrt(b) normalisation is
// folded into the quantization multiplier.  The row maximum is reduced across
// the G lanes (wave shuffles, then LDS when G > 64).  All arithmetic is fp32;
// rounding is round-half-to-even (v_rndne_f32).
//
// Also here: the W4A16 group quantizer (LoopQ abstract: plain RTN, 4-bit
// weight-only) and the channel-maximum kernels of the fold calibration.

#include <mutex>

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

// Distance from a half-integer below which a code is recomputed in float64.
// The multiplier mul = fp32(fp32(1/sqrt b) * fp32(1/scale)) is within 2^-22
// relative of the exact 1/(scale sqrt b), and fma forms v * mul exactly, so
// the fast value of r = v / (scale sqrt b) is off by at most 127.5 * 2^-22 =
// 3.0e-5; the window doubles that.
constexpr float kTieWindow = 6e-5f;

// Round-half-even of v / scale, clamped to +-qmax.  The fast path multiplies
// by the fp32 multiplier; when that product lies within kTieWindow of a
// half-integer, the quotient is recomputed in float64 so that the rounding
// decision is taken on the correctly rounded value: with exact inputs (no
// fold, no rotation) the codes then match a float64 reference exactly.
// `div` is the exact divisor (scale * sqrt(b)).
__device__ __forceinline__ float quant_code(float v, float mul, double div, float qmax) {
    const float r = v * mul;
    float q = __builtin_rintf(r);
    const float d = fabsf(fabsf(r - q) - 0.5f);
    if (d <= kTieWindow) {
        q = static_cast<float>(__builtin_rint(static_cast<double>(v) / div));
    }
    return fminf(fmaxf(q, -qmax), qmax);
}

struct RowQuantParams {
    const void* x;
    int64_t m, k, ldx;
    const float* mult;  // per-channel multiplier or nullptr
    int g;              // lanes per row (power of two, 8..256)
    int nch;            // chunk passes actually used (<= NCH)
    int had_block;      // 0/1: none
    int bits;           // 8 (int8), 4 (packed int4) or 6 (int4 grid stored as E2M3)
    void* q;            // codes out (column maxima as float bits in ROWQ_COLMAX)
    float* scale;       // per-row scale out (unused in ROWQ_STATIC and ROWQ_COLMAX)
    const float* post;  // per-channel table after the rotation (ROWQ_STATIC, ROWQ_POSTMUL)
};

// What the row kernel does after the fold and the rotation:
//   ROWQ_DYNAMIC  per-row amax scale and codes (the per-token / RTN quantizer);
//   ROWQ_STATIC   codes v / post[c] with a static per-channel scale table, no
//                 per-row scale (Omega-QVLA per-step activation table);
//   ROWQ_POSTMUL  v * post[c], then as ROWQ_DYNAMIC (weights of one step with
//                 its table folded in);
//   ROWQ_COLMAX   max over rows of |v| per column, as float bits (atomic max)
//                 into q (the table's calibration).
enum RowQuantMode { ROWQ_DYNAMIC = 0, ROWQ_STATIC = 1, ROWQ_POSTMUL = 2, ROWQ_COLMAX = 3 };

// Cross-lane butterfly stages.  The true transform value t is carried as
// w = sigma * t with a per-lane sign sigma.  At lane distance D the pair
// (a, b) must become (a + b, a - b); with s = -1 on the lane whose D bit is
// set and sigma equal on both lanes before the stage, w += s * w_partner
// leaves w = sigma' * t' with sigma' = s * sigma.  So each stage is a single
// multiply-add with the partner's value taken by DPP (D = 1, 2: quad
// permutations; D = 8: row rotation by 8; D = 4: two half-row rotations,
// each applied to the 4-lane banks it serves), and the final sign,
// (-1)^popcount(lane & (b/8 - 1)), is folded into the quantization scale.
// w += s * w[partner] for the 8 values of one chunk, the partner's value read
// through DPP (the fused v_fmac_f32_dpp reads src0 from the partner lane).
// The leading s_nop 1 gives the two wait states a DPP read needs after a
// VALU write of its source; inside the block each instruction reads a
// register no earlier instruction of the block wrote.
#define QLIN_DPP_FMAC8(CTRL)                                                           \
    asm("s_nop 1\n\t"                                                                  \
        "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
        "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"               \
        : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]),     \
          "+v"(w[6]), "+v"(w[7])                                                       \
        : "v"(sgn))

template <int D>
__device__ __forceinline__ void xlane8(float (&w)[8], float sgn) {
    if constexpr (D == 1) {
        QLIN_DPP_FMAC8("quad_perm:[1,0,3,2]");
    } else if constexpr (D == 2) {
        QLIN_DPP_FMAC8("quad_perm:[2,3,0,1]");
    } else if constexpr (D == 8) {
        QLIN_DPP_FMAC8("row_ror:8");
    } else {
        // D = 4 (no single DPP pattern: two moves would be needed) and D = 16
        // (crosses 16-lane rows): ds_swizzle, one VALU instruction per value
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = lane_xor<D>(w[e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = fmaf(t[e], sgn, w[e]);
    }
}

template <int D, int NCH>
__device__ __forceinline__ void xlane_stage(float (&v)[NCH][8], int lane) {
    const float sgn = (lane & D) ? -1.f : 1.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) xlane8<D>(v[c], sgn);
}

// ---- GeLU table for bfloat16 inputs ------------------------------------------
// gelu(g) for every bfloat16 g with 2^-20 <= |g| < 256, both signs: 28
// exponents x 128 mantissas x 2 signs, evaluated once per device in float64
// (erf) and rounded to fp32.  The range is wide enough that activations of
// any realistic scale never leave it (a value outside it sends its wave down
// a lane-divergent path).  Smaller |g| use 0.5 g + g^2 / sqrt(2 pi) (error
// below 1e-11 relative); |g| >= 256 gives g (positive) or 0 (negative).
constexpr int GELU_EF0 = 127 - 20;               // first tabulated exponent field
constexpr int GELU_NEXP = 28;
constexpr int GELU_HALF = GELU_NEXP * 128;       // tabulated entries per sign (3584)
constexpr int GELU_TAB = 2 * 4096;               // sign selects a 4096-entry half
__device__ float g_gelu_bf16_tab[GELU_TAB];

__global__ void gelu_table_init_kernel() {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= GELU_TAB) return;
    const int neg = i >= 4096;
    const int j = i & 4095;
    if (j >= GELU_HALF) {
        g_gelu_bf16_tab[i] = 0.f;
        return;
    }
    const uint32_t a = static_cast<uint32_t>(j + (GELU_EF0 << 7));
    const float g = __uint_as_float((a | (neg ? 0x8000u : 0u)) << 16);
    const double x = static_cast<double>(g);
    g_gelu_bf16_tab[i] = static_cast<float>(0.5 * x * (1.0 + erf(x * 0.70710678118654752440)));
}

// gelu of a bfloat16 value outside the table: tiny |g| by its Taylor start,
// |g| >= 256 as g (positive) or 0 (negative, -inf included); a NaN gate
// stays NaN, as in the fused GeGLU epilogue.
__device__ __forceinline__ float gelu_bf16_edge(uint32_t bits) {
    const float g = __uint_as_float(bits << 16);
    if (((bits & 0x7FFFu) >> 7) < static_cast<uint32_t>(GELU_EF0))
        return fmaf(g * g, 0.39894228040143267794f, 0.5f * g);
    return g > 0.f ? g : (g == g ? 0.f : g);
}

// Eight gelu values of gate bits w[0..3] (two bfloat16 per word).
__device__ __forceinline__ void gelu_bf16_8(const uint32_t w[4], const float* tab, float out[8]) {
    uint32_t idx[8];
    uint32_t worst = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        const uint32_t t = (bits & 0x7FFFu) - static_cast<uint32_t>(GELU_EF0 << 7);
        worst = worst > t ? worst : t;
        idx[i] = t | ((bits >> 3) & 0x1000u);   // sign bit 15 -> table half (bit 12)
    }
    if (worst < static_cast<uint32_t>(GELU_HALF)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = tab[idx[i]];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const uint32_t t = (bits & 0x7FFFu) - static_cast<uint32_t>(GELU_EF0 << 7);
            out[i] = t < static_cast<uint32_t>(GELU_HALF) ? tab[idx[i]] : gelu_bf16_edge(bits);
        }
    }
}

// 8 consecutive values of a row (GeGLU: gelu(gate) * up) from their raw
// 16-byte words: raw[0] holds the values (or the gate), raw[1] the up-half.
template <int DT>
__device__ __forceinline__ void decode8(const uint4* w, float f[8]) {
    if constexpr (DT == F32) {
        const float4 a = __builtin_bit_cast(float4, w[0]), b = __builtin_bit_cast(float4, w[1]);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == BF16) {
                f[2 * i] = __uint_as_float(u[i] << 16);
                f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            } else {
                f[2 * i] = f16_bits_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
                f[2 * i + 1] = f16_bits_to_f32(static_cast<uint16_t>(u[i] >> 16));
            }
        }
    }
}

template <int DT, bool GEGLU, int SRC, int W>
__device__ __forceinline__ void decode_chunk(const uint4 (&raw)[SRC][W], const float* gtab, float v[8]) {
    if constexpr (GEGLU && DT == BF16) {
        const uint32_t w[4] = {raw[0][0].x, raw[0][0].y, raw[0][0].z, raw[0][0].w};
        float gl[8], u[8];
        gelu_bf16_8(w, gtab, gl);
        decode8<DT>(raw[1], u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gl[i] * u[i];
    } else if constexpr (GEGLU) {
        float gg[8], u[8];
        decode8<DT>(raw[0], gg);
        decode8<DT>(raw[1], u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_erf(gg[i]) * u[i];
    } else {
        decode8<DT>(raw[0], v);
    }
}

// Packs eight codes held as the low bits of magic-biased floats (see below):
// int8 -> two dwords of bytes, int4 -> one dword of nibbles (element 2j in the
// low nibble of byte j).  v_perm_b32 gathers byte 0 of its two sources.
__device__ __forceinline__ uint2 pack8_i8(const uint32_t cb[8]) {
    const uint32_t a = __builtin_amdgcn_perm(cb[1], cb[0], 0x0C0C0400u);
    const uint32_t b = __builtin_amdgcn_perm(cb[3], cb[2], 0x04000C0Cu);
    const uint32_t c = __builtin_amdgcn_perm(cb[5], cb[4], 0x0C0C0400u);
    const uint32_t d = __builtin_amdgcn_perm(cb[7], cb[6], 0x04000C0Cu);
    return make_uint2(a | b, c | d);
}

__device__ __forceinline__ uint32_t pack8_i4(const uint32_t cb[8]) {
    // even elements -> bytes of E, odd elements -> bytes of O, then nibbles
    const uint32_t e = __builtin_amdgcn_perm(cb[2], cb[0], 0x0C0C0400u) |
                       __builtin_amdgcn_perm(cb[6], cb[4], 0x04000C0Cu);
    const uint32_t o = __builtin_amdgcn_perm(cb[3], cb[1], 0x0C0C0400u) |
                       __builtin_amdgcn_perm(cb[7], cb[5], 0x04000C0Cu);
    return (e & 0x0F0F0F0Fu) | ((o << 4) & 0xF0F0F0F0u);
}

// E2M3 fields (FP6: sign, 2 exponent bits with bias 1, 3 mantissa bits) of
// the int4-grid codes 0 .. 7, and of n - 16 for the two's complement nibbles
// n = 9 .. 15, by byte (n = 8, the code -8, never occurs: the grid is
// symmetric).  1 = 1.0 x 2^0 is 0b001000, 3 = 1.5 x 2^1 is 0b010100,
// 7 = 1.75 x 2^2 is 0b011110; negative codes set bit 5.
constexpr uint32_t kE2m3PosLo = 0x14100800u, kE2m3PosHi = 0x1E1C1A18u;
constexpr uint32_t kE2m3NegLo = 0x3A3C3E00u, kE2m3NegHi = 0x28303438u;

// Eight codes held as the low bytes of magic-biased floats -> 48 bits of
// E2M3 fields, code j at bits 6j .. 6j+5 (w.x bits 0..31, then w.y bits 0..15).
// Per byte: the field of the low three bits from the positive or the negative
// table (v_perm_b32 byte lookups), chosen by the byte's sign, which v_perm
// selectors 8 .. 11 replicate (the sign bits of bytes 1 and 3 of each source:
// x << 8 supplies bytes 0 and 2 there).
__device__ __forceinline__ uint2 pack8_e2m3(const uint32_t cb[8]) {
    const uint2 bytes = pack8_i8(cb);
    uint32_t f24[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t x = h ? bytes.y : bytes.x;
        const uint32_t sel = x & 0x07070707u;
        const uint32_t pos = __builtin_amdgcn_perm(kE2m3PosHi, kE2m3PosLo, sel);
        const uint32_t neg = __builtin_amdgcn_perm(kE2m3NegHi, kE2m3NegLo, sel);
        const uint32_t negm = __builtin_amdgcn_perm(x << 8, x, 0x090B080Au);
        const uint32_t c = (neg & negm) | (pos & ~negm);
        // four 6-bit fields from four bytes: pairs to 12 bits, then 24
        const uint32_t t = (c & 0x003F003Fu) | ((c >> 2) & 0x0FC00FC0u);
        f24[h] = (t & 0xFFFu) | ((t >> 4) & 0x00FFF000u);
    }
    return make_uint2(f24[0] | (f24[1] << 24), f24[1] >> 8);
}

// E2M3 store of a lane's eight codes at columns col .. col+7 of a row whose
// codes start at row_out (3 bytes per 4 codes).  The lanes 2j and 2j+1 hold
// consecutive chunks of the same row (their columns are 8 apart), so the pair
// forms 12 bytes at a 4-byte aligned offset and the even lane stores them.
// Both lanes of a pair must be active (same row, same column validity).
__device__ __forceinline__ void store8_e2m3(const uint32_t cb[8], uint8_t* row_out, int64_t col, int lane) {
    const uint2 w = pack8_e2m3(cb);
    // quad_perm [1, 0, 3, 2]: the partner lane's 48 bits
    const uint32_t o0 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(w.x), 0xB1, 0xF, 0xF, false));
    const uint32_t o1 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(w.y), 0xB1, 0xF, 0xF, false));
    if ((lane & 1) == 0) {
        uint32_t* out = reinterpret_cast<uint32_t*>(row_out + (col >> 3) * 6);
        out[0] = w.x;
        out[1] = (w.y & 0xFFFFu) | (o0 << 16);
        out[2] = (o0 >> 16) | (o1 << 16);
    }
}

// Codes of one chunk (eight magic-biased floats) to their storage: int8, packed
// int4 (two per byte) or E2M3 (see store8_e2m3).
__device__ __forceinline__ void store8_codes(int bits, const uint32_t cb[8], void* q, int64_t row, int64_t k,
                                             int64_t col, int lane) {
    if (bits == 8) {
        int8_t* out = static_cast<int8_t*>(q) + row * k + col;
        *reinterpret_cast<uint2*>(out) = pack8_i8(cb);
    } else if (bits == 4) {
        uint8_t* out = static_cast<uint8_t*>(q) + row * (k / 2) + col / 2;
        *reinterpret_cast<uint32_t*>(out) = pack8_i4(cb);
    } else {
        store8_e2m3(cb, static_cast<uint8_t*>(q) + row * (k / 4 * 3), col, lane);
    }
}

// Rows of k values; TPB lanes per block, g lanes per row (g <= TPB, RPB =
// TPB / g rows per block and iteration), NCH chunk passes of 8 values per
// lane.  Blocks are persistent: block i handles row groups i, i + grid, ...
// and (where registers allow) loads the next group while it rotates and
// quantizes the current one.  The fold multipliers of the lane's columns are
// loaded once.  No load sits
// behind a branch: rows past the end read the last row and columns past k
// read column 0, and their values are replaced by zeros afterwards.
template <int DT, int NCH, bool GEGLU, int TPB, int MODE = ROWQ_DYNAMIC>
__global__ __launch_bounds__(TPB) void rotate_quant_rows_kernel(RowQuantParams p) {
    static_assert(MODE == ROWQ_DYNAMIC || !GEGLU, "table modes take plain rows");
    constexpr int NW = TPB / 64;
    __shared__ float red[2][NW];
    constexpr bool LUT = GEGLU && DT == BF16;
    __shared__ float gtab[LUT ? GELU_TAB : 1];
    if constexpr (LUT) {
        for (int i = threadIdx.x; i < GELU_TAB; i += TPB) gtab[i] = g_gelu_bf16_tab[i];
        __syncthreads();
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = p.g;
    const int rpb = TPB / g;
    const int t = tid & (g - 1);
    const int b = p.had_block > 1 ? p.had_block : 1;
    constexpr int ES = (DT == F32) ? 4 : 2;
    constexpr int W = (DT == F32) ? 2 : 1;   // 16-byte words per 8 values
    constexpr int SRC = GEGLU ? 2 : 1;
    // prefetch the next group into registers while this one is processed,
    // where the doubled load registers still leave room without spills
    constexpr bool PF = NCH * SRC * W <= 4;

    // per-lane constants: which chunks hold columns, their fold multipliers, output scaling
    bool col_ok[NCH];
    int64_t col_ld[NCH];   // column of each chunk's load (0 where the chunk is unused)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t col = static_cast<int64_t>(c) * g * 8 + t * 8;
        col_ok[c] = c < p.nch && col < p.k;
        col_ld[c] = col_ok[c] ? col : 0;
    }
    float mlt[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        float4 m0 = make_float4(1.f, 1.f, 1.f, 1.f), m1 = m0;
        if (p.mult) {
            const float4* mp = reinterpret_cast<const float4*>(p.mult + col_ld[c]);
            m0 = mp[0];
            m1 = mp[1];
        }
        mlt[c][0] = m0.x; mlt[c][1] = m0.y; mlt[c][2] = m0.z; mlt[c][3] = m0.w;
        mlt[c][4] = m1.x; mlt[c][5] = m1.y; mlt[c][6] = m1.z; mlt[c][7] = m1.w;
    }
    constexpr bool HAS_POST = (MODE == ROWQ_STATIC || MODE == ROWQ_POSTMUL);
    float pst[HAS_POST ? NCH : 1][8];
    if constexpr (HAS_POST) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float4* pp = reinterpret_cast<const float4*>(p.post + col_ld[c]);
            const float4 a0 = pp[0], a1 = pp[1];
            pst[c][0] = a0.x; pst[c][1] = a0.y; pst[c][2] = a0.z; pst[c][3] = a0.w;
            pst[c][4] = a1.x; pst[c][5] = a1.y; pst[c][6] = a1.z; pst[c][7] = a1.w;
        }
    }
    // fp32 of 1/sqrt(b), correctly rounded (exact for b = 4^j)
    const float nrm = static_cast<float>(1.0 / sqrt(static_cast<double>(b)));
    const float qmax = (p.bits == 8) ? 127.f : 7.f;   // 4 and 6: the int4 grid
    // lane sign left by the cross-lane stages (lane bits below b/8)
    const int lane_bits = (b > 8) ? (lane & (b / 8 - 1)) : 0;
    const float sigma = (__builtin_popcount(lane_bits) & 1) ? -1.f : 1.f;

    auto load_rows = [&](int64_t row, uint4 (&raw)[NCH][SRC][W]) {
        const int64_t r = row < p.m ? row : p.m - 1;
        const char* xrow = static_cast<const char*>(p.x) + r * p.ldx * ES;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int sidx = 0; sidx < SRC; ++sidx)
#pragma unroll
                for (int w = 0; w < W; ++w)
                    raw[c][sidx][w] = reinterpret_cast<const uint4*>(xrow + (col_ld[c] + sidx * p.k) * ES)[w];
    };

    const int64_t stride = static_cast<int64_t>(gridDim.x) * rpb;
    int64_t row = static_cast<int64_t>(blockIdx.x) * rpb + tid / g;
    uint4 raw[NCH][SRC][W];
    load_rows(row, raw);
    int parity = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * rpb; base < p.m;
         base += stride, row += stride, parity ^= 1) {
        uint4 nxt[PF ? NCH : 1][SRC][W];
        if constexpr (PF) load_rows(row + stride, nxt);   // in flight while this group is processed

        // decode (GeGLU), fold, in-register butterflies
        float v[NCH][8];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            decode_chunk<DT, GEGLU>(raw[c], gtab, v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = col_ok[c] ? mul_rn(v[c][e], mlt[c][e]) : 0.f;
#pragma unroll
            for (int h = 1; h < 8; h <<= 1) {
                if (h < b) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if ((e & h) == 0) {
                            const float a0 = v[c][e], a1 = v[c][e + h];
                            v[c][e] = a0 + a1;
                            v[c][e + h] = a0 - a1;
                        }
                    }
                }
            }
        }
        // cross-lane stages: lane distance 1 .. b/16 (b/8 lanes hold one block)
        if (b > 8) xlane_stage<1, NCH>(v, lane);
        if (b > 16) xlane_stage<2, NCH>(v, lane);
        if (b > 32) xlane_stage<4, NCH>(v, lane);
        if (b > 64) xlane_stage<8, NCH>(v, lane);
        if (b > 128) xlane_stage<16, NCH>(v, lane);

        if constexpr (MODE == ROWQ_POSTMUL) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[c][e] *= pst[c][e];
        }
        if constexpr (MODE == ROWQ_COLMAX) {
            // |v| * nrm is the rotated value's magnitude; float bits of
            // non-negative values order like unsigned integers
            if (row < p.m) {
                uint32_t* cm = static_cast<uint32_t*>(p.q);
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (!col_ok[c]) continue;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        atomicMax(cm + col_ld[c] + e, __float_as_uint(fabsf(v[c][e]) * nrm));
                }
            }
        }

        // row maximum: lanes, then the row's waves through LDS (two slots
        // alternate between iterations, so one barrier per group suffices)
        float amax = 0.f;
        if constexpr (MODE == ROWQ_DYNAMIC || MODE == ROWQ_POSTMUL) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; e += 2) amax = max3_abs(amax, v[c][e], v[c][e + 1]);
        amax = wave_max(amax, g < 64 ? g : 64);
        if (g > 64) {
            if (lane == 0) red[parity][wave] = amax;
            __syncthreads();
            const int wpr = g >> 6;  // waves per row
            const int first = (wave / wpr) * wpr;
            amax = red[parity][first];
            for (int i = 1; i < wpr; ++i) amax = fmaxf(amax, red[parity][first + i]);
        }
        }

        if (MODE == ROWQ_STATIC && row < p.m) {
            // codes rne(t / post[c]) with t = sigma * nrm * v: the fp32 product
            // with sigma * nrm / post[c], redone on float64 quotients near a
            // half-integer; a zero table entry gives code 0
            constexpr float M = 12582912.f;
            const double sqb = sqrt(static_cast<double>(b));
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (!col_ok[c]) continue;
                const int64_t col = col_ld[c];
                float qb[8], mulc[8];
                float worst = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    mulc[e] = pst[c][e] > 0.f ? sigma * (nrm * (1.f / pst[c][e])) : 0.f;
                    qb[e] = fmaf(v[c][e], mulc[e], M);
                    worst = fmaxf(worst, fabsf(fmaf(v[c][e], mulc[e], M - qb[e])));
                }
                if (worst >= 0.5f - kTieWindow) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        qb[e] = (pst[c][e] > 0.f
                                     ? quant_code(v[c][e], mulc[e], sigma * static_cast<double>(pst[c][e]) * sqb, qmax)
                                     : 0.f) + M;
                }
                uint32_t cb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) cb[e] = __float_as_uint(__builtin_amdgcn_fmed3f(qb[e], M - qmax, M + qmax));
                store8_codes(p.bits, cb, p.q, row, p.k, col, lane);
            }
        }

        if ((MODE == ROWQ_DYNAMIC || MODE == ROWQ_POSTMUL) && row < p.m) {
            const float scale = (amax * nrm) / qmax;
            const float mul = (scale > 0.f) ? sigma * (nrm * (1.f / scale)) : 0.f;
            const double div = sigma * static_cast<double>(scale) * sqrt(static_cast<double>(b));
            if (t == 0) p.scale[row] = scale;

            // fma(v, mul, M) with M = 1.5 * 2^23 rounds v * mul to an integer
            // once, half to even (the fp32 spacing at M is 1); the code is the
            // low mantissa bits in two's complement, the clamp a med3 around M.
            constexpr float M = 12582912.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (!col_ok[c]) continue;
                const int64_t col = col_ld[c];
                float qb[8];
                float worst = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qb[e] = fmaf(v[c][e], mul, M);
                    worst = fmaxf(worst, fabsf(fmaf(v[c][e], mul, M - qb[e])));
                }
                // a value near a half-integer: the chunk's rounding is redone on
                // float64 quotients
                if (worst >= 0.5f - kTieWindow) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qb[e] = quant_code(v[c][e], mul, div, qmax) + M;
                }
                uint32_t cb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) cb[e] = __float_as_uint(__builtin_amdgcn_fmed3f(qb[e], M - qmax, M + qmax));
                store8_codes(p.bits, cb, p.q, row, p.k, col, lane);
            }
        }
        if constexpr (PF) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int sidx = 0; sidx < SRC; ++sidx)
#pragma unroll
                    for (int w = 0; w < W; ++w) raw[c][sidx][w] = nxt[c][sidx][w];
        } else {
            load_rows(row + stride, raw);
        }
    }
}

// ---- bfloat16 fast path ---------------------------------------------------------
// The same computation for bfloat16 rows whose k is a whole number of chunk
// passes, with the Hadamard block (64 or 128), the code width and the GeGLU
// pre-op fixed at compile time.  Per element it spends about 16 VALU
// instructions: the GeLU table index of two values at once with 16-bit
// packed arithmetic, 3 in-lane and 3-4 cross-lane butterflies (DPP, and the
// lane distance 4 through ds_swizzle), max3 reductions, and no clamp
// (|v / scale| <= qmax by construction, so the rounded code never leaves the
// grid).

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Lane distance 4 through the LDS crossbar (ds_swizzle, xor 4): one VALU
// instruction per value where the DPP form takes two, and this kernel is
// VALU-bound at the backbone's widths (the LDS unit is otherwise idle).
__device__ __forceinline__ void xlane4_swz(float (&w)[8], float sgn) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = lane_xor<4>(w[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = fmaf(t[e], sgn, w[e]);
}

// gelu of 8 bfloat16 gate values (four dwords) from the LDS table; values
// outside the tabulated range take the edge formula (rare: a lane-divergent
// branch).
__device__ __forceinline__ void gelu8_fast(const uint4 gw, const float* tab, float out[8]) {
    const uint32_t w[4] = {gw.x, gw.y, gw.z, gw.w};
    const us2 base = {static_cast<unsigned short>(GELU_EF0 << 7), static_cast<unsigned short>(GELU_EF0 << 7)};
    uint32_t idx[4];
    us2 worst = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const us2 tt = __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu) - base;   // v_pk_sub_u16
        worst = worst > tt ? worst : tt;                                         // v_pk_max_u16
        idx[i] = __builtin_bit_cast(uint32_t, tt) | ((w[i] >> 3) & 0x10001000u); // sign -> table half
    }
    const uint32_t wmax = worst.x > worst.y ? worst.x : worst.y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = tab[idx[i] & 0xFFFFu];
        out[2 * i + 1] = tab[idx[i] >> 16];
    }
    if (wmax >= static_cast<uint32_t>(GELU_HALF)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const uint32_t t = (bits & 0x7FFFu) - static_cast<uint32_t>(GELU_EF0 << 7);
            if (t >= static_cast<uint32_t>(GELU_HALF)) out[i] = gelu_bf16_edge(bits);
        }
    }
}

template <int NCH, bool GEGLU, int HB, int BITS, int TPB>
__global__ __launch_bounds__(TPB) void rotate_quant_bf16_kernel(RowQuantParams p) {
    static_assert(HB == 64 || HB == 128, "Hadamard block");
    constexpr int NW = TPB / 64;
    __shared__ float red[2][NW];
    __shared__ float gtab[GEGLU ? GELU_TAB : 1];
    if constexpr (GEGLU) {
        for (int i = threadIdx.x; i < GELU_TAB; i += TPB) gtab[i] = g_gelu_bf16_tab[i];
        __syncthreads();
    }
    constexpr int SRC = GEGLU ? 2 : 1;
    constexpr bool PF = NCH * SRC <= 4;          // prefetch the next group into registers
    constexpr float QMAX = BITS == 8 ? 127.f : 7.f;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = p.g;
    const int rpb = TPB / g;
    const int t = tid & (g - 1);

    float mlt[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        float4 m0 = make_float4(1.f, 1.f, 1.f, 1.f), m1 = m0;
        if (p.mult) {
            const float4* mp = reinterpret_cast<const float4*>(p.mult + static_cast<int64_t>(c) * g * 8 + t * 8);
            m0 = mp[0];
            m1 = mp[1];
        }
        mlt[c][0] = m0.x; mlt[c][1] = m0.y; mlt[c][2] = m0.z; mlt[c][3] = m0.w;
        mlt[c][4] = m1.x; mlt[c][5] = m1.y; mlt[c][6] = m1.z; mlt[c][7] = m1.w;
    }
    constexpr float NRM = HB == 64 ? 0.125f : 0.08838834764831845f;   // fp32(1/sqrt(HB))
    const float sigma = (__builtin_popcount(lane & (HB / 8 - 1)) & 1) ? -1.f : 1.f;

    auto load_rows = [&](int64_t row, uint4 (&raw)[NCH][SRC]) {
        const int64_t r = row < p.m ? row : p.m - 1;
        const uint16_t* xrow = static_cast<const uint16_t*>(p.x) + r * p.ldx;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int sidx = 0; sidx < SRC; ++sidx)
                raw[c][sidx] = *reinterpret_cast<const uint4*>(xrow + static_cast<int64_t>(c) * g * 8 + t * 8 + sidx * p.k);
    };

    const int64_t stride = static_cast<int64_t>(gridDim.x) * rpb;
    int64_t row = static_cast<int64_t>(blockIdx.x) * rpb + tid / g;
    uint4 raw[NCH][SRC];
    load_rows(row, raw);
    int parity = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * rpb; base < p.m;
         base += stride, row += stride, parity ^= 1) {
        uint4 nxt[PF ? NCH : 1][SRC];
        if constexpr (PF) load_rows(row + stride, nxt);

        float v[NCH][8];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t u[4] = {raw[c][SRC - 1].x, raw[c][SRC - 1].y, raw[c][SRC - 1].z, raw[c][SRC - 1].w};
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(u[i] << 16);
                x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            }
            if constexpr (GEGLU) {
                float gl[8];
                gelu8_fast(raw[c][0], gtab, gl);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= gl[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = mul_rn(x[e], mlt[c][e]);
#pragma unroll
            for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((e & h) == 0) {
                        const float a0 = v[c][e], a1 = v[c][e + h];
                        v[c][e] = a0 + a1;
                        v[c][e + h] = a0 - a1;
                    }
                }
            }
        }
        {
            const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f;
            const float s4 = (lane & 4) ? -1.f : 1.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                xlane8<1>(v[c], s1);
                xlane8<2>(v[c], s2);
                xlane4_swz(v[c], s4);
                if constexpr (HB == 128) xlane8<8>(v[c], (lane & 8) ? -1.f : 1.f);
            }
        }

        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; e += 2) amax = max3_abs(amax, v[c][e], v[c][e + 1]);
        amax = wave_max(amax, g < 64 ? g : 64);
        if (g > 64) {
            if (lane == 0) red[parity][wave] = amax;
            __syncthreads();
            const int wpr = g >> 6;
            const int first = (wave / wpr) * wpr;
            amax = red[parity][first];
            for (int i = 1; i < wpr; ++i) amax = fmaxf(amax, red[parity][first + i]);
        }

        if (row < p.m) {
            const float scale = (amax * NRM) / QMAX;
            const float mul = (scale > 0.f) ? sigma * (NRM * (1.f / scale)) : 0.f;
            if (t == 0) p.scale[row] = scale;
            constexpr float M = 12582912.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int64_t col = static_cast<int64_t>(c) * g * 8 + t * 8;
                float qb[8];
                float worst = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) qb[e] = fmaf(v[c][e], mul, M);
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    worst = max3_abs(worst, fmaf(v[c][e], mul, M - qb[e]), fmaf(v[c][e + 1], mul, M - qb[e + 1]));
                if (worst >= 0.5f - kTieWindow) {
                    const double div = sigma * static_cast<double>(scale) * (HB == 64 ? 8.0 : 11.313708498984761);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qb[e] = quant_code(v[c][e], mul, div, QMAX) + M;
                }
                uint32_t cb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) cb[e] = __float_as_uint(qb[e]);
                store8_codes(BITS, cb, p.q, row, p.k, col, lane);
            }
        }
        if constexpr (PF) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int sidx = 0; sidx < SRC; ++sidx) raw[c][sidx] = nxt[c][sidx];
        } else {
            load_rows(row + stride, raw);
        }
    }
}

// ---- W4A16 group quantizer ---------------------------------------------------

// float64 -> fp16 bits with a single round-half-to-even: truncate to fp32
// toward zero and mark inexactness in the last bit (round to odd), then
// round to fp16; fp32 keeps more than two extra bits, so this is exact RNE.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double d) {
    float f = static_cast<float>(d);
    if (fabs(static_cast<double>(f)) > fabs(d)) {
        f = __uint_as_float(__float_as_uint(f) - 1u);  // one step toward zero
    }
    if (static_cast<double>(f) != d) f = __uint_as_float(__float_as_uint(f) | 1u);
    return f32_to_f16_bits(f);
}

struct GroupQuantParams {
    const void* w;
    int64_t n, k;
    uint8_t* q;        // packed int4 [n][k/2]
    uint16_t* scale;   // fp16 [n][k/128]
};

// One 128-wide group is held by 16 lanes (8 values each); a block of 256
// lanes covers 16 groups, i.e. 2048 consecutive values of the flattened
// [n][k] matrix (k % 128 == 0 keeps groups inside rows).
template <int DT>
__global__ __launch_bounds__(256) void quant_groups_w4_kernel(GroupQuantParams p) {
    const int64_t total = p.n * p.k;
    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
    const bool ok = e0 < total;
    float v[8];
    constexpr int ES = (DT == F32) ? 4 : 2;
    if (ok) {
        load8<DT>(static_cast<const char*>(p.w) + e0 * ES, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max(amax, 16);
    if (!ok) return;
    const uint16_t s16 = f64_to_f16_rne(static_cast<double>(amax) / 7.0);
    const float s = f16_bits_to_f32(s16);
    const float mul = (s > 0.f) ? 1.f / s : 0.f;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = static_cast<int>(quant_code(v[i], mul, static_cast<double>(s), 7.f));
        w |= static_cast<uint32_t>(c & 0xF) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(p.q + e0 / 2) = w;
    if ((threadIdx.x & 15) == 0) p.scale[e0 / 128] = s16;
}

// ---- fold calibration: channel maxima ------------------------------------------

__global__ void fill_u32_kernel(uint32_t* a, int64_t n, uint32_t v) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) a[i] = v;
}

// Column maximum of |x| (or |gelu(gate) * up|) over rows: each thread owns 8
// consecutive columns and walks `rows_per_thread` rows, then merges with an
// integer atomicMax on the float bit pattern (valid for non-negative floats).
template <int DT, bool GEGLU>
__global__ __launch_bounds__(256) void colmax_kernel(const void* x, int64_t m, int64_t k,
                                                     int64_t ldx, int rows_per_block,
                                                     uint32_t* out) {
    const int64_t col = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
    if (col >= k) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows_per_block;
    int64_t r1 = r0 + rows_per_block;
    if (r1 > m) r1 = m;
    constexpr int ES = (DT == F32) ? 4 : 2;
    float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t r = r0; r < r1; ++r) {
        const char* rp = static_cast<const char*>(x) + (r * ldx + col) * ES;
        float v[8];
        if constexpr (GEGLU) {
            float g[8], u[8];
            load8<DT>(rp, g);
            load8<DT>(rp + k * ES, u);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = gelu_erf(g[i]) * u[i];
        } else {
            load8<DT>(rp, v);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(v[i]));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) atomicMax(out + col + i, __float_as_uint(mx[i]));
}

__global__ void fold_finish_kernel(float* s, float* inv_s, int64_t k) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= k) return;
    const float ax = __uint_as_float(reinterpret_cast<uint32_t*>(s)[i]);
    const float aw = __uint_as_float(reinterpret_cast<uint32_t*>(inv_s)[i]);
    float si = 1.f;
    if (ax > 0.f && aw > 0.f) si = static_cast<float>(sqrt(static_cast<double>(ax) / static_cast<double>(aw)));
    s[i] = si;
    inv_s[i] = 1.f / si;
}

// ---- host launchers ----------------------------------------------------------

// Compute units of the current device (cached per device).
namespace {

template <int DT, int NCH, bool GEGLU, int TPB, int MODE = ROWQ_DYNAMIC>
hipError_t launch_rows_nch(const RowQuantParams& p, hipStream_t st) {
    auto kern = rotate_quant_rows_kernel<DT, NCH, GEGLU, TPB, MODE>;
    // resident blocks per CU of this instantiation (queried once)
    static const int per_cu = [&] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, TPB, 0) != hipSuccess || n <= 0) n = 1;
        return n;
    }();
    const int rows_per_block = TPB / p.g;
    const int64_t groups = (p.m + rows_per_block - 1) / rows_per_block;
    // persistent blocks: as many as are resident at once, at most one per row group
    const int64_t slots = static_cast<int64_t>(device_cus()) * per_cu;
    dim3 grid(static_cast<unsigned>(groups < slots ? groups : slots));
    hipLaunchKernelGGL(kern, grid, dim3(TPB), 0, st, p);
    return hipGetLastError();
}

template <int DT, bool GEGLU, int TPB, int MODE = ROWQ_DYNAMIC>
hipError_t launch_rows_tpb(const RowQuantParams& p, int nch_tpl, hipStream_t st) {
    switch (nch_tpl) {
        case 1: return launch_rows_nch<DT, 1, GEGLU, TPB, MODE>(p, st);
        case 2: return launch_rows_nch<DT, 2, GEGLU, TPB, MODE>(p, st);
        case 4: return launch_rows_nch<DT, 4, GEGLU, TPB, MODE>(p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int NCH, bool GEGLU, int HB, int BITS, int TPB>
hipError_t launch_fast(const RowQuantParams& p, hipStream_t st) {
    auto kern = rotate_quant_bf16_kernel<NCH, GEGLU, HB, BITS, TPB>;
    static const int per_cu = [&] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, TPB, 0) != hipSuccess || n <= 0) n = 1;
        return n;
    }();
    const int rows_per_block = TPB / p.g;
    const int64_t groups = (p.m + rows_per_block - 1) / rows_per_block;
    const int64_t slots = static_cast<int64_t>(device_cus()) * per_cu;
    dim3 grid(static_cast<unsigned>(groups < slots ? groups : slots));
    hipLaunchKernelGGL(kern, grid, dim3(TPB), 0, st, p);
    return hipGetLastError();
}

template <bool GEGLU, int HB, int BITS, int TPB>
hipError_t launch_fast_nch(const RowQuantParams& p, hipStream_t st) {
    switch (p.nch) {
        case 1: return launch_fast<1, GEGLU, HB, BITS, TPB>(p, st);
        case 2: return launch_fast<2, GEGLU, HB, BITS, TPB>(p, st);
        case 4: return launch_fast<4, GEGLU, HB, BITS, TPB>(p, st);
    }
    return hipErrorInvalidValue;
}

template <bool GEGLU, int HB, int BITS>
hipError_t launch_fast_tpb(const RowQuantParams& p, hipStream_t st) {
    if (p.g > 256) return launch_fast_nch<GEGLU, HB, BITS, 1024>(p, st);
    return launch_fast_nch<GEGLU, HB, BITS, 256>(p, st);
}

template <bool GEGLU, int HB>
hipError_t launch_fast_bits(const RowQuantParams& p, hipStream_t st) {
    switch (p.bits) {
        case 8: return launch_fast_tpb<GEGLU, HB, 8>(p, st);
        case 4: return launch_fast_tpb<GEGLU, HB, 4>(p, st);
        case 6: return launch_fast_tpb<GEGLU, HB, 6>(p, st);
    }
    return hipErrorInvalidValue;
}

template <bool GEGLU>
hipError_t launch_fast_geglu(const RowQuantParams& p, hipStream_t st) {
    if (p.had_block == 64) return launch_fast_bits<GEGLU, 64>(p, st);
    return launch_fast_bits<GEGLU, 128>(p, st);
}

hipError_t launch_bf16_fast(const RowQuantParams& p, bool geglu, hipStream_t st) {
    return geglu ? launch_fast_geglu<true>(p, st) : launch_fast_geglu<false>(p, st);
}

template <int DT, bool GEGLU, int MODE = ROWQ_DYNAMIC>
hipError_t launch_rows_dt(const RowQuantParams& p, int nch_tpl, hipStream_t st) {
    if (p.g > 256) return launch_rows_tpb<DT, GEGLU, 1024, MODE>(p, nch_tpl, st);
    return launch_rows_tpb<DT, GEGLU, 256, MODE>(p, nch_tpl, st);
}

template <int MODE>
hipError_t launch_rows_mode(const RowQuantParams& p, int dtype, int nch_tpl, hipStream_t st) {
    switch (dtype) {
        case F16: return launch_rows_dt<F16, false, MODE>(p, nch_tpl, st);
        case BF16: return launch_rows_dt<BF16, false, MODE>(p, nch_tpl, st);
        case F32: return launch_rows_dt<F32, false, MODE>(p, nch_tpl, st);
    }
    return hipErrorInvalidValue;
}

// table = column maximum bits / qmax, in place (fp32 division)
__global__ void step_scale_finish_kernel(float* table, int64_t k, float qmax) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= k) return;
    table[i] = __uint_as_float(reinterpret_cast<uint32_t*>(table)[i]) / qmax;
}

}  // namespace

// Lanes per row: a power of two >= k / 8 up to 256 (several rows per block),
// 1024 lanes (one row per 1024-thread block) for longer rows, and 512 lanes
// (two rows per block) for 12288 < k <= 16384.  Many rows of 1024, 2048 or
// 4096 values (m * k >= 2^21) take k / 32 lanes with four chunks each instead
// (a power of two of at least 32 lanes, so a Hadamard block of up to 256
// stays in a row): at
// k = 2048 one wave per row, whose maximum then needs no block barrier, and
// four independent chunks per lane (52224 x 2048 bf16: 64 us against 87 us
// with 256 lanes per row; 816 x 4096: 6.9 us against 11.2 us).
int row_quant_lanes(int64_t k, int64_t m) {
    if ((k == 1024 || k == 2048 || k == 4096) && m * k >= (int64_t{1} << 21)) return static_cast<int>(k / 32);
    int64_t g = 8;
    while (g < 1024 && g * 8 < k) g <<= 1;
    if (g == 512) g = 1024;
    // 12288 < k <= 16384: 512 lanes with four chunks each, two rows per block
    // (measured ~9% faster than 1024 lanes x two chunks at k = 16384)
    if (k > 3 * 4096 && k <= 4 * 4096) g = 512;
    return static_cast<int>(g);
}

int row_quant_chunks(int64_t k, int g) { return static_cast<int>((k + 8LL * g - 1) / (8LL * g)); }

namespace {
std::mutex g_once_mu;
}  // namespace

hipError_t fill_once_per_device(OncePerDevice& once, hipStream_t caller, hipError_t (*fill)(hipStream_t)) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_once_mu);
    if (once.ready[dev]) return hipSuccess;
    if (caller != nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(caller, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    }
    hipStream_t own = nullptr;
    e = hipStreamCreateWithFlags(&own, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    e = fill(own);
    const hipError_t es = hipStreamSynchronize(own);
    if (e == hipSuccess) e = es;
    const hipError_t ed = hipStreamDestroy(own);
    if (e == hipSuccess) e = ed;
    if (e == hipSuccess) once.ready[dev] = true;
    return e;
}

namespace {
OncePerDevice g_gelu_tab_once;

hipError_t fill_gelu_table(hipStream_t st) {
    hipLaunchKernelGGL(gelu_table_init_kernel, dim3((GELU_TAB + 255) / 256), dim3(256), 0, st);
    return hipGetLastError();
}

// The bfloat16 GeLU table of this device, filled before first use.
hipError_t ensure_gelu_table(hipStream_t st) { return fill_once_per_device(g_gelu_tab_once, st, fill_gelu_table); }
}  // namespace

hipError_t launch_rotate_quant(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                               bool geglu, const float* mult, int had_block, int bits, void* q,
                               float* scale, hipStream_t st) {
    if (geglu && dtype == BF16) {
        hipError_t e = ensure_gelu_table(st);
        if (e != hipSuccess) return e;
    }
    RowQuantParams p;
    p.x = x; p.m = m; p.k = k; p.ldx = ldx; p.mult = mult;
    p.g = row_quant_lanes(k, m);
    p.nch = row_quant_chunks(k, p.g);
    p.had_block = had_block; p.bits = bits; p.q = q; p.scale = scale; p.post = nullptr;
    int tpl = 1;
    while (tpl < p.nch) tpl <<= 1;
    if (tpl > 4) return hipErrorInvalidValue;
    // bfloat16 rows made of whole chunk passes, Hadamard block 64 or 128
    if (dtype == BF16 && (had_block == 64 || had_block == 128) && tpl == p.nch &&
        static_cast<int64_t>(p.nch) * 8 * p.g == k && p.g >= had_block / 8)
        return launch_bf16_fast(p, geglu, st);
    if (geglu) {
        switch (dtype) {
            case F16: return launch_rows_dt<F16, true>(p, tpl, st);
            case BF16: return launch_rows_dt<BF16, true>(p, tpl, st);
            case F32: return launch_rows_dt<F32, true>(p, tpl, st);
        }
    } else {
        switch (dtype) {
            case F16: return launch_rows_dt<F16, false>(p, tpl, st);
            case BF16: return launch_rows_dt<BF16, false>(p, tpl, st);
            case F32: return launch_rows_dt<F32, false>(p, tpl, st);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_rotate_quant_table(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                     const float* mult, int had_block, int bits, const float* table,
                                     bool weights, void* q, float* scale, hipStream_t st) {
    RowQuantParams p;
    p.x = x; p.m = m; p.k = k; p.ldx = ldx; p.mult = mult;
    p.g = row_quant_lanes(k, 0);
    p.nch = row_quant_chunks(k, p.g);
    p.had_block = had_block; p.bits = bits; p.q = q; p.scale = scale; p.post = table;
    int tpl = 1;
    while (tpl < p.nch) tpl <<= 1;
    if (tpl > 4) return hipErrorInvalidValue;
    if (weights) return launch_rows_mode<ROWQ_POSTMUL>(p, dtype, tpl, st);
    return launch_rows_mode<ROWQ_STATIC>(p, dtype, tpl, st);
}

hipError_t launch_calibrate_step_scales(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                        const float* mult, int had_block, int bits, float* table,
                                        hipStream_t st) {
    RowQuantParams p;
    p.x = x; p.m = m; p.k = k; p.ldx = ldx; p.mult = mult;
    p.g = row_quant_lanes(k, 0);
    p.nch = row_quant_chunks(k, p.g);
    p.had_block = had_block; p.bits = bits; p.q = table; p.scale = nullptr; p.post = nullptr;
    int tpl = 1;
    while (tpl < p.nch) tpl <<= 1;
    if (tpl > 4) return hipErrorInvalidValue;
    const dim3 fg(static_cast<unsigned>((k + 255) / 256));
    hipLaunchKernelGGL(fill_u32_kernel, fg, dim3(256), 0, st, reinterpret_cast<uint32_t*>(table), k, 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_rows_mode<ROWQ_COLMAX>(p, dtype, tpl, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(step_scale_finish_kernel, fg, dim3(256), 0, st, table, k, bits == 8 ? 127.f : 7.f);
    return hipGetLastError();
}

hipError_t launch_quant_groups_w4(const void* w, int dtype, int64_t n, int64_t k, void* q,
                                  void* scale, hipStream_t st) {
    GroupQuantParams p{w, n, k, static_cast<uint8_t*>(q), static_cast<uint16_t*>(scale)};
    const int64_t total = n * k;
    dim3 grid(static_cast<unsigned>((total / 8 + 255) / 256));
    switch (dtype) {
        case F16: hipLaunchKernelGGL(quant_groups_w4_kernel<F16>, grid, dim3(256), 0, st, p); break;
        case BF16: hipLaunchKernelGGL(quant_groups_w4_kernel<BF16>, grid, dim3(256), 0, st, p); break;
        case F32: hipLaunchKernelGGL(quant_groups_w4_kernel<F32>, grid, dim3(256), 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

namespace {
template <int DT, bool GEGLU>
void launch_colmax(const void* x, int64_t m, int64_t k, int64_t ldx, uint32_t* out, hipStream_t st) {
    const int rows_per_block = 64;
    dim3 grid(static_cast<unsigned>((k / 8 + 255) / 256),
              static_cast<unsigned>((m + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL((colmax_kernel<DT, GEGLU>), grid, dim3(256), 0, st, x, m, k, ldx,
                       rows_per_block, out);
}

void colmax_any(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx, bool geglu,
                uint32_t* out, hipStream_t st) {
    if (geglu) {
        if (dtype == F16) launch_colmax<F16, true>(x, m, k, ldx, out, st);
        else if (dtype == BF16) launch_colmax<BF16, true>(x, m, k, ldx, out, st);
        else launch_colmax<F32, true>(x, m, k, ldx, out, st);
    } else {
        if (dtype == F16) launch_colmax<F16, false>(x, m, k, ldx, out, st);
        else if (dtype == BF16) launch_colmax<BF16, false>(x, m, k, ldx, out, st);
        else launch_colmax<F32, false>(x, m, k, ldx, out, st);
    }
}
}  // namespace

hipError_t launch_calibrate_fold(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                                 bool geglu, const void* w, int w_dtype, int64_t n, float* s,
                                 float* inv_s, hipStream_t st) {
    // s and inv_s first hold the activation / weight channel maxima as bits.
    dim3 fg(static_cast<unsigned>((k + 255) / 256));
    hipLaunchKernelGGL(fill_u32_kernel, fg, dim3(256), 0, st, reinterpret_cast<uint32_t*>(s), k, 0u);
    hipLaunchKernelGGL(fill_u32_kernel, fg, dim3(256), 0, st, reinterpret_cast<uint32_t*>(inv_s), k, 0u);
    colmax_any(x, x_dtype, m, k, ldx, geglu, reinterpret_cast<uint32_t*>(s), st);
    colmax_any(w, w_dtype, n, k, k, false, reinterpret_cast<uint32_t*>(inv_s), st);
    hipLaunchKernelGGL(fold_finish_kernel, fg, dim3(256), 0, st, s, inv_s, k);
    return hipGetLastError();
}

}  // namespace qlin
