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

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

// Round-half-even of v / scale, clamped to +-qmax.  The fast path multiplies
// by an fp32 reciprocal (relative error ~1.5 ulp); when that product lies
// within 1e-5 * max(1, |r|) of a half-integer, the quotient is recomputed in
// float64 so that the rounding decision is taken on the correctly rounded
// value: with exact inputs (no fold, no rotation) the codes then match a
// float64 reference exactly.  `div` is the exact divisor (scale * sqrt(b)).
__device__ __forceinline__ float quant_code(float v, float mul, double div, float qmax) {
    const float r = v * mul;
    float q = __builtin_rintf(r);
    const float d = fabsf(fabsf(r - q) - 0.5f);
    if (d <= 1e-5f * fmaxf(1.f, fabsf(r))) {
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
    int bits;           // 4 or 8
    void* q;            // codes out
    float* scale;       // per-row scale out
};

template <int DT, bool GEGLU>
__device__ __forceinline__ void load_row_chunk(const RowQuantParams& p, int64_t row, int64_t col,
                                               float v[8]) {
    const char* base = static_cast<const char*>(p.x);
    constexpr int ES = (DT == F32) ? 4 : 2;
    const char* r = base + (row * p.ldx + col) * ES;
    if constexpr (GEGLU) {
        float g[8], u[8];
        load8<DT>(r, g);
        load8<DT>(r + p.k * ES, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_erf(g[i]) * u[i];
    } else {
        load8<DT>(r, v);
    }
}

// Butterfly across lanes at distance MASK: lane with the bit clear keeps
// a + b, lane with the bit set keeps a - b (a = lower-index element).
template <int MASK, int NCH>
__device__ __forceinline__ void xlane_stage(float (&v)[NCH][8], int lane) {
    const bool upper = (lane & MASK) != 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float other = lane_xor<MASK>(v[c][e]);
            v[c][e] = upper ? (other - v[c][e]) : (v[c][e] + other);
        }
    }
}

template <int DT, int NCH, bool GEGLU>
__global__ __launch_bounds__(256) void rotate_quant_rows_kernel(RowQuantParams p) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = p.g;
    const int rows_per_block = 256 / g;
    const int t = tid & (g - 1);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_block + tid / g;
    const bool row_ok = row < p.m;
    const int b = p.had_block > 1 ? p.had_block : 1;

    float v[NCH][8];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t col = static_cast<int64_t>(c) * g * 8 + t * 8;
        const bool ok = row_ok && c < p.nch && col < p.k;
        if (ok) {
            load_row_chunk<DT, GEGLU>(p, row, col, v[c]);
            if (p.mult) {
                const float4* mp = reinterpret_cast<const float4*>(p.mult + col);
                float4 m0 = mp[0], m1 = mp[1];
                v[c][0] *= m0.x; v[c][1] *= m0.y; v[c][2] *= m0.z; v[c][3] *= m0.w;
                v[c][4] *= m1.x; v[c][5] *= m1.y; v[c][6] *= m1.z; v[c][7] *= m1.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
        }
        // in-register butterfly stages (distance 1, 2, 4 within the 8 values)
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
            if (h < b) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((e & h) == 0) {
                        float a0 = v[c][e], a1 = v[c][e + h];
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

#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[c][e]));

    amax = wave_max(amax, g < 64 ? g : 64);
    if (g > 64) {
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        const int wpr = g >> 6;  // waves per row
        const int first = (wave / wpr) * wpr;
        amax = red[first];
        for (int i = 1; i < wpr; ++i) amax = fmaxf(amax, red[first + i]);
    }
    if (!row_ok) return;

    // normalisation of the unnormalised transform: 1/sqrt(b)
    // fp32 of 1/sqrt(b), correctly rounded (exact for b = 4^j)
    const float nrm = static_cast<float>(1.0 / sqrt(static_cast<double>(b)));
    const float qmax = (p.bits == 8) ? 127.f : 7.f;
    const float amax_n = amax * nrm;
    const float scale = amax_n / qmax;
    const float mul = (scale > 0.f) ? nrm * (1.f / scale) : 0.f;
    const double div = static_cast<double>(scale) * sqrt(static_cast<double>(b));
    if (t == 0) p.scale[row] = scale;

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t col = static_cast<int64_t>(c) * g * 8 + t * 8;
        if (c >= p.nch || col >= p.k) continue;
        int qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = static_cast<int>(quant_code(v[c][e], mul, div, qmax));
        if (p.bits == 8) {
            uint32_t lo = (qv[0] & 0xFF) | ((qv[1] & 0xFF) << 8) | ((qv[2] & 0xFF) << 16) |
                          (static_cast<uint32_t>(qv[3] & 0xFF) << 24);
            uint32_t hi = (qv[4] & 0xFF) | ((qv[5] & 0xFF) << 8) | ((qv[6] & 0xFF) << 16) |
                          (static_cast<uint32_t>(qv[7] & 0xFF) << 24);
            int8_t* out = static_cast<int8_t*>(p.q) + row * p.k + col;
            *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) w |= static_cast<uint32_t>(qv[e] & 0xF) << (4 * e);
            uint8_t* out = static_cast<uint8_t*>(p.q) + row * (p.k / 2) + col / 2;
            *reinterpret_cast<uint32_t*>(out) = w;
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

namespace {

template <int DT, bool GEGLU>
hipError_t launch_rows_dt(const RowQuantParams& p, int nch_tpl, hipStream_t st) {
    const int rows_per_block = 256 / p.g;
    dim3 grid(static_cast<unsigned>((p.m + rows_per_block - 1) / rows_per_block));
    switch (nch_tpl) {
        case 1: hipLaunchKernelGGL((rotate_quant_rows_kernel<DT, 1, GEGLU>), grid, dim3(256), 0, st, p); break;
        case 2: hipLaunchKernelGGL((rotate_quant_rows_kernel<DT, 2, GEGLU>), grid, dim3(256), 0, st, p); break;
        case 4: hipLaunchKernelGGL((rotate_quant_rows_kernel<DT, 4, GEGLU>), grid, dim3(256), 0, st, p); break;
        case 8: hipLaunchKernelGGL((rotate_quant_rows_kernel<DT, 8, GEGLU>), grid, dim3(256), 0, st, p); break;
        case 16: hipLaunchKernelGGL((rotate_quant_rows_kernel<DT, 16, GEGLU>), grid, dim3(256), 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int row_quant_lanes(int64_t k) {
    int64_t g = 8;
    while (g < 256 && g * 8 < k) g <<= 1;
    return static_cast<int>(g);
}

int row_quant_chunks(int64_t k, int g) { return static_cast<int>((k + 8LL * g - 1) / (8LL * g)); }

hipError_t launch_rotate_quant(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                               bool geglu, const float* mult, int had_block, int bits, void* q,
                               float* scale, hipStream_t st) {
    RowQuantParams p;
    p.x = x; p.m = m; p.k = k; p.ldx = ldx; p.mult = mult;
    p.g = row_quant_lanes(k);
    p.nch = row_quant_chunks(k, p.g);
    p.had_block = had_block; p.bits = bits; p.q = q; p.scale = scale;
    int tpl = 1;
    while (tpl < p.nch) tpl <<= 1;
    if (tpl > 16) return hipErrorInvalidValue;
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
