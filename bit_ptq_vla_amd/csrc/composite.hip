// SVD-Hadamard composite rotation with the zigzag channel permutation
// (Omega-QVLA technical summary, Metodologia 1: "Rotazione SVD", "Rotazione
// Hadamard", "Implementazione a Blocchi"), for gfx950.
//
// Online (activations) and offline (weights) quantization with the composite
// rotation in place of the fast Hadamard transform: per row,
//   v[c'] = x[perm[c']] * mult[perm[c']]            (gather, optional fold)
//   v[B_j] = v[B_j] @ R_j                           (b x b rotation per block)
//   per-row symmetric quantization of v (scale = max |v| / qmax, RNE codes).
// The rotation is a dense product: dot products of b terms of fp32 operands,
// on the matrix cores with fp32 accumulation for b >= 32 (within
// gamma_b sum |x| |R| of the exact product), as fp64 sums rounded to fp32
// for b = 16.  One kernel applies block j's rotation to a tile of rows and
// writes the rotated rows (fp32) to a workspace; the row quantizer of the
// Hadamard path then quantizes them as they stand (no fold, no rotation).
//
// Offline calibration of perm and R from the weights:
//   * column norms of w * fold, fp64;
//   * zigzag: channels ranked by descending norm (lower index first on ties)
//     are dealt to the k / b blocks in snake order;
//   * per block, the Gram matrix G_j = W[:, B_j]^T W[:, B_j] (fp64) and its
//     eigenvectors by cyclic Jacobi rotations (round-robin pairs, b / 2
//     rotations per round applied together), ordered by descending
//     eigenvalue, each with its largest-magnitude entry positive; then
//     R_j = U_j H_b / sqrt(b).
// The page writes y = x W with W of shape C_in x C_out, so the U of its SVD
// acts on the input channels: in the [n][k] storage here that is the
// eigenvector matrix of W^T W, restricted to each block.

#include "device_common.h"
#include "qlin_internal.h"

namespace qlin {

namespace {

template <int DT>
__device__ __forceinline__ float load1(const void* row, int64_t i);
template <>
__device__ __forceinline__ float load1<F16>(const void* row, int64_t i) {
    return static_cast<float>(static_cast<const _Float16*>(row)[i]);
}
template <>
__device__ __forceinline__ float load1<BF16>(const void* row, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(row)[i]);
}
template <>
__device__ __forceinline__ float load1<F32>(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
}

struct CompParams {
    const void* x;
    int64_t m, k, ldx;
    const float* mult;   // fold multiplier on the original channels, or nullptr
    const int32_t* perm; // [k]
    const float* rot;    // [k/b][b][b]
    int b;
    float* v;            // out: rotated rows [m][k] fp32
};

// Block (j, column slice, row tile): CW = min(B, 64) output columns of block
// j's rotation, R[:, c0 .. c0 + CW) staged in LDS (fp32), applied to a tile of
// RT rows whose gathered, folded values are staged in LDS as the fp32
// products they are (row pitch B + 4 floats: rows of one wave fall in
// different banks).  A thread owns 4 adjacent columns of RPT rows; per four
// input channels it reads one float4 of R per channel (shared by the wave's
// row groups) and one float4 of x per row, and runs each output's fp64 FMA
// chain in channel order, so every output is the same fp64 sum as a plain
// loop over the channels.  At B = 128 two blocks fit a CU (65 KB of LDS).
template <int DT, int B, int RPT>
__global__ __launch_bounds__(256) void composite_rotate_kernel(CompParams p) {
    constexpr int CW = B < 64 ? B : 64;
    constexpr int CG = CW / 4;            // column groups of 4
    constexpr int RG = 256 / CG;          // row groups
    constexpr int RT = RG * RPT;          // rows per block
    constexpr int XP = B + 4;             // x tile pitch, floats
    extern __shared__ float lds[];
    float* rs = lds;                      // [B][CW]
    float* xs = lds + B * CW;             // [RT][XP]
    const int tid = threadIdx.x;
    const int j = blockIdx.x / (B / CW);
    const int c0 = (blockIdx.x % (B / CW)) * CW;
    const int k = static_cast<int>(p.k);
    const int64_t row0 = static_cast<int64_t>(blockIdx.y) * RT;
    {
        // R[:, c0 .. c0 + CW) of block j: B * CW / 4 float4
        constexpr int NQ = B * CW / 4;
        constexpr int PER = (NQ + 255) / 256;
        const float* rj = p.rot + static_cast<int64_t>(j) * B * B + c0;
        float4 t4[PER];
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int q = tid + 256 * t < NQ ? tid + 256 * t : NQ - 1;
            const int i = q / (CW / 4), cq = q - i * (CW / 4);
            t4[t] = *reinterpret_cast<const float4*>(rj + i * B + 4 * cq);
        }
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int q = tid + 256 * t;
            if (q < NQ) {
                const int i = q / (CW / 4), cq = q - i * (CW / 4);
                *reinterpret_cast<float4*>(rs + i * CW + 4 * cq) = t4[t];
            }
        }
    }
    {
        // gathered, folded x: a thread keeps one channel i = tid % B (256 is a
        // multiple of B) for rows tid / B + (256 / B) t: its source channel and
        // fold multiplier are loaded once, its RT * B / 256 row loads all
        // issued before the first is used
        constexpr int NR = RT * B / 256;      // rows per thread
        constexpr int RS = 256 / B;           // row stride
        const int i = tid % B, r0 = tid / B;
        int sidx = p.perm[j * B + i];
        sidx = sidx < 0 ? 0 : (sidx >= k ? k - 1 : sidx);   // (a valid permutation never clamps)
        const float f = p.mult ? p.mult[sidx] : 1.f;
        const char* xb = static_cast<const char*>(p.x);
        const int64_t pitch = p.ldx * (DT == F32 ? 4 : 2);
        float xv[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int64_t row = row0 + r0 + RS * t;
            xv[t] = load1<DT>(xb + (row < p.m ? row : 0) * pitch, sidx);
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const int64_t row = row0 + r0 + RS * t;
            xs[(r0 + RS * t) * XP + i] = row < p.m ? xv[t] * f : 0.f;
        }
    }
    __syncthreads();
    const int cg = tid % CG, rg = tid / CG;
    double acc[RPT][4];
#pragma unroll
    for (int u = 0; u < RPT; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[u][c] = 0.0;
#pragma unroll 2
    for (int i = 0; i < B; i += 4) {
        float4 r4[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) r4[ii] = *reinterpret_cast<const float4*>(rs + (i + ii) * CW + 4 * cg);
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const float4 x4 = *reinterpret_cast<const float4*>(xs + (rg + u * RG) * XP + i);
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const double xd = static_cast<double>(xv[ii]);
                acc[u][0] = __builtin_fma(xd, static_cast<double>(r4[ii].x), acc[u][0]);
                acc[u][1] = __builtin_fma(xd, static_cast<double>(r4[ii].y), acc[u][1]);
                acc[u][2] = __builtin_fma(xd, static_cast<double>(r4[ii].z), acc[u][2]);
                acc[u][3] = __builtin_fma(xd, static_cast<double>(r4[ii].w), acc[u][3]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int64_t row = row0 + rg + u * RG;
        if (row < p.m)
            *reinterpret_cast<float4*>(p.v + row * p.k + static_cast<int64_t>(j) * B + c0 + 4 * cg) =
                make_float4(static_cast<float>(acc[u][0]), static_cast<float>(acc[u][1]),
                            static_cast<float>(acc[u][2]), static_cast<float>(acc[u][3]));
    }
}

// The same rotation on the matrix cores (b = 32, 64, 128): fp32 operands,
// v_mfma_f32_32x32x2_f32 with fp32 accumulation.  A workgroup of four waves
// covers 32 * 4 / (b / 32) rows of block j; each wave one 32 x 32 output tile
// (b / 32 column tiles side by side, 128 / b row tiles).  The gathered,
// folded rows are staged in LDS (pitch b + 4 floats: the 16 lanes of a
// ds_read_b128 reach 16 distinct 16-byte bank groups); a wave's 32 columns
// of R_j are loaded into registers once.  MFMA step s pairs channel
// 8 (s / 4) + 4 h + s % 4 of both operands for lane half h, so a lane reads
// four consecutive channels of its row per four steps; the steps feed four
// accumulators in turn (independent MFMA chains), added pairwise at the end.
// Each output is thus a sum of b fp32 products with at most b fp32
// roundings: within gamma_b * sum_i |x_i| |R_ij| of the exact product of the
// fp32 operands (gamma_n = n u / (1 - n u), u = 2^-24).
typedef float v16f_c __attribute__((ext_vector_type(16)));

template <int DT, int B>
__global__ __launch_bounds__(256) void composite_rotate_mfma_kernel(CompParams p) {
    static_assert(B == 32 || B == 64 || B == 128, "32 x 32 output tiles");
    constexpr int NC = B / 32;            // column tiles
    constexpr int NR = 4 / NC;            // row tiles
    constexpr int RT = 32 * NR;           // rows per workgroup
    constexpr int P = B + 4;              // LDS row pitch, floats
    constexpr int STEPS = B / 2;          // MFMA steps (two channels each)
    __shared__ __attribute__((aligned(16))) float xs[RT * P];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = blockIdx.x;
    const int k = static_cast<int>(p.k);
    const int64_t row0 = static_cast<int64_t>(blockIdx.y) * RT;
    const int ct = wave % NC, rt = wave / NC;
    const int l32 = lane & 31, h = lane >> 5;

    // this wave's columns of R_j: rv[s] = R_j[c(s, h)][32 ct + l32]
    float rv[STEPS];
    {
        const float* rj = p.rot + static_cast<int64_t>(j) * B * B + 32 * ct + l32;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) rv[s] = rj[(8 * (s / 4) + 4 * h + (s % 4)) * B];
    }
    // gathered, folded rows: thread -> channel i = tid % B of rows tid / B + (256 / B) u
    {
        constexpr int RS = 256 / B;
        constexpr int NU = RT * B / 256;
        const int i = tid % B, r0 = tid / B;
        int sidx = p.perm[j * B + i];
        sidx = sidx < 0 ? 0 : (sidx >= k ? k - 1 : sidx);   // (a valid permutation never clamps)
        const float f = p.mult ? p.mult[sidx] : 1.f;
        const char* xb = static_cast<const char*>(p.x);
        const int64_t pitch = p.ldx * (DT == F32 ? 4 : 2);
        float xv[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int64_t row = row0 + r0 + RS * u;
            xv[u] = load1<DT>(xb + (row < p.m ? row : 0) * pitch, sidx);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int64_t row = row0 + r0 + RS * u;
            xs[(r0 + RS * u) * P + i] = row < p.m ? mul_rn(xv[u], f) : 0.f;
        }
    }
    __syncthreads();
    // four independent accumulator chains (steps s % 4), added at the end
    v16f_c acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    const float* xr = xs + (32 * rt + l32) * P + 4 * h;
#pragma unroll
    for (int t = 0; t < STEPS / 4; ++t) {
        const float4 a4 = *reinterpret_cast<const float4*>(xr + 8 * t);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, rv[4 * t + 0], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, rv[4 * t + 1], acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, rv[4 * t + 2], acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, rv[4 * t + 3], acc[3], 0, 0, 0);
    }
    v16f_c sum;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[r] = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
    // acc: column 32 ct + l32 of block j, rows 8 (r / 4) + 4 h + r % 4 of the row tile
    float* vcol = p.v + static_cast<int64_t>(j) * B + 32 * ct + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + 32 * rt + 8 * (r / 4) + 4 * h + (r % 4);
        if (row < p.m) vcol[row * p.k] = sum[r];
    }
}

// ---- calibration ------------------------------------------------------------

// Partial sums of squares of w * fold per column over a chunk of 256 rows:
// part[chunk][c] (fp64, summed afterwards in chunk order).
template <int DT>
__global__ __launch_bounds__(256) void colnorm_part_kernel(const void* w, int64_t n, int64_t k,
                                                           const float* fold, double* part) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= k) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 256;
    const int64_t r1 = r0 + 256 < n ? r0 + 256 : n;
    const double f = fold ? static_cast<double>(fold[c]) : 1.0;
    double s = 0.0;
    for (int64_t r = r0; r < r1; ++r) {
        const double v = static_cast<double>(load1<DT>(static_cast<const char*>(w) + r * k * (DT == F32 ? 4 : 2), c)) * f;
        s = __builtin_fma(v, v, s);
    }
    part[static_cast<int64_t>(blockIdx.y) * k + c] = s;
}

__global__ __launch_bounds__(256) void colnorm_sum_kernel(const double* part, int64_t chunks, int64_t k,
                                                          double* norm2) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= k) return;
    double s = 0.0;
    for (int64_t i = 0; i < chunks; ++i) s += part[i * k + c];
    norm2[c] = s;
}

// rank of channel c: channels with a larger norm, or an equal one and a
// lower index, come first; then the snake deal to its position.
__global__ __launch_bounds__(256) void zigzag_kernel(const double* norm2, int64_t k, int b, int32_t* perm) {
    __shared__ double tile[2048];
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const double mine = c < k ? norm2[c] : 0.0;
    int64_t rank = 0;
    for (int64_t t0 = 0; t0 < k; t0 += 2048) {
        __syncthreads();
        for (int i = threadIdx.x; i < 2048; i += 256) tile[i] = t0 + i < k ? norm2[t0 + i] : 0.0;
        __syncthreads();
        const int64_t lim = k - t0 < 2048 ? k - t0 : 2048;
        for (int64_t i = 0; i < lim; ++i) {
            const double o = tile[i];
            rank += (o > mine || (o == mine && t0 + i < c)) ? 1 : 0;
        }
    }
    if (c >= k) return;
    const int64_t nb = k / b;
    const int64_t t = rank / nb, i = rank - t * nb;
    const int64_t j = (t & 1) ? nb - 1 - i : i;
    perm[j * b + t] = static_cast<int32_t>(c);
}

// Gram matrix of block j of the permuted columns of w * fold:
// G[j][a][c] = sum_n v[n][perm[jb + a]] v[n][perm[jb + c]] (fp64).  Block
// (j, tile): a 16 x 16 tile of G_j, rows of w in chunks of 64 through LDS.
template <int DT>
__global__ __launch_bounds__(256) void gram_kernel(const void* w, int64_t n, int64_t k, const float* fold,
                                                   const int32_t* perm, int b, double* gram) {
    __shared__ double va[64][17], vc[64][17];
    const int j = blockIdx.x;
    const int tiles = b / 16;
    const int ta = blockIdx.y / tiles, tc = blockIdx.y - ta * tiles;
    const int ia = threadIdx.x >> 4, ic = threadIdx.x & 15;
    const int ca = perm[j * b + ta * 16 + (threadIdx.x & 15)];
    const int cc = perm[j * b + tc * 16 + (threadIdx.x & 15)];
    const double fa = fold ? static_cast<double>(fold[ca]) : 1.0;
    const double fc = fold ? static_cast<double>(fold[cc]) : 1.0;
    double acc = 0.0;
    for (int64_t r0 = 0; r0 < n; r0 += 64) {
        __syncthreads();
        // 64 rows x 16 columns of each tile: thread t loads rows t/16, t/16 + 16, ...
        for (int rr = threadIdx.x >> 4; rr < 64; rr += 16) {
            const int64_t r = r0 + rr;
            double a = 0.0, c = 0.0;
            if (r < n) {
                const char* wr = static_cast<const char*>(w) + r * k * (DT == F32 ? 4 : 2);
                a = static_cast<double>(load1<DT>(wr, ca)) * fa;
                c = static_cast<double>(load1<DT>(wr, cc)) * fc;
            }
            va[rr][threadIdx.x & 15] = a;
            vc[rr][threadIdx.x & 15] = c;
        }
        __syncthreads();
        for (int rr = 0; rr < 64; ++rr) acc = __builtin_fma(va[rr][ia], vc[rr][ic], acc);
    }
    gram[(static_cast<int64_t>(j) * b + ta * 16 + ia) * b + tc * 16 + ic] = acc;
}

// Cyclic Jacobi eigen-decomposition of one block's Gram matrix (T = double
// for b <= 64, float for b = 128 so that A and V fit LDS), then the sorted,
// sign-fixed eigenvectors times H_b / sqrt(b) into rot[j] (fp32).
// Round-robin pairing (circle method): in round r the b positions
// [0, (r + t) % (b - 1) + 1 for t = 0 .. b - 2] are paired first with last;
// the b / 2 rotations of a round touch disjoint rows and columns, so their
// row updates run together, then their column updates.  Sweeps stop when
// every off-diagonal entry is below 1e-14 (fp32: 2e-6) of the largest
// diagonal entry, or after 15 sweeps.
template <typename T>
__global__ __launch_bounds__(256) void jacobi_rot_kernel(const double* gram, int b, float* rot) {
    extern __shared__ unsigned char smem[];
    T* A = reinterpret_cast<T*>(smem);                 // [b][b]
    T* V = A + b * b;                                  // [b][b]
    __shared__ int pp[128], qq[128], order[256];
    __shared__ T cs[128], sn[128];
    __shared__ int converged;
    const int j = blockIdx.x, tid = threadIdx.x;
    const int half = b / 2;
    const double* g = gram + static_cast<int64_t>(j) * b * b;
    for (int i = tid; i < b * b; i += 256) {
        A[i] = static_cast<T>(g[i]);
        V[i] = (i / b == i % b) ? T(1) : T(0);
    }
    // converged when every off-diagonal entry is below tol times the largest
    // diagonal entry (the rounding floor of the rotations is about eps times
    // the matrix norm), or after 15 sweeps
    const T tol = sizeof(T) == 8 ? T(1e-14) : T(2e-6);
    __shared__ T dmax;
    __syncthreads();
    if (tid == 0) {
        T d = T(0);
        for (int i = 0; i < b; ++i) d = fmax(d, fabs(A[i * b + i]));
        dmax = d;
    }
    for (int sweep = 0; sweep < 15; ++sweep) {
        __syncthreads();
        if (tid == 0) converged = 1;
        __syncthreads();
        const T lim = tol * dmax;
        for (int i = tid; i < b * b; i += 256) {
            const int r = i / b, c = i - r * b;
            if (r < c && fabs(A[i]) > lim) converged = 0;
        }
        __syncthreads();
        if (converged) break;
        for (int round = 0; round < b - 1; ++round) {
            if (tid < half) {
                const int li = tid, lj = b - 1 - tid;
                const int p = li == 0 ? 0 : (round + li - 1) % (b - 1) + 1;
                const int q = (round + lj - 1) % (b - 1) + 1;
                const T apq = A[p * b + q];
                T c = T(1), s = T(0);
                if (apq != T(0)) {
                    const T tau = (A[q * b + q] - A[p * b + p]) / (T(2) * apq);
                    const T t = (tau >= T(0) ? T(1) : T(-1)) / (fabs(tau) + sqrt(T(1) + tau * tau));
                    c = T(1) / sqrt(T(1) + t * t);
                    s = t * c;
                }
                pp[tid] = p; qq[tid] = q; cs[tid] = c; sn[tid] = s;
            }
            __syncthreads();
            // rows: A <- J^T A
            for (int i = tid; i < half * b; i += 256) {
                const int pr = i / b, col = i - pr * b;
                const int p = pp[pr], q = qq[pr];
                const T c = cs[pr], s = sn[pr];
                const T ap = A[p * b + col], aq = A[q * b + col];
                A[p * b + col] = c * ap - s * aq;
                A[q * b + col] = s * ap + c * aq;
            }
            __syncthreads();
            // columns: A <- A J, V <- V J
            for (int i = tid; i < half * b; i += 256) {
                const int pr = i / b, row = i - pr * b;
                const int p = pp[pr], q = qq[pr];
                const T c = cs[pr], s = sn[pr];
                const T ap = A[row * b + p], aq = A[row * b + q];
                A[row * b + p] = c * ap - s * aq;
                A[row * b + q] = s * ap + c * aq;
                const T vp = V[row * b + p], vq = V[row * b + q];
                V[row * b + p] = c * vp - s * vq;
                V[row * b + q] = s * vp + c * vq;
            }
            __syncthreads();
        }
    }
    __syncthreads();
    // descending eigenvalues (lower index first on ties): position of column i
    if (tid < b) {
        const T d = A[tid * b + tid];
        int rank = 0;
        for (int l = 0; l < b; ++l) {
            const T e = A[l * b + l];
            rank += (e > d || (e == d && l < tid)) ? 1 : 0;
        }
        order[rank] = tid;
    }
    __syncthreads();
    // U[:, r] = +-V[:, order[r]] with its largest-magnitude entry positive,
    // then R = U H / sqrt(b), H[l][c] = (-1)^popcount(l & c)
    __shared__ T sgn[256];
    if (tid < b) {
        const int col = order[tid];
        int best = 0;
        T bv = T(-1);
        for (int r = 0; r < b; ++r) {
            const T a = fabs(V[r * b + col]);
            if (a > bv) { bv = a; best = r; }
        }
        sgn[tid] = V[best * b + col] < T(0) ? T(-1) : T(1);
    }
    __syncthreads();
    const double nrm = 1.0 / sqrt(static_cast<double>(b));
    float* out = rot + static_cast<int64_t>(j) * b * b;
    for (int i = tid; i < b * b; i += 256) {
        const int a = i / b, c = i - a * b;
        double acc = 0.0;
        for (int l = 0; l < b; ++l) {
            const double u = static_cast<double>(V[a * b + order[l]]) * static_cast<double>(sgn[l]);
            acc += (__builtin_popcount(l & c) & 1) ? -u : u;
        }
        out[i] = static_cast<float>(acc * nrm);
    }
}

template <int DT, int B, int RPT>
hipError_t launch_rot_b(const CompParams& p, hipStream_t st) {
    constexpr int CW = B < 64 ? B : 64;
    constexpr int RT = (256 / (CW / 4)) * RPT;
    const size_t lds = static_cast<size_t>(B) * CW * 4 + static_cast<size_t>(RT) * (B + 4) * 4;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(composite_rotate_kernel<DT, B, RPT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    dim3 grid(static_cast<unsigned>(p.k / B * (B / CW)), static_cast<unsigned>((p.m + RT - 1) / RT));
    hipLaunchKernelGGL((composite_rotate_kernel<DT, B, RPT>), grid, dim3(256), lds, st, p);
    return hipGetLastError();
}

// Four rows per thread when that still makes a grid of at least 256 blocks,
// else one (the action expert's few dozen rows).
template <int DT, int B>
hipError_t launch_rot_rpt(const CompParams& p, hipStream_t st) {
    constexpr int CW = B < 64 ? B : 64;
    constexpr int RT4 = (256 / (CW / 4)) * 4;
    const int64_t blocks4 = p.k / B * (B / CW) * ((p.m + RT4 - 1) / RT4);
    if (blocks4 >= 256) return launch_rot_b<DT, B, 4>(p, st);
    return launch_rot_b<DT, B, 1>(p, st);
}

template <int DT, int B>
hipError_t launch_rot_mfma(const CompParams& p, hipStream_t st) {
    constexpr int RT = 32 * (4 / (B / 32));
    dim3 grid(static_cast<unsigned>(p.k / B), static_cast<unsigned>((p.m + RT - 1) / RT));
    hipLaunchKernelGGL((composite_rotate_mfma_kernel<DT, B>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// b >= 32 on the matrix cores; b = 16 (too narrow for a 32 x 32 tile) as fp64 sums
template <int DT>
hipError_t launch_rot_dt(const CompParams& p, hipStream_t st) {
    switch (p.b) {
        case 16: return launch_rot_rpt<DT, 16>(p, st);
        case 32: return launch_rot_mfma<DT, 32>(p, st);
        case 64: return launch_rot_mfma<DT, 64>(p, st);
        case 128: return launch_rot_mfma<DT, 128>(p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_composite_quant(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx, const float* mult,
                                  const int32_t* perm, const float* rot, int b, int bits, void* q, float* scale,
                                  float* v, hipStream_t st) {
    CompParams p;
    p.x = x; p.m = m; p.k = k; p.ldx = ldx; p.mult = mult; p.perm = perm; p.rot = rot; p.b = b; p.v = v;
    hipError_t e = hipErrorInvalidValue;
    switch (dtype) {
        case F16: e = launch_rot_dt<F16>(p, st); break;
        case BF16: e = launch_rot_dt<BF16>(p, st); break;
        case F32: e = launch_rot_dt<F32>(p, st); break;
    }
    if (e != hipSuccess) return e;
    // the rotated rows are then quantized per row as they stand (no fold, no rotation)
    return launch_rotate_quant(v, F32, m, k, k, false, nullptr, 0, bits, q, scale, st);
}

hipError_t launch_calibrate_composite(const void* w, int dtype, int64_t n, int64_t k, const float* fold, int b,
                                      int32_t* perm, float* rot, void* work, hipStream_t st) {
    // work: chunks * k doubles (column partials), then k doubles (norms),
    // then k * b doubles (Gram matrices)
    const int64_t chunks = (n + 255) / 256;
    double* part = static_cast<double*>(work);
    double* norm2 = part + chunks * k;
    double* gram = norm2 + k;
    const dim3 cg(static_cast<unsigned>((k + 255) / 256), static_cast<unsigned>(chunks));
    const dim3 kg(static_cast<unsigned>((k + 255) / 256));
    const dim3 gg(static_cast<unsigned>(k / b), static_cast<unsigned>((b / 16) * (b / 16)));
    switch (dtype) {
        case F16: hipLaunchKernelGGL(colnorm_part_kernel<F16>, cg, dim3(256), 0, st, w, n, k, fold, part); break;
        case BF16: hipLaunchKernelGGL(colnorm_part_kernel<BF16>, cg, dim3(256), 0, st, w, n, k, fold, part); break;
        case F32: hipLaunchKernelGGL(colnorm_part_kernel<F32>, cg, dim3(256), 0, st, w, n, k, fold, part); break;
        default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(colnorm_sum_kernel, kg, dim3(256), 0, st, part, chunks, k, norm2);
    hipLaunchKernelGGL(zigzag_kernel, kg, dim3(256), 0, st, norm2, k, b, perm);
    switch (dtype) {
        case F16: hipLaunchKernelGGL(gram_kernel<F16>, gg, dim3(256), 0, st, w, n, k, fold, perm, b, gram); break;
        case BF16: hipLaunchKernelGGL(gram_kernel<BF16>, gg, dim3(256), 0, st, w, n, k, fold, perm, b, gram); break;
        case F32: hipLaunchKernelGGL(gram_kernel<F32>, gg, dim3(256), 0, st, w, n, k, fold, perm, b, gram); break;
    }
    if (b <= 64) {
        const size_t lds = static_cast<size_t>(2) * b * b * 8;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(jacobi_rot_kernel<double>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(jacobi_rot_kernel<double>, dim3(static_cast<unsigned>(k / b)), dim3(256), lds, st,
                           gram, b, rot);
    } else {
        const size_t lds = static_cast<size_t>(2) * b * b * 4;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(jacobi_rot_kernel<float>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(jacobi_rot_kernel<float>, dim3(static_cast<unsigned>(k / b)), dim3(256), lds, st,
                           gram, b, rot);
    }
    return hipGetLastError();
}



}  // namespace qlin
