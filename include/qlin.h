/*
 * qlin.h -- C ABI of the MI355X (gfx950) quantized linear projection library.
 *
 * The projection follows the FoldQuantVLA abstract ("FoldQuantVLA: Native
 * Low-Bit Quantization of Vision-Language-Action Models via Consistent
 * Folding"): a per-input-channel scale fold, a block Hadamard rotation and
 * dynamic per-token quantization of the activations, an integer GEMM against
 * round-to-nearest per-output-channel int4/int8 weights, and a dequantizing
 * epilogue; attention-output and FFN-down projections may run at W8A8 while
 * the rest run at W4A4.  The block form of the rotation follows the
 * Omega-QVLA technical summary (Metodologia 1, "Implementazione a Blocchi").
 * The weight-only W4A16 GEMV is the batch-1 memory-bound case of the LoopQ
 * abstract ("LoopQ: Fair, Closed-Loop Evaluation of Quantized
 * Vision-Language-Action Models").
 *
 * Conventions for every entry point
 *  - Tensor arguments are DEVICE pointers owned by the caller.  Matrices are
 *    row-major; W is [n][k] (output channel n, input channel k), so the
 *    projection is Y[m][n] = sum_k X[m][k] * W[n][k].
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Work is enqueued on it; no entry point synchronizes the device.
 *  - Arguments are validated on the host before any HIP call.  On an error
 *    the status is returned and no output is touched.  Asynchronous device
 *    faults surface at the caller's next synchronization.
 *  - Every device pointer must be 16-byte aligned; row pitches (ld*) are in
 *    elements and must keep each row 16-byte aligned.  Outputs must not
 *    overlap inputs.
 *  - m == 0 (no tokens) is a valid empty call: QLIN_OK, nothing launched.
 *  - Entry points are thread-safe.  No entry point allocates device memory:
 *    scratch (split-K partial sums, rotated rows, calibration temporaries)
 *    comes from a caller-owned workspace argument where an operation needs
 *    one, with a *_bytes query of its size.
 *  - Two lookup tables (the GeLU values of the GeGLU paths) are filled once
 *    per device by the first call that needs them, on a private stream that
 *    the library waits for; if that first call is made while `stream` is
 *    being captured into a graph it returns QLIN_ERR_CAPTURE (make one such
 *    call outside capture first).
 *  - Codes: int8 codes are int8_t[rows][k]; int4 codes are packed two per
 *    byte, uint8_t[rows][k/2], element 2j in the low nibble and 2j+1 in the
 *    high nibble, two's complement.  Both grids are symmetric: codes lie in
 *    [-7, 7] or [-127, 127].
 *  - E2M3 codes (bits == QLIN_BITS_E2M3 in the quantizers, scheme
 *    QLIN_W4A4_E2M3 in the GEMMs): the int4 grid's codes, the same integers
 *    -7 .. 7, each stored as the 6-bit FP6 E2M3 element of the OCP
 *    Microscaling (MX) v1.0 format whose value is that integer (sign bit 5,
 *    exponent bits 4..3 with bias 1, mantissa bits 2..0), packed densely
 *    little-endian: code j of a row at bits 6j .. 6j+5 of the row's bytes,
 *    uint8_t[rows][3k/4].  This is the operand format of the FP6 matrix
 *    cores; the projection's results are those of the packed-int4 form.
 *  - Rounding is round-half-to-even everywhere (codes and fp16/bf16 outputs).
 */
#ifndef QLIN_H
#define QLIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLIN_ABI_VERSION 3

typedef int32_t qlin_status;
enum {
    QLIN_OK = 0,
    QLIN_ERR_NULL = 1,        /* a required pointer is NULL                       */
    QLIN_ERR_SHAPE = 2,       /* sizes violate a stated precondition              */
    QLIN_ERR_DTYPE = 3,       /* dtype not accepted for this argument             */
    QLIN_ERR_ALIGN = 4,       /* pointer or row pitch not 16-byte aligned         */
    QLIN_ERR_UNSUPPORTED = 5, /* bits / block / group / pre-op value not supported */
    QLIN_ERR_DEVICE = 6,      /* no usable gfx950 device / HIP runtime error      */
    QLIN_ERR_LAUNCH = 7,      /* kernel launch failed (hipGetLastError)           */
    QLIN_ERR_ALIAS = 8,       /* an output overlaps an input                      */
    QLIN_ERR_CAPTURE = 9,     /* first use of a lookup table inside stream capture */
    QLIN_ERR_WORKSPACE = 10   /* workspace smaller than the call needs            */
};

typedef int32_t qlin_dtype;
enum { QLIN_F16 = 0, QLIN_BF16 = 1, QLIN_F32 = 2, QLIN_I32 = 3 };

typedef int32_t qlin_preop;
enum { QLIN_PRE_NONE = 0, QLIN_PRE_GEGLU = 1 };

/* Integer GEMM schemes: activation codes x weight codes.  QLIN_W4A4_E2M3 is
 * W4A4 with both operands in E2M3 storage (see the conventions above). */
typedef int32_t qlin_scheme;
enum { QLIN_W4A4 = 0, QLIN_W8A8 = 1, QLIN_W4A8 = 2, QLIN_W4A4_E2M3 = 3 };

/* `bits` value of the quantizers for int4-grid codes (qmax 7) written in
 * E2M3 storage; k must then be a multiple of 128. */
#define QLIN_BITS_E2M3 6

/* Version of this ABI (QLIN_ABI_VERSION). */
int32_t qlin_abi_version(void);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char* qlin_status_string(qlin_status s);

/*
 * qlin_calibrate_fold -- per-input-channel fold vector of the channel-scale
 * fold (FoldQuantVLA abstract, "channel scaling"; the balance point
 * s_j = sqrt(max_m |X[m][j]| / max_n |W[n][j]|) is the formula taken).
 *
 *   x        [m][ldx] activations, x_dtype F16/BF16/F32.  With pre == GEGLU a
 *            row holds [gate | up] (2k values, ldx >= 2k) and the channel
 *            maximum is taken over gelu(gate) * up (exact erf GeLU, fp32).
 *   w        [n][k] weights, w_dtype F16/BF16/F32 (channel j is column j).
 *   s        out float[k]: s_j in fp32 (1 where either maximum is 0).
 *   inv_s    out float[k]: 1 / s_j rounded to fp32.
 * Preconditions: m, n, k >= 1; k % 8 == 0; ldx % 8 == 0 and ldx >= k (2k
 * with GEGLU).  This is an offline calibration step, not part of the timed
 * projection.
 */
qlin_status qlin_calibrate_fold(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                int64_t ldx, qlin_preop pre, const void* w, qlin_dtype w_dtype,
                                int64_t n, float* s, float* inv_s, void* stream);

/*
 * qlin_quantize_weights -- offline weight quantization.
 *
 * group == 0 (W4A4 / W8A8 weights, FoldQuantVLA abstract "weight rounding"):
 *   w_hat = (w * fold_s) @ blockdiag(H_b / sqrt(b)) row by row, then per
 *   output channel n: w_scale[n] = fp32(max_k |w_hat[n][k]| / qmax),
 *   code = clamp(rne(w_hat / w_scale[n]), -qmax, qmax); qmax = 7 or 127.
 *   w_scale is float[n].  A zero row gives scale 0 and codes 0.
 * group == 128 (W4A16, LoopQ abstract: plain round-to-nearest, 4-bit
 *   weight-only): bits must be 4, fold_s NULL and had_block 0 or 1.  Per row n
 *   and group g: s16 = fp16_rne(max |w| / 7) over the group's 128 inputs,
 *   code = clamp(rne(w / s16), -7, 7); w_scale is uint16_t (fp16) [n][k/128].
 *
 *   w        [n][k] float weights, w_dtype F16/BF16/F32, contiguous.
 *   fold_s   float[k] fold vector or NULL (no fold).
 *   had_block Hadamard block b: 0 or 1 = none, else a power of two <= 256
 *            dividing k.  Sylvester (natural) order, orthonormal.
 *   bits     4, 8 or QLIN_BITS_E2M3 (group 0 only).   wq: out codes (layout
 *            above).
 * Preconditions: n, k >= 1; k % 8 == 0 (k % 128 == 0 for E2M3); k % group == 0.
 */
qlin_status qlin_quantize_weights(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                  const float* fold_s, int32_t had_block, int32_t bits,
                                  int32_t group, void* wq, void* w_scale, void* stream);

/*
 * qlin_rotate_quant_act -- the online activation stage (FoldQuantVLA
 * abstract: channel scaling + block Hadamard + dynamic per-token
 * quantization).  Per token row m:
 *   v = (pre(x[m]) * fold_inv_s) @ blockdiag(H_b / sqrt(b));
 *   x_scale[m] = fp32(max_k |v| / qmax); xq = clamp(rne(v / x_scale[m]), +-qmax).
 *   pre == NONE : x holds [m][ldx] with the k inputs first in each row.
 *   pre == GEGLU: x holds [gate | up] (2k values per row, ldx >= 2k) and
 *                 v is computed from gelu(gate) * up (exact erf form, fp32).
 *   x_dtype F16/BF16/F32; fold_inv_s float[k] (1/s) or NULL;
 *   had_block 0/1 = none, else a power of two <= 256 dividing k; bits 4, 8
 *   or QLIN_BITS_E2M3 (the int4 codes in E2M3 storage).
 *   xq: out codes [m][k] int8, [m][k/2] packed int4 or [m][3k/4] E2M3;
 *   x_scale: out float[m].  A zero row gives scale 0 and codes 0.
 * Preconditions: k >= 8, k % 8 == 0 (k % 128 == 0 for E2M3); ldx % 8 == 0.
 */
qlin_status qlin_rotate_quant_act(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                  int64_t ldx, qlin_preop pre, const float* fold_inv_s,
                                  int32_t had_block, int32_t bits, void* xq, float* x_scale,
                                  void* stream);

/*
 * Per-step static activation scales (Omega-QVLA technical summary,
 * Metodologia 2, "Scalatura delle Attivazioni DiT per Passo": a scale table
 * per denoising step, layer and channel, computed beforehand from
 * calibration trajectories and looked up at inference in place of one static
 * scale).  Reading taken: the table holds one scale per input channel of the
 * projection, in the rotated space where activations are quantized; since a
 * per-channel scale cannot leave the integer dot product, each step gets its
 * own weights with the table folded in, and the GEMM then takes x_scale = 1.
 * v below is the activation stage of qlin_rotate_quant_act without its
 * quantizer: v = (x[m] * fold_inv_s) @ blockdiag(H_b / sqrt(b)) (no pre-op).
 *
 * qlin_calibrate_step_scales -- one table row from a step's calibration tokens:
 *   table[c] = fp32( max_m |v[m][c]| / qmax ),  qmax = 7 (bits 4) or 127 (bits 8).
 *   x [m][ldx] (k inputs first in each row), m >= 1; table: out float[k].
 *
 * qlin_rotate_quant_act_static -- activation codes of one step:
 *   xq[m][c] = clamp(rne(v[m][c] / table[c]), +-qmax); a table entry that is
 *   not a positive finite number gives code 0.  xq as in qlin_rotate_quant_act;
 *   there is no per-row scale (the GEMM takes x_scale[m] = 1).
 *
 * qlin_quantize_weights_step -- one step's weights: per output row n,
 *   v = (w[n] * fold_s) @ blockdiag(H_b / sqrt(b)), times table[c] (finite);
 *   w_scale[n] = fp32(max_c |v| / qmax); wq = clamp(rne(v / w_scale[n]), +-qmax)
 *   (layout and zero rows as qlin_quantize_weights with group 0).
 *
 * Arguments as qlin_rotate_quant_act / qlin_quantize_weights; table is
 * float[k], 16-byte aligned, read (or written) on the device.  Preconditions:
 * k >= 8, k % 8 == 0, ldx % 8 == 0, ldx >= k; had_block 0/1 or a power of two
 * <= 256 dividing k; bits 4, 8 or QLIN_BITS_E2M3 (then k % 128 == 0).  Errors
 * as those entry points (NULL table: QLIN_ERR_NULL).
 */
qlin_status qlin_calibrate_step_scales(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                       int64_t ldx, const float* fold_inv_s, int32_t had_block,
                                       int32_t bits, float* table, void* stream);
qlin_status qlin_rotate_quant_act_static(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                         int64_t ldx, const float* fold_inv_s, int32_t had_block,
                                         int32_t bits, const float* table, void* xq, void* stream);
qlin_status qlin_quantize_weights_step(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                       const float* fold_s, int32_t had_block, int32_t bits,
                                       const float* table, void* wq, float* w_scale, void* stream);

/*
 * SVD-Hadamard composite rotation with the zigzag permutation (Omega-QVLA
 * technical summary, Metodologia 1: "Rotazione SVD", "Rotazione Hadamard",
 * "Implementazione a Blocchi").  In place of the fast Hadamard block of
 * qlin_rotate_quant_act / qlin_quantize_weights, each row is gathered by a
 * channel permutation and multiplied, block by block of b channels, by a
 * dense b x b rotation R_j:
 *   v[c'] = x[perm[c']] * fold[perm[c']];   v[B_j] = v[B_j] @ R_j
 * then quantized per row (x_scale / w_scale = fp32(max |v| / qmax), codes
 * clamp(rne(v / scale), +-qmax), layouts as the Hadamard entry points; codes
 * are in the permuted channel order on both sides, so the GEMM is unchanged).
 * Arithmetic: v[c'] is the fp32 product; for b >= 32 the dot products of b
 * fp32 terms run on the matrix cores with fp32 accumulation, each within
 * gamma_b * sum_i |v_i| |R_ij| of the exact product of its fp32 operands
 * (gamma_n = n u / (1 - n u), u = 2^-24); for b = 16 they are fp64 sums
 * rounded to fp32.  The rotated rows (fp32) are left in the caller's scratch
 * `work` (device, 16-byte aligned, rows * k floats; required).
 *
 * qlin_calibrate_composite -- perm and R from the weights w [n][k] (times
 *   fold_s): channels ranked by descending L2 norm of their column (lower
 *   index first on ties) are dealt to the k / b blocks in snake order (rank
 *   r, round t = r / (k/b), i = r % (k/b): block i on even rounds, k/b-1-i on
 *   odd ones, slot t).  Per block j, U_j = eigenvectors of the Gram matrix
 *   W[:, B_j]^T W[:, B_j] (the page's R_SVD = U of W = U S V^T with W stored
 *   C_in x C_out) by descending eigenvalue, each with its largest-magnitude
 *   entry positive; R_j = U_j H_b / sqrt(b) (Sylvester H).  Eigenvectors of
 *   repeated eigenvalues are any orthonormal basis of their space.
 *   perm: out int32[k]; rot: out float[k/b][b][b].  work: device scratch of
 *   work_bytes >= qlin_calibrate_composite_work_bytes(n, k, b) bytes, 16-byte
 *   aligned (about 8 (k b + k n / 256 + k) bytes; QLIN_ERR_WORKSPACE if
 *   smaller).
 * qlin_rotate_quant_act_composite -- activations x [m][ldx] with fold_inv_s
 *   (1/s or NULL), perm and rot as written by the calibration; xq, x_scale out.
 * qlin_quantize_weights_composite -- weights w [n][k] with fold_s (s or
 *   NULL); wq, w_scale out; work as above (n * k floats).
 * Preconditions: had_block b in {16, 32, 64, 128} dividing k; k % 8 == 0;
 * k <= 32768; bits 4, 8 or QLIN_BITS_E2M3 (then k % 128 == 0);
 * perm a permutation of 0 .. k-1 (other values are clamped into range).
 * Errors as the Hadamard entry points.
 */
int64_t qlin_calibrate_composite_work_bytes(int64_t n, int64_t k, int32_t had_block);
qlin_status qlin_calibrate_composite(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                     const float* fold_s, int32_t had_block, int32_t* perm, float* rot,
                                     void* work, int64_t work_bytes, void* stream);
qlin_status qlin_rotate_quant_act_composite(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                            int64_t ldx, const float* fold_inv_s, const int32_t* perm,
                                            const float* rot, int32_t had_block, int32_t bits, void* xq,
                                            float* x_scale, float* work, void* stream);
qlin_status qlin_quantize_weights_composite(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                            const float* fold_s, const int32_t* perm, const float* rot,
                                            int32_t had_block, int32_t bits, void* wq, float* w_scale,
                                            float* work, void* stream);

/*
 * qlin_gemm_w4a4 / qlin_gemm_w8a8 -- integer GEMM with int32 accumulation
 * and a fused dequantizing epilogue (FoldQuantVLA abstract: native integer
 * execution of the projections).
 *   acc[m][n] = sum_k xq[m][k] * wq[n][k]   (exact, int32)
 *   y[m][n]   = round_{y_dtype}(fp32(acc) * x_scale[m] * w_scale[n])
 * Per-head or per-layer calibration scalars (QuantVLA technical summary,
 * Methodology B and C) are expected pre-multiplied into w_scale.
 *   xq, wq   codes as produced by qlin_rotate_quant_act / qlin_quantize_weights
 *            (packed int4 for w4a4, int8 for w8a8), contiguous rows of k.
 *   y_dtype  F16, BF16, F32, or I32 (raw accumulators; the scales may then be NULL).
 *   y        out [m][n] contiguous.
 * Preconditions: m >= 0, n >= 1; k a multiple of 64 (for w4a4 the last
 * 64-byte stage of 128 codes is then half full and its upper half reads as
 * zeros),
 * at least one such step; k < 131072 (2^17), which keeps every int32
 * accumulator exact for any codes, -8 and -128 included.
 * These calls never split k (no scratch); a grid of few output tiles with a
 * long k (the FFN-down projection at a few hundred tokens) runs faster
 * through qlin_gemm_ws with a workspace.
 */
qlin_status qlin_gemm_w4a4(const void* xq, const float* x_scale, const void* wq,
                           const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                           qlin_dtype y_dtype, void* stream);
qlin_status qlin_gemm_w8a8(const void* xq, const float* x_scale, const void* wq,
                           const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                           qlin_dtype y_dtype, void* stream);

/*
 * qlin_gemm_w4a8 -- W4A8: int8 activation codes against packed int4 weight
 * codes (QuantVLA summary, "4. 実験結果": the setting it is evaluated in,
 * 4-bit weights and 8-bit activations).
 *   xq:      int8 [m][k] (qlin_rotate_quant_act with bits 8);
 *   wq:      uint8 [n][k/2] packed int4 (qlin_quantize_weights with bits 4);
 *   acc, y, scales, dtypes, stream and errors exactly as qlin_gemm_w4a4.
 * Preconditions: k a multiple of 128, below 131072; otherwise those of
 * qlin_gemm_w4a4.
 */
qlin_status qlin_gemm_w4a8(const void* xq, const float* x_scale, const void* wq,
                           const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                           qlin_dtype y_dtype, void* stream);

/*
 * qlin_gemm_ws -- the integer GEMM of qlin_gemm_w4a4 / _w8a8 / _w4a8
 * (scheme QLIN_W4A4, QLIN_W8A8 or QLIN_W4A8; same arguments, results and
 * preconditions) with a caller-owned workspace for split-K partial sums.
 * Scheme QLIN_W4A4_E2M3 takes both operands in E2M3 storage
 * (qlin_rotate_quant_act / qlin_quantize_weights with bits QLIN_BITS_E2M3,
 * rows of 3k/4 bytes) and gives the results of QLIN_W4A4 on the same codes:
 * it runs on the FP6 matrix cores, whose fp32 sums of grid products are
 * exact integers (|acc| <= 49 k < 2^24); k a multiple of 128, below 131072.
 * It never splits k (its workspace size is 0).
 * When the output tile grid leaves the chip under-filled and k is long, the
 * call splits k over several blocks per tile: each split writes int32 partial
 * accumulators to the workspace ([splits][m][n]) and a second kernel adds
 * them in split order (exact integer sums, so the result is bit-identical to
 * the unsplit GEMM) and applies the epilogue.
 *   workspace        device memory, 16-byte aligned, contents overwritten; or
 *                    NULL with workspace_bytes 0 (then no split, as
 *                    qlin_gemm_w4a4 and co.).
 *   workspace_bytes  its size; at least qlin_gemm_workspace_bytes(scheme, m, n, k)
 *                    when workspace is not NULL, else QLIN_ERR_WORKSPACE.
 * Two calls in flight on different streams need different workspaces.
 * qlin_gemm_workspace_bytes returns the bytes the split plan of that shape
 * needs (0 when it takes no split), or -1 for an invalid scheme or shape.
 */
int64_t qlin_gemm_workspace_bytes(qlin_scheme scheme, int64_t m, int64_t n, int64_t k);
qlin_status qlin_gemm_ws(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                         const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                         qlin_dtype y_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qlin_gemm_static_ws -- qlin_gemm_ws for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * device allocation): the split-K partials go to a static device array of
 * QLIN_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, instead of a workspace argument.  Arguments,
 * results, preconditions and errors as qlin_gemm_ws; the plan is the one
 * qlin_gemm_ws takes with a large enough workspace, and a shape whose
 * partials exceed QLIN_STATIC_SCRATCH_BYTES (qlin_gemm_workspace_bytes tells)
 * returns QLIN_ERR_WORKSPACE.  Allocates nothing.  Every call on a GPU shares
 * that GPU's array and it keeps the last call's contents (nothing in it needs
 * clearing: each partial is written before it is read), so calls that
 * overlap on one GPU (concurrent streams) race and must be serialized by the
 * caller.
 */
#define QLIN_STATIC_SCRATCH_BYTES (16LL << 20)
qlin_status qlin_gemm_static_ws(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                                const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                                qlin_dtype y_dtype, void* stream);

/*
 * qlin_gemm_w4a4_geglu -- the backbone MLP's gate and up projections with the
 * gated GeLU fused into the epilogue (FoldQuantVLA abstract: the projections
 * run natively in integer arithmetic; the gated GeLU joins them here so that
 * only h, not gate and up, goes to memory).
 *   wq, w_scale: the gate and up weights quantized together (qlin_quantize_weights
 *            with bits 4), their rows interleaved in blocks of 32: rows
 *            64c .. 64c+31 are gate rows 32c .. 32c+31 and rows 64c+32 .. 64c+63
 *            are up rows 32c .. 32c+31.  n2 = 2 f rows.
 *   g, u     = fp32(acc) * x_scale[m] * w_scale[row], each rounded to bfloat16
 *            (as an unfused chain would store them);
 *   h[m][c]  = round_{h_dtype}(gelu(g[m][c]) * u[m][c]), c = 0 .. f-1, h
 *            contiguous [m][f]; gelu is the erf form, evaluated in fp32 to
 *            within about one fp32 rounding; h_dtype F16, BF16 or F32.
 * Preconditions: m >= 0; n2 a multiple of 64; k a multiple of 64 (128 for
 * E2M3 codes in qlin_gemm_geglu), below 131072.  Errors: NULL pointers
 * (QLIN_ERR_NULL), other dtypes
 * (QLIN_ERR_DTYPE), shapes (QLIN_ERR_SHAPE), pointers not 16-byte aligned
 * (QLIN_ERR_ALIGN), h overlapping an input (QLIN_ERR_ALIAS); m == 0 returns
 * QLIN_OK without touching the device.  The first call on a device also
 * fills a static 8 KB GeLU table there (see the conventions above).
 */
qlin_status qlin_gemm_w4a4_geglu(const void* xq, const float* x_scale, const void* wq,
                                 const float* w_scale, int64_t m, int64_t n2, int64_t k, void* h,
                                 qlin_dtype h_dtype, void* stream);

/*
 * qlin_gemm_geglu -- qlin_gemm_w4a4_geglu for a given code storage: scheme
 * QLIN_W4A4 (packed int4, identical to qlin_gemm_w4a4_geglu) or
 * QLIN_W4A4_E2M3 (both operands in E2M3 storage, rows of 3k/4 bytes; the
 * same h for the same codes).  Other schemes: QLIN_ERR_UNSUPPORTED.
 * Arguments, results, preconditions and errors as qlin_gemm_w4a4_geglu.
 */
qlin_status qlin_gemm_geglu(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                            const float* w_scale, int64_t m, int64_t n2, int64_t k, void* h,
                            qlin_dtype h_dtype, void* stream);

/*
 * qlin_gemv_w4a16 -- weight-only int4 projection for small batches (LoopQ
 * abstract: batch-1 weight-only kernels of the memory-bound action expert).
 *   y[m][n] = fp16_rne( sum_k x[m][k] * code[n][k] * s16[n][k / group] ),
 *   products and sums in fp32.
 *   x        [m][k] fp16, contiguous.   wq: packed int4 [n][k/2].
 *   w_scale  fp16 [n][k/group] (uint16_t storage).   y: out fp16 [m][n].
 * Preconditions: 1 <= m <= 64 (m == 0 is an empty call); n >= 1;
 * group == 128; k % group == 0; k <= 32768.
 */
qlin_status qlin_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                            int64_t n, int64_t k, int32_t group, void* y, void* stream);

/*
 * qlin_stream_read -- measurement aid, not a step of the projection: reads
 * `bytes` bytes at src once with 16-byte loads spread over the whole device
 * and writes the xor of the words a workgroup read to sink (one uint32 per
 * workgroup, at most QLIN_STREAM_READ_SINK_WORDS).  Its rate on the bytes a
 * memory-bound call reads (the packed weights and scales of
 * qlin_gemv_w4a16) is the streaming-read ceiling that call is compared with
 * (LoopQ abstract: the batch-1 projections of the action expert are
 * memory-bound).
 *   src   device, 16-byte aligned; bytes a positive multiple of 16.
 *   sink  device uint32[QLIN_STREAM_READ_SINK_WORDS], 16-byte aligned, not
 *         overlapping src.
 * Errors: QLIN_ERR_NULL, QLIN_ERR_SHAPE, QLIN_ERR_ALIGN, QLIN_ERR_ALIAS.
 */
#define QLIN_STREAM_READ_SINK_WORDS 4096
qlin_status qlin_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
