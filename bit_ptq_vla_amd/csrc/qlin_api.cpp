// Host side of the qlin C ABI: argument validation (before any HIP call),
// device check, launch, and HIP error mapping.  Declarations and the meaning
// of every argument are in include/qlin.h.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/qlin.h"
#include "qlin_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unchecked, 1 = gfx950, 2 = other device
int g_device_ok[kMaxDevices] = {0};
std::mutex g_device_mu;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t dtype_size(qlin_dtype d) {
    switch (d) {
        case QLIN_F16: case QLIN_BF16: return 2;
        case QLIN_F32: case QLIN_I32: return 4;
    }
    return 0;
}

bool is_float_in(qlin_dtype d) { return d == QLIN_F16 || d == QLIN_BF16 || d == QLIN_F32; }

bool pow2_block_ok(int32_t b) { return b == 0 || b == 1 || (b > 1 && b <= 256 && (b & (b - 1)) == 0); }

struct Span {
    const void* p;
    int64_t bytes;
};

bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

bool any_overlap(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}

// Checks (once per device, cached) that the current device is a gfx950.
qlin_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QLIN_ERR_DEVICE;
    if (dev >= kMaxDevices) return QLIN_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_device_mu);
    if (g_device_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QLIN_ERR_DEVICE;
        g_device_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    return g_device_ok[dev] == 1 ? QLIN_OK : QLIN_ERR_DEVICE;
}

qlin_status map_err(hipError_t e) {
    if (e == hipSuccess) return QLIN_OK;
    if (e == hipErrorStreamCaptureUnsupported) return QLIN_ERR_CAPTURE;
    return QLIN_ERR_LAUNCH;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Largest k the activation / weight row kernel holds in registers:
// 256 lanes x 16 chunks x 8 values.
constexpr int64_t kMaxRowK = 32768;

// GEMM k bound (exclusive): 2^17.
constexpr int64_t kMaxGemmK = 131072;

// Code widths of the quantizers: int8, packed int4, or int4 codes in E2M3
// storage (k a multiple of 128 there, the GEMM's stage).
bool bits_ok(int32_t bits) { return bits == 4 || bits == 8 || bits == QLIN_BITS_E2M3; }
bool bits_k_ok(int32_t bits, int64_t k) { return bits != QLIN_BITS_E2M3 || k % 128 == 0; }
int64_t code_bytes(int64_t rows, int64_t k, int32_t bits) {
    if (bits == 8) return rows * k;
    if (bits == 4) return rows * (k / 2);
    return rows * (k / 4 * 3);
}

// Step of k the GEMM schemes take: 64 (W8A8, and W4A4, whose last 64-byte
// stage of 128 codes may then be half full), 128 for W4A8 (a stage holds
// 128 k of both operands) and E2M3 (128 codes per 96-byte stage).
int64_t gemm_k_step(bool int4, bool a8, bool f6) { return (f6 || (int4 && a8)) ? 128 : 64; }

// Shape checks of the integer GEMM schemes (before any pointer check).
bool gemm_shape_ok(int64_t m, int64_t n, int64_t k, int64_t kstep) {
    if (m < 0 || n < 1 || k < kstep || (k % kstep) != 0) return false;
    // k < 2^17: the accumulator, 256 * acc for W4A4 and 16 * acc for W4A8,
    // stays below 2^31 in magnitude for any codes (|code| <= 8 int4, 128 int8)
    if (k >= kMaxGemmK) return false;
    return m <= 0x7FFFFFFF && n <= 0x7FFFFFFF;
}

// Split-K partial bytes of the plan a call with a workspace takes (0: no split).
int64_t gemm_ws_need(int64_t m, int64_t n, int64_t k, bool int4, bool a8, bool f6) {
    if (f6) return 0;                                     // the E2M3 kernels never split
    if (m == 0 || m <= qlin::kSkinnyIntMaxM) return 0;   // the small-M kernel never splits
    return qlin::plan_gemm(m, n, k, int4, a8, true).ws_bytes;
}

// Split-K scratch of a GEMM call: none (no split), the caller's workspace, or
// the library's static device array.
enum class Scratch { None, Caller, Static };

qlin_status gemm_common(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                        int64_t m, int64_t n, int64_t k, void* y, qlin_dtype y_dtype, Scratch mode, void* ws,
                        int64_t ws_bytes, void* stream, bool int4, bool a8, bool f6) {
    const bool use_static = mode == Scratch::Static;
    if (!xq && m > 0) return QLIN_ERR_NULL;
    if (!wq || !y) return QLIN_ERR_NULL;
    if (y_dtype != QLIN_I32 && ((!x_scale && m > 0) || !w_scale)) return QLIN_ERR_NULL;
    if (y_dtype != QLIN_F16 && y_dtype != QLIN_BF16 && y_dtype != QLIN_F32 && y_dtype != QLIN_I32)
        return QLIN_ERR_DTYPE;
    if (!gemm_shape_ok(m, n, k, gemm_k_step(int4, a8, f6))) return QLIN_ERR_SHAPE;
    if (ws_bytes < 0) return QLIN_ERR_SHAPE;
    if (!ws && ws_bytes > 0) return QLIN_ERR_NULL;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(x_scale) || !aligned16(w_scale) ||
        !aligned16(ws))
        return QLIN_ERR_ALIGN;
    const int64_t need = ws ? gemm_ws_need(m, n, k, int4, a8, f6) : 0;
    if (ws && ws_bytes < need) return QLIN_ERR_WORKSPACE;
    const int64_t kb = f6 ? k / 4 * 3 : int4 ? k / 2 : k;
    const int64_t ka = f6 ? k / 4 * 3 : (int4 && !a8) ? k / 2 : k;
    const Span outs[2] = {{y, m * n * dtype_size(y_dtype)}, {ws, ws ? ws_bytes : 0}};
    const Span ins[4] = {{xq, m * ka}, {wq, n * kb}, {x_scale, m * 4}, {w_scale, n * 4}};
    if (any_overlap(outs, 2, ins, 4)) return QLIN_ERR_ALIAS;
    if (use_static && gemm_ws_need(m, n, k, int4, a8, f6) > QLIN_STATIC_SCRATCH_BYTES) return QLIN_ERR_WORKSPACE;
    if (m == 0) return QLIN_OK;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    hipStream_t s = as_stream(stream);
    if (f6)
        return map_err(qlin::launch_gemm_f6(qlin::plan_gemm_f6(m, n, k, false), xq, x_scale, wq, w_scale, m, n, k,
                                            y, y_dtype, false, s));
    if (m <= qlin::kSkinnyIntMaxM)
        return map_err(qlin::launch_skinny_int(xq, x_scale, wq, w_scale, m, n, k, int4, a8, y, y_dtype, s));
    if (use_static) {
        int32_t* scratch_dev = nullptr;
        if (qlin::static_scratch(&scratch_dev) != hipSuccess) return QLIN_ERR_DEVICE;
        const qlin::GemmPlan plan = qlin::plan_gemm(m, n, k, int4, a8, true);
        return map_err(qlin::launch_gemm(plan, xq, x_scale, wq, w_scale, m, n, k, int4, a8, y, y_dtype,
                                         scratch_dev, s));
    }
    const qlin::GemmPlan plan = qlin::plan_gemm(m, n, k, int4, a8, ws != nullptr);
    return map_err(qlin::launch_gemm(plan, xq, x_scale, wq, w_scale, m, n, k, int4, a8, y, y_dtype,
                                     static_cast<int32_t*>(ws), s));
}

bool scheme_flags(qlin_scheme scheme, bool* int4, bool* a8, bool* f6) {
    *f6 = false;
    switch (scheme) {
        case QLIN_W4A4: *int4 = true; *a8 = false; return true;
        case QLIN_W8A8: *int4 = false; *a8 = false; return true;
        case QLIN_W4A8: *int4 = true; *a8 = true; return true;
        case QLIN_W4A4_E2M3: *int4 = true; *a8 = false; *f6 = true; return true;
    }
    return false;
}

// Shared checks of the per-step table entry points (rows of k values, no pre-op).
qlin_status table_rows_check(const void* x, qlin_dtype dt, int64_t rows, int64_t k, int64_t ldx,
                             const float* fold, int32_t had_block, int32_t bits, const void* table) {
    if (!table) return QLIN_ERR_NULL;
    if (rows > 0 && !x) return QLIN_ERR_NULL;
    if (!is_float_in(dt)) return QLIN_ERR_DTYPE;
    if (!bits_ok(bits)) return QLIN_ERR_UNSUPPORTED;
    if (!pow2_block_ok(had_block)) return QLIN_ERR_UNSUPPORTED;
    if (rows < 0 || k < 8 || (k % 8) != 0 || (ldx % 8) != 0 || ldx < k) return QLIN_ERR_SHAPE;
    if (!bits_k_ok(bits, k)) return QLIN_ERR_SHAPE;
    if (had_block > 1 && (k % had_block) != 0) return QLIN_ERR_SHAPE;
    if (k > kMaxRowK) return QLIN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(fold) || !aligned16(table)) return QLIN_ERR_ALIGN;
    return QLIN_OK;
}

// Shared checks of the composite-rotation entry points.
qlin_status composite_check(const void* x, qlin_dtype dt, int64_t rows, int64_t k, int64_t ldx, int32_t b) {
    if (rows > 0 && !x) return QLIN_ERR_NULL;
    if (!is_float_in(dt)) return QLIN_ERR_DTYPE;
    if (b != 16 && b != 32 && b != 64 && b != 128) return QLIN_ERR_UNSUPPORTED;
    if (rows < 0 || k < b || (k % b) != 0 || (k % 8) != 0 || (ldx % 8) != 0 || ldx < k) return QLIN_ERR_SHAPE;
    if (k > kMaxRowK) return QLIN_ERR_SHAPE;
    return QLIN_OK;
}

// The rotated rows (fp32 [rows][k]) go through the caller's workspace.
qlin_status composite_run(const void* x, qlin_dtype dt, int64_t rows, int64_t k, int64_t ldx, const float* mult,
                          const int32_t* perm, const float* rot, int32_t b, int32_t bits, void* q, float* scale,
                          float* work, void* stream) {
    return map_err(qlin::launch_composite_quant(x, dt, rows, k, ldx, mult, perm, rot, b, bits, q, scale, work,
                                                as_stream(stream)));
}

}  // namespace

extern "C" {

int32_t qlin_abi_version(void) { return QLIN_ABI_VERSION; }

const char* qlin_status_string(qlin_status s) {
    switch (s) {
        case QLIN_OK: return "ok";
        case QLIN_ERR_NULL: return "null pointer";
        case QLIN_ERR_SHAPE: return "invalid shape";
        case QLIN_ERR_DTYPE: return "unsupported dtype";
        case QLIN_ERR_ALIGN: return "pointer or row pitch not 16-byte aligned";
        case QLIN_ERR_UNSUPPORTED: return "unsupported bits, block, group or pre-op";
        case QLIN_ERR_DEVICE: return "no usable gfx950 device or HIP runtime error";
        case QLIN_ERR_LAUNCH: return "kernel launch failed";
        case QLIN_ERR_ALIAS: return "output overlaps an input";
        case QLIN_ERR_CAPTURE: return "first use of a lookup table inside stream capture";
        case QLIN_ERR_WORKSPACE: return "workspace smaller than the call needs";
    }
    return "unknown status";
}

qlin_status qlin_calibrate_fold(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k, int64_t ldx,
                                qlin_preop pre, const void* w, qlin_dtype w_dtype, int64_t n, float* s,
                                float* inv_s, void* stream) {
    if (!x || !w || !s || !inv_s) return QLIN_ERR_NULL;
    if (!is_float_in(x_dtype) || !is_float_in(w_dtype)) return QLIN_ERR_DTYPE;
    if (pre != QLIN_PRE_NONE && pre != QLIN_PRE_GEGLU) return QLIN_ERR_UNSUPPORTED;
    const int64_t width = (pre == QLIN_PRE_GEGLU) ? 2 * k : k;
    if (m < 1 || n < 1 || k < 8 || (k % 8) != 0 || (ldx % 8) != 0 || ldx < width) return QLIN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(inv_s)) return QLIN_ERR_ALIGN;
    const Span outs[2] = {{s, k * 4}, {inv_s, k * 4}};
    const Span ins[2] = {{x, ((m - 1) * ldx + width) * dtype_size(x_dtype)}, {w, n * k * dtype_size(w_dtype)}};
    if (any_overlap(outs, 2, ins, 2)) return QLIN_ERR_ALIAS;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_calibrate_fold(x, x_dtype, m, k, ldx, pre == QLIN_PRE_GEGLU, w, w_dtype,
                                               n, s, inv_s, as_stream(stream)));
}

qlin_status qlin_quantize_weights(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                  const float* fold_s, int32_t had_block, int32_t bits, int32_t group,
                                  void* wq, void* w_scale, void* stream) {
    if (!w || !wq || !w_scale) return QLIN_ERR_NULL;
    if (!is_float_in(w_dtype)) return QLIN_ERR_DTYPE;
    if (!bits_ok(bits)) return QLIN_ERR_UNSUPPORTED;
    if (!pow2_block_ok(had_block)) return QLIN_ERR_UNSUPPORTED;
    if (group != 0 && group != 128) return QLIN_ERR_UNSUPPORTED;
    if (group == 128 && (bits != 4 || fold_s != nullptr || had_block > 1)) return QLIN_ERR_UNSUPPORTED;
    if (n < 1 || k < 8 || (k % 8) != 0) return QLIN_ERR_SHAPE;
    if (!bits_k_ok(bits, k)) return QLIN_ERR_SHAPE;
    if (group && (k % group) != 0) return QLIN_ERR_SHAPE;
    if (had_block > 1 && (k % had_block) != 0) return QLIN_ERR_SHAPE;
    if (!group && k > kMaxRowK) return QLIN_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(fold_s)) return QLIN_ERR_ALIGN;
    const int64_t scale_bytes = group ? n * (k / group) * 2 : n * 4;
    const Span outs[2] = {{wq, code_bytes(n, k, bits)}, {w_scale, scale_bytes}};
    const Span ins[2] = {{w, n * k * dtype_size(w_dtype)}, {fold_s, fold_s ? k * 4 : 0}};
    if (any_overlap(outs, 2, ins, 2)) return QLIN_ERR_ALIAS;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    hipStream_t s = as_stream(stream);
    if (group) return map_err(qlin::launch_quant_groups_w4(w, w_dtype, n, k, wq, w_scale, s));
    return map_err(qlin::launch_rotate_quant(w, w_dtype, n, k, k, false, fold_s, had_block, bits, wq,
                                             static_cast<float*>(w_scale), s));
}

qlin_status qlin_rotate_quant_act(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k, int64_t ldx,
                                  qlin_preop pre, const float* fold_inv_s, int32_t had_block, int32_t bits,
                                  void* xq, float* x_scale, void* stream) {
    if (m > 0 && (!x || !xq || !x_scale)) return QLIN_ERR_NULL;
    if (!is_float_in(x_dtype)) return QLIN_ERR_DTYPE;
    if (!bits_ok(bits)) return QLIN_ERR_UNSUPPORTED;
    if (!pow2_block_ok(had_block)) return QLIN_ERR_UNSUPPORTED;
    if (pre != QLIN_PRE_NONE && pre != QLIN_PRE_GEGLU) return QLIN_ERR_UNSUPPORTED;
    const int64_t width = (pre == QLIN_PRE_GEGLU) ? 2 * k : k;
    if (m < 0 || k < 8 || (k % 8) != 0 || (ldx % 8) != 0 || ldx < width) return QLIN_ERR_SHAPE;
    if (!bits_k_ok(bits, k)) return QLIN_ERR_SHAPE;
    if (had_block > 1 && (k % had_block) != 0) return QLIN_ERR_SHAPE;
    if (k > kMaxRowK) return QLIN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || !aligned16(fold_inv_s)) return QLIN_ERR_ALIGN;
    const Span outs[2] = {{xq, code_bytes(m, k, bits)}, {x_scale, m * 4}};
    const Span ins[2] = {{x, m > 0 ? ((m - 1) * ldx + width) * dtype_size(x_dtype) : 0},
                         {fold_inv_s, fold_inv_s ? k * 4 : 0}};
    if (any_overlap(outs, 2, ins, 2)) return QLIN_ERR_ALIAS;
    if (m == 0) return QLIN_OK;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_rotate_quant(x, x_dtype, m, k, ldx, pre == QLIN_PRE_GEGLU, fold_inv_s,
                                             had_block, bits, xq, x_scale, as_stream(stream)));
}

qlin_status qlin_calibrate_step_scales(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k, int64_t ldx,
                                       const float* fold_inv_s, int32_t had_block, int32_t bits,
                                       float* table, void* stream) {
    qlin_status st = table_rows_check(x, x_dtype, m, k, ldx, fold_inv_s, had_block, bits, table);
    if (st != QLIN_OK) return st;
    if (m < 1) return QLIN_ERR_SHAPE;
    const Span outs[1] = {{table, k * 4}};
    const Span ins[2] = {{x, ((m - 1) * ldx + k) * dtype_size(x_dtype)}, {fold_inv_s, fold_inv_s ? k * 4 : 0}};
    if (any_overlap(outs, 1, ins, 2)) return QLIN_ERR_ALIAS;
    st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_calibrate_step_scales(x, x_dtype, m, k, ldx, fold_inv_s, had_block, bits,
                                                      table, as_stream(stream)));
}

qlin_status qlin_rotate_quant_act_static(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k, int64_t ldx,
                                         const float* fold_inv_s, int32_t had_block, int32_t bits,
                                         const float* table, void* xq, void* stream) {
    qlin_status st = table_rows_check(x, x_dtype, m, k, ldx, fold_inv_s, had_block, bits, table);
    if (st != QLIN_OK) return st;
    if (m > 0 && !xq) return QLIN_ERR_NULL;
    if (!aligned16(xq)) return QLIN_ERR_ALIGN;
    const Span outs[1] = {{xq, code_bytes(m, k, bits)}};
    const Span ins[3] = {{x, m > 0 ? ((m - 1) * ldx + k) * dtype_size(x_dtype) : 0},
                         {fold_inv_s, fold_inv_s ? k * 4 : 0}, {table, k * 4}};
    if (any_overlap(outs, 1, ins, 3)) return QLIN_ERR_ALIAS;
    if (m == 0) return QLIN_OK;
    st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_rotate_quant_table(x, x_dtype, m, k, ldx, fold_inv_s, had_block, bits, table,
                                                   false, xq, nullptr, as_stream(stream)));
}

qlin_status qlin_quantize_weights_step(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                       const float* fold_s, int32_t had_block, int32_t bits,
                                       const float* table, void* wq, float* w_scale, void* stream) {
    qlin_status st = table_rows_check(w, w_dtype, n, k, k, fold_s, had_block, bits, table);
    if (st != QLIN_OK) return st;
    if (!wq || !w_scale) return QLIN_ERR_NULL;
    if (n < 1) return QLIN_ERR_SHAPE;
    if (!aligned16(wq) || !aligned16(w_scale)) return QLIN_ERR_ALIGN;
    const Span outs[2] = {{wq, code_bytes(n, k, bits)}, {w_scale, n * 4}};
    const Span ins[3] = {{w, n * k * dtype_size(w_dtype)}, {fold_s, fold_s ? k * 4 : 0}, {table, k * 4}};
    if (any_overlap(outs, 2, ins, 3)) return QLIN_ERR_ALIAS;
    st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_rotate_quant_table(w, w_dtype, n, k, k, fold_s, had_block, bits, table, true,
                                                   wq, w_scale, as_stream(stream)));
}

int64_t qlin_calibrate_composite_work_bytes(int64_t n, int64_t k, int32_t had_block) {
    if (n < 1 || k < 1 || (had_block != 16 && had_block != 32 && had_block != 64 && had_block != 128) ||
        k % had_block != 0 || k > kMaxRowK)
        return -1;
    return qlin::composite_calib_work_bytes(n, k, had_block);
}

qlin_status qlin_calibrate_composite(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                     const float* fold_s, int32_t had_block, int32_t* perm, float* rot,
                                     void* work, int64_t work_bytes, void* stream) {
    qlin_status st = composite_check(w, w_dtype, n, k, k, had_block);
    if (st != QLIN_OK) return st;
    if (!w || !perm || !rot || !work) return QLIN_ERR_NULL;
    if (n < 1) return QLIN_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(fold_s) || !aligned16(perm) || !aligned16(rot) || !aligned16(work))
        return QLIN_ERR_ALIGN;
    if (work_bytes < qlin::composite_calib_work_bytes(n, k, had_block)) return QLIN_ERR_WORKSPACE;
    const Span outs[3] = {{perm, k * 4}, {rot, k * had_block * 4}, {work, work_bytes}};
    const Span ins[2] = {{w, n * k * dtype_size(w_dtype)}, {fold_s, fold_s ? k * 4 : 0}};
    if (any_overlap(outs, 3, ins, 2)) return QLIN_ERR_ALIAS;
    st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_calibrate_composite(w, w_dtype, n, k, fold_s, had_block, perm, rot, work,
                                                    as_stream(stream)));
}

qlin_status qlin_rotate_quant_act_composite(const void* x, qlin_dtype x_dtype, int64_t m, int64_t k,
                                            int64_t ldx, const float* fold_inv_s, const int32_t* perm,
                                            const float* rot, int32_t had_block, int32_t bits, void* xq,
                                            float* x_scale, float* work, void* stream) {
    qlin_status st = composite_check(x, x_dtype, m, k, ldx, had_block);
    if (st != QLIN_OK) return st;
    if (!perm || !rot) return QLIN_ERR_NULL;
    if (m > 0 && (!xq || !x_scale || !work)) return QLIN_ERR_NULL;
    if (!bits_ok(bits)) return QLIN_ERR_UNSUPPORTED;
    if (!bits_k_ok(bits, k)) return QLIN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(fold_inv_s) || !aligned16(perm) || !aligned16(rot) || !aligned16(xq) ||
        !aligned16(x_scale) || !aligned16(work))
        return QLIN_ERR_ALIGN;
    const Span outs[3] = {{xq, code_bytes(m, k, bits)}, {x_scale, m * 4}, {work, m * k * 4}};
    const Span ins[4] = {{x, m > 0 ? ((m - 1) * ldx + k) * dtype_size(x_dtype) : 0},
                         {fold_inv_s, fold_inv_s ? k * 4 : 0}, {perm, k * 4}, {rot, k * had_block * 4}};
    if (any_overlap(outs, 3, ins, 4)) return QLIN_ERR_ALIAS;
    if (m == 0) return QLIN_OK;
    st = check_device();
    if (st != QLIN_OK) return st;
    return composite_run(x, x_dtype, m, k, ldx, fold_inv_s, perm, rot, had_block, bits, xq, x_scale, work, stream);
}

qlin_status qlin_quantize_weights_composite(const void* w, qlin_dtype w_dtype, int64_t n, int64_t k,
                                            const float* fold_s, const int32_t* perm, const float* rot,
                                            int32_t had_block, int32_t bits, void* wq, float* w_scale,
                                            float* work, void* stream) {
    qlin_status st = composite_check(w, w_dtype, n, k, k, had_block);
    if (st != QLIN_OK) return st;
    if (!w || !perm || !rot || !wq || !w_scale || !work) return QLIN_ERR_NULL;
    if (n < 1) return QLIN_ERR_SHAPE;
    if (!bits_ok(bits)) return QLIN_ERR_UNSUPPORTED;
    if (!bits_k_ok(bits, k)) return QLIN_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(fold_s) || !aligned16(perm) || !aligned16(rot) || !aligned16(wq) ||
        !aligned16(w_scale) || !aligned16(work))
        return QLIN_ERR_ALIGN;
    const Span outs[3] = {{wq, code_bytes(n, k, bits)}, {w_scale, n * 4}, {work, n * k * 4}};
    const Span ins[4] = {{w, n * k * dtype_size(w_dtype)}, {fold_s, fold_s ? k * 4 : 0}, {perm, k * 4},
                         {rot, k * had_block * 4}};
    if (any_overlap(outs, 3, ins, 4)) return QLIN_ERR_ALIAS;
    st = check_device();
    if (st != QLIN_OK) return st;
    return composite_run(w, w_dtype, n, k, k, fold_s, perm, rot, had_block, bits, wq, w_scale, work, stream);
}

qlin_status qlin_gemm_w4a4(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                           int64_t m, int64_t n, int64_t k, void* y, qlin_dtype y_dtype, void* stream) {
    return gemm_common(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, Scratch::None, nullptr, 0, stream, true, false,
                       false);
}

qlin_status qlin_gemm_w8a8(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                           int64_t m, int64_t n, int64_t k, void* y, qlin_dtype y_dtype, void* stream) {
    return gemm_common(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, Scratch::None, nullptr, 0, stream, false,
                       false, false);
}

qlin_status qlin_gemm_w4a8(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                           int64_t m, int64_t n, int64_t k, void* y, qlin_dtype y_dtype, void* stream) {
    return gemm_common(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, Scratch::None, nullptr, 0, stream, true, true,
                       false);
}

int64_t qlin_gemm_workspace_bytes(qlin_scheme scheme, int64_t m, int64_t n, int64_t k) {
    bool int4 = false, a8 = false, f6 = false;
    if (!scheme_flags(scheme, &int4, &a8, &f6)) return -1;
    if (!gemm_shape_ok(m, n, k, gemm_k_step(int4, a8, f6))) return -1;
    return gemm_ws_need(m, n, k, int4, a8, f6);
}

qlin_status qlin_gemm_ws(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                         const float* w_scale, int64_t m, int64_t n, int64_t k, void* y, qlin_dtype y_dtype,
                         void* workspace, int64_t workspace_bytes, void* stream) {
    bool int4 = false, a8 = false, f6 = false;
    if (!scheme_flags(scheme, &int4, &a8, &f6)) return QLIN_ERR_UNSUPPORTED;
    return gemm_common(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, Scratch::Caller, workspace, workspace_bytes,
                       stream, int4, a8, f6);
}

qlin_status qlin_gemm_w4a4_geglu(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                                 int64_t m, int64_t n2, int64_t k, void* h, qlin_dtype h_dtype, void* stream) {
    return qlin_gemm_geglu(QLIN_W4A4, xq, x_scale, wq, w_scale, m, n2, k, h, h_dtype, stream);
}

qlin_status qlin_gemm_geglu(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                            const float* w_scale, int64_t m, int64_t n2, int64_t k, void* h, qlin_dtype h_dtype,
                            void* stream) {
    if (scheme != QLIN_W4A4 && scheme != QLIN_W4A4_E2M3) return QLIN_ERR_UNSUPPORTED;
    const bool f6 = scheme == QLIN_W4A4_E2M3;
    if (!xq && m > 0) return QLIN_ERR_NULL;
    if (!wq || !h || !w_scale || (!x_scale && m > 0)) return QLIN_ERR_NULL;
    if (h_dtype != QLIN_F16 && h_dtype != QLIN_BF16 && h_dtype != QLIN_F32) return QLIN_ERR_DTYPE;
    const int64_t kstep = gemm_k_step(true, false, f6);
    if (m < 0 || n2 < 64 || (n2 % 64) != 0 || k < kstep || (k % kstep) != 0 || k >= kMaxGemmK) return QLIN_ERR_SHAPE;
    if (m > 0x7FFFFFFF || n2 > 0x7FFFFFFF) return QLIN_ERR_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(h) || !aligned16(x_scale) || !aligned16(w_scale))
        return QLIN_ERR_ALIGN;
    const int64_t kb = f6 ? k / 4 * 3 : k / 2;
    const Span outs[1] = {{h, m * (n2 / 2) * dtype_size(h_dtype)}};
    const Span ins[4] = {{xq, m * kb}, {wq, n2 * kb}, {x_scale, m * 4}, {w_scale, n2 * 4}};
    if (any_overlap(outs, 1, ins, 4)) return QLIN_ERR_ALIAS;
    if (m == 0) return QLIN_OK;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    hipStream_t s = as_stream(stream);
    if (f6)
        return map_err(qlin::launch_gemm_f6(qlin::plan_gemm_f6(m, n2, k, true), xq, x_scale, wq, w_scale, m, n2, k,
                                            h, h_dtype, true, s));
    return map_err(qlin::launch_gemm_geglu(xq, x_scale, wq, w_scale, m, n2, k, true, h, h_dtype, s));
}

qlin_status qlin_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m, int64_t n,
                            int64_t k, int32_t group, void* y, void* stream) {
    if (m > 0 && (!x || !y)) return QLIN_ERR_NULL;
    if (!wq || !w_scale) return QLIN_ERR_NULL;
    if (group != 128) return QLIN_ERR_UNSUPPORTED;
    if (m < 0 || m > 64 || n < 1 || k < group || (k % group) != 0 || k > 32768) return QLIN_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y)) return QLIN_ERR_ALIGN;
    const Span outs[1] = {{y, m * n * 2}};
    const Span ins[3] = {{x, m * k * 2}, {wq, n * k / 2}, {w_scale, n * (k / group) * 2}};
    if (any_overlap(outs, 1, ins, 3)) return QLIN_ERR_ALIAS;
    if (m == 0) return QLIN_OK;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_gemv_w4a16(x, wq, w_scale, m, n, k, group, y, as_stream(stream)));
}

qlin_status qlin_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink) return QLIN_ERR_NULL;
    if (bytes < 16 || (bytes % 16) != 0) return QLIN_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(sink)) return QLIN_ERR_ALIGN;
    const Span outs[1] = {{sink, QLIN_STREAM_READ_SINK_WORDS * 4}};
    const Span ins[1] = {{src, bytes}};
    if (any_overlap(outs, 1, ins, 1)) return QLIN_ERR_ALIAS;
    qlin_status st = check_device();
    if (st != QLIN_OK) return st;
    return map_err(qlin::launch_stream_read(src, bytes, sink, QLIN_STREAM_READ_SINK_WORDS, as_stream(stream)));
}

qlin_status qlin_gemm_static_ws(qlin_scheme scheme, const void* xq, const float* x_scale, const void* wq,
                                const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                                qlin_dtype y_dtype, void* stream) {
    bool int4 = false, a8 = false, f6 = false;
    if (!scheme_flags(scheme, &int4, &a8, &f6)) return QLIN_ERR_UNSUPPORTED;
    return gemm_common(xq, x_scale, wq, w_scale, m, n, k, y, y_dtype, Scratch::Static, nullptr, 0, stream, int4,
                       a8, f6);
}

}  // extern "C"
