// Internal launchers of the qlin library (host side).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qlin {

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();

// Device-resident lookup tables filled once per device.  The first call on a
// device runs `fill` on a private stream and waits for it, so every later call
// on any stream or thread reads the finished table; a table is never in use
// while it is written.  A first call made while `caller` is being captured
// into a graph returns hipErrorStreamCaptureUnsupported (the fill cannot go
// into the caller's graph, and the host wait is not allowed there); later
// calls, captured or not, return hipSuccess at once.
struct OncePerDevice {
    bool ready[64] = {false};
};
hipError_t fill_once_per_device(OncePerDevice& once, hipStream_t caller, hipError_t (*fill)(hipStream_t));

int row_quant_lanes(int64_t k, int64_t m);
int row_quant_chunks(int64_t k, int g);

hipError_t launch_rotate_quant(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                               bool geglu, const float* mult, int had_block, int bits, void* q,
                               float* scale, hipStream_t st);

hipError_t launch_quant_groups_w4(const void* w, int dtype, int64_t n, int64_t k, void* q,
                                  void* scale, hipStream_t st);

// Per-step static activation table: codes v / table[c] (weights == false, no
// per-row scale), or one step's weights v * table[c] then per-row RTN
// (weights == true, scale out).  Plain rows only (no GeGLU pre-op).
hipError_t launch_rotate_quant_table(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                     const float* mult, int had_block, int bits, const float* table,
                                     bool weights, void* q, float* scale, hipStream_t st);

// table[c] = max over the m rows of |rotate(x * mult)[., c]| / qmax.
hipError_t launch_calibrate_step_scales(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx,
                                        const float* mult, int had_block, int bits, float* table,
                                        hipStream_t st);

// SVD-Hadamard composite rotation (b in 16..128): rows gathered by perm,
// folded, rotated per block by rot[k/b][b][b] into v (fp32 [m][k], caller's
// workspace), then per-row quantized.
hipError_t launch_composite_quant(const void* x, int dtype, int64_t m, int64_t k, int64_t ldx, const float* mult,
                                  const int32_t* perm, const float* rot, int b, int bits, void* q, float* scale,
                                  float* v, hipStream_t st);
// Calibration of perm and rot from weights [n][k] (times fold); `work` holds
// composite_calib_work_bytes(n, k, b) bytes.
int64_t composite_calib_work_bytes(int64_t n, int64_t k, int b);
hipError_t launch_calibrate_composite(const void* w, int dtype, int64_t n, int64_t k, const float* fold, int b,
                                      int32_t* perm, float* rot, void* work, hipStream_t st);

hipError_t launch_calibrate_fold(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                                 bool geglu, const void* w, int w_dtype, int64_t n, float* s,
                                 float* inv_s, hipStream_t st);

// Integer GEMM.  int4 == true: the weights are packed int4 codes, and so are
// the activations unless a8.
// ws: int32 workspace of splits * m * n elements when splits > 1.
struct GemmPlan {
    int bm, bn;     // block tile
    int splits;     // split-K factor (1 = fused epilogue)
    bool deep;      // grid fits one block per CU: one block per CU with a deeper DMA ring
    int group_m;    // tile order: 0 = rows fastest, else groups of group_m tile rows
    int64_t ws_bytes;
    int64_t m_tail; // 256 x 256 plans: the last m_tail rows run as 128 x 128 tiles in a second launch
};
// a8 (with int4): int8 activations against int4 weights (W4A8).  Split-K
// only when allow_split (the caller supplies the partials' workspace).
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, bool int4, bool a8, bool allow_split);
hipError_t launch_gemm(const GemmPlan& plan, const void* xq, const float* x_scale, const void* wq,
                       const float* w_scale, int64_t m, int64_t n, int64_t k, bool int4, bool a8, void* y,
                       int y_dtype, int32_t* ws, hipStream_t st);
// The library's static split-K scratch (kStaticScratchBytes per device):
// its device address on the current device, looked up on first use.
constexpr int64_t kStaticScratchBytes = 16LL << 20;
hipError_t static_scratch(int32_t** ptr);
// Gate|up GEMM with the GeGLU epilogue: n interleaved rows (blocks of 32 gate
// rows then 32 up rows), y [m][n/2] = gelu(g) * u.  int4 only, no split-K.
hipError_t launch_gemm_geglu(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                             int64_t m, int64_t n, int64_t k, bool int4, void* y, int y_dtype,
                             hipStream_t st);

// W4A4 with the codes stored as FP6 E2M3 fields (3 bytes per 4 codes) on the
// scaled FP6 MFMA; k a multiple of 128; no split-K.  geglu: the gate|up
// layout and epilogue of launch_gemm_geglu.
GemmPlan plan_gemm_f6(int64_t m, int64_t n, int64_t k, bool geglu);
hipError_t launch_gemm_f6(const GemmPlan& plan, const void* xq, const float* x_scale, const void* wq,
                          const float* w_scale, int64_t m, int64_t n, int64_t k, void* y, int y_dtype, bool geglu,
                          hipStream_t st);

// Streaming read of bytes (a multiple of 16) at src; one word per block to sink.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, hipStream_t st);

hipError_t launch_gemv_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                             int64_t n, int64_t k, int group, void* y, hipStream_t st);

// The same projection on the matrix cores, for 3 < m <= 64; group 128.
hipError_t launch_skinny_w4a16(const void* x, const void* wq, const void* w_scale, int64_t m,
                               int64_t n, int64_t k, void* y, hipStream_t st);

// Integer projection (W4A4 / W8A8 / W4A8 as int4, a8 select) for m <= 64:
// 16-column blocks, k split over eight waves; same results as launch_gemm.
constexpr int64_t kSkinnyIntMaxM = 64;
hipError_t launch_skinny_int(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                             int64_t m, int64_t n, int64_t k, bool int4, bool a8, void* y, int y_dtype,
                             hipStream_t st);

}  // namespace qlin
