// Host-side planning of the qlin kernels: the device's compute-unit count,
// the GEMM tile / split-K plans and the composite calibration's scratch size.
// Plain C++ over the HIP runtime API (no device code), so that the argument
// validation of the C ABI can be built and tested without the kernels.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <mutex>

#include "qlin_internal.h"

namespace qlin {

namespace {
constexpr int STAGE_BYTES = 64;   // bytes of one row per pipeline stage of the integer GEMM
}  // namespace

int device_cus() {
    static std::mutex mu;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, bool int4, bool a8, bool allow_split) {
    // 128-row tiles, 256 columns wide when N is large (fewer L2 -> LDS bytes
    // per MFMA), two blocks per CU (one block's per-stage barrier and LDS
    // latency is covered by the other block's MFMAs).
    // (int8 keeps 128 columns: its 128 x 256 tile would spill at two blocks per
    // CU; so does W4A8, whose 128 x 256 stage would not leave room for 3 stages.)
    GemmPlan g;
    g.m_tail = 0;
    const int64_t cus = device_cus();
    const int64_t kbytes = int4 ? k / 2 : k;
    const int64_t stages = (kbytes + STAGE_BYTES - 1) / STAGE_BYTES;
    g.group_m = 0;
    // int8 activations with 256 x 256 tiles for at least 3/4 of the CUs: one
    // block per CU, each wave a 128 x 128 accumulator tile (half the LDS bytes
    // per MFMA of a 64 x 128 wave tile), tiles in 4-row groups.  Below one
    // tile per CU this still beats the 128 x 128 two-block plan, whose tiles
    // do about 0.6x the work per CU-second: at 6528 x 2048 (208 tiles on 256
    // CUs) o takes 37 us against 50-52 us, down 223 us against 330-335 us.  (W4A4 stays on the two-
    // blocks-per-CU tiles below: its int4 unpack and epilogue VALU work is
    // covered there by the co-resident block's MFMAs; measured 45.6% against
    // 40.7% of the int8 peak for the 52224 x 32768 x 2048 gate|up GEMM.)
    const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
    if (tiles256 * 4 >= cus * 3 && (!int4 || a8)) {
        g.bm = g.bn = 256;
        g.splits = 1;
        g.deep = false;
        g.group_m = 4;
        g.ws_bytes = 0;
        // When the last round of 256 x 256 tiles would fill at most half of
        // the CUs, its rows run instead as 128 x 128 tiles, two blocks per
        // CU, in a second launch: the whole chip then shares them, rather
        // than most CUs idling through a last round.  At 52224 x 2048 that is
        // 6.375 rounds: 6 rounds of 256 x 256 tiles and 3072 rows (384 small
        // tiles on 512 block slots).
        const int64_t tn = (n + 255) / 256, tm = (m + 255) / 256;
        if (cus % tn == 0) {
            const int64_t per_round = cus / tn;               // tile rows of one full round
            const int64_t full = tm / per_round * per_round;  // tile rows in full rounds
            if (full > 0 && tm > full && (tm - full) * 2 <= per_round) g.m_tail = m - full * 256;
        }
        return g;
    }
    // int8 x int8 grids that fill at most half the CUs with 128 x 128 tiles
    // but half to all of them with 64 x 64 tiles (the 7B decoder's 4096-row
    // weights at 256 tokens): 64 x 64 tiles, one block per CU with the deep
    // ring, no split.  Each block then pulls half the bytes of a 128 x 128
    // block through its ring, whose bytes in flight bound a CU's rate here
    // (cold weights, 256 x 4096 x 4096: 12.8 us against 21.9 us).  Long-k
    // grids smaller than that keep split-K: 64-byte stages of 2 MFMAs per
    // wave are then barrier-bound.  With a workspace, k past 128 stages also
    // keeps split-K (256 x 4096 x 11008: four splits and the reduction,
    // 26.7 us, against 28.5 us for 64 x 64 tiles).
    if (!int4 && !a8 && (!allow_split || stages <= 128)) {
        const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
        const int64_t t64 = ((m + 63) / 64) * ((n + 63) / 64);
        // up to two rounds of them when k is short (at most 64 stages): at
        // 816 x 2048 x 2048 (416 tiles) 11.1 us against 14.5 us for 112
        // tiles of 128 x 128, at 600 x 2048 x 4096 15.3 us against 21.2 us;
        // longer k keeps one round (816 x 2048 x 16384: 72 us against 68 us)
        if (t128 * 2 <= cus && t64 * 2 >= cus && (t64 <= cus || (stages <= 64 && t64 <= 2 * cus))) {
            g.bm = g.bn = 64;
            g.splits = 1;
            g.deep = true;
            g.ws_bytes = 0;
            return g;
        }
    }
    g.bm = 128;
    g.bn = (n >= 4096 && int4 && !a8) ? 256 : 128;
    const int64_t slots = 2 * cus;   // two resident blocks per CU
    // split K only when the tile grid fills under half of the block slots,
    // keeping at least 16 stages (1 KiB of k per row) in every split
    auto split_for = [&](int64_t t) {
        int s = 1;
        if (allow_split && t * 2 <= slots) {
            while (t * s * 2 <= slots && stages / (s * 2) >= 16) s *= 2;
        }
        return s;
    };
    // The wide tiles only when they, with their splits, fill every CU: at
    // 816 x 6144 x 2048 (no split) their 168 tiles leave 88 CUs idle, and
    // 336 tiles of 128 x 128 (two blocks per CU) take 23.1-23.6 us against
    // 25.8-26.0 us.
    if (g.bn == 256) {
        const int64_t t = ((m + 127) / 128) * ((n + 255) / 256);
        if (t * split_for(t) < cus) g.bn = 128;
    }
    const int64_t tiles = ((m + g.bm - 1) / g.bm) * ((n + g.bn - 1) / g.bn);
    int splits = split_for(tiles);
    // int8 x int8 with few tiles: the largest split that still gives every
    // block a CU of its own (the deep ring below), when it fills at least 3/4
    // of the CUs.  At 816 x 2048 x 16384 that is two splits on 224 CUs: the
    // GEMM takes the time of four splits at two blocks per CU (38.1 us) and
    // the reduction reads half the partials (4.8 us instead of 7.2 us).
    if (allow_split && !int4 && !a8) {
        int deep_splits = 1;
        while (tiles * deep_splits * 2 <= cus && stages / (deep_splits * 2) >= 16) deep_splits *= 2;
        if (deep_splits >= 2 && tiles * deep_splits * 4 >= cus * 3 && tiles * splits > cus) splits = deep_splits;
    }
    g.splits = splits;
    // Many rounds of tiles: groups of 8 tile rows (see gemm_i8_kernel's tile order)
    if (tiles * splits >= 2 * slots) g.group_m = 8;
    // A grid of at most one block per CU gets the whole LDS for a deeper ring:
    // with one wave per SIMD nothing else covers the DMA latency.
    g.deep = tiles * splits <= cus;
    g.ws_bytes = (splits > 1) ? static_cast<int64_t>(splits) * m * n * 4 : 0;
    return g;
}

GemmPlan plan_gemm_f6(int64_t m, int64_t n, int64_t k, bool geglu) {
    (void)k;
    GemmPlan g;
    const int64_t cus = device_cus();
    g.splits = 1;
    g.deep = false;
    g.ws_bytes = 0;
    g.m_tail = 0;
    const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
    if (tiles256 >= cus && geglu) {   // the fused GeGLU: 128 x 256 tiles, two blocks per CU
        g.bm = 128;
        g.bn = 256;
        g.group_m = 8;
        return g;
    }
    if (tiles256 >= cus) {   // at least one 256 x 256 tile per CU
        g.bm = g.bn = 256;
        g.group_m = 4;
        return g;
    }
    g.bm = g.bn = 128;
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    g.group_m = tiles >= 4 * cus ? 8 : 0;
    return g;
}

int64_t composite_calib_work_bytes(int64_t n, int64_t k, int b) {
    const int64_t chunks = (n + 255) / 256;
    return (chunks * k + k + k * b) * 8;
}

}  // namespace qlin
