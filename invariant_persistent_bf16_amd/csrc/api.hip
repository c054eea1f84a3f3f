// C-ABI entry points of the batch-invariant contraction library (declared in
// include/bi.h).  Every argument is checked on the host before any HIP call,
// so a rejected call touches neither the device nor the stream; accepted
// calls enqueue kernels on the caller's stream and return without waiting.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "../../include/bi.h"
#include "conv_pack.hpp"
#include "attn_probs.hpp"
#include "decode.hpp"
#include "prefill.hpp"
#include "gemm_bf16.hpp"
#include "gemm_small.hpp"
#include "gemm_f32.hpp"
#include "softmax.hpp"
#include "rowops.hpp"
#include "internal.hpp"

namespace bi {

// ------------------------------------------------------------ device info
// Per-device compute-unit count, read once (0 = not yet read, -1 = not gfx950).
static std::atomic<int> g_cu_count[64];

int device_cu_count(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BI_ERR_DEVICE;
    if (dev < 0 || dev >= 64) return BI_ERR_DEVICE;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BI_ERR_DEVICE;
        n = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? prop.multiProcessorCount : -1;
        if (n == 0) n = -1;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    if (n < 0) return BI_ERR_DEVICE;
    *cus = n;
    return BI_OK;
}

static int launch_status() { return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH; }

static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------- GEMM
// Output dtypes: binary32 always; bfloat16 for bfloat16 or binary32 operands;
// binary16 for binary16 operands.
static bool gemm_out_ok(int in, int out) {
    if (out == BI_F32) return true;
    if (out == BI_BF16) return in == BI_BF16 || in == BI_F32;
    if (out == BI_F16) return in == BI_F16;
    return false;
}

int gemm_check(const GemmDesc& d) {
    if (d.in_dtype != BI_F32 && d.in_dtype != BI_BF16 && d.in_dtype != BI_F16) return BI_ERR_DTYPE;
    if (!gemm_out_ok(d.in_dtype, d.out_dtype)) return BI_ERR_DTYPE;
    if (d.G1 < 0 || d.G2 < 1 || d.M < 0 || d.N < 0 || d.K < 0) return BI_ERR_SHAPE;
    if (d.G1 == 0 || d.M == 0 || d.N == 0) return BI_OK;   // nothing to compute
    if (!d.C) return BI_ERR_NULL;
    if (d.K > 0 && (!d.A || !d.B)) return BI_ERR_NULL;
    const int64_t strides[] = {d.sA1, d.sA2, d.sAm, d.sAk, d.sB1, d.sB2, d.sBk, d.sBn,
                               d.sBias2, d.sC1, d.sC2, d.sCm, d.sCn};
    for (int64_t s : strides)
        if (s < 0) return BI_ERR_LAYOUT;
    if (d.sCn != 1) return BI_ERR_LAYOUT;
    const int osz = d.out_dtype == BI_F32 ? 4 : 2;
    if (!aligned(d.C, osz)) return BI_ERR_LAYOUT;
    if (d.in_dtype != BI_F32) {
        if (d.K > 0) {
            if (d.K % 8 != 0) return BI_ERR_LAYOUT;
            if (d.sAk != 1 || (d.M > 1 && d.sAm % 8 != 0) || !aligned(d.A, 16)) return BI_ERR_LAYOUT;
            if (d.sA1 % 8 != 0 || d.sA2 % 8 != 0) return BI_ERR_LAYOUT;
            if (!aligned(d.B, 16) || d.sB1 % 8 != 0 || d.sB2 % 8 != 0) return BI_ERR_LAYOUT;
            const bool kc = d.sBk == 1 && (d.N == 1 || d.sBn % 8 == 0);
            const bool nc = d.sBn == 1 && d.sBk % 8 == 0 && d.N % 8 == 0;
            if (!kc && !nc) return BI_ERR_LAYOUT;
            // Byte offsets inside one tile are 32-bit buffer offsets below 2^31.
            const int64_t lim = (1ll << 30) - 512;
            if (d.sAm * G16_BM > lim || (kc ? d.sBn * G16_BN : d.sBk * G16_BK) > lim)
                return BI_ERR_UNSUPPORTED;
            if ((d.sCm * 128 + 128) * osz > lim) return BI_ERR_UNSUPPORTED;   // 32-bit epilogue offsets
            // The K advance is a 32-bit scalar byte offset.
            if ((d.K + 64) * (kc ? 1 : d.sBk) * 2 > lim) return BI_ERR_UNSUPPORTED;
        }
        if (d.bias && !aligned(d.bias, 2)) return BI_ERR_LAYOUT;
    } else {
        if (d.K > 0 && (!aligned(d.A, 4) || !aligned(d.B, 4))) return BI_ERR_LAYOUT;
        // The tiled kernels address a step's operands with 32-bit byte offsets
        // from the tile's first row (column) and the step's first k.
        const int64_t lim = 1ll << 31;
        if (d.K > 0 && ((63 * d.sAm + 31 * d.sAk) * 4 + 4 >= lim || (63 * d.sBn + 31 * d.sBk) * 4 + 4 >= lim))
            return BI_ERR_UNSUPPORTED;
        if (d.bias && !aligned(d.bias, 4)) return BI_ERR_LAYOUT;
    }
    const int64_t bm = d.in_dtype != BI_F32 ? G16_BM : G32_BM;
    const int64_t bn = d.in_dtype != BI_F32 ? G16_BN : G32_BN;
    if (d.G1 > (1ll << 30) || d.G2 > (1ll << 30) || d.K > (1ll << 30)) return BI_ERR_UNSUPPORTED;
    const int64_t tiles = cdiv(d.M, bm) * cdiv(d.N, bn);
    const int64_t slices = d.G1 * d.G2;
    if (slices > (1ll << 30) || tiles > (1ll << 30) || tiles * slices > (1ll << 30))
        return BI_ERR_UNSUPPORTED;
    return BI_OK;
}

// The kernel for a 16-bit product, a function of the shape alone (every
// choice gives the same bits): 0 = the persistent kernel with 256x256 tiles,
// 1 = with 128x256 tiles, 2 = with 256x128 tiles (N <= 128), 3 = with 128x128
// tiles, 4 = with 192x256 tiles, 32 / 64 / 128 = the small-tile kernel with
// blocks of that many rows.  Estimated times fitted to measurements on MI355X
// (GPU time of the addmm with K = 4096, N = 14336 and of the patch
// convolution's GEMM, K = 592): a persistent tile costs, per round of one
// tile per compute unit, a fixed part (launch, prologue and epilogue, growing
// with the tile's area) plus a part per 32-wide K step: 13.1 + 0.464 nk us
// (256x256), 10.3 + 0.456 nk (192x256), 8.2 + 0.296 nk (128x256), 4.7 +
// 0.225 nk (128x128); the 192x256 and 128x128 tiles are considered only while
// their tiles fit in one round; N <= 128 compares 256x128 and 128x256 tiles
// at 6 + 0.30 nk per round.  The small-tile waves sustain about 8 TB/s of
// operand reads from L2 (each block reads its rows of A and its 64 columns
// of B over the whole of K) and need 0.16 / 0.20 / 0.38 us per K step (32,
// 64, 128 rows) for each block per compute unit, plus 2 us, when latency
// bound.  Only products with at most two rounds of 256x256 tiles are
// considered for the others (larger ones keep the 256x256 tile).
// The binary32 split-chain kernels address a 16x16 block's operands with
// 32-bit byte offsets from the block's first row / column: 15 rows (columns)
// plus K + 512 steps of the K stride (the loads run up to two stages of 256
// past K, clamped) must stay below 2^31 bytes.
static bool split32_fits(const GemmDesc& d) {
    const int64_t lim = 1ll << 31;
    return (15 * d.sAm + (d.K + 512) * d.sAk) * 4 < lim && (15 * d.sBn + (d.K + 512) * d.sBk) * 4 < lim;
}

// Operand layouts the split kernel stages in 16-byte pieces.  A: k
// contiguous, every row and slice start 16-byte aligned, K a multiple of 4
// (a piece never straddles K).  B: columns contiguous, every k row and slice
// start 16-byte aligned, N a multiple of 4 (a piece never straddles N).
static bool split32_stage_a(const GemmDesc& d) {
    return d.sAk == 1 && (d.M == 1 || d.sAm % 4 == 0) && d.K % 4 == 0 && aligned(d.A, 16) &&
           d.sA1 % 4 == 0 && d.sA2 % 4 == 0;
}
static bool split32_stage_b(const GemmDesc& d) {
    return d.sBn == 1 && d.sBk % 4 == 0 && d.N % 4 == 0 && aligned(d.B, 16) && d.sB1 % 4 == 0 &&
           d.sB2 % 4 == 0;
}

int gemm_tile_rows(const GemmDesc& d, int cus) {
    const int64_t slices = d.G1 * d.G2;
    // Binary32: 64x64 tiles; 32x32 tiles where those do not fill the compute
    // units; 16x16 blocks with the K chains on separate waves (returned as
    // 16) where even the 32x32 tiles would occupy fewer than half of them and
    // the blocks' byte offsets fit the split kernel's 32-bit buffer offsets.
    if (d.in_dtype == BI_F32) {
        if (slices * cdiv(d.M, G32_BM) * cdiv(d.N, G32_BN) >= cus) return 0;
        if (2 * slices * cdiv(d.M, 32) * cdiv(d.N, 32) >= cus || !split32_fits(d)) return 32;
        return 16;
    }
    const int64_t tiles = slices * cdiv(d.M, G16_BM) * cdiv(d.N, G16_BN);
    // N <= 128 fills half of a 256-wide tile: the 256x128 tile (returned as 2)
    // does the same rows with half the MFMA work and B traffic.
    const bool narrow = d.N <= 128;
    if (tiles >= 2 * (int64_t)cus) return narrow ? 2 : 0;
    const double nk = (double)cdiv(d.K, G16_BK);
    const int64_t tiles128 = slices * cdiv(d.M, 128) * cdiv(d.N, G16_BN);
    double best;
    int best_rows;
    if (narrow) {
        best = 6.0 + 0.30 * nk * (double)cdiv(tiles, cus);
        best_rows = 2;
        const double t1 = 6.0 + 0.30 * nk * (double)cdiv(tiles128, cus);
        if (t1 < best) { best = t1; best_rows = 1; }
    } else {
        best = (double)cdiv(tiles, cus) * (13.1 + 0.464 * nk);
        best_rows = 0;
        const double t1 = (double)cdiv(tiles128, cus) * (8.2 + 0.296 * nk);
        if (t1 < best) { best = t1; best_rows = 1; }
        if (slices * cdiv(d.M, 192) * cdiv(d.N, G16_BN) <= cus) {
            const double t4 = 10.3 + 0.456 * nk;
            if (t4 < best) { best = t4; best_rows = 4; }
        }
    }
    if (slices * cdiv(d.M, 128) * cdiv(d.N, 128) <= cus) {
        const double t3 = 4.7 + 0.225 * nk;
        if (t3 < best) { best = t3; best_rows = 3; }
    }
    if (tiles >= cus) return best_rows;
    // Small tiles: A is read once per GS_COLS columns, B once per row block;
    // a K step costs more for taller blocks and when blocks outnumber the CUs.
    const int64_t nblk = cdiv(d.N, GS_COLS);
    for (int rows : {32, 64, 128}) {
        if (rows > 32 && d.M <= rows / 2) break;   // a taller block only adds empty rows
        const int64_t blocks = slices * cdiv(d.M, rows) * nblk;
        const double bytes = (double)(slices * d.M * nblk + blocks * GS_COLS) * (double)(nk * G16_BK) * 2.0;
        const double per_step = rows == 32 ? 0.16 : rows == 64 ? 0.20 : 0.38;
        const double t = std::max(bytes / 8.0e6, 2.0 + per_step * (double)nk * (double)cdiv(blocks, cus));
        if (t < best) { best = t; best_rows = rows; }
    }
    return best_rows;
}

// Events that the caller asked every kernel of the library to carry
// (bi_set_launch_events): the first kernel launched after the request records
// start when it begins, every kernel records stop when it ends, so stop ends
// up at the end of the last one.  Per host thread; empty in normal use.
static thread_local LaunchEvents t_events = {nullptr, nullptr};
static thread_local bool t_events_first = false;

// Every kernel launch of the entry points goes through here.
template <typename Kern, typename... Args>
static void launch_kernel(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
    if (t_events.stop) {
        hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, st, t_events_first ? t_events.start : nullptr,
                              t_events.stop, 0, args...);
        t_events_first = false;
    } else {
        hipLaunchKernelGGL(kern, grid, block, lds, st, args...);
    }
}

// One kernel launch of the GEMM, with the dispatch's own start / end events
// when ev is given.
template <typename Kern, typename... Args>
static void launch_gemm_kernel(Kern kern, dim3 grid, dim3 block, hipStream_t st, const LaunchEvents* ev,
                               Args... args) {
    if (ev) hipExtLaunchKernelGGL(kern, grid, block, 0, st, ev->start, ev->stop, 0, args...);
    else    launch_kernel(kern, grid, block, 0, st, args...);
}

template <bool KC, int O16, bool F16>
static void gemm_small_launch(const GemmParams& p, int rows, int cvec4, hipStream_t st, const LaunchEvents* ev) {
    typedef void (*KernS)(GemmParams, int);
    const KernS k = rows == 128 ? gemm_bf16_small<KC, O16, F16, 4>
                  : rows == 64  ? gemm_bf16_small<KC, O16, F16, 2>
                                : gemm_bf16_small<KC, O16, F16, 1>;
    const int grid = (int)(cdiv(p.total_tiles, 8) * 8);
    launch_gemm_kernel(k, dim3(grid), dim3(GS_THREADS), st, ev, p, cvec4);
}

// Launch an already checked GEMM.  grid_override > 0 forces the persistent
// grid size and tile_rows >= 0 the kernel (both used only to show that the
// result does not depend on them).
int gemm_launch(const GemmDesc& d, hipStream_t st, int grid_override, int tile_rows, const LaunchEvents* ev) {
    if (d.G1 == 0 || d.M == 0 || d.N == 0) return BI_OK;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    const bool out_bf16 = d.out_dtype == BI_BF16;
    if (d.in_dtype != BI_F32) {
        const bool out16 = d.out_dtype != BI_F32;
        const bool kc = d.K == 0 || (d.sBk == 1 && (d.N == 1 || d.sBn % 8 == 0));
        const int rows = tile_rows >= 0 ? tile_rows : grid_override > 0 ? 0 : gemm_tile_rows(d, cus);
        if (rows != 0 && rows != 1 && rows != 2 && rows != 3 && rows != 4 && rows != 32 && rows != 64 &&
            rows != 128)
            return BI_ERR_UNSUPPORTED;
        if (rows > 4) {
            GemmParams p;
            p.A = (const uint16_t*)d.A; p.B = (const uint16_t*)d.B;
            p.bias = (const uint16_t*)d.bias; p.C = d.C;
            p.M = d.M; p.N = d.N; p.K = d.K;
            p.sAm = d.sAm; p.sBk = d.sBk; p.sBn = d.sBn; p.sCm = d.sCm;
            p.G2 = d.G2;
            p.sA1 = d.sA1; p.sA2 = d.sA2; p.sB1 = d.sB1; p.sB2 = d.sB2;
            p.sC1 = d.sC1; p.sC2 = d.sC2; p.sBias2 = d.sBias2; p.bias_rows = d.bias_rows;
            p.tiles_m = (int)cdiv(d.M, rows);
            p.tiles_n = (int)cdiv(d.N, GS_COLS);
            p.tiles_per_slice = p.tiles_m * p.tiles_n;
            const int64_t total = (int64_t)p.tiles_per_slice * d.G1 * d.G2;
            if (total > (1ll << 30)) return BI_ERR_UNSUPPORTED;
            p.total_tiles = (int)total;
            const int osz = out16 ? 2 : 4;
            const int cvec4 = aligned(d.C, 4 * osz) && d.N % 4 == 0 && d.sCm % 4 == 0 && d.sC1 % 4 == 0 &&
                              d.sC2 % 4 == 0;
            const bool f16 = d.in_dtype == BI_F16;
            if (f16) {
                if (kc) { if (out16) gemm_small_launch<true, 1, true>(p, rows, cvec4, st, ev);
                          else       gemm_small_launch<true, 0, true>(p, rows, cvec4, st, ev); }
                else    { if (out16) gemm_small_launch<false, 1, true>(p, rows, cvec4, st, ev);
                          else       gemm_small_launch<false, 0, true>(p, rows, cvec4, st, ev); }
            } else {
                if (kc) { if (out16) gemm_small_launch<true, 1, false>(p, rows, cvec4, st, ev);
                          else       gemm_small_launch<true, 0, false>(p, rows, cvec4, st, ev); }
                else    { if (out16) gemm_small_launch<false, 1, false>(p, rows, cvec4, st, ev);
                          else       gemm_small_launch<false, 0, false>(p, rows, cvec4, st, ev); }
            }
            return launch_status();
        }
        GemmParams p;
        p.A = (const uint16_t*)d.A; p.B = (const uint16_t*)d.B;
        p.bias = (const uint16_t*)d.bias; p.C = d.C;
        p.M = d.M; p.N = d.N; p.K = d.K;
        p.sAm = d.sAm; p.sBk = d.sBk; p.sBn = d.sBn; p.sCm = d.sCm;
        p.G2 = d.G2;
        p.sA1 = d.sA1; p.sA2 = d.sA2; p.sB1 = d.sB1; p.sB2 = d.sB2;
        p.sC1 = d.sC1; p.sC2 = d.sC2; p.sBias2 = d.sBias2; p.bias_rows = d.bias_rows;
        const int bm = rows == 1 || rows == 3 ? 128 : rows == 4 ? 192 : G16_BM;
        const int bn = rows == 2 || rows == 3 ? 128 : G16_BN;
        p.tiles_m = (int)cdiv(d.M, bm);
        p.tiles_n = (int)cdiv(d.N, bn);
        p.tiles_per_slice = p.tiles_m * p.tiles_n;
        const int64_t total = (int64_t)p.tiles_per_slice * d.G1 * d.G2;
        if (total > (1ll << 30)) return BI_ERR_UNSUPPORTED;
        p.total_tiles = (int)total;
        const int grid = grid_override > 0 ? grid_override : (p.total_tiles < cus ? p.total_tiles : cus);
        const int osz = out16 ? 2 : 4;
        const int vel = 16 / osz;   // elements per 16-byte chunk
        const bool cvec = aligned(d.C, 16) && d.N % vel == 0 && d.sCm % vel == 0 && d.sC1 % vel == 0 &&
                          d.sC2 % vel == 0;
        const int f16 = d.in_dtype == BI_F16;
        const Gemm16Kern kern = rows == 1 ? gemm16_kernel_128x256(f16, kc, out16, cvec)
                              : rows == 2 ? gemm16_kernel_256x128(f16, kc, out16, cvec)
                              : rows == 3 ? gemm16_kernel_128x128(f16, kc, out16, cvec)
                              : rows == 4 ? gemm16_kernel_192x256(f16, kc, out16, cvec)
                                          : gemm16_kernel_256x256(f16, kc, out16, cvec);
        launch_gemm_kernel(kern, dim3(grid), dim3(G16_THREADS), st, ev, p);
    } else {
        GemmF32Params p;
        p.A = (const float*)d.A; p.B = (const float*)d.B; p.bias = (const float*)d.bias; p.C = d.C;
        p.M = d.M; p.N = d.N; p.K = d.K;
        p.sAm = d.sAm; p.sAk = d.sAk; p.sBk = d.sBk; p.sBn = d.sBn; p.sCm = d.sCm;
        p.G2 = d.G2;
        p.sA1 = d.sA1; p.sA2 = d.sA2; p.sB1 = d.sB1; p.sB2 = d.sB2;
        p.sC1 = d.sC1; p.sC2 = d.sC2; p.sBias2 = d.sBias2; p.bias_rows = d.bias_rows;
        // 64x64 tiles, or 32x32 tiles where the 64x64 ones do not fill the
        // compute units (same per-element arithmetic, same bits).
        const int rows = tile_rows >= 0 ? tile_rows : grid_override > 0 ? 0 : gemm_tile_rows(d, cus);
        if (rows != 0 && rows != 32 && (rows < 16 || rows > 19)) return BI_ERR_UNSUPPORTED;
        if (rows >= 16 && rows <= 19 && d.K > 0) {
            if (!split32_fits(d)) return BI_ERR_UNSUPPORTED;
            // one workgroup per 16x16 block (and slice); K = 0 (a bias or
            // zero fill) takes the 32x32 tiles below
            const int64_t blocks = d.G1 * d.G2 * cdiv(d.M, 16) * cdiv(d.N, 16);
            if (blocks > (1ll << 30)) return BI_ERR_UNSUPPORTED;
            typedef void (*KernS)(GemmF32Params);
            static const KernS kerns[2][2][2] = {
                {{gemm_f32_split_chains<0, false, false>, gemm_f32_split_chains<1, false, false>},
                 {gemm_f32_split_chains<0, false, true>, gemm_f32_split_chains<1, false, true>}},
                {{gemm_f32_split_chains<0, true, false>, gemm_f32_split_chains<1, true, false>},
                 {gemm_f32_split_chains<0, true, true>, gemm_f32_split_chains<1, true, true>}}};
            // 16: each operand staged where its layout allows; 17: neither;
            // 18: B only; 19: A only
            const bool sa = (rows == 16 || rows == 19) && split32_stage_a(d);
            const bool sb = (rows == 16 || rows == 18) && split32_stage_b(d);
            launch_gemm_kernel(kerns[sa][sb][out_bf16], dim3((unsigned)blocks), dim3(256), st, ev, p);
            return launch_status();
        }
        const int bt = rows == 0 ? G32_BM : 32;
        p.tiles_m = (int)cdiv(d.M, bt);
        p.tiles_n = (int)cdiv(d.N, bt);
        p.tiles_per_slice = p.tiles_m * p.tiles_n;
        const int64_t total = (int64_t)p.tiles_per_slice * d.G1 * d.G2;
        if (total > (1ll << 30)) return BI_ERR_UNSUPPORTED;
        p.total_tiles = (int)total;
        const int cap = 4 * cus;
        const int grid = grid_override > 0 ? grid_override : (p.total_tiles < cap ? p.total_tiles : cap);
        // The K tail variant only where K is not a multiple of the K step (the
        // arithmetic of both is the same MFMA chain over the same zero-padded K).
        const bool ktail = d.K % G32_BK != 0;
        typedef void (*Kern32)(GemmF32Params);
        static const Kern32 kerns32[2][2][2] = {
            {{gemm_f32_persistent<0, false, 32>, gemm_f32_persistent<0, true, 32>},
             {gemm_f32_persistent<1, false, 32>, gemm_f32_persistent<1, true, 32>}},
            {{gemm_f32_persistent<0, false, 16>, gemm_f32_persistent<0, true, 16>},
             {gemm_f32_persistent<1, false, 16>, gemm_f32_persistent<1, true, 16>}}};
        launch_gemm_kernel(kerns32[rows != 0][out_bf16][ktail], dim3(grid), dim3(G32_THREADS), st, ev, p);
    }
    return launch_status();
}

GemmDesc mm_desc(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
                 const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C,
                 int64_t sCm, int64_t sCn, int in_dtype, int out_dtype) {
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = 1; d.G2 = 1; d.M = M; d.N = N; d.K = K;
    d.A = A; d.sAm = sAm; d.sAk = sAk;
    d.B = B; d.sBk = sBk; d.sBn = sBn;
    d.bias = bias; d.C = C; d.sCm = sCm; d.sCn = sCn;
    d.in_dtype = in_dtype; d.out_dtype = out_dtype;
    return d;
}

GemmDesc bmm_desc(int64_t G, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
                  const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
                  void* C, int64_t sCg, int64_t sCm, int64_t sCn, int in_dtype, int out_dtype) {
    GemmDesc d = mm_desc(M, N, K, A, sAm, sAk, B, sBk, sBn, nullptr, C, sCm, sCn, in_dtype, out_dtype);
    d.G1 = G; d.sA1 = sAg; d.sB1 = sBg; d.sC1 = sCg;
    return d;
}

// ------------------------------------------------------------------- conv
int conv_geometry(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t Kh,
                  int64_t Kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                  int64_t dw, int64_t groups, int in_dtype, ConvGeom* g, size_t* ws_bytes) {
    if (in_dtype != BI_F32 && in_dtype != BI_BF16 && in_dtype != BI_F16) return BI_ERR_DTYPE;
    if (N < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || Kh < 1 || Kw < 1) return BI_ERR_SHAPE;
    if (sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || groups < 1) return BI_ERR_SHAPE;
    if (Cin % groups != 0 || Cout % groups != 0) return BI_ERR_SHAPE;
    const int64_t ohn = H + 2 * ph - dh * (Kh - 1) - 1, own = W + 2 * pw - dw * (Kw - 1) - 1;
    if (ohn < 0 || own < 0) return BI_ERR_SHAPE;
    ConvGeom c;
    c.N = N; c.Cin = Cin; c.H = H; c.W = W; c.Cout = Cout; c.Kh = Kh; c.Kw = Kw;
    c.sh = sh; c.sw = sw; c.ph = ph; c.pw = pw; c.dh = dh; c.dw = dw; c.groups = groups;
    c.OH = ohn / sh + 1; c.OW = own / sw + 1; c.L = c.OH * c.OW;
    c.cig = Cin / groups; c.cog = Cout / groups;
    c.Kg = c.cig * Kh * Kw;
    c.Kp = cdiv(c.Kg, 8) * 8;
    const int64_t esz = in_dtype == BI_F32 ? 4 : 2;
    const int64_t wbytes = cdiv(Cout * c.Kp * esz, 256) * 256;
    const int64_t ubytes = N * groups * c.L * c.Kp * esz;
    if (g) *g = c;
    if (ws_bytes) *ws_bytes = (size_t)(wbytes + ubytes);
    return BI_OK;
}

// Launch a row operation: the lane count and the number of chunks held in
// registers are chosen by cols alone (so a row's reduction tree never depends
// on the number of rows); vector access is chosen by alignment and does not
// change the bits.
template <int OP>
int row_op_launch(int64_t rows, int64_t cols, const void* x, int64_t ldx, const void* w, float eps,
                  void* y, int64_t ldy, int in_dtype, int out_dtype, hipStream_t st) {
    const bool ib = in_dtype == BI_BF16, ob = out_dtype == BI_BF16;
    const uintptr_t vin = ib ? 8 : 16, vout = ob ? 8 : 16;
    const bool vec = cols % 4 == 0 && aligned(x, vin) && (rows == 1 || ldx % 4 == 0) &&
                     (OP == RO_MEAN || (aligned(y, vout) && (rows == 1 || ldy % 4 == 0))) &&
                     (OP != RO_RMS || aligned(w, vin));
    typedef void (*Kern)(const void*, int64_t, const void*, float, void*, int64_t, int64_t, int, int);
    // [regime][input bfloat16][vector]
    static const Kern kerns[4][2][2] = {
        {{row_op_kernel<64, 4, false, OP, false>, row_op_kernel<64, 4, false, OP, true>},
         {row_op_kernel<64, 4, true, OP, false>, row_op_kernel<64, 4, true, OP, true>}},
        {{row_op_kernel<64, 16, false, OP, false>, row_op_kernel<64, 16, false, OP, true>},
         {row_op_kernel<64, 16, true, OP, false>, row_op_kernel<64, 16, true, OP, true>}},
        {{row_op_kernel<256, 16, false, OP, false>, row_op_kernel<256, 16, false, OP, true>},
         {row_op_kernel<256, 16, true, OP, false>, row_op_kernel<256, 16, true, OP, true>}},
        {{row_op_kernel<256, 0, false, OP, false>, row_op_kernel<256, 0, false, OP, true>},
         {row_op_kernel<256, 0, true, OP, false>, row_op_kernel<256, 0, true, OP, true>}}};
    const int regime = cols <= 1024 ? 0 : cols <= 4096 ? 1 : cols <= 16384 ? 2 : 3;
    const int64_t rpb = regime < 2 ? 4 : 1;
    const Kern kern = kerns[regime][ib ? 1 : 0][vec ? 1 : 0];
    int64_t blocks = std::min<int64_t>((rows + rpb - 1) / rpb, 1ll << 30);
    // RMSNorm with a wave per row holds the row and its weights in registers,
    // which leaves room for two or three waves per SIMD: there the grid is
    // capped at the workgroups resident at once and each wave loops over
    // rows, so no SIMD idles while a finished workgroup's successor starts
    // (4-22 % less time on MI355X for 256 to 4096 columns, warm or cold
    // caches; log-softmax and the mean gain nothing from it).  Each row's arithmetic
    // is unchanged, and so are the bits.
    if (OP == RO_RMS && regime < 2) {
        static std::atomic<int> per_cu[2][2][2];   // resident workgroups per CU, 0 until asked
        std::atomic<int>& slot = per_cu[regime][ib ? 1 : 0][vec ? 1 : 0];
        int occ = slot.load(std::memory_order_relaxed);
        if (occ == 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, 0) != hipSuccess || occ < 1)
                return BI_ERR_LAUNCH;
            slot.store(occ, std::memory_order_relaxed);
        }
        int cus = 0;
        const int rc = device_cu_count(&cus);
        if (rc != BI_OK) return rc;
        blocks = std::min<int64_t>(blocks, (int64_t)occ * cus);
    }
    const dim3 grid((unsigned)blocks);
    launch_kernel(kern, grid, dim3(256), 0, st, x, ldx, w, eps, y, ldy, rows, (int)cols, ob ? 1 : 0);
    return launch_status();
}

// Shared argument checks of the row operations (y_rows: the output has one
// row per input row with ldy, else one value per row).
int row_op_check(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* y, int64_t ldy,
                 int in_dtype, int out_dtype, bool y_rows) {
    if ((in_dtype != BI_F32 && in_dtype != BI_BF16) || (out_dtype != BI_F32 && out_dtype != BI_BF16))
        return BI_ERR_DTYPE;
    if (rows < 0 || cols < 0) return BI_ERR_SHAPE;
    if (cols > (1ll << 24) || rows > (1ll << 40)) return BI_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return BI_OK;
    if (!x || !y) return BI_ERR_NULL;
    if (ldx < 0 || (rows > 1 && ldx < cols)) return BI_ERR_LAYOUT;
    if (y_rows && (ldy < 0 || (rows > 1 && ldy < cols))) return BI_ERR_LAYOUT;
    if (!aligned(x, in_dtype == BI_BF16 ? 2 : 4) || !aligned(y, out_dtype == BI_BF16 ? 2 : 4))
        return BI_ERR_LAYOUT;
    return BI_OK;
}

template <int D>
static void decode_paged_launch(dim3 g1, dim3 g2, hipStream_t st, bool uni, const void* q, const void* kc,
                                const void* vc, const int32_t* bt, int64_t max_pages, const int32_t* sl,
                                int H, int log2p, int num_pages, int max_seq, int maxchunks, float* wsf,
                                float scale, void* out, int64_t BH, int out_dtype) {
    auto kern = uni ? decode_chunk_paged_kernel<D, true> : decode_chunk_paged_kernel<D, false>;
    launch_kernel(kern, g1, dim3(DEC_THREADS), 0, st, (const uint16_t*)q, (const uint16_t*)kc,
                  (const uint16_t*)vc, bt, max_pages, sl, H, log2p, num_pages, max_seq, maxchunks, (int)BH, wsf,
                  scale);
    auto merge = out_dtype == BI_BF16 ? decode_merge_kernel<D, 1> : decode_merge_kernel<D, 0>;
    launch_kernel(merge, g2, dim3(256), 0, st, (const float*)wsf, out, BH, maxchunks, sl, H, max_seq);
}

}  // namespace bi

using namespace bi;

// ================================================================ C ABI
extern "C" {

const char* bi_status_string(int status) {
    switch (status) {
        case BI_OK: return "BI_OK";
        case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
        case BI_ERR_SHAPE: return "BI_ERR_SHAPE: negative or inconsistent sizes";
        case BI_ERR_DTYPE: return "BI_ERR_DTYPE: dtype not accepted by this entry point";
        case BI_ERR_LAYOUT: return "BI_ERR_LAYOUT: strides or alignment not supported";
        case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: request outside what is implemented";
        case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: workspace NULL, too small or misaligned";
        case BI_ERR_LAUNCH: return "BI_ERR_LAUNCH: the HIP runtime refused a launch";
        case BI_ERR_DEVICE: return "BI_ERR_DEVICE: no usable gfx950 device is current";
        case BI_ERR_SCRATCH: return "BI_ERR_SCRATCH: the call needs more than the library's static scratch";
        default: return "unknown bi_status";
    }
}

int bi_mm(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
          const void* B, int64_t sBk, int64_t sBn, void* C, int64_t sCm, int64_t sCn,
          int in_dtype, int out_dtype, void* stream) {
    GemmDesc d = mm_desc(M, N, K, A, sAm, sAk, B, sBk, sBn, nullptr, C, sCm, sCn, in_dtype, out_dtype);
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    return gemm_launch(d, (hipStream_t)stream, 0);
}

int bi_addmm(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
             const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C, int64_t sCm,
             int64_t sCn, int in_dtype, int out_dtype, void* stream) {
    GemmDesc d = mm_desc(M, N, K, A, sAm, sAk, B, sBk, sBn, bias, C, sCm, sCn, in_dtype, out_dtype);
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    return gemm_launch(d, (hipStream_t)stream, 0);
}

int bi_bmm(int64_t G, int64_t M, int64_t N, int64_t K, const void* A, int64_t sAg, int64_t sAm,
           int64_t sAk, const void* B, int64_t sBg, int64_t sBk, int64_t sBn, void* C, int64_t sCg,
           int64_t sCm, int64_t sCn, int in_dtype, int out_dtype, void* stream) {
    GemmDesc d = bmm_desc(G, M, N, K, A, sAg, sAm, sAk, B, sBg, sBk, sBn, C, sCg, sCm, sCn,
                          in_dtype, out_dtype);
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    return gemm_launch(d, (hipStream_t)stream, 0);
}

size_t bi_conv2d_workspace_bytes(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                 int64_t Kh, int64_t Kw, int64_t sh, int64_t sw, int64_t ph,
                                 int64_t pw, int64_t dh, int64_t dw, int64_t groups, int in_dtype) {
    size_t bytes = 0;
    if (conv_geometry(N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw, dh, dw, groups, in_dtype,
                      nullptr, &bytes) != BI_OK)
        return 0;
    return bytes;
}

int bi_conv2d(int64_t N, int64_t Cin, int64_t H, int64_t W, const void* x, int64_t Cout,
              int64_t Kh, int64_t Kw, const void* w, const void* bias, int64_t sh, int64_t sw,
              int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t groups, void* y, void* ws,
              size_t ws_bytes, int in_dtype, int out_dtype, void* stream) {
    ConvGeom g;
    size_t need = 0;
    int rc = conv_geometry(N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw, dh, dw, groups, in_dtype,
                           &g, &need);
    if (rc != BI_OK) return rc;
    if (!gemm_out_ok(in_dtype, out_dtype)) return BI_ERR_DTYPE;
    if (N == 0) return BI_OK;
    if (!x || !w || !y) return BI_ERR_NULL;
    if (!ws) return BI_ERR_WORKSPACE;
    if (ws_bytes < need || !aligned(ws, 256)) return BI_ERR_WORKSPACE;
    const int64_t esz = in_dtype == BI_F32 ? 4 : 2;
    if (!aligned(x, esz) || !aligned(w, esz) || (bias && !aligned(bias, esz)) ||
        !aligned(y, out_dtype == BI_F32 ? 4 : 2))
        return BI_ERR_LAYOUT;
    // The GEMM over (sample, group) slices: A = packed weight, B = unfold (K-contiguous).
    uint8_t* wp = (uint8_t*)ws;
    uint8_t* u = wp + cdiv(Cout * g.Kp * esz, 256) * 256;
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = N; d.G2 = groups; d.M = g.cog; d.N = g.L; d.K = g.Kp;
    d.A = wp; d.sA1 = 0; d.sA2 = g.cog * g.Kp; d.sAm = g.Kp; d.sAk = 1;
    d.B = u; d.sB1 = groups * g.L * g.Kp; d.sB2 = g.L * g.Kp; d.sBk = 1; d.sBn = g.Kp;
    d.bias = bias; d.sBias2 = g.cog; d.bias_rows = 1;
    d.C = y; d.sC1 = Cout * g.L; d.sC2 = g.cog * g.L; d.sCm = g.L; d.sCn = 1;
    d.in_dtype = in_dtype; d.out_dtype = out_dtype;
    rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    int cus = 0;
    rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t wchunks = Cout * (g.Kp / 8);
    const int64_t uchunks = N * groups * g.L * (g.Kp / 8);
    const int wgrid = (int)std::min<int64_t>(cdiv(wchunks, 256), 8 * cus);
    const int ugrid = (int)std::min<int64_t>(cdiv(uchunks, 256), 64 * cus);
    const int64_t lim32 = (1ll << 31) - 1;
    const bool idx32 = N * Cin * H * W <= lim32 && N * groups * g.L * g.Kp + Cout * g.Kp <= lim32 &&
                       g.OH * sh + (Kh - 1) * dh <= lim32 && g.OW * sw + (Kw - 1) * dw <= lim32 &&
                       N * Cin <= lim32 / std::max<int64_t>(H * W, 1);
    // The patch geometry (16-bit, no padding or dilation, one group, even
    // Kw / column stride / W, 4-byte aligned input and weight): the
    // specialised pack and unfold, if its magic-number divisions are exact
    // for every numerator (x * d < 2^32) and its offset table fits in LDS.
    const int64_t nchunk = g.Kp / 8;
    const bool patch = in_dtype != BI_F32 && ph == 0 && pw == 0 && dh == 1 && dw == 1 && groups == 1 &&
                       Kw % 2 == 0 && sw % 2 == 0 && W % 2 == 0 && aligned(x, 4) && aligned(w, 4) && idx32 &&
                       (wchunks + uchunks) * nchunk < (1ll << 32) && N * g.L * g.L < (1ll << 32) &&
                       g.L * g.OW < (1ll << 32) && nchunk * 16 <= 32 * 1024;
    // Row blocks (one workgroup per output row of locations): the input rows
    // and U's rows in whole 16-byte pieces, the blocks within 48 KiB of LDS.
    const int64_t blk = Kh * W;
    const int64_t rows_lds = nchunk * 16 + Cin * blk * 2;
    const int64_t rowblocks = N * g.OH;
    const bool patch_rows = patch && aligned(x, 16) && (blk * 2) % 16 == 0 && (H * W * 2) % 16 == 0 &&
                            (sh * W * 2) % 16 == 0 && rows_lds <= 48 * 1024 && rowblocks <= lim32 / 256 &&
                            Cin * (blk / 8) * (blk / 8) < (1ll << 32) && g.OW * nchunk * nchunk < (1ll << 32);
    if (patch_rows) {
        ConvPatchRows gr;
        gr.Cin = (int)Cin; gr.H = (int)H; gr.W = (int)W; gr.OH = (int)g.OH; gr.OW = (int)g.OW;
        gr.sh = (int)sh; gr.sw = (int)sw; gr.Kh = (int)Kh; gr.Kw = (int)Kw; gr.Kg = (int)g.Kg; gr.Kp = (int)g.Kp;
        gr.nchunk = (int)nchunk; gr.blk = (int)blk; gr.pieces = (int)(blk / 8); gr.wchunks = (int)wchunks;
        gr.rowblocks = (int)rowblocks;
        auto magic = [](int64_t d) { return (uint64_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d); };
        gr.m_nchunk = magic(nchunk); gr.m_pieces = magic(blk / 8);
        const int grid = (int)std::max<int64_t>(rowblocks, cdiv(wchunks, 256));
        launch_kernel(conv_prepare_patch_rows, dim3(grid), dim3(256), (size_t)rows_lds, st,
                      (const uint16_t*)w, (uint16_t*)wp, (const uint16_t*)x, (uint16_t*)u, gr);
    } else if (patch) {
        ConvPatch16 gp;
        gp.Cin = (int)Cin; gp.H = (int)H; gp.W = (int)W; gp.L = (int)g.L; gp.OW = (int)g.OW;
        gp.sh = (int)sh; gp.sw = (int)sw; gp.Kh = (int)Kh; gp.Kw = (int)Kw; gp.Kg = (int)g.Kg; gp.Kp = (int)g.Kp;
        gp.nchunk = (int)nchunk; gp.wchunks = (int)wchunks; gp.total = (int)(wchunks + uchunks);
        auto magic = [](int64_t d) { return (uint64_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d); };
        gp.m_nchunk = magic(nchunk); gp.m_L = magic(g.L); gp.m_OW = magic(g.OW);
        // one piece per thread up to 16 workgroups per CU (at 32 SigLIP images,
        // 2701 workgroups: 6.7 us, against 6.8-7.1 us with 2-16 per CU and
        // each workgroup's offset table spread over more pieces)
        const int pgrid = (int)std::min<int64_t>(cdiv(wchunks + uchunks, 256), 16 * cus);
        launch_kernel(conv_prepare_patch16, dim3(pgrid), dim3(256), (size_t)(nchunk * 16), st,
                      (const uint16_t*)w, (uint16_t*)wp, (const uint16_t*)x, (uint16_t*)u, gp);
    } else if (idx32) {
        ConvGeom32 g32;
        g32.N = (int)N; g32.Cin = (int)Cin; g32.H = (int)H; g32.W = (int)W; g32.Cout = (int)Cout;
        g32.Kh = (int)Kh; g32.Kw = (int)Kw; g32.sh = (int)sh; g32.sw = (int)sw; g32.ph = (int)ph; g32.pw = (int)pw;
        g32.dh = (int)dh; g32.dw = (int)dw; g32.groups = (int)groups; g32.OW = (int)g.OW; g32.L = (int)g.L;
        g32.cig = (int)g.cig; g32.Kg = (int)g.Kg; g32.Kp = (int)g.Kp;
        const int pgrid = (int)std::min<int64_t>(cdiv(wchunks + uchunks, 256), 64 * cus);
        if (in_dtype != BI_F32)
            launch_kernel((conv_prepare32<uint16_t>), dim3(pgrid), dim3(256), 0, st,
                          (const uint16_t*)w, (uint16_t*)wp, (const uint16_t*)x, (uint16_t*)u, g32);
        else
            launch_kernel((conv_prepare32<float>), dim3(pgrid), dim3(256), 0, st,
                          (const float*)w, (float*)wp, (const float*)x, (float*)u, g32);
    } else if (in_dtype != BI_F32) {
        launch_kernel((conv_pack_weight<uint16_t>), dim3(wgrid), dim3(256), 0, st,
                      (const uint16_t*)w, (uint16_t*)wp, g);
        launch_kernel((conv_unfold<uint16_t>), dim3(ugrid), dim3(256), 0, st,
                      (const uint16_t*)x, (uint16_t*)u, g);
    } else {
        launch_kernel((conv_pack_weight<float>), dim3(wgrid), dim3(256), 0, st,
                      (const float*)w, (float*)wp, g);
        launch_kernel((conv_unfold<float>), dim3(ugrid), dim3(256), 0, st,
                      (const float*)x, (float*)u, g);
    }
    rc = launch_status();
    if (rc != BI_OK) return rc;
    return gemm_launch(d, st, 0);
}

int bi_decode_chunk_tokens(void) { return DEC_CHUNK; }

size_t bi_decode_attn_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D) {
    if (B < 0 || H < 0 || S < 1 || D < 1) return 0;
    return (size_t)(B * H * cdiv(S, DEC_CHUNK) * (2 + D) * 4);
}

}  // extern "C"

namespace bi {

// Checks of bi_decode_attn's arguments other than the workspace (1: nothing
// to compute).
static int decode_check(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                        const void* v, void* out, int in_dtype, int out_dtype) {
    if (in_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (B < 0 || H < 0 || S < 1) return BI_ERR_SHAPE;
    if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return 1;
    if (!q || !k || !v || !out) return BI_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(out, out_dtype == BI_BF16 ? 2 : 4))
        return BI_ERR_LAYOUT;
    if (B * H * cdiv(S, DEC_CHUNK) > (1ll << 31) - 1 || B * H * D > (1ll << 40)) return BI_ERR_UNSUPPORTED;
    // Per-(b, h) K and V byte offsets (up to one chunk past S) are 32-bit.
    if ((S + DEC_CHUNK) * D * 2 >= (1ll << 31)) return BI_ERR_UNSUPPORTED;
    return BI_OK;
}

// The chunk and merge launches of an already checked decode, with the chunk
// triples in wsf.
static int decode_launch(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                         const void* v, void* out, float scale, float* wsf, int out_dtype, void* stream) {
    const int64_t nchunk = cdiv(S, DEC_CHUNK);
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t BH = B * H;
    const dim3 g1((unsigned)(BH * nchunk));
    const dim3 g2((unsigned)cdiv(BH * D, 256));
    const int sn = (int)nchunk;
    if (D == 64) {
        launch_kernel((decode_chunk_kernel<64>), g1, dim3(DEC_THREADS), 0, st,
                      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wsf, S, sn, DEC_CHUNK, scale);
        if (out_dtype == BI_BF16) launch_kernel((decode_merge_kernel<64, 1>), g2, dim3(256), 0, st, wsf, out, BH, sn, nullptr, 1, 0);
        else                      launch_kernel((decode_merge_kernel<64, 0>), g2, dim3(256), 0, st, wsf, out, BH, sn, nullptr, 1, 0);
    } else {
        launch_kernel((decode_chunk_kernel<128>), g1, dim3(DEC_THREADS), 0, st,
                      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wsf, S, sn, DEC_CHUNK, scale);
        if (out_dtype == BI_BF16) launch_kernel((decode_merge_kernel<128, 1>), g2, dim3(256), 0, st, wsf, out, BH, sn, nullptr, 1, 0);
        else                      launch_kernel((decode_merge_kernel<128, 0>), g2, dim3(256), 0, st, wsf, out, BH, sn, nullptr, 1, 0);
    }
    return launch_status();
}

// Device memory of bi_decode_attn_noalloc's chunk triples: one copy per GPU,
// allocated when the code object is loaded and held until the process ends.
// Host code never passes this name to a kernel (on the host it is only a
// handle): the device address comes from hipGetSymbolAddress, once per
// device, on that device's first call.
static __device__ __align__(256) float scratch[BI_DECODE_SCRATCH_BYTES / 4];
static std::atomic<float*> g_scratch_ptr[64];

static int scratch_ptr(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BI_ERR_DEVICE;
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return BI_ERR_DEVICE;
        p = (float*)a;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return BI_OK;
}

}  // namespace bi

extern "C" {

int bi_decode_attn(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                   const void* v, void* out, float scale, void* ws, size_t ws_bytes,
                   int in_dtype, int out_dtype, void* stream) {
    int rc = decode_check(B, H, S, D, q, k, v, out, in_dtype, out_dtype);
    if (rc != BI_OK) return rc == 1 ? BI_OK : rc;
    if (!ws) return BI_ERR_WORKSPACE;
    if (ws_bytes < bi_decode_attn_workspace_bytes(B, H, S, D) || !aligned(ws, 16))
        return BI_ERR_WORKSPACE;
    return decode_launch(B, H, S, D, q, k, v, out, scale, (float*)ws, out_dtype, stream);
}

int bi_decode_attn_noalloc(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                           const void* v, void* out, float scale, int in_dtype, int out_dtype,
                           void* stream) {
    int rc = decode_check(B, H, S, D, q, k, v, out, in_dtype, out_dtype);
    if (rc != BI_OK) return rc == 1 ? BI_OK : rc;
    if (bi_decode_attn_workspace_bytes(B, H, S, D) > (size_t)BI_DECODE_SCRATCH_BYTES) return BI_ERR_SCRATCH;
    float* wsf = nullptr;
    rc = scratch_ptr(&wsf);
    if (rc != BI_OK) return rc;
    // Every chunk writes its triple before the merge reads it: nothing in the
    // scratch needs clearing between calls.
    return decode_launch(B, H, S, D, q, k, v, out, scale, wsf, out_dtype, stream);
}

size_t bi_decode_attn_paged_workspace_bytes(int64_t B, int64_t H, int64_t max_seq_len, int64_t D) {
    if (B < 0 || H < 0 || max_seq_len < 1 || D < 1) return 0;
    return (size_t)(B * H * cdiv(max_seq_len, DEC_CHUNK) * (2 + D) * 4);
}

int bi_decode_attn_paged(int64_t B, int64_t H, int64_t D, const void* q, const void* k_cache,
                         const void* v_cache, int64_t num_pages, int64_t page_size,
                         const int32_t* block_table, int64_t max_pages, const int32_t* seq_lens,
                         int64_t max_seq_len, void* out, float scale, void* ws, size_t ws_bytes,
                         int in_dtype, int out_dtype, void* stream) {
    if (in_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (B < 0 || H < 0 || num_pages < 1 || max_pages < 1 || max_seq_len < 1) return BI_ERR_SHAPE;
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return BI_ERR_SHAPE;
    if (max_seq_len > max_pages * page_size) return BI_ERR_SHAPE;
    if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return BI_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return BI_ERR_NULL;
    if (!ws) return BI_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(out, out_dtype == BI_BF16 ? 2 : 4))
        return BI_ERR_LAYOUT;
    const int64_t maxchunks = cdiv(max_seq_len, DEC_CHUNK);
    // Token indices and in-page offsets are 32-bit; page ids are int32.
    if (B * H * maxchunks > (1ll << 31) - 1 || B * H * D > (1ll << 40) || H > (1 << 30) ||
        max_seq_len + DEC_CHUNK >= (1ll << 31) || page_size * D * 2 >= (1ll << 31) ||
        num_pages > (1ll << 31) - 1 || B * max_pages > (1ll << 40))
        return BI_ERR_UNSUPPORTED;
    if (ws_bytes < bi_decode_attn_paged_workspace_bytes(B, H, max_seq_len, D) || !aligned(ws, 16))
        return BI_ERR_WORKSPACE;
    int log2p = 0;
    while ((1ll << log2p) < page_size) ++log2p;
    hipStream_t st = (hipStream_t)stream;
    const int64_t BH = B * H;
    const dim3 g1((unsigned)(BH * maxchunks));
    const dim3 g2((unsigned)cdiv(BH * D, 256));
    // One page holds all of a wave-wide load's tokens (512 / D of them).
    const bool uni = page_size >= 512 / D;
    if (D == 64)
        decode_paged_launch<64>(g1, g2, st, uni, q, k_cache, v_cache, block_table, max_pages, seq_lens, (int)H,
                                log2p, (int)num_pages, (int)max_seq_len, (int)maxchunks, (float*)ws, scale, out,
                                BH, out_dtype);
    else
        decode_paged_launch<128>(g1, g2, st, uni, q, k_cache, v_cache, block_table, max_pages, seq_lens, (int)H,
                                 log2p, (int)num_pages, (int)max_seq_len, (int)maxchunks, (float*)ws, scale, out,
                                 BH, out_dtype);
    return launch_status();
}

size_t bi_prefill_attn_paged_workspace_bytes(int64_t total_q, int64_t H, int64_t max_kv_len, int64_t D) {
    if (total_q < 0 || H < 0 || max_kv_len < 1 || D < 1) return 0;
    const int64_t nch = cdiv(max_kv_len, PF_CHUNK);
    return nch > 1 ? (size_t)(nch * H * (4 + D) * total_q * 4) : 0;
}

int bi_prefill_attn_paged(int64_t B, int64_t H, int64_t D, const void* q, int64_t total_q,
                          const int32_t* cu_q, const int32_t* q_pos0, int64_t max_q,
                          const void* k_cache, const void* v_cache, int64_t num_pages, int64_t page_size,
                          const int32_t* block_table, int64_t max_pages, int64_t max_kv_len,
                          void* out, float scale, void* ws, size_t ws_bytes,
                          int in_dtype, int out_dtype, void* stream) {
    if (in_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (B < 0 || H < 0 || total_q < 0 || max_q < 1 || num_pages < 1 || max_pages < 1 || max_kv_len < 1)
        return BI_ERR_SHAPE;
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return BI_ERR_SHAPE;
    if (max_kv_len > max_pages * page_size) return BI_ERR_SHAPE;
    if (D != 128) return BI_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || total_q == 0) return BI_OK;
    if (!q || !cu_q || !q_pos0 || !k_cache || !v_cache || !block_table || !out) return BI_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(cu_q, 4) ||
        !aligned(q_pos0, 4) || !aligned(block_table, 4) || !aligned(out, 16))
        return BI_ERR_LAYOUT;
    const int64_t maxchunks = cdiv(max_kv_len, PF_CHUNK);
    const int64_t ntiles = cdiv(max_q, PF_QT);
    // Positions, in-page offsets and page ids are 32-bit; row offsets 64-bit.
    if (maxchunks * B * ntiles * H > (1ll << 31) - 1 || max_q > (1ll << 30) || H > (1 << 20) ||
        max_kv_len + PF_CHUNK >= (1ll << 31) || page_size * D * 2 >= (1ll << 31) ||
        num_pages > (1ll << 31) - 1 || B > (1 << 30) || cdiv(total_q * H * (D / 4), 256) > (1ll << 31) - 1)
        return BI_ERR_UNSUPPORTED;
    const size_t need = bi_prefill_attn_paged_workspace_bytes(total_q, H, max_kv_len, D);
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return BI_ERR_WORKSPACE;
    int log2p = 0;
    while ((1ll << log2p) < page_size) ++log2p;
    PfArgs a;
    a.q = (const uint16_t*)q;
    a.kc = (const uint8_t*)k_cache;
    a.vc = (const uint8_t*)v_cache;
    a.table = block_table;
    a.cu_q = cu_q;
    a.q_pos0 = q_pos0;
    a.ws = (float*)ws;
    a.out = out;
    a.total_q = total_q;
    a.max_pages = max_pages;
    a.B = (int)B;
    a.H = (int)H;
    a.log2p = log2p;
    a.num_pages = (int)num_pages;
    a.max_q = (int)max_q;
    a.max_kv = (int)max_kv_len;
    a.ntiles = (int)ntiles;
    a.cscale = (float)((double)scale * 1.4426950408889634);
    hipStream_t st = (hipStream_t)stream;
    const dim3 g1((unsigned)(maxchunks * B * ntiles * H));
    if (out_dtype == BI_BF16) launch_kernel((prefill_chunk_kernel<128, 1>), g1, dim3(PF_THREADS), 0, st, a);
    else                      launch_kernel((prefill_chunk_kernel<128, 0>), g1, dim3(PF_THREADS), 0, st, a);
    if (maxchunks > 1) {
        const dim3 g2((unsigned)cdiv(total_q * H * (D / 4), 256));
        if (out_dtype == BI_BF16) launch_kernel((prefill_merge_kernel<128, 1>), g2, dim3(256), 0, st, a);
        else                      launch_kernel((prefill_merge_kernel<128, 0>), g2, dim3(256), 0, st, a);
    }
    return launch_status();
}

int bi_softmax_rows(int64_t rows, int64_t cols, const void* S, int64_t ldS, float scale, void* P,
                    int64_t ldP, int out_dtype, void* stream) {
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (rows < 0 || cols < 0) return BI_ERR_SHAPE;
    if (cols > (1ll << 24)) return BI_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return BI_OK;
    if (!S || !P) return BI_ERR_NULL;
    if ((rows > 1 && (ldS < cols || ldP < cols)) || ldS < 0 || ldP < 0) return BI_ERR_LAYOUT;
    if (!aligned(S, 4) || !aligned(P, out_dtype == BI_BF16 ? 2 : 4)) return BI_ERR_LAYOUT;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid((unsigned)std::min<int64_t>((rows + 3) / 4, 1ll << 30));
    const float* s = (const float*)S;
    const bool ob = out_dtype == BI_BF16;
    const bool vec = cols % 4 == 0 && aligned(S, 16) && (rows == 1 || ldS % 4 == 0) &&
                     aligned(P, ob ? 8 : 16) && (rows == 1 || ldP % 4 == 0);
    const int nch = cols <= 1024 ? 4 : cols <= 4096 ? 16 : 0;
    typedef void (*Kern)(const float*, int64_t, float, void*, int64_t, int64_t, int);
    // [nch 4/16/0][vec][out_bf16]
    static const Kern kerns[3][2][2] = {
        {{softmax_rows_kernel<4, false, 0>, softmax_rows_kernel<4, false, 1>},
         {softmax_rows_kernel<4, true, 0>, softmax_rows_kernel<4, true, 1>}},
        {{softmax_rows_kernel<16, false, 0>, softmax_rows_kernel<16, false, 1>},
         {softmax_rows_kernel<16, true, 0>, softmax_rows_kernel<16, true, 1>}},
        {{softmax_rows_kernel<0, false, 0>, softmax_rows_kernel<0, false, 1>},
         {softmax_rows_kernel<0, true, 0>, softmax_rows_kernel<0, true, 1>}}};
    const Kern k = kerns[nch == 4 ? 0 : nch == 16 ? 1 : 2][vec ? 1 : 0][ob ? 1 : 0];
    launch_kernel(k, grid, dim3(SM_THREADS), 0, st, s, ldS, scale, P, ldP, rows, (int)cols);
    return launch_status();
}

int bi_attention_probs(int64_t G, int64_t T, int64_t Tk, int64_t D, const void* Q, int64_t sQg,
                       int64_t sQt, const void* K, int64_t sKg, int64_t sKt, float scale, void* P,
                       int64_t sPg, int64_t sPt, void* stream) {
    if (G < 0 || T < 0 || Tk < 0 || D < 0) return BI_ERR_SHAPE;
    if ((D != 64 && D != 128) || (Tk != 256 && Tk != 512 && Tk != 768 && Tk != 1024)) return BI_ERR_UNSUPPORTED;
    if (G == 0 || T == 0) return BI_OK;
    if (!Q || !K || !P) return BI_ERR_NULL;
    if (sQg < 0 || sQt < 0 || sKg < 0 || sKt < 0 || sPg < 0 || sPt < 0) return BI_ERR_LAYOUT;
    // 16-byte fragments of Q and K rows, 8-byte chunks of P rows
    if (!aligned(Q, 16) || !aligned(K, 16) || sQg % 8 || sQt % 8 || sKg % 8 || sKt % 8) return BI_ERR_LAYOUT;
    if (!aligned(P, 8) || sPg % 4 || sPt % 4) return BI_ERR_LAYOUT;
    if ((T > 1 && (sQt < D || sPt < Tk)) || sKt < D) return BI_ERR_LAYOUT;
    if (G > (1ll << 24) || T > (1ll << 30)) return BI_ERR_UNSUPPORTED;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    AttnProbsParams a;
    a.Q = (const uint16_t*)Q; a.K = (const uint16_t*)K; a.P = (uint16_t*)P;
    a.sQg = sQg; a.sQt = sQt; a.sKg = sKg; a.sKt = sKt; a.sPg = sPg; a.sPt = sPt;
    a.G = (int)G; a.T = (int)T; a.scale = scale;
    // one workgroup per CU: split a slice's query blocks when there are fewer slices than CUs
    const int64_t nblocks = cdiv(T, AP_ROWS);
    a.splits = (int)std::max<int64_t>(1, std::min<int64_t>(nblocks, cdiv(cus, G)));
    const int64_t grid = G * a.splits;
    if (grid > (1ll << 30)) return BI_ERR_UNSUPPORTED;
    typedef void (*Kern)(AttnProbsParams);
    static const Kern kerns[2][4] = {
        {attn_probs_kernel<64, 256>, attn_probs_kernel<64, 512>, attn_probs_kernel<64, 768>, attn_probs_kernel<64, 1024>},
        {attn_probs_kernel<128, 256>, attn_probs_kernel<128, 512>, attn_probs_kernel<128, 768>,
         attn_probs_kernel<128, 1024>}};
    launch_kernel(kerns[D == 128][Tk / 256 - 1], dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, a);
    return launch_status();
}

int bi_rms_norm(int64_t rows, int64_t cols, const void* x, int64_t ldx, const void* w, float eps,
                void* y, int64_t ldy, int in_dtype, int out_dtype, void* stream) {
    int rc = row_op_check(rows, cols, x, ldx, y, ldy, in_dtype, out_dtype, true);
    if (rc != BI_OK || rows == 0 || cols == 0) return rc;
    if (!w) return BI_ERR_NULL;
    if (!aligned(w, in_dtype == BI_BF16 ? 2 : 4)) return BI_ERR_LAYOUT;
    if (!(eps >= 0.0f) || eps == INFINITY) return BI_ERR_SHAPE;
    int cus = 0;
    rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    return row_op_launch<RO_RMS>(rows, cols, x, ldx, w, eps, y, ldy, in_dtype, out_dtype, (hipStream_t)stream);
}

int bi_log_softmax_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* y, int64_t ldy,
                        int in_dtype, int out_dtype, void* stream) {
    int rc = row_op_check(rows, cols, x, ldx, y, ldy, in_dtype, out_dtype, true);
    if (rc != BI_OK || rows == 0 || cols == 0) return rc;
    int cus = 0;
    rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    return row_op_launch<RO_LOGSOFTMAX>(rows, cols, x, ldx, nullptr, 0.0f, y, ldy, in_dtype, out_dtype,
                                        (hipStream_t)stream);
}

int bi_mean_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* y, int in_dtype, int out_dtype,
                 void* stream) {
    if (rows > 0 && cols == 0) return BI_ERR_SHAPE;   // the mean of no values is undefined
    int rc = row_op_check(rows, cols, x, ldx, y, 1, in_dtype, out_dtype, false);
    if (rc != BI_OK || rows == 0) return rc;
    int cus = 0;
    rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    return row_op_launch<RO_MEAN>(rows, cols, x, ldx, nullptr, 0.0f, y, 1, in_dtype, out_dtype, (hipStream_t)stream);
}

int bi_set_launch_events(void* start, void* stop) {
    t_events = stop ? LaunchEvents{(hipEvent_t)start, (hipEvent_t)stop} : LaunchEvents{nullptr, nullptr};
    t_events_first = stop != nullptr;
    return BI_OK;
}

}  // extern "C"
