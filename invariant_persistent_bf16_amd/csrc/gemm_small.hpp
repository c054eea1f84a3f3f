// Small-tile 16-bit GEMM for gfx950: the same arithmetic as
// gemm_bf16_persistent, for products whose 256x256 tiles would leave most
// compute units idle (a batch-1 linear, a one-image patch convolution).
//
// Why the bits are those of the persistent kernel.  In both kernels output
// element (i, j) is one chain of v_mfma_f32_32x32x16 instructions (bf16 or
// f16 by the operands), two per 32-wide K step (K 0..15 of the step, then
// 16..31), K ascending from a zero accumulator, with the B fragment as the
// instruction's first operand and, in every lane, the same eight consecutive
// K values of row i of A and column j of B in the same register positions;
// the K tail is zero-filled to the 32-wide step; the bias is added once to
// the finished binary32 sum (the unused row or column part is -0.0, an exact
// identity) and the value is rounded once.  The tile size only decides which
// wave computes which outputs, so the two kernels agree bit for bit, and the
// choice between them (a function of the shape) cannot make a row depend on
// the rest of the batch.  This is the reading the batch-invariance pages'
// fixed configuration rests on ("Unmasking the True Culprit ...", section
// "Why This Achieves Batch Invariance": the reduction order of an element
// must not depend on the batch), kept while the tile is chosen by shape.
//
// Hardware mapping.  One wave per workgroup computes a (32 WM) x (32 WN)
// block of C: WM x WN accumulator blocks of 32x32; each A fragment serves the
// WN column blocks and each B fragment the WM row blocks.  Operands are read
// straight into registers with 16-byte buffer loads, D steps ahead of their
// use (D steps x (WM + WN) x 32 bytes per lane in flight), so a wave streams
// its slab of B at the rate HBM gives it without barriers.  WN = 2: an
// N-contiguous B is then read as whole 128-byte lines of each K row, and A
// is read once per 64 columns rather than per 32.
//  * A, and a K-contiguous B: lane l loads row (column) l % 32, K values
//    8 (l / 32) .. +7 of each 16-wide half-step: the MFMA operand itself.
//  * an N-contiguous B: per 32-column block, lane l loads 8 columns of K rows
//    l / 4 and 16 + l / 4 of the step (a 2 KiB [32 K, 32 N] block per step),
//    writes them to the block's LDS buffer in row order, and builds its
//    fragments with
//    ds_read_b64_tr_b16 (within 16 lanes, lane t receives element t % 4 of the
//    8 bytes addressed by lanes 4 j + t / 4): lane 16 g + 4 j + u addresses K
//    row 16 kk + 8 (g / 2) + 4 h + j, columns 16 (g % 2) + 4 u .. +3, so lane
//    16 g + t receives column 16 (g % 2) + t, K values 16 kk + 8 (g / 2) + 4 h
//    .. +3, half h of the operand.
// Lanes past M, N or K read through the out-of-range buffer offset (zeros, no
// memory access); columns of an N-contiguous B past N are read from the last
// valid 8 (never stored).  Workgroups are renumbered so that consecutive
// blocks (which share lines of an N-contiguous B and rows of A) run on the
// same XCD.
#pragma once

#include "gemm_bf16.hpp"

namespace bi {

constexpr int GS_THREADS = 64;

// Column blocks per wave, and the width of a wave's block of C.
constexpr int GS_WN = 2;
constexpr int GS_COLS = 32 * GS_WN;

// Steps of operands in flight per wave.
template <int WM, int WN>
constexpr int gs_depth() { return WM == 1 ? 8 : WM == 2 ? (WN == 1 ? 8 : 6) : 4; }

typedef short gs_v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) gs_v4i16_t gs_lds_v4i16_t;

// CVEC4: four consecutive outputs of a lane may be stored as one access
// (C aligned to 4 elements' bytes; N, sCm, sC1, sC2 multiples of 4).
// WN: 32-column blocks per wave; with an N-contiguous B each block has its
// own 2 KiB LDS transpose buffer (per slot parity).
// p.tiles_m / tiles_n / tiles_per_slice / total_tiles count (32 WM) x (32 WN) blocks.
template <bool B_KCONTIG, int OUT16, bool F16, int WM, int WN = GS_WN>
__global__ void __launch_bounds__(GS_THREADS)
gemm_bf16_small(GemmParams p, int cvec4) {
    constexpr int D = gs_depth<WM, WN>();
    static_assert(D % 2 == 0, "the LDS double buffer alternates with the step");
    __shared__ __attribute__((aligned(16))) uint8_t smem[B_KCONTIG ? 16 : 2 * WN * 2048];

    // Grid padded to a multiple of 8; XCD x = w % 8 takes blocks
    // x * (grid / 8) .. (x + 1) * (grid / 8) - 1.
    const int w = blockIdx.x;
    const int task = (w % 8) * (int)(gridDim.x / 8) + w / 8;
    if (task >= p.total_tiles) return;

    const int lane = threadIdx.x;
    const int l32 = lane & 31, lh = lane >> 5;
    const int s = task / p.tiles_per_slice;
    const int t = task - s * p.tiles_per_slice;
    const int pid_m = t / p.tiles_n;
    const int pid_n = t - pid_m * p.tiles_n;
    const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
    const int64_t m0 = (int64_t)pid_m * (32 * WM), n0 = (int64_t)pid_n * (32 * WN);
    const uint16_t* Ab = p.A + s1 * p.sA1 + s2 * p.sA2 + m0 * p.sAm;
    const uint16_t* Bb = B_KCONTIG ? p.B + s1 * p.sB1 + s2 * p.sB2 + n0 * p.sBn
                                   : p.B + s1 * p.sB1 + s2 * p.sB2 + n0;
    const __amdgpu_buffer_rsrc_t rsA = g16_rsrc(Ab), rsB = g16_rsrc(Bb);
    const int K32 = (int)p.K;
    const int nk = (K32 + G16_BK - 1) / G16_BK;

    // Per-lane byte offsets from the block's base (fixed for the block); each
    // step adds a uniform byte offset.  The host bounds all of them below 2^31.
    uint32_t a_off[WM];
#pragma unroll
    for (int im = 0; im < WM; ++im)
        a_off[im] = m0 + 32 * im + l32 < p.M ? (uint32_t)(((32 * im + l32) * (int)p.sAm + 8 * lh) * 2) : G16_OOB;
    uint32_t b_off[WN][2];
    if constexpr (B_KCONTIG) {
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            const int n = 32 * b + l32;
            b_off[b][0] = n0 + n < p.N ? (uint32_t)((n * (int)p.sBn + 8 * lh) * 2) : G16_OOB;
            b_off[b][1] = b_off[b][0] == G16_OOB ? G16_OOB : b_off[b][0] + 32;
        }
    } else {
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            const int col = min(32 * b + 8 * (lane & 3), (int)(p.N - 8 - n0));
#pragma unroll
            for (int j = 0; j < 2; ++j) b_off[b][j] = (uint32_t)((((lane >> 2) + 16 * j) * (int)p.sBk + col) * 2);
        }
    }
    const uint32_t kstepB = B_KCONTIG ? 2u * G16_BK : (uint32_t)(2 * G16_BK * p.sBk);

    // Operands of D steps: ra[slot][im][kk]; rb[slot][b][kk] (K-contiguous
    // fragments) or rb[slot][b][j] (N-contiguous rows j*16 + lane/4 of block b).
    u32x4_t ra[D][WM][2];
    u32x4_t rb[D][WN][2];
    // Load step kt into slot; steps past the last read step nk (all lanes out
    // of range), which keeps the scalar offset within the host's bound.
    auto load = [&](int kt, auto slotc) {
        constexpr int slot = decltype(slotc)::value;
        const int kl = min(kt, nk);
        const int kleft = K32 - kl * G16_BK;
#pragma unroll
        for (int im = 0; im < WM; ++im)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                ra[slot][im][kk] = __builtin_amdgcn_raw_buffer_load_b128(
                    rsA, (int)(16 * kk + 8 * lh < kleft ? a_off[im] + 32 * kk : G16_OOB), kl * (2 * G16_BK), 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                const bool ok = B_KCONTIG ? 16 * j + 8 * lh < kleft : (lane >> 2) + 16 * j < kleft;
                rb[slot][b][j] = __builtin_amdgcn_raw_buffer_load_b128(rsB, (int)(ok ? b_off[b][j] : G16_OOB),
                                                                       (int)((uint32_t)kl * kstepB), 0);
            }
    };

    // N-contiguous B: LDS addresses of this lane's transposing reads
    // (kk, h) in buffer 0 of block 0; block b adds 2 KiB b, buffer 1 2 KiB WN.
    uint32_t tr_addr = 0;
    if constexpr (!B_KCONTIG) {
        const int g = lane >> 4, j = (lane >> 2) & 3, u = lane & 3;
        tr_addr = g16_lds_addr(smem) + (8 * (g >> 1) + j) * 64 + (16 * (g & 1) + 4 * u) * 2;
    }

    f32x16_t acc[WM][WN];
#pragma unroll
    for (int im = 0; im < WM; ++im)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[im][b][r] = 0.0f;

    auto compute = [&](auto slotc) {
        constexpr int slot = decltype(slotc)::value;
        u32x4_t bf[WN][2];
        if constexpr (B_KCONTIG) {
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                bf[b][0] = rb[slot][b][0];
                bf[b][1] = rb[slot][b][1];
            }
        } else {
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                uint8_t* buf = smem + ((slot & 1) * WN + b) * 2048;
                *(u32x4_t*)(buf + 16 * lane) = rb[slot][b][0];
                *(u32x4_t*)(buf + 1024 + 16 * lane) = rb[slot][b][1];
            }
#pragma unroll
            for (int b = 0; b < WN; ++b)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t a = tr_addr + ((slot & 1) * WN + b) * 2048 + kk * 1024 + h * 256;
                        const gs_v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gs_lds_v4i16_t*)(size_t)a);
                        const u32x2_t d = __builtin_bit_cast(u32x2_t, v);
                        bf[b][kk][2 * h] = d[0];
                        bf[b][kk][2 * h + 1] = d[1];
                    }
        }
        // Each accumulator takes kk = 0, then kk = 1, whatever WM and WN are.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int b = 0; b < WN; ++b)
#pragma unroll
                for (int im = 0; im < WM; ++im) {
                    if constexpr (F16)
                        acc[im][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            as_f16x8(bf[b][kk]), as_f16x8(ra[slot][im][kk]), acc[im][b], 0, 0, 0);
                    else
                        acc[im][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(bf[b][kk]), as_bf16x8(ra[slot][im][kk]), acc[im][b], 0, 0, 0);
                }
    };

    // Full groups of D steps as one straight-line block (each step's loads
    // reuse the slot it has just consumed, and the fences keep them there),
    // then the last nk % D steps, whose operands are already in flight.
    g16_static_for<0, D>([&](auto u) { load(decltype(u)::value, u); });
    int kt = 0;
    for (; kt + D <= nk; kt += D) {
        g16_static_for<0, D>([&](auto u) {
            compute(u);
            load(kt + decltype(u)::value + D, u);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    g16_static_for<0, D - 1>([&](auto u) {
        if (kt + decltype(u)::value < nk) compute(u);
    });

    // ---- epilogue: lane l, register 4 g + j of block (im, b) is C[m0 + 32 im
    // + l % 32][n0 + 32 b + 8 g + 4 (l / 32) + j]; + bias (binary32, once),
    // round once.
    using OutT = typename std::conditional<OUT16 != 0, uint16_t, float>::type;
    constexpr int ESZ = (int)sizeof(OutT);
    OutT* Cw = (OutT*)p.C + s1 * p.sC1 + s2 * p.sC2 + m0 * p.sCm + n0;
    const __amdgpu_buffer_rsrc_t rsC = g16_rsrc(Cw);
    const int sCm = (int)p.sCm;
    const uint16_t* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
    float brow[WM], bcol[WN][16];
#pragma unroll
    for (int im = 0; im < WM; ++im) brow[im] = -0.0f;
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) bcol[b][q] = -0.0f;
    if (bb) {
        if (p.bias_rows) {
#pragma unroll
            for (int im = 0; im < WM; ++im) brow[im] = h16_to_f32<F16>(bb[min<int64_t>(m0 + 32 * im + l32, p.M - 1)]);
        } else {
#pragma unroll
            for (int b = 0; b < WN; ++b)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    bcol[b][q] = h16_to_f32<F16>(bb[min<int64_t>(n0 + 32 * b + 8 * (q / 4) + 4 * lh + q % 4, p.N - 1)]);
        }
    }
    const int rows_valid = (int)min<int64_t>(p.M - m0, 32 * WM);
    const int cols_valid = (int)min<int64_t>(p.N - n0, 32 * WN);
#pragma unroll
    for (int im = 0; im < WM; ++im) {
        const int r = 32 * im + l32;
        const bool row_ok = r < rows_valid;
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4_t v = {acc[im][b][4 * g], acc[im][b][4 * g + 1], acc[im][b][4 * g + 2], acc[im][b][4 * g + 3]};
            v += brow[im];
            v += f32x4_t{bcol[b][4 * g], bcol[b][4 * g + 1], bcol[b][4 * g + 2], bcol[b][4 * g + 3]};
            const int c = 32 * b + 8 * g + 4 * lh;
            if (cvec4) {
                const uint32_t off = row_ok && c < cols_valid ? (uint32_t)((r * sCm + c) * ESZ) : G16_OOB;
                if constexpr (OUT16)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2_t{pack16x2<F16>(v[0], v[1]), pack16x2<F16>(v[2], v[3])}, rsC, (int)off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rsC, (int)off, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t off = row_ok && c + j < cols_valid ? (uint32_t)((r * sCm + c + j) * ESZ) : G16_OOB;
                    if constexpr (OUT16)
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pack16x2<F16>(v[j], 0.0f), rsC, (int)off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), rsC, (int)off, 0, 0);
                }
            }
        }
    }
}

}  // namespace bi
