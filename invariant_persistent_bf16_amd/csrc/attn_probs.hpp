// P = softmax(scale * Q K^T) in one kernel, with the bits of the two-stage
// path (the invariant bmm for S = Q K^T in binary32, then the row softmax),
// without writing S to memory.
//
// Batch-invariant attention ("Batch-Invariant Kernel Design: Conv2d and
// Attention BMM", section "Kernel 2: Attention BMM") computes the scores with
// the invariant bmm and normalises each row with the row-per-program softmax
// ("Unmasking the True Culprit ...", section "Beyond Matrix
// Multiplication").  Both fix their reduction orders by the non-batch shape,
// so a kernel that runs the same two orders gives the same bits while S
// never leaves the chip:
//   * S[i, j] is the chain of v_mfma_f32_32x32x16_bf16 over the D/16 slices
//     of d, ascending, from +0.0, with the key fragment as the instruction's
//     first operand and the query fragment as its second, as in the GEMM
//     (so each lane holds four consecutive keys of one query row);
//   * the softmax of row i is the one of softmax_rows_kernel: x = S * scale
//     (binary32), lane l of the row's wave owns the 4-key chunks l, l + 64,
//     l + 128, l + 192 and folds them in ascending order, then the same xor
//     butterflies (wave_max / wave_sum), exponential, reciprocal and
//     Markstein-corrected quotient, and the same rounding to bfloat16.
//
// One workgroup (4 waves) per (slice, range of 32-row query blocks), one per
// compute unit.  Wave w keeps its quarter of the slice's keys (Tk / 4 keys,
// all of d) in registers for the whole range, so K is read once per
// workgroup; per query block it loads the 32 query rows' fragments, runs its
// Tk / 128 blocks of 32 keys (D / 16 MFMAs each), writes the block's scores
// to LDS ([32][Tk + 4] binary32), and after a barrier each wave normalises 8
// rows from LDS, four at a time, and stores them as bfloat16 (non-temporal:
// P is far larger than the caches).  Query rows past T read the last row and
// are not stored.  At 256 slices of 1024 x 1024 x 128 the vector work of the
// softmax (eight operations and one exponential per score, fixed by the
// reference's arithmetic) takes about half of the kernel's time, the MFMAs
// about a ninth.
#pragma once

#include "common.hpp"
#include "rowio.hpp"
#include "softmax.hpp"

namespace bi {

constexpr int AP_ROWS = 32;              // query rows per block
constexpr int AP_TK_MAX = 1024;          // keys per slice (LDS: 32 x 1028 binary32)
constexpr int AP_PITCH = AP_TK_MAX + 4;  // row pitch of the score block in LDS
constexpr int AP_RG = 4;                 // rows a wave normalises together

struct AttnProbsParams {
    const uint16_t* Q;   // (g, t, d) at Q[g*sQg + t*sQt + d]
    const uint16_t* K;   // (g, j, d) at K[g*sKg + j*sKt + d]
    uint16_t* P;         // (g, t, j) at P[g*sPg + t*sPt + j]
    int64_t sQg, sQt, sKg, sKt, sPg, sPt;
    int G, T;
    float scale;
    int splits;          // workgroups per slice; each takes a contiguous range of query blocks
};

// D: head dimension (16-wide slices), TK: keys per slice (a multiple of 256).
template <int D, int TK>
__global__ void __launch_bounds__(256, 1)
attn_probs_kernel(AttnProbsParams p) {
    static_assert(D % 16 == 0 && D <= 128 && TK % 256 == 0 && TK <= AP_TK_MAX, "shape");
    constexpr int NS = D / 16;          // MFMA slices of d
    constexpr int NBLK = TK / 128;      // 32-key blocks per wave
    constexpr int NCH = TK / 256;       // 4-key chunks per lane and row in the softmax
    __shared__ __attribute__((aligned(16))) float sS[AP_ROWS * AP_PITCH];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.x / p.splits;
    const int part = blockIdx.x - g * p.splits;
    const int nblocks = (p.T + AP_ROWS - 1) / AP_ROWS;
    const int per = (nblocks + p.splits - 1) / p.splits;
    const int b0 = part * per, b1 = min(nblocks, b0 + per);
    if (b0 >= b1) return;   // uniform over the workgroup, before any barrier

    const uint16_t* Qg = p.Q + (int64_t)g * p.sQg;
    const uint16_t* Kg = p.K + (int64_t)g * p.sKg;
    const int key0 = wave * (TK / 4);
    const int lr = lane & 31, lh = lane >> 5;   // fragment row (query / key), 8-wide half of a slice

    // The wave's keys: block j, slice s -> K[key0 + 32 j + lr][16 s + 8 lh .. + 7].
    u32x4_t kf[NBLK][NS];
#pragma unroll
    for (int j = 0; j < NBLK; ++j)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            kf[j][s] = *(const u32x4_t*)(Kg + (int64_t)(key0 + 32 * j + lr) * p.sKt + 16 * s + 8 * lh);

    auto load_q = [&](u32x4_t (&qf)[NS], int blk) {
        const int t = min(blk * AP_ROWS + lr, p.T - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4_t*)(Qg + (int64_t)t * p.sQt + 16 * s + 8 * lh);
    };
    u32x4_t qf[NS];
    load_q(qf, b0);

    for (int blk = b0; blk < b1; ++blk) {
        // ---- scores of the block: this wave's keys, all 32 query rows
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            f32x16_t acc;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const f32x16_t zero = {};
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[j][s]), as_bf16x8(qf[s]),
                                                             s == 0 ? zero : acc, 0, 0, 0);
            }
            // lane: query row lr, keys 32 j + 8 q + 4 lh .. + 3 in registers 4q .. 4q + 3
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(f32x4_t*)&sS[lr * AP_PITCH + key0 + 32 * j + 8 * q + 4 * lh] =
                    f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
        if (blk + 1 < b1) load_q(qf, blk + 1);   // the next block's queries, under the softmax
        __syncthreads();

        // ---- softmax of rows 8 wave .. 8 wave + 7 of the block, AP_RG rows at
        // a time so that their reductions' cross-lane exchanges overlap (each
        // row's own sequence of operations is the reference's)
#pragma unroll 1
        for (int r0 = 0; r0 < 8; r0 += AP_RG) {
            f32x4_t x[AP_RG][NCH];
            float m[AP_RG], sum[AP_RG], rsum[AP_RG];
            // every score of the AP_RG rows read before the first is used, so
            // the LDS reads overlap instead of each waiting for the last
#pragma unroll
            for (int q = 0; q < AP_RG; ++q)
#pragma unroll
                for (int v = 0; v < NCH; ++v)
                    x[q][v] = *(const f32x4_t*)&sS[(8 * wave + r0 + q) * AP_PITCH + 4 * (lane + 64 * v)];
#pragma unroll
            for (int q = 0; q < AP_RG; ++q) {
#pragma unroll
                for (int v = 0; v < NCH; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[q][v][e] *= p.scale;
                m[q] = -INFINITY;
#pragma unroll
                for (int v = 0; v < NCH; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) m[q] = fmaxf(m[q], x[q][v][e]);
            }
#pragma unroll
            for (int q = 0; q < AP_RG; ++q) m[q] = wave_max(m[q]);
#pragma unroll
            for (int q = 0; q < AP_RG; ++q) {
                sum[q] = 0.0f;
#pragma unroll
                for (int v = 0; v < NCH; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[q][v][e] = sm_exp(x[q][v][e] - m[q]);
                        sum[q] += x[q][v][e];
                    }
            }
#pragma unroll
            for (int q = 0; q < AP_RG; ++q) sum[q] = wave_sum(sum[q]);
#pragma unroll
            for (int q = 0; q < AP_RG; ++q) {
                rsum[q] = 1.0f / sum[q];
                const int t = blk * AP_ROWS + 8 * wave + r0 + q;
                // rows past T: the store range is empty (nothing written)
                const __amdgpu_buffer_rsrc_t rp = row_rsrc(p.P + (int64_t)g * p.sPg + (int64_t)min(t, p.T - 1) * p.sPt,
                                                           t < p.T ? (int64_t)TK * 2 : 0);
#pragma unroll
                for (int v = 0; v < NCH; ++v) {
                    f32x4_t y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = sm_div(x[q][v][e], sum[q], rsum[q]);
                    row_store<true, 2>(rp, lane + 64 * v, y, true);
                }
            }
        }
        __syncthreads();   // the block's scores are read before the next block overwrites them
    }
}

}  // namespace bi
