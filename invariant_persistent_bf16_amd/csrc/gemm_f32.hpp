// Persistent binary32 GEMM for gfx950: C = A @ B (+ bias) on the fp32 matrix
// cores (v_mfma_f32_16x16x4f32), binary32 operands, binary32 accumulation.
//
// The binary32 configuration of the persistent matmul: each output element
// is reduced by one chain of v_mfma_f32_16x16x4f32 instructions over 4-wide
// K slices in ascending order from zero (lane l supplies k = l / 16 of each
// slice for both operands), rows/columns past M/N read from clamped
// addresses and never stored, the K tail zero-filled, the bias added once at
// the end.  Operands keep their binary32 precision: nothing is rounded to a
// narrower type.  Two tile sizes run this same per-element arithmetic and
// give the same bits: 64x64 outputs per workgroup (each of 4 waves a 32x32
// block as 2x2 MFMA blocks of 16x16), and 32x32 (each wave one 16x16 block)
// for products whose 64x64 tiles would leave most compute units idle; the
// host picks by shape.  The 16x16x4 instruction has the 32x32x2 one's rate
// but a chain of K/4 steps of 8 passes instead of K/2 steps of 16, so a
// small product whose time is its chain length runs four times shorter.
//
// Operands may have any element strides (the loads are scalar and coalesced
// along whichever stride is 1), so transposed views need no copy.  Loads run
// three K steps ahead of their LDS store in four register sets, issued
// unconditionally (past the last step they re-read it), so the compiler's
// waits cover exactly the set being stored; the address of each element is
// fixed per tile and a step adds a uniform offset.  Per step that leaves one
// address add per load beside the MFMAs (the K-tail variant, used only when
// K is not a multiple of the step, clamps k per element and zeroes the tail).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int G32_BM = 64;   // the large tile; the small one is 32x32
constexpr int G32_BN = 64;
constexpr int G32_BK = 32;
constexpr int G32_THREADS = 256;
constexpr int G32_GROUP_M = 8;

struct GemmF32Params {
    const float* A;     // (i, k) at A[i*sAm + k*sAk]
    const float* B;     // (k, j) at B[k*sBk + j*sBn]
    const float* bias;  // [N] (or [M] if bias_rows) or nullptr
    void* C;            // (i, j) at C[i*sCm + j]
    int64_t M, N, K;
    int64_t sAm, sAk, sBk, sBn, sCm;
    int64_t G2;
    int64_t sA1, sA2, sB1, sB2, sC1, sC2, sBias2;
    int tiles_m, tiles_n, tiles_per_slice, total_tiles;
    int bias_rows;      // 1: bias indexed by row (conv output channel), 0: by column
};

// WT: rows (and columns) of one wave's block, 32 (2x2 MFMA blocks, 64x64
// tile) or 16 (one MFMA block, 32x32 tile); p.tiles_* count tiles of 2 WT.
template <int OUT_BF16, bool KTAIL, int WT = 32>
__global__ void __launch_bounds__(G32_THREADS)
gemm_f32_persistent(GemmF32Params p) {
    constexpr int BM = 2 * WT, BN = 2 * WT;
    constexpr int NB = WT / 16;                        // MFMA blocks per wave side
    constexpr int NE = BM * G32_BK / G32_THREADS;      // elements per thread per operand and step
    // LDS holds A as [k][m] and B as [k][n] so that the 16 lanes feeding one
    // MFMA operand read 16 consecutive words.
    __shared__ float sA[2][G32_BK][BM + 4];
    __shared__ float sB[2][G32_BK][BN + 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (int)((p.K + G32_BK - 1) / G32_BK);
    const int grid = gridDim.x;
    const int w = blockIdx.x;
    const int wr = (grid % 8 == 0) ? (w % 8) * (grid / 8) + (w / 8) : w;
    const bool a_kfast = p.sAk == 1;
    const bool b_kfast = p.sBk == 1 && p.sBn != 1;

    for (int tile = wr; tile < p.total_tiles; tile += grid) {
        const int s = tile / p.tiles_per_slice;
        const int t = tile - s * p.tiles_per_slice;
        const int width = G32_GROUP_M * p.tiles_n;
        const int first_m = (t / width) * G32_GROUP_M;
        const int gsz = min(p.tiles_m - first_m, G32_GROUP_M);
        const int pid_m = first_m + (t % width) % gsz;
        const int pid_n = (t % width) / gsz;
        const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
        const int64_t m0 = (int64_t)pid_m * BM, n0 = (int64_t)pid_n * BN;
        const float* Ab = p.A + s1 * p.sA1 + s2 * p.sA2;
        const float* Bb = p.B + s1 * p.sB1 + s2 * p.sB2;

        f32x4_t acc[NB][NB];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj) acc[bi][bj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        // Loads run three K steps ahead of their LDS store: step j's operands
        // go to register set j % 4, issued at the start of step j - 3.  Every
        // step issues its loads (past the last step it re-reads the last one,
        // unused), so the code is straight-line and each store waits only for
        // its own set.  The K tail (k >= K, read from a clamped address)
        // becomes zero at the store.
        float ra[4][NE], rb[4][NE];
        // Per element of the thread's share of a step: its address at k = 0 of
        // the tile, fixed for the tile; a step adds the uniform k0 times the K
        // stride.  KTAIL (K not a multiple of the step): the element's k is
        // clamped to K - 1 (32-bit: the host bounds K times the strides below
        // 2^31) and the tail becomes zero at the store.
        const float* pa[NE];
        const float* pb[NE];
        int ka[NE], kb_[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int idx = tid + G32_THREADS * i;
            const int mm = a_kfast ? idx / G32_BK : idx % BM;
            ka[i] = a_kfast ? idx % G32_BK : idx / BM;
            const int64_t r = min(m0 + mm, p.M - 1);
            const int nn = b_kfast ? idx / G32_BK : idx % BN;
            kb_[i] = b_kfast ? idx % G32_BK : idx / BN;
            const int64_t c = min(n0 + nn, p.N - 1);
            if constexpr (KTAIL) {
                pa[i] = Ab + r * p.sAm;
                pb[i] = Bb + c * p.sBn;
            } else {
                pa[i] = Ab + r * p.sAm + ka[i] * p.sAk;
                pb[i] = Bb + c * p.sBn + kb_[i] * p.sBk;
            }
        }
        const int K1 = (int)p.K - 1, sAk = (int)p.sAk, sBk = (int)p.sBk;
        auto load_tile = [&](int kt, auto uc) {
            constexpr int u = decltype(uc)::value;
            const int k0 = min(kt, nk - 1) * G32_BK;
            if constexpr (KTAIL) {
#pragma unroll
                for (int i = 0; i < NE; ++i) ra[u][i] = pa[i][min(k0 + ka[i], K1) * sAk];
#pragma unroll
                for (int i = 0; i < NE; ++i) rb[u][i] = pb[i][min(k0 + kb_[i], K1) * sBk];
            } else {
                const int64_t oa = (int64_t)k0 * p.sAk, ob = (int64_t)k0 * p.sBk;
#pragma unroll
                for (int i = 0; i < NE; ++i) ra[u][i] = pa[i][oa];
#pragma unroll
                for (int i = 0; i < NE; ++i) rb[u][i] = pb[i][ob];
            }
        };
        auto store_tile = [&](int kt, auto uc) {
            constexpr int u = decltype(uc)::value, st = u & 1;
            const int kl = (int)p.K - kt * G32_BK;   // valid k within this step
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int mm = a_kfast ? idx / G32_BK : idx % BM;
                sA[st][ka[i]][mm] = !KTAIL || ka[i] < kl ? ra[u][i] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int nn = b_kfast ? idx / G32_BK : idx % BN;
                sB[st][kb_[i]][nn] = !KTAIL || kb_[i] < kl ? rb[u][i] : 0.0f;
            }
        };
        // Block (bi, bj) of the wave: rows wm WT + 16 bi .., columns wn WT + 16 bj ..;
        // lane l feeds row (column) l % 16 with k = 4 ks + l / 16.
        auto compute_tile = [&](int st) {
#pragma unroll
            for (int ks = 0; ks < G32_BK / 4; ++ks) {
                const int k = ks * 4 + (lane >> 4);
                float a[NB], b[NB];
#pragma unroll
                for (int bi = 0; bi < NB; ++bi) a[bi] = sA[st][k][wm * WT + 16 * bi + (lane & 15)];
#pragma unroll
                for (int bj = 0; bj < NB; ++bj) b[bj] = sB[st][k][wn * WT + 16 * bj + (lane & 15)];
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < NB; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
            }
        };
        // Step t (set u = t % 4, LDS stage t % 2): loads of step t + 3 into set
        // (u + 3) % 4, the MFMAs of step t, the store of step t + 1, barrier.
        auto step = [&](int t, auto uc) {
            constexpr int u = decltype(uc)::value;
            load_tile(t + 3, std::integral_constant<int, (u + 3) % 4>{});
            compute_tile(u & 1);
            store_tile(t + 1, std::integral_constant<int, (u + 1) % 4>{});
            __syncthreads();
        };

        if (nk > 0) {
            load_tile(0, std::integral_constant<int, 0>{});
            load_tile(1, std::integral_constant<int, 1>{});
            load_tile(2, std::integral_constant<int, 2>{});
            store_tile(0, std::integral_constant<int, 0>{});
            __syncthreads();
            // Four steps per trip (register sets are named statically), then the
            // remaining zero to three steps.  The last step's store (of step nk)
            // writes zeros into a stage that is not read again.
            int t = 0;
            for (; t + 4 <= nk; t += 4) {
                step(t, std::integral_constant<int, 0>{});
                step(t + 1, std::integral_constant<int, 1>{});
                step(t + 2, std::integral_constant<int, 2>{});
                step(t + 3, std::integral_constant<int, 3>{});
            }
            if (t < nk) step(t, std::integral_constant<int, 0>{});
            if (t + 1 < nk) step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < nk) step(t + 2, std::integral_constant<int, 2>{});
        }

        // Lane l, register r of block (bi, bj): row 16 bi + 4 (l / 16) + r,
        // column 16 bj + l % 16 of the wave's block.
        void* Cb = (OUT_BF16 ? (void*)((uint16_t*)p.C + s1 * p.sC1 + s2 * p.sC2)
                             : (void*)((float*)p.C + s1 * p.sC1 + s2 * p.sC2));
        const float* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) {
            const int64_t col = n0 + wn * WT + 16 * bj + (lane & 15);
            const float bv = (bb && !p.bias_rows && col < p.N) ? bb[col] : 0.0f;
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m0 + wm * WT + 16 * bi + 4 * (lane >> 4) + r;
                    if (row < p.M && col < p.N) {
                        float v = acc[bi][bj][r];
                        if (bb) v += p.bias_rows ? bb[row] : bv;
                        store_out<OUT_BF16>(Cb, row * p.sCm + col, v);
                    }
                }
        }
    }
}

}  // namespace bi
