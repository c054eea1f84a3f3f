// Persistent binary32 GEMM for gfx950: C = A @ B (+ bias) on the fp32 matrix
// cores (v_mfma_f32_32x32x2f32), binary32 operands, binary32 accumulation.
//
// The binary32 configuration of the persistent matmul: one fixed tile
// (64x64 outputs, K step 32) for every call, each output element reduced by
// one chain of MFMA instructions over 2-wide K slices in ascending order from
// zero, rows/columns past M/N read from clamped addresses and never stored,
// the K tail zero-filled, the bias added once at the end.  Operands keep their
// binary32 precision: nothing is rounded to a narrower type.
//
// Operands may have any element strides (the loads are scalar and coalesced
// along whichever stride is 1), so transposed views need no copy.  Loads run
// three K steps ahead of their LDS store in four register sets, issued
// unconditionally (past the last step they re-read it), so the compiler's
// waits cover exactly the set being stored; the address of each element is
// fixed per tile and a step adds a uniform offset.  Per step that leaves one
// address add per load beside the 16 MFMAs (the K-tail variant, used only when
// K is not a multiple of the step, clamps k per element and zeroes the tail).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int G32_BM = 64;
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

template <int OUT_BF16, bool KTAIL>
__global__ void __launch_bounds__(G32_THREADS)
gemm_f32_persistent(GemmF32Params p) {
    // LDS holds A as [k][m] and B as [k][n] so that the 32 lanes feeding one
    // MFMA operand read 32 consecutive words.
    __shared__ float sA[2][G32_BK][G32_BM + 4];
    __shared__ float sB[2][G32_BK][G32_BN + 4];

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
        const int64_t m0 = (int64_t)pid_m * G32_BM, n0 = (int64_t)pid_n * G32_BN;
        const float* Ab = p.A + s1 * p.sA1 + s2 * p.sA2;
        const float* Bb = p.B + s1 * p.sB1 + s2 * p.sB2;

        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

        // Loads run three K steps ahead of their LDS store: step j's operands
        // go to register set j % 4, issued at the start of step j - 3.  Every
        // step issues its loads (past the last step it re-reads the last one,
        // unused), so the code is straight-line and each store waits only for
        // its own set.  The K tail (k >= K, read from a clamped address)
        // becomes zero at the store.
        float ra[4][8], rb[4][8];
        // Per element of the thread's share of a step: its address at k = 0 of
        // the tile, fixed for the tile; a step adds the uniform k0 times the K
        // stride.  KTAIL (K not a multiple of the step): the element's k is
        // clamped to K - 1 (32-bit: the host bounds K times the strides below
        // 2^31) and the tail becomes zero at the store.
        const float* pa[8];
        const float* pb[8];
        int ka[8], kb_[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + G32_THREADS * i;
            const int mm = a_kfast ? idx / G32_BK : idx % G32_BM;
            ka[i] = a_kfast ? idx % G32_BK : idx / G32_BM;
            const int64_t r = min(m0 + mm, p.M - 1);
            const int nn = b_kfast ? idx / G32_BK : idx % G32_BN;
            kb_[i] = b_kfast ? idx % G32_BK : idx / G32_BN;
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
                for (int i = 0; i < 8; ++i) ra[u][i] = pa[i][min(k0 + ka[i], K1) * sAk];
#pragma unroll
                for (int i = 0; i < 8; ++i) rb[u][i] = pb[i][min(k0 + kb_[i], K1) * sBk];
            } else {
                const int64_t oa = (int64_t)k0 * p.sAk, ob = (int64_t)k0 * p.sBk;
#pragma unroll
                for (int i = 0; i < 8; ++i) ra[u][i] = pa[i][oa];
#pragma unroll
                for (int i = 0; i < 8; ++i) rb[u][i] = pb[i][ob];
            }
        };
        auto store_tile = [&](int kt, auto uc) {
            constexpr int u = decltype(uc)::value, st = u & 1;
            const int kl = (int)p.K - kt * G32_BK;   // valid k within this step
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int mm = a_kfast ? idx / G32_BK : idx % G32_BM;
                sA[st][ka[i]][mm] = !KTAIL || ka[i] < kl ? ra[u][i] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int nn = b_kfast ? idx / G32_BK : idx % G32_BN;
                sB[st][kb_[i]][nn] = !KTAIL || kb_[i] < kl ? rb[u][i] : 0.0f;
            }
        };
        auto compute_tile = [&](int st) {
#pragma unroll
            for (int ks = 0; ks < G32_BK / 2; ++ks) {
                const int k = ks * 2 + (lane >> 5);
                const float a = sA[st][k][wm * 32 + (lane & 31)];
                const float b = sB[st][k][wn * 32 + (lane & 31)];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
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

        void* Cb = (OUT_BF16 ? (void*)((uint16_t*)p.C + s1 * p.sC1 + s2 * p.sC2)
                             : (void*)((float*)p.C + s1 * p.sC1 + s2 * p.sC2));
        const int64_t col = n0 + wn * 32 + (lane & 31);
        const float* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
        const float bv = (bb && !p.bias_rows && col < p.N) ? bb[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < p.M && col < p.N) {
                float v = acc[r];
                if (bb) v += p.bias_rows ? bb[row] : bv;
                store_out<OUT_BF16>(Cb, row * p.sCm + col, v);
            }
        }
    }
}

}  // namespace bi
