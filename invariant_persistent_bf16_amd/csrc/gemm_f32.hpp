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
// along whichever stride is 1), so transposed views need no copy.
#pragma once

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

template <int OUT_BF16>
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

        float ra[8], rb[8];
        auto load_tile = [&](int kt) {
            const int64_t k0 = (int64_t)kt * G32_BK;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int mm = a_kfast ? idx / G32_BK : idx % G32_BM;
                const int kk = a_kfast ? idx % G32_BK : idx / G32_BM;
                int64_t r = m0 + mm;
                r = r < p.M ? r : p.M - 1;
                const int64_t k = k0 + kk;
                ra[i] = k < p.K ? Ab[r * p.sAm + k * p.sAk] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int nn = b_kfast ? idx / G32_BK : idx % G32_BN;
                const int kk = b_kfast ? idx % G32_BK : idx / G32_BN;
                int64_t c = n0 + nn;
                c = c < p.N ? c : p.N - 1;
                const int64_t k = k0 + kk;
                rb[i] = k < p.K ? Bb[k * p.sBk + c * p.sBn] : 0.0f;
            }
        };
        auto store_tile = [&](int st) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int mm = a_kfast ? idx / G32_BK : idx % G32_BM;
                const int kk = a_kfast ? idx % G32_BK : idx / G32_BM;
                sA[st][kk][mm] = ra[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int nn = b_kfast ? idx / G32_BK : idx % G32_BN;
                const int kk = b_kfast ? idx % G32_BK : idx / G32_BN;
                sB[st][kk][nn] = rb[i];
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

        if (nk > 0) {
            load_tile(0);
            store_tile(0);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const bool more = kt + 1 < nk;
                if (more) load_tile(kt + 1);
                compute_tile(kt & 1);
                if (more) store_tile((kt + 1) & 1);
                __syncthreads();
            }
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
