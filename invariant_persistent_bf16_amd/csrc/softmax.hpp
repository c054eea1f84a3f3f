// Row softmax of a scaled binary32 matrix: P[r, :] = softmax(scale * S[r, :]).
//
// One workgroup (256 threads, 4 waves) owns one row for its whole
// computation, the row-per-program scheme of the batch-invariant softmax
// kernels ("Unmasking the True Culprit ...", section "Beyond Matrix
// Multiplication").  The reduction tree depends only on `cols`:
//   thread t holds elements t, t+256, t+512, ... (ascending), folds them
//   left to right; a xor-butterfly over the 64 lanes of each wave (every lane
//   ends with the same bits); the 4 wave partials added as ((w0+w1)+w2)+w3.
// The maximum is exact in any order; exp is the correctly rounded-to-1-ulp
// expf of the device math library; the division is IEEE.
#pragma once

#include "common.hpp"

namespace bi {

constexpr int SM_THREADS = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// VPT > 0: each thread keeps its VPT values in registers (cols <= 256*VPT).
// VPT == 0: any cols; the row is re-read for each pass.
template <int VPT, int OUT_BF16>
__global__ void __launch_bounds__(SM_THREADS)
softmax_rows_kernel(const float* __restrict__ S, int64_t ldS, float scale,
                    void* __restrict__ P, int64_t ldP, int64_t rows, int64_t cols) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const float* s = S + row * ldS;
        float x[VPT > 0 ? VPT : 1];
        float m = -INFINITY;
        if constexpr (VPT > 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int64_t j = tid + (int64_t)SM_THREADS * v;
                x[v] = j < cols ? scale * s[j] : -INFINITY;
                m = fmaxf(m, x[v]);
            }
        } else {
            for (int64_t j = tid; j < cols; j += SM_THREADS) m = fmaxf(m, scale * s[j]);
        }
        m = wave_max(m);
        if (lane == 0) red[0][wave] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

        float sum = 0.0f;
        if constexpr (VPT > 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                x[v] = expf(x[v] - m);   // padding lanes: expf(-inf) = 0
                sum += x[v];
            }
        } else {
            for (int64_t j = tid; j < cols; j += SM_THREADS) sum += expf(scale * s[j] - m);
        }
        sum = wave_sum(sum);
        if (lane == 0) red[1][wave] = sum;
        __syncthreads();
        sum = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];

        if constexpr (VPT > 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int64_t j = tid + (int64_t)SM_THREADS * v;
                if (j < cols) store_out<OUT_BF16>(P, row * ldP + j, x[v] / sum);
            }
        } else {
            for (int64_t j = tid; j < cols; j += SM_THREADS)
                store_out<OUT_BF16>(P, row * ldP + j, expf(scale * s[j] - m) / sum);
        }
        __syncthreads();   // red[] is reused by the next row
    }
}

}  // namespace bi
