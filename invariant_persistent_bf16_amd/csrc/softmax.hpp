// Row softmax of a scaled binary32 matrix: P[r, :] = softmax(scale * S[r, :]).
//
// One wave (64 lanes) owns one row for its whole computation, the
// row-per-program scheme of the batch-invariant softmax kernels ("Unmasking
// the True Culprit ...", section "Beyond Matrix Multiplication"); a
// workgroup holds four independent rows, one per wave, with no LDS and no
// barrier.  The reduction tree depends only on `cols`:
//   element j belongs to chunk c = j / 4; lane c % 64 owns chunk c; a lane
//   folds its elements left to right in ascending j; then a xor-butterfly
//   over the 64 lanes (offsets 32, 16, ..., 1; every lane ends with the same
//   bits).
// The same element-to-lane map is used whether the row is read with 16-byte
// loads (aligned rows, cols % 4 == 0) or element loads, so the bits do not
// depend on alignment either.  The maximum is exact in any order; exp is the
// device math library's expf; the division is IEEE.
#pragma once

#include "common.hpp"

namespace bi {

constexpr int SM_THREADS = 256;   // 4 rows per workgroup

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

// NCH > 0: the lane keeps its NCH chunks (4 * NCH values) in registers, so
// cols <= 256 * NCH; NCH == 0: any cols, the row is re-read for each pass.
// VEC: S rows and P rows allow 16-byte (S, binary32 P) or 8-byte (bfloat16 P)
// accesses and cols % 4 == 0.
template <int NCH, bool VEC, int OUT_BF16>
__global__ void __launch_bounds__(SM_THREADS)
softmax_rows_kernel(const float* __restrict__ S, int64_t ldS, float scale,
                    void* __restrict__ P, int64_t ldP, int64_t rows, int64_t cols) {
    const int lane = threadIdx.x & 63;
    const int64_t nchunk = (cols + 3) / 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
        const float* s = S + row * ldS;
        // Chunk c of the row, scaled, with -inf past cols.
        auto load = [&](int64_t c) {
            f32x4_t x;
            if constexpr (VEC) {
                if (c < nchunk) x = *(const f32x4_t*)(s + 4 * c) * scale;
                else            x = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t j = 4 * c + e;
                    x[e] = j < cols ? scale * s[j] : -INFINITY;
                }
            }
            return x;
        };
        auto store = [&](int64_t c, f32x4_t y) {
            if constexpr (VEC) {
                if (c < nchunk) {
                    if constexpr (OUT_BF16) {
                        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                        const u32x2_t w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
                        *(u32x2_t*)((uint16_t*)P + row * ldP + 4 * c) = w;
                    } else {
                        *(f32x4_t*)((float*)P + row * ldP + 4 * c) = y;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t j = 4 * c + e;
                    if (j < cols) store_out<OUT_BF16>(P, row * ldP + j, y[e]);
                }
            }
        };

        float m = -INFINITY;
        if constexpr (NCH > 0) {
            f32x4_t x[NCH];
#pragma unroll
            for (int v = 0; v < NCH; ++v) {
                x[v] = load(lane + 64 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, x[v][e]);
            }
            m = wave_max(m);
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < NCH; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[v][e] = expf(x[v][e] - m);   // past cols: expf(-inf) = 0
                    sum += x[v][e];
                }
            sum = wave_sum(sum);
#pragma unroll
            for (int v = 0; v < NCH; ++v) {
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = x[v][e] / sum;
                store(lane + 64 * v, y);
            }
        } else {
            for (int64_t c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, x[e]);
            }
            m = wave_max(m);
            float sum = 0.0f;
            for (int64_t c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
#pragma unroll
                for (int e = 0; e < 4; ++e) sum += expf(x[e] - m);
            }
            sum = wave_sum(sum);
            for (int64_t c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = expf(x[e] - m) / sum;
                store(c, y);
            }
        }
    }
}

}  // namespace bi
