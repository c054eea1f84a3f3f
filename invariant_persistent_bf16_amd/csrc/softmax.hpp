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
// depend on alignment either.  The maximum is exact in any order.
// exp(y), y = x - max <= 0, is computed as the hardware base-2 exponential
// (v_exp_f32, about 1 ulp) of the binary32 product y * log2(e); the rounding
// of that product adds a relative error of about |y| * 2^-24, at most ~1e-6
// for terms above 2^-30 of the largest.  The division by the sum uses
// Markstein's correction of the quotient (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", 1990): with
// y = 1/sum correctly rounded (one IEEE division per row), q = x*y,
// r = fma(-q, sum, x) (exact), q' = fma(r, y, q) is the correctly rounded
// x / sum when nothing underflows.  A GPU check against IEEE division found
// no difference for x in [2^-100, 1] and sum in [1, 2^20) (2^32 random pairs,
// and every binary32 x in [2^-30, 1] for eight sums); for x below that, a
// term under 2^-100 of the row's largest, q' may differ in the last place.
// The library expf and an IEEE division per score would cost about twenty
// vector instructions per score and make the kernel bound by the vector ALUs
// instead of by HBM.  P is written non-temporally, and S read so when the row
// stays in registers (S [G*T, T] and P are far larger than the caches; this
// took the kernel from 5.8 to 6.4 TB/s at 262144 rows of 1024).  Rows too long
// for registers are re-read, so their first read keeps the default policy.
#pragma once

#include "common.hpp"
#include "rowio.hpp"
#include "wave.hpp"

namespace bi {

constexpr int SM_THREADS = 256;   // 4 rows per workgroup
constexpr float SM_LOG2E = 1.44269504088896340736f;

// exp(y) for y <= 0 (y = -inf gives 0).
__device__ __forceinline__ float sm_exp(float y) { return __builtin_amdgcn_exp2f(y * SM_LOG2E); }
// x / s given y = 1/s correctly rounded (Markstein's correction).
__device__ __forceinline__ float sm_div(float x, float s, float y) {
    const float q = x * y;
    return __builtin_fmaf(__builtin_fmaf(-q, s, x), y, q);
}

// NCH > 0: the lane keeps its NCH chunks (4 * NCH values) in registers, so
// cols <= 256 * NCH; NCH == 0: any cols, the row is re-read for each pass.
// VEC: rows allow 16-byte reads of S and 16-byte (binary32 P) or 8-byte
// (bfloat16 P) writes, and cols % 4 == 0.  Accesses go through rowio.hpp
// (no access in a branch; positions past cols read as -inf).
template <int NCH, bool VEC, int OUT_BF16>
__global__ void __launch_bounds__(SM_THREADS)
softmax_rows_kernel(const float* __restrict__ S, int64_t ldS, float scale,
                    void* __restrict__ P, int64_t ldP, int64_t rows, int cols) {
    const int lane = threadIdx.x & 63;
    const int nchunk = (cols + 3) / 4;
    constexpr int OSZ = OUT_BF16 ? 2 : 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(S + row * ldS, (int64_t)cols * 4);
        const __amdgpu_buffer_rsrc_t rp = row_rsrc((const uint8_t*)P + row * ldP * OSZ, (int64_t)cols * OSZ);
        auto load = [&](int c) { return row_load<false, VEC, true, (NCH > 0 ? 2 : 0)>(rs, c, cols, -INFINITY, scale); };

        float m = -INFINITY;
        if constexpr (NCH > 0) {
            f32x4_t x[NCH];
#pragma unroll
            for (int v = 0; v < NCH; ++v) x[v] = load(lane + 64 * v);
#pragma unroll
            for (int v = 0; v < NCH; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, x[v][e]);
            m = wave_max(m);
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < NCH; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[v][e] = sm_exp(x[v][e] - m);   // past cols: exp(-inf) = 0
                    sum += x[v][e];
                }
            sum = wave_sum(sum);
            const float rsum = 1.0f / sum;
#pragma unroll
            for (int v = 0; v < NCH; ++v) {
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = sm_div(x[v][e], sum, rsum);
                row_store<VEC, 2>(rp, lane + 64 * v, y, OUT_BF16 != 0);
            }
        } else {
            for (int c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, x[e]);
            }
            m = wave_max(m);
            float sum = 0.0f;
            for (int c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
#pragma unroll
                for (int e = 0; e < 4; ++e) sum += sm_exp(x[e] - m);
            }
            sum = wave_sum(sum);
            const float rsum = 1.0f / sum;
            for (int c = lane; c < nchunk; c += 64) {
                const f32x4_t x = load(c);
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = sm_div(sm_exp(x[e] - m), sum, rsum);
                row_store<VEC, 2>(rp, c, y, OUT_BF16 != 0);
            }
        }
    }
}

}  // namespace bi
