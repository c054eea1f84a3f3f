// Row-per-program reductions beside the matmul, each row reduced in an order
// fixed by its length alone ("Unmasking the True Culprit ...", section "Beyond
// Matrix Multiplication": RMSNorm and log-softmax; the deterministic-inference
// handbook, section "与 batch 无关：固定切分": normalisation, softmax and mean
// each reduced by one block per row, never split across blocks because rows
// are few):
//   RMSNorm      y_j = (x_j * r) * w_j,  r = 1 / sqrt(sum_i x_i^2 / cols + eps)
//   log-softmax  y_j = (x_j - m) - log(sum_i exp(x_i - m)),  m = max_i x_i
//   row mean     y   = sum_i x_i / cols
// in binary32 (bfloat16 inputs widen exactly).
//
// Reduction tree (a function of cols only): element j lies in chunk c = j/4;
// chunk c belongs to lane c % L of the row's L lanes (L = 64: one wave per
// row, four rows per workgroup; L = 256: one workgroup per row for rows
// longer than 4096); a lane folds its elements left to right in ascending j;
// then a xor-butterfly over the wave (offsets 32 .. 1) and, for L = 256, the
// four wave partials added as ((w0 + w1) + w2) + w3.  Positions past cols hold
// an exact identity of the fold (-0.0 for sums, -inf for the maximum), so the
// register path (chunks held for the whole row) and the re-reading path fold
// the same values in the same order, and vector and element loads (aligned or
// not) give the same bits.  sqrt, the divisions and log are the device
// library's correctly rounded / ~1 ulp functions without fast-math; exp is the
// hardware base-2 exponential of (x - m) * log2(e) as in the softmax.
#pragma once

#include "rowio.hpp"
#include "softmax.hpp"

namespace bi {

constexpr int RO_RMS = 0, RO_LOGSOFTMAX = 1, RO_MEAN = 2;

// L lanes per row, NCH chunks per lane held in registers (0: re-read the row
// for each pass), bfloat16 or binary32 input, vector or element accesses
// (rowio.hpp: no access in a branch, positions past cols read as the fold's
// identity, writes past cols dropped).
template <int L, int NCH, bool IN_BF16, int OP, bool VEC>
__global__ void __launch_bounds__(256)
row_op_kernel(const void* __restrict__ X, int64_t ldx, const void* __restrict__ Wt, float eps,
              void* __restrict__ Y, int64_t ldy, int64_t rows, int cols, int out_bf16) {
    __shared__ float red[4];
    constexpr int RPB = 256 / L;                         // rows per workgroup
    constexpr int ISZ = IN_BF16 ? 2 : 4;
    const int tid = threadIdx.x;
    const int li = L == 64 ? (tid & 63) : tid;           // lane within the row
    const int wave = tid >> 6;
    const int nchunk = (cols + 3) / 4;
    const int osz = out_bf16 ? 2 : 4;
    constexpr float PAD_SUM = -0.0f;
    constexpr float PAD = OP == RO_LOGSOFTMAX ? -INFINITY : PAD_SUM;

    auto rsum = [&](float v) {
        v = wave_sum(v);
        if constexpr (L == 256) {
            if ((tid & 63) == 0) red[wave] = v;
            __syncthreads();
            v = ((red[0] + red[1]) + red[2]) + red[3];
            __syncthreads();
        }
        return v;
    };
    auto rmax = [&](float v) {
        v = wave_max(v);
        if constexpr (L == 256) {
            if ((tid & 63) == 0) red[wave] = v;
            __syncthreads();
            v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            __syncthreads();
        }
        return v;
    };
    const __amdgpu_buffer_rsrc_t rw = row_rsrc(OP == RO_RMS ? Wt : X, (int64_t)cols * ISZ);

    for (int64_t row = (int64_t)blockIdx.x * RPB + (L == 64 ? wave : 0); row < rows; row += (int64_t)gridDim.x * RPB) {
        const __amdgpu_buffer_rsrc_t rx = row_rsrc((const uint8_t*)X + row * ldx * ISZ, (int64_t)cols * ISZ);
        auto ldx4 = [&](int c) { return row_load<IN_BF16, VEC>(rx, c, cols, PAD); };

        if constexpr (OP == RO_MEAN) {
            float s = PAD_SUM;
            if constexpr (NCH > 0) {
                f32x4_t xs[NCH];
#pragma unroll
                for (int v = 0; v < NCH; ++v) xs[v] = ldx4(li + L * v);
#pragma unroll
                for (int v = 0; v < NCH; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += xs[v][e];
            } else {
                for (int c = li; c < nchunk; c += L) {
                    const f32x4_t x = ldx4(c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += x[e];
                }
            }
            s = rsum(s);
            if (li == 0) {
                const float m = s / (float)cols;
                if (out_bf16) ((uint16_t*)Y)[row] = f32_to_bf16_rne(m);
                else          ((float*)Y)[row] = m;
            }
        } else {
            const __amdgpu_buffer_rsrc_t ry = row_rsrc((uint8_t*)Y + row * ldy * osz, (int64_t)cols * osz);
            if constexpr (OP == RO_RMS) {
                float ss = PAD_SUM;
                f32x4_t xs[NCH > 0 ? NCH : 1];
                if constexpr (NCH > 0) {
#pragma unroll
                    for (int v = 0; v < NCH; ++v) xs[v] = ldx4(li + L * v);
#pragma unroll
                    for (int v = 0; v < NCH; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e) ss += xs[v][e] * xs[v][e];
                } else {
                    for (int c = li; c < nchunk; c += L) {
                        const f32x4_t x = ldx4(c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) ss += x[e] * x[e];
                    }
                }
                ss = rsum(ss);
                const float r = 1.0f / sqrtf(ss / (float)cols + eps);
                auto out = [&](int c, f32x4_t x) {
                    const f32x4_t w = row_load<IN_BF16, VEC>(rw, c, cols, 0.0f);
                    f32x4_t y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = (x[e] * r) * w[e];
                    row_store<VEC>(ry, c, y, out_bf16 != 0);
                };
                if constexpr (NCH > 0) {
#pragma unroll
                    for (int v = 0; v < NCH; ++v) out(li + L * v, xs[v]);
                } else {
                    for (int c = li; c < nchunk; c += L) out(c, ldx4(c));
                }
            } else {   // log-softmax
                float m = -INFINITY;
                f32x4_t xs[NCH > 0 ? NCH : 1];
                if constexpr (NCH > 0) {
#pragma unroll
                    for (int v = 0; v < NCH; ++v) xs[v] = ldx4(li + L * v);
#pragma unroll
                    for (int v = 0; v < NCH; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e) m = fmaxf(m, xs[v][e]);
                } else {
                    for (int c = li; c < nchunk; c += L) {
                        const f32x4_t x = ldx4(c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) m = fmaxf(m, x[e]);
                    }
                }
                m = rmax(m);
                float s = PAD_SUM;
                if constexpr (NCH > 0) {
#pragma unroll
                    for (int v = 0; v < NCH; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e) s += sm_exp(xs[v][e] - m);   // past cols: exp(-inf) = 0
                } else {
                    for (int c = li; c < nchunk; c += L) {
                        const f32x4_t x = ldx4(c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) s += sm_exp(x[e] - m);
                    }
                }
                s = rsum(s);
                const float ls = logf(s);
                auto out = [&](int c, f32x4_t x) {
                    f32x4_t y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = (x[e] - m) - ls;
                    // Non-temporal: log-probabilities over a vocabulary are far
                    // larger than the caches.  (Inputs, and RMSNorm's output,
                    // keep the default policy: a layer's activations are
                    // typically still in the 256 MB cache when the next op reads them.)
                    row_store<VEC, 2>(ry, c, y, out_bf16 != 0);
                };
                if constexpr (NCH > 0) {
#pragma unroll
                    for (int v = 0; v < NCH; ++v) out(li + L * v, xs[v]);
                } else {
                    for (int c = li; c < nchunk; c += L) out(c, ldx4(c));
                }
            }
        }
    }
}

}  // namespace bi
