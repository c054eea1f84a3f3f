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

#include "softmax.hpp"

namespace bi {

constexpr int RO_RMS = 0, RO_LOGSOFTMAX = 1, RO_MEAN = 2;

// L lanes per row, NCH chunks per lane held in registers (0: re-read the row
// for each pass), bfloat16 or binary32 input.
template <int L, int NCH, bool IN_BF16, int OP>
__global__ void __launch_bounds__(256)
row_op_kernel(const void* __restrict__ X, int64_t ldx, const void* __restrict__ Wt, float eps,
              void* __restrict__ Y, int64_t ldy, int64_t rows, int64_t cols, int vec, int out_bf16) {
    __shared__ float red[4];
    constexpr int RPB = 256 / L;                         // rows per workgroup
    const int tid = threadIdx.x;
    const int li = L == 64 ? (tid & 63) : tid;           // lane within the row
    const int wave = tid >> 6;
    const int64_t nchunk = (cols + 3) / 4;
    constexpr float PAD_SUM = -0.0f;
    const float pad = OP == RO_LOGSOFTMAX ? -INFINITY : PAD_SUM;

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
    // Chunk c of a row of T (bfloat16 or binary32) with `fill` past cols.
    auto load = [&](const void* base, int64_t c, float fill, bool bf16, bool v4) {
        f32x4_t x;
        if (c < nchunk && v4) {
            if (bf16) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                const u32x2_t w = *(const u32x2_t*)((const uint16_t*)base + 4 * c);
                x = f32x4_t{bf16lo_to_f32(w[0]), bf16hi_to_f32(w[0]), bf16lo_to_f32(w[1]), bf16hi_to_f32(w[1])};
            } else {
                x = *(const f32x4_t*)((const float*)base + 4 * c);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = 4 * c + e;
                x[e] = j < cols ? (bf16 ? bf16_to_f32(((const uint16_t*)base)[j]) : ((const float*)base)[j]) : fill;
            }
        }
        return x;
    };
    auto store = [&](void* base, int64_t c, f32x4_t y) {
        if (c < nchunk && vec) {
            if (out_bf16) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                *(u32x2_t*)((uint16_t*)base + 4 * c) = u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            } else {
                *(f32x4_t*)((float*)base + 4 * c) = y;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = 4 * c + e;
                if (j < cols) {
                    if (out_bf16) ((uint16_t*)base)[j] = f32_to_bf16_rne(y[e]);
                    else          ((float*)base)[j] = y[e];
                }
            }
        }
    };

    for (int64_t row = (int64_t)blockIdx.x * RPB + (L == 64 ? wave : 0); row < rows; row += (int64_t)gridDim.x * RPB) {
        const void* xr = IN_BF16 ? (const void*)((const uint16_t*)X + row * ldx) : (const void*)((const float*)X + row * ldx);
        void* yr = out_bf16 ? (void*)((uint16_t*)Y + row * ldy) : (void*)((float*)Y + row * ldy);
        auto ldx4 = [&](int64_t c) { return load(xr, c, pad, IN_BF16, vec != 0); };

        if constexpr (OP == RO_MEAN) {
            float s = PAD_SUM;
            if constexpr (NCH > 0) {
#pragma unroll
                for (int v = 0; v < NCH; ++v) {
                    const f32x4_t x = ldx4(li + (int64_t)L * v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += x[e];
                }
            } else {
                for (int64_t c = li; c < nchunk; c += L) {
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
        } else if constexpr (OP == RO_RMS) {
            auto ldw4 = [&](int64_t c) { return load(Wt, c, 0.0f, IN_BF16, vec != 0); };
            float ss = PAD_SUM;
            f32x4_t xs[NCH > 0 ? NCH : 1];
            if constexpr (NCH > 0) {
#pragma unroll
                for (int v = 0; v < NCH; ++v) {
                    xs[v] = ldx4(li + (int64_t)L * v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ss += xs[v][e] * xs[v][e];
                }
            } else {
                for (int64_t c = li; c < nchunk; c += L) {
                    const f32x4_t x = ldx4(c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ss += x[e] * x[e];
                }
            }
            ss = rsum(ss);
            const float r = 1.0f / sqrtf(ss / (float)cols + eps);
            auto out = [&](int64_t c, f32x4_t x) {
                const f32x4_t w = ldw4(c);
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (x[e] * r) * w[e];
                store(yr, c, y);
            };
            if constexpr (NCH > 0) {
#pragma unroll
                for (int v = 0; v < NCH; ++v) out(li + (int64_t)L * v, xs[v]);
            } else {
                for (int64_t c = li; c < nchunk; c += L) out(c, ldx4(c));
            }
        } else {   // log-softmax
            float m = -INFINITY;
            f32x4_t xs[NCH > 0 ? NCH : 1];
            if constexpr (NCH > 0) {
#pragma unroll
                for (int v = 0; v < NCH; ++v) {
                    xs[v] = ldx4(li + (int64_t)L * v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) m = fmaxf(m, xs[v][e]);
                }
            } else {
                for (int64_t c = li; c < nchunk; c += L) {
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
                for (int64_t c = li; c < nchunk; c += L) {
                    const f32x4_t x = ldx4(c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += sm_exp(x[e] - m);
                }
            }
            s = rsum(s);
            const float ls = logf(s);
            auto out = [&](int64_t c, f32x4_t x) {
                f32x4_t y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (x[e] - m) - ls;
                store(yr, c, y);
            };
            if constexpr (NCH > 0) {
#pragma unroll
                for (int v = 0; v < NCH; ++v) out(li + (int64_t)L * v, xs[v]);
            } else {
                for (int64_t c = li; c < nchunk; c += L) out(c, ldx4(c));
            }
        }
    }
}

}  // namespace bi
