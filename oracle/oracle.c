/*
 * Reference oracle for the batch-invariant dense-contraction path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU statement of what the GPU path computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, loads or calls it, and it shares no source,
 * header, helper or table with the HIP code.
 *
 * Conventions
 *   - Every input arrives as the exact bits the GPU receives: dtype 0 is IEEE
 *     binary32, dtype 1 is bfloat16 stored as raw uint16 bits.  Both are
 *     widened exactly to double and every sum below is taken in double, in the
 *     order written (reduction index ascending), with no blocking or reordering.
 *   - Strides are element strides (int64).
 *   - Optional subset lists (rows / slices / samples / requests) let the tests
 *     check chosen outputs of full-size problems; NULL means "all".
 *   - Outputs are double, densely packed in the order of the subset list.
 *
 * Sources (the pages this code restates):
 *   [TM]  "Unmasking the True Culprit: Why Temperature=0 Doesn't Mean
 *         Deterministic LLM Inference" (blog.sugiv.fyi), section "Technical
 *         Deep Dive: Batch Invariant Kernels": the persistent matmul kernel
 *         listing and the matmul_persistent host wrapper (tile accumulation in
 *         float32 over an ascending K loop, optional bias), and "Beyond Matrix
 *         Multiplication": the row-per-program log-softmax kernel.
 *   [VLA] "Batch-Invariant VLAs" (cybernetic-physics.pages.dev), sections
 *         "Weird nn.Conv2d behavior" (SigLIP patch embedding: 3->1152
 *         channels, 14x14 kernel, stride 14, no padding) and "Replacing
 *         nn.Conv2d" (per-sample unfold, flattened kernel matmul, bias add).
 *   [KD]  "Batch-Invariant Kernel Design: Conv2d and Attention BMM"
 *         (cybernetic-physics.pages.dev), sections "Kernel 1: Conv2d"
 *         (unfold matrix [Cin*Kh*Kw, locations]; stride, padding, dilation
 *         and groups) and "Kernel 2: Attention BMM" (flattened [B*H, T, D]
 *         operands, one grid row per batch element).
 *   [HB]  "确定性推理：让结果与 batch 无关" (anrans.github.io ai-infra-handbooks),
 *         section "根源：浮点加法的顺序": the split-K GEMM simulation and the
 *         flash-decoding simulation (per-chunk (max, sum, p@V), LSE merge,
 *         fixed 2048-token chunks), with their printed outputs.
 *
 * Parity pins: every exported function is pinned by the CPU tests against
 * closed forms, brute force, independent library routines and the values the
 * pages print.  No function here is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F16 2

/* bfloat16 is the top half of a binary32: widen by placing the 16 bits high. */
/* IEEE binary16 bits -> its exact value: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24), exponent 31 is
 * infinity (fraction 0) or NaN. */
static double f16_value(uint16_t h) {
    const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

static double widen(const void* p, int dtype, int64_t i) {
    if (dtype == OR_F16) return f16_value(((const uint16_t*)p)[i]);
    if (dtype == OR_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float*)p)[i];
}

/* Round a double to the nearest bfloat16 value, ties to even, in one step
 * (no detour through binary32, which would round twice).  bfloat16 has an
 * 8-bit significand and binary32's exponent range; below 2^-126 its spacing
 * is the fixed subnormal quantum 2^-133.  Overflow goes to +-inf. */
double oracle_bf16_rne(double x) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    (void)frexp(fabs(x), &e);              /* |x| = m * 2^e with m in [0.5, 1) */
    int q = e - 8;                         /* value of the last significand bit */
    if (q < -133) q = -133;
    double r = ldexp(rint(ldexp(fabs(x), -q)), q);   /* rint: ties to even */
    if (r >= ldexp(1.0, 128) - ldexp(1.0, 128 - 9)) /* >= max + half ulp */
        r = INFINITY;
    return x < 0 ? -r : r;
}

/* Widen one element (exposed so tests can pin the bit conversion). */
double oracle_widen(const void* p, int dtype, int64_t i) { return widen(p, dtype, i); }

/* ---------------------------------------------------------------- GEMM ----
 * [TM] matmul kernel and host wrapper: C = A @ B (+ bias), A [M,K], B [K,N],
 * reduction over k in ascending order; the bias of the addmm form is added
 * once to the finished sum.
 *   C[i,j] = sum_{k=0}^{K-1} A[i,k] * B[k,j]  (+ bias[j])
 * The i-k-j loop order below keeps each C[i,j] summed over k ascending. */
void oracle_mm(int64_t M, int64_t N, int64_t K,
               const void* A, int64_t sAm, int64_t sAk,
               const void* B, int64_t sBk, int64_t sBn,
               const void* bias, int dtype,
               const int64_t* rows, int64_t nrows, double* C) {
    int64_t nr = rows ? nrows : M;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        int64_t i = rows ? rows[r] : r;
        double* c = C + r * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = widen(A, dtype, i * sAm + k * sAk);
            for (int64_t j = 0; j < N; ++j) c[j] += a * widen(B, dtype, k * sBk + j * sBn);
        }
        if (bias)
            for (int64_t j = 0; j < N; ++j) c[j] += widen(bias, dtype, j);
    }
    (void)M;
}

/* [KD] Kernel 2 / [VLA] loop_bmm: a batched product is the plain product of
 * each batch element g on its own, C[g] = A[g] @ B[g]. */
void oracle_bmm(int64_t G, int64_t M, int64_t N, int64_t K,
                const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
                const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
                int dtype, const int64_t* slices, int64_t nslices, double* C) {
    int64_t ns = slices ? nslices : G;
    for (int64_t s = 0; s < ns; ++s) {
        int64_t g = slices ? slices[s] : s;
        const char* a = (const char*)A + (size_t)(g * sAg) * (dtype == OR_F32 ? 4 : 2);
        const char* b = (const char*)B + (size_t)(g * sBg) * (dtype == OR_F32 ? 4 : 2);
        oracle_mm(M, N, K, a, sAm, sAk, b, sBk, sBn, NULL, dtype, NULL, 0, C + s * M * N);
    }
}

/* ---------------------------------------------------------------- conv ----
 * Output size of a 2-D convolution along one axis. */
int64_t oracle_conv_out(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d) {
    return (in + 2 * p - d * (k - 1) - 1) / s + 1;
}

/* Direct convolution, the seven nested loops.  [VLA] "Weird nn.Conv2d
 * behavior" states the independence of every output patch; [KD] Kernel 1
 * lists the supported options (stride, padding, dilation, groups):
 *   y[n,co,oh,ow] = bias[co] + sum_{ci<Cin/G} sum_{kh<Kh} sum_{kw<Kw}
 *        x[n, g*Cin/G + ci, oh*sh + kh*dh - ph, ow*sw + kw*dw - pw]
 *        * w[co, ci, kh, kw],            g = co / (Cout/G),
 * where x outside the image counts as zero.  The reduction runs ci, kh, kw
 * ascending (ci outermost), the order of the flattened kernel. */
void oracle_conv2d_direct(int64_t N, int64_t Cin, int64_t H, int64_t W, const void* x,
                          int64_t Cout, int64_t Kh, int64_t Kw, const void* w,
                          const void* bias, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                          int64_t dh, int64_t dw, int64_t groups, int dtype,
                          const int64_t* samples, int64_t nsamples, double* y) {
    int64_t OH = oracle_conv_out(H, Kh, sh, ph, dh), OW = oracle_conv_out(W, Kw, sw, pw, dw);
    int64_t cig = Cin / groups, cog = Cout / groups;
    int64_t ns = samples ? nsamples : N;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < ns; ++s) {
        for (int64_t co = 0; co < Cout; ++co) {
            int64_t n = samples ? samples[s] : s;
            int64_t g = co / cog;
            for (int64_t oh = 0; oh < OH; ++oh) {
                for (int64_t ow = 0; ow < OW; ++ow) {
                    double acc = 0.0;
                    for (int64_t ci = 0; ci < cig; ++ci)
                        for (int64_t kh = 0; kh < Kh; ++kh)
                            for (int64_t kw = 0; kw < Kw; ++kw) {
                                int64_t ih = oh * sh + kh * dh - ph;
                                int64_t iw = ow * sw + kw * dw - pw;
                                double xv = 0.0;
                                if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                    xv = widen(x, dtype, ((n * Cin + g * cig + ci) * H + ih) * W + iw);
                                acc += xv * widen(w, dtype, ((co * cig + ci) * Kh + kh) * Kw + kw);
                            }
                    if (bias) acc += widen(bias, dtype, co);
                    y[((s * Cout + co) * OH + oh) * OW + ow] = acc;
                }
            }
        }
    }
}

/* The same convolution by the second route the pages describe ([VLA]
 * "Replacing nn.Conv2d", [KD] Kernel 1): build the unfold matrix of one
 * sample, U[k, l] with k = ci*Kh*Kw + kh*Kw + kw and l = oh*OW + ow, then
 * multiply the flattened kernel [Cout/G, Cin/G*Kh*Kw] of each group by it and
 * add the bias.  Used only to cross-check the direct form. */
void oracle_conv2d_unfold(int64_t N, int64_t Cin, int64_t H, int64_t W, const void* x,
                          int64_t Cout, int64_t Kh, int64_t Kw, const void* w,
                          const void* bias, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                          int64_t dh, int64_t dw, int64_t groups, int dtype,
                          const int64_t* samples, int64_t nsamples, double* y) {
    int64_t OH = oracle_conv_out(H, Kh, sh, ph, dh), OW = oracle_conv_out(W, Kw, sw, pw, dw);
    int64_t L = OH * OW, cig = Cin / groups, cog = Cout / groups, Kg = cig * Kh * Kw;
    int64_t ns = samples ? nsamples : N;
    double* U = (double*)malloc(sizeof(double) * (size_t)(Kg * L));
    for (int64_t s = 0; s < ns; ++s) {
        int64_t n = samples ? samples[s] : s;
        for (int64_t g = 0; g < groups; ++g) {
            for (int64_t ci = 0; ci < cig; ++ci)
                for (int64_t kh = 0; kh < Kh; ++kh)
                    for (int64_t kw = 0; kw < Kw; ++kw) {
                        int64_t k = (ci * Kh + kh) * Kw + kw;
                        for (int64_t oh = 0; oh < OH; ++oh)
                            for (int64_t ow = 0; ow < OW; ++ow) {
                                int64_t ih = oh * sh + kh * dh - ph, iw = ow * sw + kw * dw - pw;
                                U[k * L + oh * OW + ow] =
                                    (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                        ? widen(x, dtype, ((n * Cin + g * cig + ci) * H + ih) * W + iw)
                                        : 0.0;
                            }
                    }
            for (int64_t c = 0; c < cog; ++c) {
                int64_t co = g * cog + c;
                double* out = y + (s * Cout + co) * L;
                for (int64_t l = 0; l < L; ++l) out[l] = 0.0;
                for (int64_t k = 0; k < Kg; ++k) {
                    double wv = widen(w, dtype, co * Kg + k);
                    for (int64_t l = 0; l < L; ++l) out[l] += wv * U[k * L + l];
                }
                if (bias)
                    for (int64_t l = 0; l < L; ++l) out[l] += widen(bias, dtype, co);
            }
        }
    }
    free(U);
}

/* ------------------------------------------------------------- softmax ----
 * Row softmax of a scaled fp32 score matrix, the row-per-program reduction of
 * [TM] "Beyond Matrix Multiplication" (max, then exponentials and their sum):
 *   x_j = scale * S[r, j];  m = max_j x_j;  P[r, j] = exp(x_j - m) / sum_j exp(x_j - m)
 * (the log-softmax listing subtracts log(sum); the softmax divides by sum). */
void oracle_softmax_rows(int64_t rows, int64_t cols, const float* S, int64_t ldS,
                         double scale, double* P) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* s = S + r * ldS;
        double* p = P + r * cols;
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j) {
            double xv = scale * (double)s[j];
            if (xv > m) m = xv;
        }
        double sum = 0.0;
        for (int64_t j = 0; j < cols; ++j) { p[j] = exp(scale * (double)s[j] - m); sum += p[j]; }
        for (int64_t j = 0; j < cols; ++j) p[j] /= sum;
    }
}

/* ------------------------------------------------------------- row ops ----
 * The row-per-program reductions beside the matmul: [TM] "Beyond Matrix
 * Multiplication" gives RMSNorm over the last dimension,
 *   y_j = x_j * (1 / sqrt(mean_i(x_i^2) + eps)) * w_j,
 * and log-softmax, y_j = (x_j - m) - log(sum_i exp(x_i - m)), m = max_i x_i;
 * [TM]'s list of overridden operators and [HB] "与 batch 无关：固定切分" (each
 * normalisation, softmax and mean reduced by one block per row in a fixed
 * order) add the row mean, y = sum_i x_i / cols.  Row r of x is
 * x[r * ldx + i] (dtype 0 binary32 or 1 bfloat16); outputs are dense doubles,
 * cols per row (one per row for the mean). */
void oracle_rms_norm(int64_t rows, int64_t cols, const void* x, int64_t ldx, int dtype,
                     const void* w, double eps, double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            const double v = widen(x, dtype, r * ldx + i);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / (double)cols + eps);
        for (int64_t j = 0; j < cols; ++j)
            y[r * cols + j] = widen(x, dtype, r * ldx + j) * inv * widen(w, dtype, j);
    }
}

void oracle_log_softmax_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, int dtype,
                             double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int64_t i = 0; i < cols; ++i) {
            const double v = widen(x, dtype, r * ldx + i);
            if (v > m) m = v;
        }
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i) sum += exp(widen(x, dtype, r * ldx + i) - m);
        const double ls = log(sum);
        for (int64_t j = 0; j < cols; ++j) y[r * cols + j] = (widen(x, dtype, r * ldx + j) - m) - ls;
    }
}

void oracle_mean_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, int dtype, double* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i) sum += widen(x, dtype, r * ldx + i);
        y[r] = sum / (double)cols;
    }
}

/* ------------------------------------------------------------ attention ----
 * [KD] Kernel 2: for each flattened batch element g, S = Q[g] @ K[g]^T,
 * P = softmax(scale * S) over each row, O = P @ V[g].  Q, K, V are [G, T, D]
 * contiguous.  If p_bf16 is set, P is rounded to bfloat16 (ties to even)
 * before the second product, because the method feeds a bfloat16 P into the
 * bfloat16 batched product (the persistent wrapper requires equal operand
 * dtypes, [TM] matmul_persistent). */
void oracle_attention(int64_t G, int64_t T, int64_t D, const void* Q, const void* K,
                      const void* V, double scale, int dtype, int p_bf16,
                      const int64_t* slices, int64_t nslices, double* O) {
    int64_t ns = slices ? nslices : G;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < ns; ++s) {
        int64_t g = slices ? slices[s] : s;
        double* srow = (double*)malloc(sizeof(double) * (size_t)T);
        for (int64_t t = 0; t < T; ++t) {
            double m = -INFINITY;
            for (int64_t j = 0; j < T; ++j) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += widen(Q, dtype, (g * T + t) * D + d) * widen(K, dtype, (g * T + j) * D + d);
                srow[j] = scale * acc;
                if (srow[j] > m) m = srow[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < T; ++j) { srow[j] = exp(srow[j] - m); sum += srow[j]; }
            for (int64_t j = 0; j < T; ++j) {
                srow[j] /= sum;
                if (p_bf16) srow[j] = oracle_bf16_rne(srow[j]);
            }
            double* o = O + (s * T + t) * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t j = 0; j < T; ++j)
                for (int64_t d = 0; d < D; ++d) o[d] += srow[j] * widen(V, dtype, (g * T + j) * D + d);
        }
        free(srow);
    }
}

/* --------------------------------------------------------------- decode ----
 * Single-query attention for each (b, h): q [B,H,D], K and V [B,H,S,D].
 * Unsplit definition:
 *   s_t = scale * q . k_t;  out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s). */
void oracle_decode(int64_t B, int64_t H, int64_t S, int64_t D, const void* q,
                   const void* k, const void* v, double scale, int dtype,
                   const int64_t* reqs, int64_t nreqs, double* out) {
    int64_t nr = reqs ? nreqs : B;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        for (int64_t h = 0; h < H; ++h) {
            int64_t b = reqs ? reqs[r] : r;
            int64_t bh = b * H + h;
            double* sc = (double*)malloc(sizeof(double) * (size_t)S);
            double m = -INFINITY;
            for (int64_t t = 0; t < S; ++t) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += widen(q, dtype, bh * D + d) * widen(k, dtype, (bh * S + t) * D + d);
                sc[t] = scale * acc;
                if (sc[t] > m) m = sc[t];
            }
            double den = 0.0;
            double* o = out + (r * H + h) * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < S; ++t) {
                double p = exp(sc[t] - m);
                den += p;
                for (int64_t d = 0; d < D; ++d) o[d] += p * widen(v, dtype, (bh * S + t) * D + d);
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= den;
            free(sc);
        }
    }
}

/* Decode over a paged KV cache with per-request lengths: the same unsplit
 * attention as oracle_decode for request b over its first seq_lens[b] tokens,
 * token t of request b read from page block_table[b * max_pages + t / P] at
 * slot t % P of the cache laid out [num_pages, H, P, D] (the storage the
 * handbook's serving frameworks page their KV cache in; [HB] "框架里的开关" and
 * "与 batch 无关：固定切分": prefix cache and chunked prefill must not change a
 * request's bits).  out [B, H, D]; a request with seq_lens[b] == 0 gets NaN. */
void oracle_decode_paged(int64_t B, int64_t H, int64_t D, const void* q, const void* kc,
                         const void* vc, const int32_t* block_table, int64_t max_pages,
                         const int32_t* seq_lens, int64_t P, double scale, int dtype, double* out) {
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t S = seq_lens[b];
            double* o = out + (b * H + h) * D;
            double* sc = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
            double m = -INFINITY;
            for (int64_t t = 0; t < S; ++t) {
                const int64_t row = ((int64_t)block_table[b * max_pages + t / P] * H + h) * P + t % P;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += widen(q, dtype, (b * H + h) * D + d) * widen(kc, dtype, row * D + d);
                sc[t] = scale * acc;
                if (sc[t] > m) m = sc[t];
            }
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < S; ++t) {
                const int64_t row = ((int64_t)block_table[b * max_pages + t / P] * H + h) * P + t % P;
                const double p = exp(sc[t] - m);
                den += p;
                for (int64_t d = 0; d < D; ++d) o[d] += p * widen(vc, dtype, row * D + d);
            }
            for (int64_t d = 0; d < D; ++d) o[d] = S > 0 ? o[d] / den : NAN;
            free(sc);
        }
    }
}

/* Causal prefill attention over a paged KV cache, for chunked prefill with a
 * prefix cache ([HB] "与 batch 无关：固定切分", the items on attention and on
 * chunked prefill with the prefix cache: a request's attention must not depend
 * on how its prompt was cut into prefill chunks or where its KV came from).
 * Request b owns query rows cu_q[b] .. cu_q[b+1]-1 of q [total_q, H, D]; row
 * cu_q[b] + j sits at absolute position pos = q_pos0[b] + j and attends to the
 * request's keys 0 .. pos (inclusive), key t read from page
 * block_table[b * max_pages + t / P], slot t % P of the caches
 * [num_pages, H, P, D].  Unsplit fp64 attention; out [total_q, H, D]. */
void oracle_prefill_paged(int64_t B, int64_t H, int64_t D, const void* q, const int32_t* cu_q,
                          const int32_t* q_pos0, const void* kc, const void* vc,
                          const int32_t* block_table, int64_t max_pages, int64_t P, double scale,
                          int dtype, double* out) {
    const int64_t total = cu_q[B];
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < total; ++r) {
        for (int64_t h = 0; h < H; ++h) {
            int64_t b = 0;
            while (cu_q[b + 1] <= r) ++b;
            const int64_t S = (int64_t)q_pos0[b] + (r - cu_q[b]) + 1;   /* keys 0 .. pos */
            const int32_t* bt = block_table + b * max_pages;
            double* o = out + (r * H + h) * D;
            double* sc = (double*)malloc(sizeof(double) * (size_t)S);
            double m = -INFINITY;
            for (int64_t t = 0; t < S; ++t) {
                const int64_t row = ((int64_t)bt[t / P] * H + h) * P + t % P;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += widen(q, dtype, (r * H + h) * D + d) * widen(kc, dtype, row * D + d);
                sc[t] = scale * acc;
                if (sc[t] > m) m = sc[t];
            }
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = 0; t < S; ++t) {
                const int64_t row = ((int64_t)bt[t / P] * H + h) * P + t % P;
                const double p = exp(sc[t] - m);
                den += p;
                for (int64_t d = 0; d < D; ++d) o[d] += p * widen(vc, dtype, row * D + d);
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= den;
            free(sc);
        }
    }
}

/* [HB] flash-decoding with fixed-length chunks.  The KV sequence is cut into
 * consecutive chunks of `chunk` tokens from position 0 (the last may be
 * shorter).  Each chunk c keeps the triple
 *   m_c = max_{t in c} s_t,  l_c = sum_{t in c} exp(s_t - m_c),
 *   o_c = sum_{t in c} exp(s_t - m_c) v_t,
 * and the triples are merged in ascending chunk order:
 *   M = max_c m_c,  out = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c.
 * If trip is non-NULL the triples are also written there, [nr, H, nchunk, 2+D]. */
void oracle_decode_chunked(int64_t B, int64_t H, int64_t S, int64_t D, const void* q,
                           const void* k, const void* v, double scale, int dtype,
                           int64_t chunk, const int64_t* reqs, int64_t nreqs,
                           double* out, double* trip) {
    int64_t nr = reqs ? nreqs : B;
    int64_t nc = (S + chunk - 1) / chunk;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; ++r) {
        for (int64_t h = 0; h < H; ++h) {
            int64_t b = reqs ? reqs[r] : r;
            int64_t bh = b * H + h;
            double* sc = (double*)malloc(sizeof(double) * (size_t)chunk);
            double* mc = (double*)malloc(sizeof(double) * (size_t)nc);
            double* lc = (double*)malloc(sizeof(double) * (size_t)nc);
            double* oc = (double*)malloc(sizeof(double) * (size_t)(nc * D));
            for (int64_t c = 0; c < nc; ++c) {
                int64_t t0 = c * chunk, t1 = t0 + chunk < S ? t0 + chunk : S;
                double m = -INFINITY;
                for (int64_t t = t0; t < t1; ++t) {
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        acc += widen(q, dtype, bh * D + d) * widen(k, dtype, (bh * S + t) * D + d);
                    sc[t - t0] = scale * acc;
                    if (sc[t - t0] > m) m = sc[t - t0];
                }
                double l = 0.0;
                double* o = oc + c * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t t = t0; t < t1; ++t) {
                    double p = exp(sc[t - t0] - m);
                    l += p;
                    for (int64_t d = 0; d < D; ++d) o[d] += p * widen(v, dtype, (bh * S + t) * D + d);
                }
                mc[c] = m;
                lc[c] = l;
                if (trip) {
                    double* tp = trip + ((r * H + h) * nc + c) * (2 + D);
                    tp[0] = m;
                    tp[1] = l;
                    for (int64_t d = 0; d < D; ++d) tp[2 + d] = o[d];
                }
            }
            double Mx = -INFINITY;
            for (int64_t c = 0; c < nc; ++c) if (mc[c] > Mx) Mx = mc[c];
            double den = 0.0;
            double* res = out + (r * H + h) * D;
            for (int64_t d = 0; d < D; ++d) res[d] = 0.0;
            for (int64_t c = 0; c < nc; ++c) {
                double wgt = exp(mc[c] - Mx);
                den += wgt * lc[c];
                for (int64_t d = 0; d < D; ++d) res[d] += wgt * oc[c * D + d];
            }
            for (int64_t d = 0; d < D; ++d) res[d] /= den;
            free(sc); free(mc); free(lc); free(oc);
        }
    }
}

/* ------------------------------------------------ fp32 simulations ----
 * These two routines restate, in binary32, the two CPU experiments of [HB]
 * "根源：浮点加法的顺序" whose printed booleans the tests pin.  They model the
 * batch-DEPENDENT schedules the method replaces and are used only to show
 * that the invariance checks can tell a changed reduction order apart.
 *
 * Split-K GEMM: each row is computed on its own; the K range [0, K) is cut
 * at floor(linspace(0, K, splits+1)) and each part's dot product is taken
 * separately (k ascending), then the parts are added in part order. */
void sim_splitk_gemm_f32(int64_t M, int64_t N, int64_t K, const float* X, const float* W,
                         int64_t splits, float* out) {
    int64_t* bnd = (int64_t*)malloc(sizeof(int64_t) * (size_t)(splits + 1));
    for (int64_t s = 0; s <= splits; ++s)
        bnd[s] = (int64_t)floor((double)K * (double)s / (double)splits);
    float* part = (float*)malloc(sizeof(float) * (size_t)N);
    for (int64_t i = 0; i < M; ++i) {
        float* o = out + i * N;
        for (int64_t s = 0; s < splits; ++s) {
            for (int64_t j = 0; j < N; ++j) part[j] = 0.0f;
            for (int64_t k = bnd[s]; k < bnd[s + 1]; ++k) {
                float a = X[i * K + k];
                for (int64_t j = 0; j < N; ++j) part[j] = part[j] + a * W[k * N + j];
            }
            for (int64_t j = 0; j < N; ++j) o[j] = (s == 0) ? part[j] : o[j] + part[j];
        }
    }
    free(part);
    free(bnd);
}

/* Flash-decoding with a given number of parts, single head, binary32: the
 * sequence is cut like torch.tensor_split (the first S % splits parts hold
 * one extra token), each part keeps (max, sum of exp, exp-weighted V sum)
 * and the parts are merged by the log-sum-exp rule in part order. */
void sim_decode_splits_f32(int64_t S, int64_t D, const float* q, const float* Kc,
                           const float* Vc, float scale, int64_t splits, float* out) {
    float* num = (float*)calloc((size_t)D, sizeof(float));
    float* ms = (float*)malloc(sizeof(float) * (size_t)splits);
    float* ls = (float*)malloc(sizeof(float) * (size_t)splits);
    float* os = (float*)malloc(sizeof(float) * (size_t)(splits * D));
    float* sc = (float*)malloc(sizeof(float) * (size_t)S);
    int64_t base = S / splits, extra = S % splits, t0 = 0;
    for (int64_t p = 0; p < splits; ++p) {
        int64_t len = base + (p < extra ? 1 : 0);
        float m = -INFINITY;
        for (int64_t t = t0; t < t0 + len; ++t) {
            float acc = 0.0f;
            for (int64_t d = 0; d < D; ++d) acc = acc + Kc[t * D + d] * q[d];
            sc[t] = acc * scale;
            if (sc[t] > m) m = sc[t];
        }
        float l = 0.0f;
        for (int64_t d = 0; d < D; ++d) os[p * D + d] = 0.0f;
        for (int64_t t = t0; t < t0 + len; ++t) {
            float e = expf(sc[t] - m);
            l = l + e;
            for (int64_t d = 0; d < D; ++d) os[p * D + d] = os[p * D + d] + e * Vc[t * D + d];
        }
        ms[p] = m;
        ls[p] = l;
        t0 += len;
    }
    float Mx = -INFINITY;
    for (int64_t p = 0; p < splits; ++p) if (ms[p] > Mx) Mx = ms[p];
    float den = 0.0f;
    for (int64_t p = 0; p < splits; ++p) {
        float w = expf(ms[p] - Mx);
        den = den + w * ls[p];
        for (int64_t d = 0; d < D; ++d) num[d] = num[d] + w * os[p * D + d];
    }
    for (int64_t d = 0; d < D; ++d) out[d] = num[d] / den;
    free(num); free(ms); free(ls); free(os); free(sc);
}

/* Element-wise oracle_bf16_rne over an array (tests round many values). */
void oracle_bf16_rne_array(const double* x, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}

/* Thread count of the OpenMP loops over independent outputs, for timing the
 * oracle on one core or on all of them; no result depends on it.  n < 1
 * leaves it unchanged.  Returns the count now in force. */
int oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
