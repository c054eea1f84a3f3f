// Fixed-length split-KV decode attention (flash decoding with chunks of a
// fixed token count), after the deterministic-inference handbook page
// (anrans.github.io), section "根源：浮点加法的顺序" and its batch-invariance
// rules: the KV sequence of each (b, h) is cut into chunks of DEC_CHUNK tokens
// counted from position 0, each chunk yields the triple
//     m_c = max_t s_t,  l_c = sum_t exp(s_t - m_c),  o_c = sum_t exp(s_t - m_c) v_t,
// with s_t = scale * (q . k_t), and the triples are merged in ascending chunk
// order by the log-sum-exp rule.  Nothing depends on B: the chunking, the
// per-chunk reduction trees and the merge order are functions of S and D only.
//
// Kernel 1 (one workgroup of 8 waves per (b, h, chunk); 256 tokens per wave):
//   lanes are grouped by LPT = D/8 lanes per token, each lane holding 8 of the
//   D dimensions (one 16-byte load of a K or V row); a wave load covers
//   64/LPT consecutive tokens = 1 KiB of contiguous HBM.
//   * q . k_t: 8 fused multiply-adds per lane (dimension ascending), then a
//     xor-butterfly over the LPT lanes of the token (identical bits in each).
//   * m_c: exact maximum (order-free) over the wave and then the 8 waves.
//   * p_t = expf(s_t - m_c); l and o: each lane folds its tokens in ascending
//     order, then a xor-butterfly over the token groups of the wave, then the
//     8 wave partials are added in wave order.  l and o use the same tree, so
//     V = 1 gives o_c = l_c bit for bit.
// Kernel 2 (one lane per (b, h, d)): M = max_c m_c, w_c = expf(m_c - M),
//   num = sum_c w_c o_c[d], den = sum_c w_c l_c (c ascending, same operation
//   for both), out = num / den (IEEE division).
#pragma once

#include "common.hpp"
#include "rowio.hpp"

namespace bi {

constexpr int DEC_CHUNK = 2048;
constexpr int DEC_WAVES = 8;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_TOK_PER_WAVE = DEC_CHUNK / DEC_WAVES;   // 256

// `chunk` is the chunk length in tokens (a multiple of 8, at most DEC_CHUNK);
// the product path always passes DEC_CHUNK.  Wave w of chunk c owns tokens
// [c*chunk + w*chunk/8, c*chunk + (w+1)*chunk/8).
template <int D>
__global__ void __launch_bounds__(DEC_THREADS)
decode_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, float* __restrict__ ws,
                    int64_t S, int nchunk, int chunk, float scale) {
    constexpr int LPT = D / 8;               // lanes per token
    constexpr int TPI = 64 / LPT;            // tokens per wave-wide load
    constexpr int NI = DEC_TOK_PER_WAVE / TPI;
    // Loads in flight per lane: all of the wave's K (or V) loads for D = 64,
    // half for D = 128 (register budget); one workgroup per CU then keeps
    // 256 KiB of K or V in flight, which hides HBM latency without a second
    // workgroup (whose extra concurrent streams measured slower).
    constexpr int BATCH = NI < 32 ? NI : 32;
    static_assert(NI % BATCH == 0, "tile shape");

    __shared__ float red_m[DEC_WAVES];
    __shared__ float red_l[DEC_WAVES];
    __shared__ float red_o[DEC_WAVES][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPT;              // which 8 dimensions
    const int tg = lane / LPT;               // token slot within a load
    const int64_t bh = blockIdx.x / nchunk;
    const int c = blockIdx.x - (int)(bh * nchunk);
    const int tw = chunk / DEC_WAVES;                       // tokens of this wave
    const int64_t w0 = (int64_t)c * chunk + (int64_t)wave * tw;
    const int64_t t0 = w0 + tg;
    const int64_t t_end = min(S, w0 + tw);

    // K and V rows of this (b, h) as buffers ending at token S: loads need no
    // branch (tokens past S read zero; their scores are masked below) and all
    // of a batch's loads are in flight together.  The host bounds S*D*2 below
    // 2^31.  Loads are non-temporal (K and V are read once).
    const __amdgpu_buffer_rsrc_t rk = row_rsrc(k + (bh * S) * D, S * D * 2);
    const __amdgpu_buffer_rsrc_t rv = row_rsrc(v + (bh * S) * D, S * D * 2);
    const int lane_off = sub * 16;

    float qf[8];
    {
        const u32x4_t qv = *(const u32x4_t*)(q + bh * D + sub * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16lo_to_f32(qv[e]);
            qf[2 * e + 1] = bf16hi_to_f32(qv[e]);
        }
    }

    // ---- scores
    float sc[NI];
    float m = -INFINITY;
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += BATCH) {
        u32x4_t kr[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int t = (int)(t0 + (int64_t)(i0 + b) * TPI);
            kr[b] = __builtin_amdgcn_raw_buffer_load_b128(rk, t * (D * 2) + lane_off, 0, 2);
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(qf[2 * e], bf16lo_to_f32(kr[b][e]), acc);
                acc = fmaf(qf[2 * e + 1], bf16hi_to_f32(kr[b][e]), acc);
            }
#pragma unroll
            for (int o = 1; o < LPT; o <<= 1) acc += __shfl_xor(acc, o, 64);
            const int64_t t = t0 + (int64_t)(i0 + b) * TPI;
            sc[i0 + b] = t < t_end ? acc * scale : -INFINITY;
            m = fmaxf(m, sc[i0 + b]);
        }
    }
    // The first batch of V loads is issued before the chunk maximum (V does
    // not depend on it), so its latency overlaps the cross-wave reduction.
    u32x4_t vr0[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        const int t = (int)(t0 + (int64_t)b * TPI);
        vr0[b] = __builtin_amdgcn_raw_buffer_load_b128(rv, t * (D * 2) + lane_off, 0, 2);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red_m[wave] = m;
    __syncthreads();
    m = red_m[0];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) m = fmaxf(m, red_m[w]);

    // ---- exponentials, their sum and the weighted V sum
    float l = 0.0f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += BATCH) {
        u32x4_t vr[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int t = (int)(t0 + (int64_t)(i0 + b) * TPI);
            vr[b] = i0 == 0 ? vr0[b] : __builtin_amdgcn_raw_buffer_load_b128(rv, t * (D * 2) + lane_off, 0, 2);
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const float pt = expf(sc[i0 + b] - m);
            l = fmaf(pt, 1.0f, l);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = fmaf(pt, bf16lo_to_f32(vr[b][e]), o[2 * e]);
                o[2 * e + 1] = fmaf(pt, bf16hi_to_f32(vr[b][e]), o[2 * e + 1]);
            }
        }
    }
    // Fold the token groups of the wave (lane bits above the LPT lanes).
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
        l += __shfl_xor(l, off, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off, 64);
    }
    if (lane == 0) red_l[wave] = l;
    if (tg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red_o[wave][sub * 8 + e] = o[e];
    }
    __syncthreads();
    // Wave partials in wave order; thread d < D finishes dimension d.
    float* trip = ws + (bh * nchunk + c) * (int64_t)(2 + D);
    if (tid < D) {
        float od = red_o[0][tid];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) od += red_o[w][tid];
        trip[2 + tid] = od;
    }
    if (tid == 0) {
        float lt = red_l[0];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) lt += red_l[w];
        trip[0] = m;
        trip[1] = lt;
    }
}

template <int D, int OUT_BF16>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws, void* __restrict__ out, int64_t BH, int nchunk) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= BH * D) return;
    const int64_t bh = i / D;
    const int d = (int)(i - bh * D);
    const float* tp = ws + bh * nchunk * (int64_t)(2 + D);
    float M = tp[0];
    for (int c = 1; c < nchunk; ++c) M = fmaxf(M, tp[c * (2 + D)]);
    float num = 0.0f, den = 0.0f;
    for (int c = 0; c < nchunk; ++c) {
        const float* t = tp + c * (2 + D);
        const float w = expf(t[0] - M);
        num = fmaf(w, t[2 + d], num);
        den = fmaf(w, t[1], den);
    }
    store_out<OUT_BF16>(out, i, num / den);
}

}  // namespace bi
