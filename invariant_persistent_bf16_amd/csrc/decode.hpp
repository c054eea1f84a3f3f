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
// The same chunk arithmetic serves contiguous caches [B, H, S, D] and paged
// caches [num_pages, H, P, D] with a per-request length (the handbook's
// serving rules, sections "框架里的开关" and "与 batch 无关：固定切分": chunked
// prefill and the prefix cache must not change a request's bits); only the
// address of a token's row differs.
// Kernel 2 (one lane per (b, h, d)): M = max_c m_c, w_c = expf(m_c - M),
//   num = sum_c w_c o_c[d], den = sum_c w_c l_c (c ascending, same operation
//   for both), out = num / den (IEEE division).
#pragma once

#include "common.hpp"
#include "rowio.hpp"
#include "wave.hpp"

namespace bi {

constexpr int DEC_CHUNK = 2048;
constexpr int DEC_WAVES = 8;
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_TOK_PER_WAVE = DEC_CHUNK / DEC_WAVES;   // 256

// Access to the K and V rows of one (b, h): row t as the 16 bytes of this
// lane's 8 dimensions.  Contiguous caches [B, H, S, D]: the rows of (b, h) are
// one buffer ending at token S, so rows past S read zero (their scores are
// masked) with no branch; the host bounds S*D*2 below 2^31.  Loads are
// non-temporal (K and V are read once).
template <int D>
struct DecContigKV {
    static constexpr bool MASK_V = false;
    static constexpr bool FENCE_BATCHES = false;
    static constexpr bool SKIP_EMPTY_WAVES = false;
    __amdgpu_buffer_rsrc_t rk, rv;
    int lane_off;
    __device__ __forceinline__ u32x4_t k(int t) const {
        return __builtin_amdgcn_raw_buffer_load_b128(rk, t * (D * 2) + lane_off, 0, 2);
    }
    __device__ __forceinline__ u32x4_t v(int t) const {
        return __builtin_amdgcn_raw_buffer_load_b128(rv, t * (D * 2) + lane_off, 0, 2);
    }
};

// Paged caches [num_pages, H, P, D] (P = 2^log2p tokens per page): token t of
// the request lives in page table[t >> log2p], slot t & (P - 1).  A token past
// the request's last one (t > tmax) takes the last token's page with its own
// slot: a valid address in the cache whose content is not the request's, so
// its score is masked and its V row replaced by zero (MASK_V), which gives the
// contiguous kernel's bits (there such rows read as zero).  A page id outside
// [0, num_pages) reads page 0 (no access leaves the cache).
//
// A wave-wide load covers the TPI = 512/D consecutive tokens t_l0 + tg (tg =
// lane / (D/8), t_l0 a multiple of TPI); lane l reads dimensions
// (l % (D/8)) * 8 .. + 7 of its token.  The page ids of the wave's 256 tokens
// are read once, before the K loads:
//   UNI (P >= TPI): the load's tokens are consecutive slots of one page, so
//     the address is a scalar (page + slot of t_l0) plus lane * 16 bytes; lane
//     j holds the wave's (j+1)-th page id (at most 64 pages) and the load
//     takes its page from the lane (t_l0's page - first);
//   otherwise (P < TPI): lane l's page is (t_l0 >> log2p) + (tg >> log2p) and
//     its slot tg & (P - 1); the wave's page ids (up to 256) sit in LDS.
// K and V use separate copies of the per-lane values, opaque to the compiler,
// so that a V row's address is recomputed rather than all of the K phase's
// addresses kept live until the V phase.
template <int D, bool UNI>
struct DecPagedKV {
    static constexpr bool MASK_V = true;
    static constexpr bool FENCE_BATCHES = true;
    static constexpr bool SKIP_EMPTY_WAVES = true;
    const uint8_t* kb;   // cache base + h * P * D * 2
    const uint8_t* vb;
    int64_t page_bytes;  // H * P * D * 2
    int tmax, log2p, first, last_rel;
    int lane_page[2];    // UNI: page id of lane j's slot; otherwise tg >> log2p
    uint32_t lane_off[2];    // lane's byte offset from the slot of t_l0 (UNI) or the page
    const int* wave_pages;   // P < TPI: the wave's page ids in LDS

    // Page ids of tokens [w0, w0 + 256) clamped to tmax, from `first` on.
    __device__ __forceinline__ void prepare(const int32_t* __restrict__ table, int num_pages, int64_t w0,
                                            int* lds_wave) {
        const int lane = threadIdx.x & 63;
        const int tg = lane / (D / 8), sub = lane % (D / 8);
        first = (int)(min(w0, (int64_t)tmax) >> log2p);
        const int last = tmax >> log2p;
        last_rel = last - first;
        if constexpr (UNI) {
            const int pg = table[min(first + lane, last)];
            lane_page[0] = (unsigned)pg < (unsigned)num_pages ? pg : 0;
            lane_off[0] = (uint32_t)lane * 16u;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pg = table[min(first + lane + 64 * j, last)];
                lds_wave[lane + 64 * j] = (unsigned)pg < (unsigned)num_pages ? pg : 0;
            }
            wave_pages = lds_wave;
            lane_page[0] = tg >> log2p;
            lane_off[0] = (uint32_t)((tg & ((1 << log2p) - 1)) * (D * 2) + sub * 16);
        }
        lane_page[1] = lane_page[0];
        lane_off[1] = lane_off[0];
        asm volatile("" : "+v"(lane_page[1]), "+v"(lane_off[1]));
    }
    template <int KV>
    __device__ __forceinline__ u32x4_t row(const uint8_t* b, int t) const {
        const int t_l0 = __builtin_amdgcn_readfirstlane(t);   // lane 0 holds the load's first token
        const int rel = (min(t_l0, tmax) >> log2p) - first;
        const uint8_t* p;
        if constexpr (UNI) {
            const int pg = __builtin_amdgcn_readlane(lane_page[KV], rel);
            p = b + (int64_t)pg * page_bytes + (int64_t)((t_l0 & ((1 << log2p) - 1)) * (D * 2));
        } else {
            const int pg = wave_pages[min(rel + lane_page[KV], last_rel)];
            p = b + (int64_t)pg * page_bytes;
        }
        return __builtin_nontemporal_load((const u32x4_t*)(p + lane_off[KV]));
    }
    __device__ __forceinline__ u32x4_t k(int t) const { return row<0>(kb, t); }
    __device__ __forceinline__ u32x4_t v(int t) const { return row<1>(vb, t); }
};

// The triple (m_c, l_c, o_c) of one chunk of one (b, h): wave w owns tokens
// [w0, w0 + tw) with w0 = c*chunk + w*tw, tw = chunk/8; tokens at or past
// t_end are masked.  The arithmetic does not depend on how K and V are stored,
// so a paged request and the same values stored contiguously give the same bits.
// TW: tokens per wave (DEC_TOK_PER_WAVE for every product kernel; a smaller
// TW only serves the benchmark's split-KV comparison, whose parts are shorter).
// STORE_AUX: cache policy of the triple's stores (0 for every product kernel;
// the comparison writes its triples through to memory for another workgroup).
template <int D, int BATCH_MAX, class KV, int TW = DEC_TOK_PER_WAVE, int STORE_AUX = 0>
__device__ __forceinline__ void decode_chunk_body(const KV& kv, const uint16_t* __restrict__ qrow,
                                                  float* __restrict__ trip, int64_t w0, int64_t t_end,
                                                  float scale) {
    constexpr int LPT = D / 8;               // lanes per token
    constexpr int TPI = 64 / LPT;            // tokens per wave-wide load
    constexpr int NI = TW / TPI;
    static_assert(TW % TPI == 0 && TW <= DEC_TOK_PER_WAVE, "tokens per wave");
    // Loads in flight per lane (BATCH_MAX = 32: all of the wave's K (or V)
    // loads for D = 64, half for D = 128, as the register budget allows); one
    // workgroup per CU then keeps 256 KiB of K or V in flight, which hides HBM
    // latency without a second workgroup (whose extra concurrent streams
    // measured slower).  The batch only groups loads: it does not change the
    // arithmetic.
    constexpr int BATCH = NI < BATCH_MAX ? NI : BATCH_MAX;
    static_assert(NI % BATCH == 0, "tile shape");

    __shared__ float red_m[DEC_WAVES];
    __shared__ float red_l[DEC_WAVES];
    __shared__ float red_o[DEC_WAVES][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPT;              // which 8 dimensions
    const int tg = lane / LPT;               // token slot within a load
    const int64_t t0 = w0 + tg;
    // Token t0 + i*TPI is inside the request and the wave's range iff
    // tg < nv - i*TPI (a 32-bit compare with a wave-uniform bound).
    const int nv = __builtin_amdgcn_readfirstlane((int)max(t_end - w0, (int64_t)0));

    float qf[8];
    {
        const u32x4_t qv = *(const u32x4_t*)(qrow + sub * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16lo_to_f32(qv[e]);
            qf[2 * e + 1] = bf16hi_to_f32(qv[e]);
        }
    }

    // ---- scores
    // SKIP_EMPTY_WAVES: a wave with no token of the request (nv == 0: past its
    // end in its last chunk) skips its loads; its partials stay m = -inf,
    // l = 0, o = 0, which is what its masked tokens would give.
    const bool run = !KV::SKIP_EMPTY_WAVES || nv > 0;
    float sc[NI];
    float m = -INFINITY;
    u32x4_t vr0[BATCH];
    if (run) {
#pragma unroll
        for (int i0 = 0; i0 < NI; i0 += BATCH) {
            u32x4_t kr[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) kr[b] = kv.k((int)(t0 + (int64_t)(i0 + b) * TPI));
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = fmaf(qf[2 * e], bf16lo_to_f32(kr[b][e]), acc);
                    acc = fmaf(qf[2 * e + 1], bf16hi_to_f32(kr[b][e]), acc);
                }
                acc = xor_sum_steps<1, LPT>(acc);
                sc[i0 + b] = tg < nv - (i0 + b) * TPI ? acc * scale : -INFINITY;
                m = fmaxf(m, sc[i0 + b]);
            }
            // FENCE_BATCHES: keep the next batch's loads after this batch's use
            // (the register budget holds one batch, not two).
            if constexpr (KV::FENCE_BATCHES && BATCH < NI) __builtin_amdgcn_sched_barrier(0);
        }
        // The first batch of V loads is issued before the chunk maximum (V
        // does not depend on it), so its latency overlaps the cross-wave
        // reduction.
#pragma unroll
        for (int b = 0; b < BATCH; ++b) vr0[b] = kv.v((int)(t0 + (int64_t)b * TPI));
    }
    m = wave_max(m);
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
    if (run) {
#pragma unroll
        for (int i0 = 0; i0 < NI; i0 += BATCH) {
            u32x4_t vr[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                vr[b] = i0 == 0 ? vr0[b] : kv.v((int)(t0 + (int64_t)(i0 + b) * TPI));
                if constexpr (KV::MASK_V)
                    if (tg >= nv - (i0 + b) * TPI) vr[b] = u32x4_t{0u, 0u, 0u, 0u};
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
            if constexpr (KV::FENCE_BATCHES && BATCH < NI) __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Fold the token groups of the wave (lane bits above the LPT lanes).
    l = xor_sum_steps<LPT, 64>(l);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = xor_sum_steps<LPT, 64>(o[e]);
    if (lane == 0) red_l[wave] = l;
    if (tg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red_o[wave][sub * 8 + e] = o[e];
    }
    __syncthreads();
    // Wave partials in wave order; thread d < D finishes dimension d.
    auto put = [&](int i, float x) {
        if constexpr (STORE_AUX == 0) {
            trip[i] = x;
        } else {
            const __amdgpu_buffer_rsrc_t rt = row_rsrc(trip, (2 + D) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rt, 4 * i, 0, STORE_AUX);
        }
    };
    if (tid < D) {
        float od = red_o[0][tid];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) od += red_o[w][tid];
        put(2 + tid, od);
    }
    if (tid == 0) {
        float lt = red_l[0];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) lt += red_l[w];
        put(0, m);
        put(1, lt);
    }
}

// Contiguous caches.  `chunk` is the chunk length in tokens (a multiple of 8,
// at most DEC_CHUNK); the product path always passes DEC_CHUNK.  Workgroup
// (bh, c) writes triple bh * nchunk + c of ws.
template <int D>
__global__ void __launch_bounds__(DEC_THREADS)
decode_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, float* __restrict__ ws,
                    int64_t S, int nchunk, int chunk, float scale) {
    const int64_t bh = blockIdx.x / nchunk;
    const int c = blockIdx.x - (int)(bh * nchunk);
    const int tw = chunk / DEC_WAVES;
    const int64_t w0 = (int64_t)c * chunk + (int64_t)(threadIdx.x >> 6) * tw;
    DecContigKV<D> kv;
    kv.rk = row_rsrc(k + (bh * S) * D, S * D * 2);
    kv.rv = row_rsrc(v + (bh * S) * D, S * D * 2);
    kv.lane_off = (threadIdx.x & 63) % (D / 8) * 16;
    decode_chunk_body<D, 32>(kv, q + bh * D, ws + (bh * nchunk + c) * (int64_t)(2 + D), w0,
                         min(S, w0 + tw), scale);
}

// Paged caches with per-request lengths.  Grid: B * H * maxchunks workgroups
// (workgroup c * B * H + bh: chunk c of (b, h) = bh), maxchunks =
// ceil(max_seq / DEC_CHUNK); request b's length is seq_lens[b]
// clamped to [0, max_seq] and its chunks c >= ceil(len / DEC_CHUNK) exit at
// once.  Chunk boundaries are absolute multiples of DEC_CHUNK, so a request
// gives the bits of the contiguous kernel with S = its length, whatever the
// other requests, the table's width or the page placement.
template <int D, bool UNI>
__global__ void __launch_bounds__(DEC_THREADS)
decode_chunk_paged_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                          const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table,
                          int64_t max_pages, const int32_t* __restrict__ seq_lens, int H,
                          int log2p, int num_pages, int max_seq, int maxchunks, int BH,
                          float* __restrict__ ws, float scale) {
    // Chunk-major order: consecutive workgroups are different (b, h) of the
    // same chunk index.  Workgroups are dealt round-robin to the XCDs, so with
    // (b, h)-major order XCD x would get only chunk indices c = x mod
    // maxchunks, and the XCDs holding the late chunks (absent for short
    // requests) would idle while the others do all the work.
    const int c = blockIdx.x / BH;
    const int64_t bh = blockIdx.x - (int64_t)c * BH;
    const int64_t b = bh / H;
    const int h = (int)(bh - b * H);
    const int len = min(max(seq_lens[b], 0), max_seq);
    if ((int64_t)c * DEC_CHUNK >= len) return;   // whole workgroup
    constexpr int TW = DEC_CHUNK / DEC_WAVES;
    const int64_t w0 = (int64_t)c * DEC_CHUNK + (int64_t)(threadIdx.x >> 6) * TW;
    const int64_t head_bytes = ((int64_t)D * 2) << log2p;
    DecPagedKV<D, UNI> kv;
    kv.kb = (const uint8_t*)kc + h * head_bytes;
    kv.vb = (const uint8_t*)vc + h * head_bytes;
    kv.page_bytes = head_bytes * H;
    kv.tmax = len - 1;
    kv.log2p = log2p;
    if constexpr (UNI) {
        kv.prepare(block_table + b * max_pages, num_pages, w0, nullptr);
    } else {
        __shared__ int pages[DEC_WAVES][DEC_CHUNK / DEC_WAVES];
        kv.prepare(block_table + b * max_pages, num_pages, w0, pages[threadIdx.x >> 6]);
        __syncthreads();
    }
    // Page addressing takes registers: smaller load batches where needed.
    decode_chunk_body<D, UNI ? (D == 64 ? 32 : 16) : 16>(kv, q + bh * D, ws + (bh * maxchunks + c) * (int64_t)(2 + D), w0,
                         min((int64_t)len, w0 + TW), scale);
}

// Merge of the chunk triples of each (b, h), `stride` triples apart per
// (b, h).  Contiguous: nchunk triples each.  Paged (seq_lens != null): request
// b has ceil(len_b / DEC_CHUNK) of them, len_b clamped as in the chunk kernel;
// a request of length 0 gets 0/0 = NaN.
template <int D, int OUT_BF16>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws, void* __restrict__ out, int64_t BH, int stride,
                    const int32_t* __restrict__ seq_lens, int H, int max_seq) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= BH * D) return;
    const int64_t bh = i / D;
    const int d = (int)(i - bh * D);
    int n = stride;
    if (seq_lens) n = (min(max(seq_lens[bh / H], 0), max_seq) + DEC_CHUNK - 1) / DEC_CHUNK;
    const float* tp = ws + bh * stride * (int64_t)(2 + D);
    float M = -INFINITY;
    for (int c = 0; c < n; ++c) M = fmaxf(M, tp[c * (2 + D)]);
    float num = 0.0f, den = 0.0f;
    for (int c = 0; c < n; ++c) {
        const float* t = tp + c * (2 + D);
        const float w = expf(t[0] - M);
        num = fmaf(w, t[2 + d], num);
        den = fmaf(w, t[1], den);
    }
    store_out<OUT_BF16>(out, i, num / den);
}

}  // namespace bi
