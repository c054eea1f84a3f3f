// Causal prefill attention over a paged KV cache with the KV split at a fixed
// length of 4096 tokens (the deterministic-inference handbook page, section
// "与 batch 无关：固定切分": attention splits KV by a fixed token count, 4096 for
// prefill, never by a count of parts chosen from the load; chunked prefill and
// the prefix cache must leave a request's attention unchanged).
//
// Request b owns query rows cu_q[b] .. cu_q[b+1]-1 of q [total_q, H, D]; row
// cu_q[b] + j sits at position pos = q_pos0[b] + j and attends to the
// request's keys 0 .. pos, key t in page table[b][t >> log2p], slot
// t & (P - 1) of the caches [num_pages, H, P, D].  The keys are cut into
// chunks [4096c, 4096c + 4096); chunk c of a query yields the triple
//     m_c = max_t x_t,  l_c = sum_t 2^(x_t - m_c),  o_c = sum_t 2^(x_t - m_c) v_t
// with x_t = (q . k_t) * (scale * log2 e) (the base-2 form of the softmax), and
// the triples are merged in ascending chunk order:
//     M = max_c m_c,  out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
// Every step of a query's arithmetic is a function of its position and the
// keys alone, never of the other queries in its tile or batch: so a prompt
// prefilled in one call, in several chunks, or after a prefix-cache hit gives
// the same bits for each query.
//
// Kernel 1, one workgroup of 8 waves per (chunk, request, 256-query tile,
// head); wave w owns 32 queries.  The chunk's keys advance in blocks of 64
// through a 3-stage LDS ring (K and V, 32 KiB per stage), copied HBM -> LDS by
// global_load_lds_dwordx4 two blocks ahead of use.  Per block and wave:
//   * S^T = K Q^T on the MFMA (v_mfma_f32_32x32x16_bf16, D/16 slices in
//     ascending d): lane l then holds query l % 32 and 32 of the 64 keys, so a
//     query's maximum and sum are a lane's own values plus one exchange with
//     lane l ^ 32;
//   * online softmax within the chunk with a reference m that moves only when
//     the block maximum exceeds it by more than 8 (m' = block max then, else
//     m' = m, so every 2^(x - m') < 2^8): l' = l * 2^(m - m') + sum 2^(x - m'),
//     o' = o * 2^(m - m') + P V, keys of the block in a fixed order,
//     2^(x - m') evaluated as 2^fma(q.k, c, -m'); masked keys (t > pos) give
//     exactly 0.  The chunk triple is then (m, l, o) for a reference m at most
//     the chunk maximum, which the merge takes as it takes the maximum;
//   * O^T += V^T P^T on the MFMA, P^T straight from the score registers as
//     two bfloat16 terms (hi = bf16(p), lo = bf16(p - hi); two MFMAs, so p
//     enters the binary32 sums to about 2^-17), V^T read with
//     ds_read_b64_tr_b16 (gfx950's transposing LDS read).  The MFMA's 16-key slices take the keys of a lane
//     half in the order the score registers hold them, so V's rows sit in LDS
//     with bits 2 and 3 of the key index swapped.
// A query with one chunk (pos < 4096) writes out = o / l itself (the merge of
// one triple gives these bits); others write their triples to ws
// [chunk][H][total_q][4 + D], and kernel 2 merges them.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int PF_CHUNK = 4096;
constexpr int PF_KB = 64;                  // keys per block
constexpr int PF_WAVES = 8;
constexpr int PF_QT = PF_WAVES * 32;       // queries per tile
constexpr int PF_THREADS = PF_WAVES * 64;
constexpr int PF_NSTAGE = 4;

typedef __attribute__((address_space(3))) void pf_lds_t;
typedef short pf_v4i16_t __attribute__((ext_vector_type(4)));

struct PfArgs {
    const uint16_t* q;
    const uint8_t* kc;
    const uint8_t* vc;
    const int32_t* table;
    const int32_t* cu_q;
    const int32_t* q_pos0;
    float* ws;
    void* out;
    int64_t total_q, max_pages;
    int B, H, log2p, num_pages, max_q, max_kv, ntiles;
    float cscale;   // scale * log2(e)
};

// Geometry of request b, device values clamped into range: rows
// [r0, r0 + n) of q; query j at position min(p0 + j, max_kv - 1).
struct PfReq {
    int64_t r0;
    int n, p0;
};
__device__ __forceinline__ PfReq pf_request(const PfArgs& a, int b) {
    PfReq r;
    const int64_t lo = min(max((int64_t)a.cu_q[b], (int64_t)0), a.total_q);
    const int64_t hi = min(max((int64_t)a.cu_q[b + 1], lo), a.total_q);
    r.r0 = lo;
    r.n = (int)min(hi - lo, (int64_t)a.max_q);
    r.p0 = min(max(a.q_pos0[b], 0), a.max_kv - 1);
    return r;
}

// s_waitcnt vmcnt(V) with expcnt and lgkmcnt left free (gfx9 encoding).
template <int V>
__device__ __forceinline__ void pf_wait_vm() {
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}

// s_waitcnt lgkmcnt(min(N, 15)) (the counter has 4 bits; waiting for fewer
// outstanding reads than asked is still safe), tied to the register `v` that
// the caller is about to use, so no use of v can be scheduled before it.
template <int N, class T>
__device__ __forceinline__ void pf_wait_lgkm(T& v) {
    constexpr int n = N < 15 ? N : 15;
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(n));
}
// LDS fragment reads as inline assembly: the compiler would otherwise wait for
// every copy still in flight into the ring (it cannot tell the stages apart)
// before each read.  Their results are waited for explicitly (pf_wait_lgkm);
// volatile asm statements keep their order, and LDS reads complete in order.
template <int OFF>
__device__ __forceinline__ u32x4_t pf_read128(uint32_t addr) {
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
typedef uint32_t pf_u32x2_t __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ pf_u32x2_t pf_read_tr(uint32_t addr) {
    pf_u32x2_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int I, int N, class F>
__device__ __forceinline__ void pf_static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        pf_static_for<I + 1, N>(f);
    }
}

// The value of lane l and of lane l ^ 32, as a pair in either order
// (v_permlane32_swap, one instruction; max and sum of the pair are symmetric).
__device__ __forceinline__ float pf_max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pf_sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int pf_swap23(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D, int OUT_BF16>
__global__ void __launch_bounds__(PF_THREADS)
prefill_chunk_kernel(PfArgs a) {
    constexpr int ROWB = D * 2;                // bytes of one K or V row
    constexpr int BLK = PF_KB * ROWB;          // one K (or V) block
    constexpr int STAGE = 2 * BLK;
    constexpr int NS = D / 16;                 // 16-wide d slices of S^T
    constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
    static_assert(D == 128, "LDS swizzles below assume 256-byte rows");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[PF_NSTAGE * STAGE];
    __shared__ int pids[PF_CHUNK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;

    // Workgroup -> (chunk c, request b, tile t, head h); heads fastest, so
    // that the round-robin dealing of workgroups to the 8 XCDs keeps every
    // tile of a head on one XCD (its K and V shared in that L2); the causal
    // tiles with the most keys first.
    int wi = blockIdx.x;
    const int h = wi % a.H;
    wi /= a.H;
    const int t = a.ntiles - 1 - wi % a.ntiles;
    wi /= a.ntiles;
    const int b = wi % a.B;
    const int c = wi / a.B;

    const PfReq rq = pf_request(a, b);
    const int q_lo = t * PF_QT;
    if (q_lo >= rq.n) return;
    const int q_hi = min(q_lo + PF_QT, rq.n) - 1;
    const int pos_hi = min(rq.p0 + q_hi, a.max_kv - 1);
    const int kc0 = c * PF_CHUNK;
    if (kc0 > pos_hi) return;
    const int kend = min(kc0 + PF_CHUNK, pos_hi + 1);     // keys [kc0, kend)
    const int nblk = (kend - kc0 + PF_KB - 1) / PF_KB;

    // Page ids of the chunk's keys (ids outside the cache read page 0).
    const int pfirst = kc0 >> a.log2p;
    const int np = ((kend - 1) >> a.log2p) - pfirst + 1;
    const int32_t* trow = a.table + (int64_t)b * a.max_pages + pfirst;
    for (int i = tid; i < np; i += PF_THREADS) {
        const int pg = trow[i];
        pids[i] = (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
    }
    __syncthreads();

    // This lane's query (rows past the request read its last row and are
    // not written) and the wave's position range.
    const int wq0 = q_lo + 32 * wave;
    const bool wave_on = wq0 < rq.n;
    const int qi = wq0 + (lane & 31);
    const bool q_ok = qi < rq.n;
    const int64_t row = rq.r0 + min(qi, rq.n - 1);
    const int pos = min(rq.p0 + min(qi, rq.n - 1), a.max_kv - 1);
    const int wpos_lo = min(rq.p0 + min(wq0, rq.n - 1), a.max_kv - 1);
    const int wpos_hi = min(rq.p0 + min(wq0 + 31, rq.n - 1), a.max_kv - 1);

    // Q as the B operand of S^T: lane l holds q[l % 32][16s + 8 hl .. + 7].
    u32x4_t qf[NS];
    {
        const uint16_t* qrow = a.q + (row * a.H + h) * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4_t*)(qrow + 16 * s);
    }

    // K block in LDS: row = key (256 bytes), 16-byte chunk c at c ^ (row & 15).
    // V block: row rho holds key swap23(rho), chunk c at c ^ 4 (rho & 3).
    const int pmask = (1 << a.log2p) - 1;
    // The lane's row and chunk are recomputed from an opaque copy of the lane
    // id at each call, so that none of the address arithmetic is kept live
    // across the block loop (registers are the limit there).
    auto copy_block = [&](int j, int st) {
        const int kbase = kc0 + j * PF_KB;
        uint8_t* kdst = smem + st * STAGE;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int p = ln & 15;
        const int g16 = 16 * (wave >> 1);   // the 16-row group holding the wave's K and V rows
        if (a.log2p >= 4 && kbase + g16 + 15 < kend) {
            // Pages of 16 or more tokens start at multiples of 16, so the
            // group's 16 keys lie in one page: the page and the group's first
            // row are wave-uniform, and a lane adds only its row within the
            // group and its 16-byte chunk (32-bit offsets from a scalar base).
            const int key0 = kbase + g16;
            const int pg = __builtin_amdgcn_readfirstlane(pids[(key0 >> a.log2p) - pfirst]);
            const int64_t row0 = (((int64_t)pg * a.H + h) << a.log2p) + (key0 & pmask);
            const uint8_t* kb = a.kc + row0 * ROWB;
            const uint8_t* vb = a.vc + row0 * ROWB;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rho = 8 * wave + 4 * i + (ln >> 4);
                const uint32_t rk = rho & 15, rv = pf_swap23(rho) & 15;
                __builtin_amdgcn_global_load_lds((const void*)(kb + (rk * ROWB + ((p ^ rk) << 4))),
                                                 (pf_lds_t*)(kdst + (8 * wave + 4 * i) * ROWB), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void*)(vb + (rv * ROWB + ((p ^ (4 * (rho & 3))) << 4))),
                                                 (pf_lds_t*)(kdst + BLK + (8 * wave + 4 * i) * ROWB), 16, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rho = 8 * wave + 4 * i + (ln >> 4);
            {
                const int key = min(kbase + rho, kend - 1);
                const int pg = pids[(key >> a.log2p) - pfirst];
                const uint8_t* src = a.kc + ((((int64_t)pg * a.H + h) << a.log2p) + (key & pmask)) * ROWB +
                                     ((p ^ (rho & 15)) << 4);
                __builtin_amdgcn_global_load_lds((const void*)src, (pf_lds_t*)(kdst + (8 * wave + 4 * i) * ROWB),
                                                 16, 0, 0);
            }
            {
                const int key = min(kbase + pf_swap23(rho), kend - 1);
                const int pg = pids[(key >> a.log2p) - pfirst];
                const uint8_t* src = a.vc + ((((int64_t)pg * a.H + h) << a.log2p) + (key & pmask)) * ROWB +
                                     ((p ^ (4 * (rho & 3))) << 4);
                __builtin_amdgcn_global_load_lds((const void*)src,
                                                 (pf_lds_t*)(kdst + BLK + (8 * wave + 4 * i) * ROWB), 16, 0, 0);
            }
        }
    };

    // Per-lane LDS offsets of the fragments.
    //  K (srcA of S^T): row 32 kb + l % 32, chunk (2s + hl) ^ (l & 15).
    //  V^T (srcA of O^T, transposing reads): within a 16-lane group g, lane li
    //  addresses row 8 hl + (li >> 2) (+ 4 for the second half of the 8 keys,
    //  + 16 per 16-key slice) and the 8 bytes of d block db at chunk
    //  4 (db ^ (li >> 2)) + 2 (g & 1) + ((li & 3) >> 1), half li & 1.
    // K fragment s: row l % 32, chunk (2s | hl) ^ (l & 15) = (2s ^ (l & 14)) | (hl ^ (l & 1)),
    // i.e. byte offset k0 + ((32 s) ^ ke).  V^T fragment db: v0 + ((64 db) ^ vz).
    // (Two registers per operand instead of one per fragment.)
    const uint32_t k0 = (lane & 31) * ROWB + ((hl ^ (lane & 1)) << 4);
    const uint32_t ke = (lane & 14) << 4;
    uint32_t v0, vz;
    {
        const int g = lane >> 4, li = lane & 15, z = li >> 2;
        v0 = BLK + (8 * hl + z) * ROWB + ((2 * (g & 1) + ((li & 3) >> 1)) << 4) + (li & 1) * 8;
        vz = z << 6;
    }

    const uint32_t lds0 = (uint32_t)(size_t)((const __attribute__((address_space(3))) uint8_t*)smem);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;

    // Blocks 0 .. nlive - 1 of the chunk hold keys that precede the wave's
    // last query; the wave skips the others.
    const int nlive = !wave_on || wpos_hi < kc0 ? 0 : min(nblk, (wpos_hi - kc0) / PF_KB + 1);
    f32x16_t sacc[2];        // S^T of a block, from its S^T products to its softmax step
    u32x4_t pb[4], pl[4];    // P^T of a block (hi and lo terms), from its softmax step to its P.V products

    // S^T = K Q^T of block i.
    auto qk = [&](int i) {
        const uint32_t sk = lds0 + (i % PF_NSTAGE) * STAGE + k0;
        u32x4_t kf[2][NS];
        pf_static_for<0, 2 * NS>([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            kf[k / NS][k % NS] = pf_read128<(k / NS) * 32 * ROWB>(sk + (((k % NS) << 5) ^ ke));
        });
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
        pf_static_for<0, 2 * NS>([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            pf_wait_lgkm<2 * NS - 1 - k>(kf[k / NS][k % NS]);
            sacc[k / NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[k / NS][k % NS]),
                                                                   as_bf16x8(qf[k % NS]), sacc[k / NS], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // O^T += V^T P^T of block i over its 4 slices of 16 keys.
    auto pv = [&](int i) {
        const uint32_t sv = lds0 + (i % PF_NSTAGE) * STAGE + v0;
        pf_u32x2_t vf[NDB][4][2];
        pf_static_for<0, NDB * 8>([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            constexpr int db = k / 8, u = (k / 2) % 4, hr = k % 2;
            vf[db][u][hr] = pf_read_tr<u * 16 * ROWB + hr * 4 * ROWB>(sv + ((db << 6) ^ vz));
        });
        pf_static_for<0, NDB * 4>([&](auto ic) {
            constexpr int k = decltype(ic)::value, db = k / 4, u = k % 4;
            pf_wait_lgkm<(NDB * 4 - 1 - k) * 2>(vf[db][u][1]);
            pf_wait_lgkm<(NDB * 4 - 1 - k) * 2>(vf[db][u][0]);
            const u32x4_t v = {vf[db][u][0][0], vf[db][u][0][1], vf[db][u][1][0], vf[db][u][1][1]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v), as_bf16x8(pb[u]), o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v), as_bf16x8(pl[u]), o[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // P.V of block i - 1 with S^T of block i: each K read is issued once a
    // P.V pair has consumed its V^T fragment (reads complete in order; the
    // wait counts include the K reads issued after each pair's V^T reads).
    auto pvqk = [&](int i) {
        const uint32_t sv = lds0 + ((i - 1) % PF_NSTAGE) * STAGE + v0;
        const uint32_t sk = lds0 + (i % PF_NSTAGE) * STAGE + k0;
        pf_u32x2_t vf[NDB][4][2];
        u32x4_t kf[2][NS];
        pf_static_for<0, NDB * 8>([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            constexpr int db = k / 8, u = (k / 2) % 4, hr = k % 2;
            vf[db][u][hr] = pf_read_tr<u * 16 * ROWB + hr * 4 * ROWB>(sv + ((db << 6) ^ vz));
        });
        static_assert(NDB * 4 == 2 * NS, "one K read per P.V pair");
        pf_static_for<0, NDB * 4>([&](auto ic) {
            constexpr int k = decltype(ic)::value, db = k / 4, u = k % 4;
            pf_wait_lgkm<(NDB * 4 - 1 - k) * 2 + k>(vf[db][u][1]);
            pf_wait_lgkm<(NDB * 4 - 1 - k) * 2 + k>(vf[db][u][0]);
            const u32x4_t v = {vf[db][u][0][0], vf[db][u][0][1], vf[db][u][1][0], vf[db][u][1][1]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v), as_bf16x8(pb[u]), o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v), as_bf16x8(pl[u]), o[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            kf[k / NS][k % NS] = pf_read128<(k / NS) * 32 * ROWB>(sk + (((k % NS) << 5) ^ ke));
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
        pf_static_for<0, 2 * NS>([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            pf_wait_lgkm<2 * NS - 1 - k>(kf[k / NS][k % NS]);
            sacc[k / NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[k / NS][k % NS]),
                                                                   as_bf16x8(qf[k % NS]), sacc[k / NS], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // The online-softmax step of block i.  Key of (kb, r): kbase + 32 kb +
    // 8 (r >> 2) + 4 hl + (r & 3).  The block maximum is taken on the raw dot
    // products and scaled once: c * max(s) = max(c * s) in binary32 (c > 0,
    // rounding is monotonic).  o holds blocks 0 .. i - 1 here.
    auto softmax = [&](int i) {
        const int kbase = kc0 + i * PF_KB;
        // Keys past the query's position: -inf.  Only the blocks that reach
        // past the wave's first position need it; the volatile statement keeps
        // this a branch (selected on every block it would cost ~100
        // instructions).  Key kbase + 4 hl + kr, kr = 32 kb + 8 (r >> 2) + (r & 3).
        if (kbase + PF_KB - 1 > wpos_lo) {
            int lim = pos - kbase - 4 * hl;
            asm volatile("" : "+v"(lim));
            // (lim - kr) < 0 selects -inf through a sign mask and a bitfield
            // insert; the opaque mask keeps the compiler from turning this
            // into 32 compares held in scalar register pairs at once.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    uint32_t m = (uint32_t)((lim - (32 * kb + 8 * (r >> 2) + (r & 3))) >> 31);
                    asm volatile("" : "+v"(m));
                    sacc[kb][r] = __uint_as_float((m & 0xff800000u) | (~m & __float_as_uint(sacc[kb][r])));
                }
        }
        float mb = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mb = fmaxf(mb, sacc[kb][r]);
        mb = pf_max_xor32(mb);
        // The reference m moves only when the block's maximum exceeds it by
        // more than 8 (so every 2^(x - m) stays below 2^8): per query, from its
        // own scores, so the order stays a function of the query alone.
        const float m_blk = mb * a.cscale;
        const float m_new = m_blk > m_run + 8.0f ? m_blk : m_run;
        // No key of the chunk yet (m_new = -inf): subtract 0 instead, so that
        // every 2^(x - m) is 2^-inf = 0 and alpha = 0 (o and l are still 0).
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        // P as two bfloat16 terms, hi = bf16(p) and lo = bf16(p - hi): their
        // products with the bfloat16 V are exact in the binary32 MFMA sums, so
        // P V carries p to about 2^-17 instead of bfloat16's 2^-9.
        // p = 2^(s * c - m) with one rounding (fused multiply-add).
        float ps = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], a.cscale, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], a.cscale, -m_use));
                ps += p0;
                ps += p1;
                const uint32_t hi = pack_bf16x2(p0, p1);
                pb[2 * kb + (r >> 3)][(r & 7) >> 1] = hi;
                pl[2 * kb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0 - bf16lo_to_f32(hi), p1 - bf16hi_to_f32(hi));
            }
        l_run = l_run * alpha + ps;
        // o * 1 = o: skip the rescale when no query of the wave moved its reference.
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
    };

    // Steps i = 0 .. nblk, each two phases separated by workgroup barriers.
    // Waves 0-3 run {P.V of block i - 1, S^T of block i} then the softmax
    // step of block i; waves 4-7 (on the same four SIMDs) run the softmax
    // step of block i - 1 then {P.V of block i - 1, S^T of block i}, one phase
    // behind, so that on each SIMD one wave's softmax overlaps the other's
    // MFMAs.  Block b is copied at the start of step b - 2 into stage b % 4,
    // whose previous block (b - 4) was last read in the second phase of step
    // b - 3, and waited for at the end of step b - 1.  Per query the order of
    // operations is that of a plain loop over blocks (S^T, softmax step,
    // o = o * alpha + P V), whatever the phase offset.  Each group's steps are
    // straight-line code (first block, full steps, the last P.V, then steps
    // with no live block), so no score or P register is live where it is not used.
    auto begin = [&](int i) {
        if (i + 2 < nblk) copy_block(i + 2, (i + 2) % PF_NSTAGE);
    };
    auto mid = [&]() { __builtin_amdgcn_s_barrier(); };
    // Block i + 1 landed (block i + 2's four copies may still fly).
    auto end = [&](int i) {
        if (i + 2 < nblk) pf_wait_vm<4>();
        else              pf_wait_vm<0>();
        __builtin_amdgcn_s_barrier();
    };
    copy_block(0, 0);
    if (nblk > 1) copy_block(1, 1);
    if (nblk > 1) pf_wait_vm<4>();
    else          pf_wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    int i = 0;
    if (wave < PF_WAVES / 2) {
        if (nlive > 0) {
            begin(0); qk(0); mid(); softmax(0); end(0);
            for (i = 1; i < nlive; ++i) { begin(i); pvqk(i); mid(); softmax(i); end(i); }
            begin(i); pv(i - 1); mid(); end(i); ++i;
        }
    } else {
        if (nlive > 0) {
            begin(0); mid(); qk(0); end(0);
            for (i = 1; i < nlive; ++i) { begin(i); softmax(i - 1); mid(); pvqk(i); end(i); }
            begin(i); softmax(i - 1); mid(); pv(i - 1); end(i); ++i;
        }
    }
    for (; i <= nblk; ++i) { begin(i); mid(); end(i); }

    // ---- results of this chunk for the queries that have keys in it
    if (!wave_on) return;
    const float l_tot = pf_sum_xor32(l_run);
    if (!q_ok || pos < kc0) return;
    const int nch = pos / PF_CHUNK + 1;
    // The query's row again, from an opaque lane id, so that the 64-bit row
    // is not kept live across the block loop.
    int ln_o = lane;
    asm volatile("" : "+v"(ln_o));
    const int64_t row_o = rq.r0 + min(wq0 + (ln_o & 31), rq.n - 1);
    if (nch == 1) {
        // out[row][h][d], d = 32 db + 8 (r >> 2) + 4 hl + (r & 3).
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t e = (row_o * a.H + h) * D + 32 * db + 8 * g + 4 * hl;
                f32x4_t v;
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = o[db][4 * g + k] / l_tot;
                if constexpr (OUT_BF16) {
                    typedef uint32_t u32x2_t_ __attribute__((ext_vector_type(2)));
                    *(u32x2_t_*)((uint16_t*)a.out + e) = u32x2_t_{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {
                    *(f32x4_t*)((float*)a.out + e) = v;
                }
            }
    } else {
        // Triple row [m, l, -, -, o[0 .. D)] of this (chunk, head, query).
        float* w = a.ws + (((int64_t)c * a.H + h) * a.total_q + row_o) * (4 + D);
        if (hl == 0) *(f32x4_t*)w = f32x4_t{m_run, l_tot, 0.0f, 0.0f};
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(f32x4_t*)(w + 4 + 32 * db + 8 * g + 4 * hl) =
                    f32x4_t{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    }
}

// Merge of the chunk triples of the queries with more than one chunk, in
// ascending chunk order: M = max m_c, den = sum 2^(m_c - M) l_c,
// num_d = sum 2^(m_c - M) o_c[d], out_d = num_d / den.  One thread per (query
// row, head, 4 consecutive d); the request of a row is found by bisection of
// cu_q.  Triple rows are [m, l, -, -, o[0 .. D)] (ws [chunk][H][total_q][4 + D]).
template <int D, int OUT_BF16>
__global__ void __launch_bounds__(256)
prefill_merge_kernel(PfArgs a) {
    constexpr int Q4 = D / 4;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= a.total_q * a.H * Q4) return;
    const int d4 = (int)(i % Q4);
    const int64_t rh = i / Q4;
    const int h = (int)(rh % a.H);
    const int64_t row = rh / a.H;
    // request of this row: the last b with cu_q[b] <= row (clamped as in kernel 1)
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (min(max((int64_t)a.cu_q[mid], (int64_t)0), a.total_q) <= row) lo = mid;
        else hi = mid - 1;
    }
    const PfReq rq = pf_request(a, lo);
    const int64_t qi = row - rq.r0;
    if (qi < 0 || qi >= rq.n) return;
    const int pos = min(rq.p0 + (int)qi, a.max_kv - 1);
    const int nch = pos / PF_CHUNK + 1;
    if (nch == 1) return;
    const int64_t cstride = (int64_t)a.H * a.total_q * (4 + D);
    const float* w = a.ws + ((int64_t)h * a.total_q + row) * (4 + D);
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, w[c * cstride]);
    f32x4_t num = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
    for (int c = 0; c < nch; ++c) {
        const float* wc = w + c * cstride;
        const float f = __builtin_amdgcn_exp2f(wc[0] - M);
        den = fmaf(f, wc[1], den);
        const f32x4_t ov = *(const f32x4_t*)(wc + 4 + 4 * d4);
#pragma unroll
        for (int k = 0; k < 4; ++k) num[k] = fmaf(f, ov[k], num[k]);
    }
    f32x4_t v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = num[k] / den;
    const int64_t e = (row * a.H + h) * D + 4 * d4;
    if constexpr (OUT_BF16) {
        typedef uint32_t u32x2_t_ __attribute__((ext_vector_type(2)));
        *(u32x2_t_*)((uint16_t*)a.out + e) = u32x2_t_{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
        *(f32x4_t*)((float*)a.out + e) = v;
    }
}

}  // namespace bi
