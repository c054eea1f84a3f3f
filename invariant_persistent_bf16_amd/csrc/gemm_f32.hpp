// Persistent binary32 GEMM for gfx950: C = A @ B (+ bias) on the fp32 matrix
// cores (v_mfma_f32_16x16x4f32), binary32 operands, binary32 accumulation.
//
// The binary32 configuration of the persistent matmul: each output element
// is reduced over 4-wide K slices (one v_mfma_f32_16x16x4f32 each; lane l
// supplies k = l / 16 of each slice for both operands) by four accumulation
// chains: slice j goes to chain j mod 4, each chain adds its slices in
// ascending order starting from zero, and the chains are summed as
// ((c0 + c1) + c2) + c3 at the end; then the bias is added once.  The order
// is a function of K alone (never of M, the tile or the grid).  Rows/columns
// past M/N read from clamped addresses and are never stored, the K tail is
// zero-filled (a zero slice leaves a chain unchanged).  Operands keep their
// binary32 precision: nothing is rounded to a narrower type.  Three kernels
// run this same per-element arithmetic and give the same bits; the host
// picks by shape: 64x64 outputs per workgroup (each of 4 waves a 32x32 block
// as 2x2 MFMA blocks of 16x16, its four chains interleaved), 32x32 (each wave
// one 16x16 block) where the 64x64 tiles would leave most compute units idle,
// and gemm_f32_split_chains below (one 16x16 block per workgroup, one chain
// per wave) where even the 32x32 tiles would.  Four chains make an
// element's dependent MFMA sequence K/16 steps long instead of K/4.
//
// Operands may have any element strides (the loads are 4-byte buffer loads
// coalesced along whichever stride is 1), so transposed views need no copy.
// Loads run three K steps ahead of their LDS store in four register sets,
// issued unconditionally (past the last step they re-read it), so the
// compiler's waits cover exactly the set being stored; each element's byte
// offset from the tile's first row (column) is fixed per tile and a step
// moves the wave-uniform base.  The 64x64 tile without a K tail fits 256
// registers per lane, so two of its workgroups share a compute unit (the
// grid is up to four workgroups per CU).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int G32_BM = 64;   // the large tile; the small one is 32x32
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

// Buffer loads: a wave-uniform base in the descriptor, 32-bit byte offsets
// per lane; an offset of GS32_OOB (past the 2^31 - 1 byte record count)
// reads zero.
constexpr uint32_t GS32_OOB = 0x80000000u;  // buffer offset that reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gs32_rsrc(const float* base) {
    const uint64_t v = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, 0x7fffffff, 0x00020000);
}

// WT: rows (and columns) of one wave's block, 32 (2x2 MFMA blocks, 64x64
// tile) or 16 (one MFMA block, 32x32 tile); p.tiles_* count tiles of 2 WT.
template <int OUT_BF16, bool KTAIL, int WT = 32>
__global__ void __launch_bounds__(G32_THREADS)
gemm_f32_persistent(GemmF32Params p) {
    constexpr int BM = 2 * WT, BN = 2 * WT;
    constexpr int NB = WT / 16;                        // MFMA blocks per wave side
    constexpr int NE = BM * G32_BK / G32_THREADS;      // elements per thread per operand and step
    // LDS holds A as [k][m] and B as [k][n] so that the 16 lanes feeding one
    // MFMA operand read 16 consecutive words.
    __shared__ float sA[2][G32_BK][BM + 4];
    __shared__ float sB[2][G32_BK][BN + 4];

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
        const int64_t m0 = (int64_t)pid_m * BM, n0 = (int64_t)pid_n * BN;
        const float* Ab = p.A + s1 * p.sA1 + s2 * p.sA2;
        const float* Bb = p.B + s1 * p.sB1 + s2 * p.sB2;

        // acc[c]: chain c (4-wide K slices c, c + 4, c + 8, ...).
        f32x4_t acc[4][NB][NB];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                for (int bj = 0; bj < NB; ++bj) acc[c][bi][bj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

        // Loads run three K steps ahead of their LDS store: step j's operands
        // go to register set j % 4, issued at the start of step j - 3.  Every
        // step issues its loads (past the last step they re-read it, unused),
        // so the code is straight-line and each store waits only for its own
        // set.
        float ra[4][NE], rb[4][NE];
        // Per element of the thread's share of a step: its byte offset from
        // the tile's first row (column) at the step's first k, fixed for the
        // tile (32-bit: the host bounds 64 rows and 32 k of the strides below
        // 2^31 bytes); a step moves the wave-uniform base by k0 times the K
        // stride.  Rows and columns past M / N read clamped addresses (never
        // stored); KTAIL (K not a multiple of the step): k >= K gets the
        // out-of-range offset and reads zero.
        const float* At = Ab + m0 * p.sAm;
        const float* Bt = Bb + n0 * p.sBn;
        uint32_t oa[NE], ob[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int idx = tid + G32_THREADS * i;
            const int mm = a_kfast ? idx / G32_BK : idx % BM;
            const int ka = a_kfast ? idx % G32_BK : idx / BM;
            const int nn = b_kfast ? idx / G32_BK : idx % BN;
            const int kb = b_kfast ? idx % G32_BK : idx / BN;
            oa[i] = (uint32_t)((min(m0 + mm, p.M - 1) - m0) * p.sAm + (int64_t)ka * p.sAk) * 4u;
            ob[i] = (uint32_t)((min(n0 + nn, p.N - 1) - n0) * p.sBn + (int64_t)kb * p.sBk) * 4u;
        }
        auto load_tile = [&](int kt, auto uc) {
            constexpr int u = decltype(uc)::value;
            const int k0 = min(kt, nk - 1) * G32_BK;
            const __amdgpu_buffer_rsrc_t rA = gs32_rsrc(At + (int64_t)k0 * p.sAk);
            const __amdgpu_buffer_rsrc_t rB = gs32_rsrc(Bt + (int64_t)k0 * p.sBk);
            // only the last step has a K tail; the others load unchecked (the
            // branch is uniform and both sides issue the same loads in order)
            const int kl = KTAIL && k0 + G32_BK > p.K ? (int)p.K - k0 : G32_BK;
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int ka = a_kfast ? idx % G32_BK : idx / BM;
                ra[u][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rA, !KTAIL || ka < kl ? oa[i] : GS32_OOB, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int kb = b_kfast ? idx % G32_BK : idx / BN;
                rb[u][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rB, !KTAIL || kb < kl ? ob[i] : GS32_OOB, 0, 0));
            }
        };
        auto store_tile = [&](int kt, auto uc) {
            constexpr int u = decltype(uc)::value, st = u & 1;
            // past the last step the stored values belong to a stage that is
            // never read again; the K tail already reads zero
            (void)kt;
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int mm = a_kfast ? idx / G32_BK : idx % BM;
                const int ka = a_kfast ? idx % G32_BK : idx / BM;
                sA[st][ka][mm] = ra[u][i];
            }
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int idx = tid + G32_THREADS * i;
                const int nn = b_kfast ? idx / G32_BK : idx % BN;
                const int kb = b_kfast ? idx % G32_BK : idx / BN;
                sB[st][kb][nn] = rb[u][i];
            }
        };
        // Block (bi, bj) of the wave: rows wm WT + 16 bi .., columns wn WT + 16 bj ..;
        // lane l feeds row (column) l % 16 with k = 4 ks + l / 16.
        auto compute_tile = [&](int st) {
#pragma unroll
            for (int ks = 0; ks < G32_BK / 4; ++ks) {
                const int k = ks * 4 + (lane >> 4);
                float a[NB], b[NB];
#pragma unroll
                for (int bi = 0; bi < NB; ++bi) a[bi] = sA[st][k][wm * WT + 16 * bi + (lane & 15)];
#pragma unroll
                for (int bj = 0; bj < NB; ++bj) b[bj] = sB[st][k][wn * WT + 16 * bj + (lane & 15)];
                // slice kt * 8 + ks: chain ks % 4 (the step holds 8 slices)
                const int c = ks & 3;
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < NB; ++bj)
                        acc[c][bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[bi], b[bj], acc[c][bi][bj], 0, 0, 0);
            }
        };
        // Step t (set u = t % 4, LDS stage t % 2): loads of step t + 3 into set
        // (u + 3) % 4, the MFMAs of step t, the store of step t + 1, barrier.
        auto step = [&](int t, auto uc) {
            constexpr int u = decltype(uc)::value;
            load_tile(t + 3, std::integral_constant<int, (u + 3) % 4>{});
            // keep the loads at the top of the step (the scheduler would sink
            // them below the MFMAs, leaving two steps instead of three to
            // cover their latency)
            __builtin_amdgcn_sched_barrier(0);
            compute_tile(u & 1);
            store_tile(t + 1, std::integral_constant<int, (u + 1) % 4>{});
            __syncthreads();
        };

        if (nk > 0) {
            load_tile(0, std::integral_constant<int, 0>{});
            load_tile(1, std::integral_constant<int, 1>{});
            load_tile(2, std::integral_constant<int, 2>{});
            store_tile(0, std::integral_constant<int, 0>{});
            __syncthreads();
            // Four steps per trip (register sets are named statically), then the
            // remaining zero to three steps.  The last step's store (of step nk)
            // writes zeros into a stage that is not read again.
            int t = 0;
            for (; t + 4 <= nk; t += 4) {
                step(t, std::integral_constant<int, 0>{});
                step(t + 1, std::integral_constant<int, 1>{});
                step(t + 2, std::integral_constant<int, 2>{});
                step(t + 3, std::integral_constant<int, 3>{});
            }
            if (t < nk) step(t, std::integral_constant<int, 0>{});
            if (t + 1 < nk) step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < nk) step(t + 2, std::integral_constant<int, 2>{});
        }

        // Lane l, register r of block (bi, bj): row 16 bi + 4 (l / 16) + r,
        // column 16 bj + l % 16 of the wave's block.
        void* Cb = (OUT_BF16 ? (void*)((uint16_t*)p.C + s1 * p.sC1 + s2 * p.sC2)
                             : (void*)((float*)p.C + s1 * p.sC1 + s2 * p.sC2));
        const float* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) {
            const int64_t col = n0 + wn * WT + 16 * bj + (lane & 15);
            const float bv = (bb && !p.bias_rows && col < p.N) ? bb[col] : 0.0f;
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m0 + wm * WT + 16 * bi + 4 * (lane >> 4) + r;
                    if (row < p.M && col < p.N) {
                        float v = ((acc[0][bi][bj][r] + acc[1][bi][bj][r]) + acc[2][bi][bj][r]) + acc[3][bi][bj][r];
                        if (bb) v += p.bias_rows ? bb[row] : bv;
                        store_out<OUT_BF16>(Cb, row * p.sCm + col, v);
                    }
                }
        }
    }
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void gs32_static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        gs32_static_for<N, I + 1>(f);
    }
}

// The same per-element arithmetic for products too small to fill the
// compute units with 32x32 tiles (a few rows times a narrow weight): one
// workgroup per 16x16 output block, wave c running chain c (slices c, c + 4,
// c + 8, ... in ascending order from zero), so four waves share an output
// block's K work instead of one wave running all four chains.  At the end
// the four chains meet in LDS and wave 0 forms ((c0 + c1) + c2) + c3, adds
// the bias once and stores.  The slices a chain owns and their order depend
// on K alone, so the bits are those of gemm_f32_persistent for every M.
//
// K runs in stages of GS32_KS.  An operand in its usual layout is staged:
// the workgroup fetches the stage's 16 x GS32_KS block of A (k contiguous)
// or GS32_KS x 16 block of B (columns contiguous) with one 16-byte load per
// lane and piece, stores it to LDS, and each wave reads its chain's words
// there.  Otherwise (ASTAGE / BSTAGE false: other strides or alignments)
// each wave loads its own MFMA operands with 4-byte loads (lane l: row or
// column l % 16, k = 4j + l / 16 of slice j).  A 4-byte load costs about as
// much issue time as a 16-byte one, so staging cuts the load instructions
// per stage from 4 * GS32_KS / 16 to GS32_KS / 16 per operand and
// workgroup.  The loads run GS32_SETS - 1 stages ahead in as many register
// sets; staged data goes to LDS two stages ahead and is read from LDS one
// stage ahead (two slots, one barrier per stage), both under the MFMAs of
// the current stage.  Loads past K, staged pieces of rows past M and of
// columns past N get an out-of-range offset and read zero; direct loads of
// rows and columns past M / N read clamped addresses.  Those rows and
// columns only feed outputs that are never stored.  The last stage runs all
// of its GS32_KS / 16 MFMAs per wave, the slices past K being zero (a zero
// slice leaves a chain unchanged, as in the K tail of the tiled kernels).
// Byte offsets are 32-bit (the host only picks this kernel when 15 rows plus
// K + 512 steps of the strides stay below 2^31 bytes).
constexpr int GS32_KS = 128;               // k per stage
constexpr int GS32_SETS = 8;               // register sets (even: the LDS slot is the set's parity)
constexpr int GS32_MIX = 8;                // MFMAs of a stage followed by a share of its memory instructions

template <int OUT_BF16, bool ASTAGE, bool BSTAGE, int KS = GS32_KS, int R = GS32_SETS>
__global__ void __launch_bounds__(256)
gemm_f32_split_chains(GemmF32Params p) {
    static_assert(R % 2 == 0 && R >= 4, "the LDS slot of stage t is t % 2 = (t % R) % 2; stores run 2 stages ahead");
    constexpr int MIX = GS32_MIX < KS / 16 ? GS32_MIX : KS / 16;   // MFMAs followed by a memory share
    constexpr int AP = KS + 4;            // A's LDS row pitch in words (row m starts at bank 4m)
    constexpr int NJ = KS / 16;           // MFMAs per wave and stage
    constexpr int APR = KS / 4;           // 16-byte pieces of A per row and stage
    constexpr int NA = ASTAGE ? 16 * APR / 256 : NJ;   // A loads per thread and stage
    constexpr int NB = BSTAGE ? KS * 4 / 256 : NJ;     // B loads per thread and stage
    static_assert(16 * APR % 256 == 0 && KS * 4 % 256 == 0, "stage shape");
    __shared__ float sA[ASTAGE ? 2 : 1][ASTAGE ? 16 : 1][ASTAGE ? AP : 1];
    __shared__ float sB[BSTAGE ? 2 : 1][BSTAGE ? KS : 1][16];
    __shared__ f32x4_t part[3][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's chain
    const int blocks_n = (int)((p.N + 15) / 16);
    const int blocks_m = (int)((p.M + 15) / 16);
    const int per_slice = blocks_m * blocks_n;
    const int blk = blockIdx.x;
    const int s = blk / per_slice;
    const int t0 = blk - s * per_slice;
    const int64_t m0 = (int64_t)(t0 / blocks_n) * 16, n0 = (int64_t)(t0 % blocks_n) * 16;
    const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
    const __amdgpu_buffer_rsrc_t rsA = gs32_rsrc(p.A + s1 * p.sA1 + s2 * p.sA2 + m0 * p.sAm);
    const __amdgpu_buffer_rsrc_t rsB = gs32_rsrc(p.B + s1 * p.sB1 + s2 * p.sB2 + n0 * p.sBn);
    const int K = (int)p.K;
    const int nk = (K + KS - 1) / KS;
    // The lane's k within slice c (its k in slice 4i + c is k0 + 16 i, and
    // i = NJ t + jj in stage t) and the first i past K.
    const int k0 = 4 * c + (lane >> 4);
    const int ilim = k0 < K ? (K - k0 + 15) / 16 : 0;

    // Per-thread byte offsets (the stage adds a uniform offset).  Staged A:
    // piece q = 256 r + tid is row q / APR, k 4 (q % APR) of the stage.
    // Staged B: piece q is k row q / 4 of the stage, columns 4 (q % 4) ...
    // Direct: the lane's row (column) and k0.
    // Rows past M are never stored and only feed their own output rows, so
    // their staged pieces are not fetched (zeros instead of clamped copies).
    uint32_t aoff[ASTAGE ? NA : 1], boff[BSTAGE ? NB : 1];
    int bkrow[BSTAGE ? NB : 1];
    uint32_t va = 0, vb = 0;
    const int apiece = tid % APR;
    if constexpr (ASTAGE) {
#pragma unroll
        for (int r = 0; r < NA; ++r)
            aoff[r] = m0 + (256 * r + tid) / APR < p.M
                          ? (uint32_t)(((256 * r + tid) / APR) * p.sAm * 4 + 16 * apiece) : GS32_OOB;
    } else {
        va = (uint32_t)((min(m0 + (lane & 15), p.M - 1) - m0) * p.sAm + (int64_t)k0 * p.sAk) * 4u;
    }
    if constexpr (BSTAGE) {
        const bool col_ok = n0 + 4 * (tid & 3) < p.N;
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            bkrow[r] = (256 * r + tid) >> 2;
            boff[r] = col_ok ? (uint32_t)(bkrow[r] * p.sBk * 4 + 16 * (tid & 3)) : GS32_OOB;
        }
    } else {
        vb = (uint32_t)((min(n0 + (lane & 15), p.N - 1) - n0) * p.sBn + (int64_t)k0 * p.sBk) * 4u;
    }
    const uint32_t stepA = 64u * (uint32_t)p.sAk, stepB = 64u * (uint32_t)p.sBk;

    typedef std::conditional_t<ASTAGE, f32x4_t, float> ta_t;
    typedef std::conditional_t<BSTAGE, f32x4_t, float> tb_t;
    ta_t ra[R][NA];
    tb_t rb[R][NB];
    // The memory instructions of a stage, one per item: NLD loads (A's
    // first), NST LDS stores of staged pieces, NRD LDS reads of staged words.
    constexpr int NLD = NA + NB;
    constexpr int NST = (ASTAGE ? NA : 0) + (BSTAGE ? NB : 0);
    constexpr int NRD = (ASTAGE ? NJ : 0) + (BSTAGE ? NJ : 0);
    auto load_item = [&](int t, auto uc, auto ic) {
        constexpr int u = decltype(uc)::value, i = decltype(ic)::value;
        // the stage is wave-uniform; readfirstlane keeps its offsets in SGPRs
        const uint32_t tc = (uint32_t)__builtin_amdgcn_readfirstlane(min(t, nk));
        if constexpr (i < NA) {
            if constexpr (ASTAGE)
                ra[u][i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    rsA, t * KS + 4 * apiece < K ? aoff[i] : GS32_OOB, tc * (KS * 4), 0));
            else
                ra[u][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rsA, NJ * t + i < ilim ? va : GS32_OOB, (tc * NJ + i) * stepA, 0));
        } else {
            constexpr int r = i - NA;
            if constexpr (BSTAGE)
                rb[u][r] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    rsB, t * KS + bkrow[r] < K ? boff[r] : GS32_OOB, tc * (KS * 4) * (uint32_t)p.sBk, 0));
            else
                rb[u][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rsB, NJ * t + r < ilim ? vb : GS32_OOB, (tc * NJ + r) * stepB, 0));
        }
    };
    auto store_item = [&](int slot, auto uc, auto ic) {
        constexpr int u = decltype(uc)::value, i = decltype(ic)::value;
        if constexpr (ASTAGE && i < NA) {
            *(f32x4_t*)&sA[slot][(256 * i + tid) / APR][4 * apiece] = ra[u][i];
        } else if constexpr (BSTAGE) {
            constexpr int r = ASTAGE ? i - NA : i;
            *(f32x4_t*)&sB[slot][bkrow[r]][4 * (tid & 3)] = rb[u][r];
        }
    };
    // a staged stage's words, read from LDS one step before its MFMAs
    float av[2][ASTAGE ? NJ : 1], bv[2][BSTAGE ? NJ : 1];
    auto read_item = [&](int slot, auto vc, auto ic) {
        constexpr int v = decltype(vc)::value, i = decltype(ic)::value;
        if constexpr (ASTAGE && i < NJ) {
            av[v][i] = sA[slot][lane & 15][16 * i + k0];
        } else if constexpr (BSTAGE) {
            constexpr int jj = ASTAGE ? i - NJ : i;
            bv[v][jj] = sB[slot][16 * jj + k0][lane & 15];
        }
    };
    auto load = [&](int t, auto uc) { gs32_static_for<NLD>([&](auto ic) { load_item(t, uc, ic); }); };
    auto store = [&](int slot, auto uc) { gs32_static_for<NST>([&](auto ic) { store_item(slot, uc, ic); }); };
    auto read = [&](int slot, auto vc) { gs32_static_for<NRD>([&](auto ic) { read_item(slot, vc, ic); }); };
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto mfma = [&](auto uc, auto jc) {
        constexpr int u = decltype(uc)::value, v = u & 1, jj = decltype(jc)::value;
        float a, b;
        if constexpr (ASTAGE) a = av[v][jj]; else a = ra[u][jj];
        if constexpr (BSTAGE) b = bv[v][jj]; else b = rb[u][jj];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    };
    // Step t (u = t % R; stage s lives in register set s % R and LDS slot
    // s % 2): read stage t + 1's words from LDS, store stage t + 2's staged
    // pieces into the slot stage t has left (its words were read in step
    // t - 1, before that step's barrier), issue the loads of stage t + R - 1,
    // run the MFMAs of stage t (words read one step earlier, or the direct
    // loads of set u), barrier.  A wave issues in order and each MFMA waits
    // for the one before it, so the memory instructions go between the first
    // GS32_MIX MFMAs, a share after each, and run under the chain; a store
    // waits for loads issued R - 3 steps earlier.  The loop runs whole groups
    // of R steps; in the steps past the last stage only the MFMAs are
    // skipped (loads read zeros, stores go to slots that are not read
    // again), so every group is the same straight-line code and the register
    // sets stay in place across the loop.
    auto memory_share = [&](int t, auto uc, auto gc) {
        constexpr int u = decltype(uc)::value, g = decltype(gc)::value;
        gs32_static_for<NRD>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i * MIX / NRD == g) read_item((u + 1) & 1, std::integral_constant<int, (u + 1) & 1>{}, ic);
        });
        gs32_static_for<NST>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i * MIX / NST == g) store_item(u & 1, std::integral_constant<int, (u + 2) % R>{}, ic);
        });
        gs32_static_for<NLD>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i * MIX / NLD == g) load_item(t + R - 1, std::integral_constant<int, (u + R - 1) % R>{}, ic);
        });
    };
    auto step = [&](int t, auto uc) {
        if (t < nk) {
            gs32_static_for<NJ>([&](auto jc) {
                constexpr int jj = decltype(jc)::value;
                mfma(uc, jc);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (jj < MIX) {
                    memory_share(t, uc, jc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        } else {
            gs32_static_for<MIX>([&](auto gc) { memory_share(t, uc, gc); });
        }
        __syncthreads();
    };
    gs32_static_for<R - 1>([&](auto uc) { load(decltype(uc)::value, uc); });
    store(0, std::integral_constant<int, 0>{});
    store(1, std::integral_constant<int, 1>{});
    __syncthreads();
    read(0, std::integral_constant<int, 0>{});
    __syncthreads();   // stage 0's words are in registers before step 0 stores over them
    for (int t = 0; t < nk; t += R)
        gs32_static_for<R>([&](auto uc) { step(t + decltype(uc)::value, uc); });

    if (c > 0) part[c - 1][lane] = acc;
    __syncthreads();
    if (c == 0) {
        const f32x4_t c1 = part[0][lane], c2 = part[1][lane], c3 = part[2][lane];
        // Lane l, register r: row 4 (l / 16) + r, column l % 16 of the block.
        void* Cb = (OUT_BF16 ? (void*)((uint16_t*)p.C + s1 * p.sC1 + s2 * p.sC2)
                             : (void*)((float*)p.C + s1 * p.sC1 + s2 * p.sC2));
        const float* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
        const int64_t col = n0 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + 4 * (lane >> 4) + r;
            if (row < p.M && col < p.N) {
                float v = ((acc[r] + c1[r]) + c2[r]) + c3[r];
                if (bb) v += p.bias_rows ? bb[row] : bb[col];
                store_out<OUT_BF16>(Cb, row * p.sCm + col, v);
            }
        }
    }
}

}  // namespace bi
