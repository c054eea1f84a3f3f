// Persistent bfloat16 GEMM for gfx950 (CDNA4): C = A @ B (+ bias), binary32
// accumulation on the matrix cores.
//
// Batch invariance (the property of the persistent matmul in "Unmasking the
// True Culprit ...", section "Why This Achieves Batch Invariance": fixed block
// sizes, each output tile reduced inside one core, the same K order, no
// split-K) holds here by construction:
//   * one tile shape and one K step for every call (constants below);
//   * output element (i, j) is accumulated by a single chain of
//     v_mfma_f32_32x32x16_bf16 instructions, one per 16-wide K slice, K
//     ascending, starting from zero; its operands are row i of A and column j
//     of B only, so neither the other rows of the tile nor M, the slice count
//     or the grid can change its bits;
//   * rows past M, columns past N and K past K are loaded as zeros (or, for
//     columns of an N-contiguous B, from the last valid column) and never
//     stored; zero K terms are exact;
//   * the bias (if any) is added once to the finished binary32 sum, then the
//     value is rounded once to the output dtype.
//
// Hardware mapping.  A 256x256 output tile per workgroup of 4 waves (2x2),
// each wave owning 128x128 = 4x4 MFMA blocks of 32x32 (256 binary32
// accumulators per lane, held in AGPRs).  Operand tiles of 64 K-elements are
// copied HBM -> LDS by buffer_load_dwordx4 ... lds (no staging registers;
// a lane whose 16 bytes fall outside the operand gets an out-of-range offset
// and the hardware writes zeros), double buffered (2 x 64 KiB).
// LDS holds [A stage 0 | A stage 1 | B stage 0 | B stage 1], 32 KiB each.
//   * A, and a K-contiguous B: LDS rows of 128 bytes (64 K values of one M row
//     or N column); the eight 16-byte chunks of row r sit at chunk c ^ s(r),
//     s(r) = (r ^ r>>3) & 7, so the 16-byte fragment reads of neighbouring
//     lanes fall in distinct banks.  Fragments are ds_read_b128.
//   * an N-contiguous B (a [K, N] weight): LDS rows of 512 bytes (256 N values
//     of one K row), chunk c of row k at c ^ 4(k & 3).  Fragments are built by
//     two ds_read_b64_tr_b16 (gfx950's transposing LDS read: within a group of
//     16 lanes, lane t receives element t%4 of the 8 bytes addressed by lanes
//     4j + t/4, j = 0..3), giving each lane 8 consecutive K values of its N
//     column: the MFMA B operand, without a VALU transpose.
// The persistent grid is min(tiles, compute units); workgroup w is renumbered
// so that the 8 XCDs (which receive workgroups round-robin) each work on a
// compact 2-D block of tiles, sharing A and B panels in that XCD's L2.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int G16_BM = 256;
constexpr int G16_BN = 256;
constexpr int G16_BK = 64;
constexpr int G16_THREADS = 256;
constexpr int G16_GROUP_M = 8;
constexpr int G16_STAGE_BYTES = G16_BM * G16_BK * 2;   // one operand tile: 32 KiB
constexpr int G16_LDS_BYTES = 4 * G16_STAGE_BYTES;     // {A, B} x 2 stages: 128 KiB
constexpr uint32_t G16_OOB = 0x80000000u;              // buffer offset that reads as zero
constexpr int32_t G16_RECORDS = 0x7fffffff;

struct GemmParams {
    const uint16_t* A;     // element (i, k) at A[i*sAm + k]
    const uint16_t* B;     // element (k, j) at B[k*sBk + j*sBn]
    const uint16_t* bias;  // [N] (or [M] if bias_rows) or nullptr
    void* C;               // element (i, j) at C[i*sCm + j]
    int64_t M, N, K;
    int64_t sAm, sBk, sBn, sCm;
    // Slice s in [0, G1*G2): s1 = s / G2, s2 = s % G2; operand offsets
    // s1*sX1 + s2*sX2 (elements).  bias offset s2*sBias2.
    int64_t G2;
    int64_t sA1, sA2, sB1, sB2, sC1, sC2, sBias2;
    int tiles_m, tiles_n, tiles_per_slice, total_tiles;
    int bias_rows;         // 1: bias indexed by row (conv output channel), 0: by column
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Buffer descriptor of a wave-uniform base address (kept in SGPRs).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t g16_rsrc(const void* base) {
    const uint64_t v = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    void* u = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, G16_RECORDS, 0x00020000);
}
// 64 lanes x 16 bytes: lane L's bytes [base + voff, +16) land at lds + 16 L.
__device__ __forceinline__ void g16_dma(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ int g16_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Scheduling hint for one 16-MFMA slice: one MFMA, then one LDS read, NDS
// times; then the remaining MFMAs (orders instructions only).
template <int NDS>
__device__ __forceinline__ void g16_interleave() {
#pragma unroll
    for (int q = 0; q < NDS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16 - NDS, 0);
}

template <bool B_KCONTIG, int OUT_BF16>
__global__ void __launch_bounds__(G16_THREADS, 1)
gemm_bf16_persistent(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G16_LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index as a scalar so that LDS destinations are wave-uniform.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (int)((p.K + G16_BK - 1) / G16_BK);
    const int K32 = (int)p.K;   // the host bounds K below 2^31

    const int grid = gridDim.x;
    const int w = blockIdx.x;
    const int wr = (grid % 8 == 0) ? (w % 8) * (grid / 8) + (w / 8) : w;

    // Per-lane LDS fragment bases (see load_frags).
    const uint8_t* a_fb[4];
    const uint8_t* b_fb[4];
    {
        const int R0 = wm * 128 + (lane & 31);
        const int x = (lane >> 5) ^ g16_swz(R0);
#pragma unroll
        for (int j = 0; j < 4; ++j) a_fb[j] = smem + R0 * 128 + ((x ^ (2 * j)) << 4);
        if constexpr (B_KCONTIG) {
            const int N0 = wn * 128 + (lane & 31);
            const int xb = (lane >> 5) ^ g16_swz(N0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b_fb[j] = smem + 2 * G16_STAGE_BYTES + N0 * 128 + ((xb ^ (2 * j)) << 4);
        } else {
            const int g = lane >> 4, li = lane & 15, z = li >> 2;
            const int y = 2 * (g & 1) + ((li & 3) >> 1);
#pragma unroll
            for (int in = 0; in < 4; ++in)
                b_fb[in] = smem + 2 * G16_STAGE_BYTES + (8 * (g >> 1) + z) * 512 +
                           (16 * wn + 4 * (in ^ z) + y) * 16 + (li & 1) * 8;
        }
    }

    for (int tile = wr; tile < p.total_tiles; tile += grid) {
        // ---- tile coordinates (scheduling only; no effect on arithmetic)
        const int s = tile / p.tiles_per_slice;
        const int t = tile - s * p.tiles_per_slice;
        const int width = G16_GROUP_M * p.tiles_n;
        const int first_m = (t / width) * G16_GROUP_M;
        const int gsz = min(p.tiles_m - first_m, G16_GROUP_M);
        const int pid_m = first_m + (t % width) % gsz;
        const int pid_n = (t % width) / gsz;
        const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
        const int64_t m0 = (int64_t)pid_m * G16_BM, n0 = (int64_t)pid_n * G16_BN;
        const uint16_t* Ab = p.A + s1 * p.sA1 + s2 * p.sA2 + m0 * p.sAm;
        const uint16_t* Bb;
        if constexpr (B_KCONTIG) Bb = p.B + s1 * p.sB1 + s2 * p.sB2 + n0 * p.sBn;
        else                     Bb = p.B + s1 * p.sB1 + s2 * p.sB2 + n0;

        // ---- DMA source offsets (bytes, relative to the k-tile base; 32-bit,
        // the host guarantees every in-tile offset is below 2^31).  They are
        // recomputed in every K step from two per-lane values (cheaper than
        // keeping sixteen offsets live through the K loop).
        // A (and K-contiguous B): wave w, copy i covers LDS rows 64w + 8i + lane/8;
        // the lane writes physical chunk lane&7, i.e. logical chunk
        // (lane&7) ^ s(row) = (lane&7) ^ (lane/8) ^ i.
        // N-contiguous B: copy i covers K rows 16w + 2i + lane/32; the lane
        // writes physical chunk lane&31 of that row, i.e. logical chunk
        // (lane&31) ^ 4(krow&3) (krow&3 = 2(i&1) + lane/32), clamped to the
        // last valid 8 columns.
        const int r_lo = lane >> 3;
        const int u_lo = (lane & 7) ^ r_lo;
        const int a_row0 = 64 * wave + r_lo;
        const int a_rows_left = (int)min<int64_t>(p.M - m0 - a_row0, 1 << 20);
        const int a_rowstep = (int)p.sAm * 16;                 // bytes per 8 rows
        const int a_base = a_row0 * (int)p.sAm * 2;
        int b_rows_left = 0, b_rowstep = 0, b_base = 0, ncl = 0;
        const int bn_krow0 = 16 * wave + (lane >> 5);
        if constexpr (B_KCONTIG) {
            b_rows_left = (int)min<int64_t>(p.N - n0 - a_row0, 1 << 20);
            b_rowstep = (int)p.sBn * 16;
            b_base = a_row0 * (int)p.sBn * 2;
        } else {
            b_rowstep = (int)p.sBk * 4;                         // bytes per 2 K rows
            b_base = bn_krow0 * (int)p.sBk * 2;
            ncl = (int)min<int64_t>(p.N - 8 - n0, 248);
        }

        f32x16_t acc[4][4];
#pragma unroll
        for (int im = 0; im < 4; ++im)
#pragma unroll
            for (int in = 0; in < 4; ++in)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[im][in][r] = 0.0f;

        auto issue_tile = [&](int kt, int stage) {
            const int64_t k0 = (int64_t)kt * G16_BK;
            uint8_t* sA = smem + stage * G16_STAGE_BYTES;
            uint8_t* sB = smem + (2 + stage) * G16_STAGE_BYTES;
            const int kleft = min(K32 - (int)k0, G16_BK);   // K values left in this tile
            int ab = a_base, ul = u_lo;
            asm volatile("" : "+v"(ab), "+v"(ul));          // recompute offsets in this step
            const __amdgpu_buffer_rsrc_t ra = g16_rsrc(Ab + k0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c8 = (ul ^ i) << 3;
                const bool ok = a_rows_left > 8 * i && c8 < kleft;
                g16_dma(ra, sA + (wave * 8 + i) * 1024, ok ? (uint32_t)(ab + i * a_rowstep + c8 * 2) : G16_OOB);
            }
            int bb0 = b_base;
            asm volatile("" : "+v"(bb0));
            if constexpr (B_KCONTIG) {
                const __amdgpu_buffer_rsrc_t rb = g16_rsrc(Bb + k0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c8 = (ul ^ i) << 3;
                    const bool ok = b_rows_left > 8 * i && c8 < kleft;
                    g16_dma(rb, sB + (wave * 8 + i) * 1024, ok ? (uint32_t)(bb0 + i * b_rowstep + c8 * 2) : G16_OOB);
                }
            } else {
                const __amdgpu_buffer_rsrc_t rb = g16_rsrc(Bb + k0 * p.sBk);
                const int p31 = lane & 31, hi = lane >> 5;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int col = min((p31 ^ (4 * (2 * (i & 1) + hi))) << 3, ncl);
                    const bool ok = bn_krow0 + 2 * i < kleft;
                    g16_dma(rb, sB + (wave * 8 + i) * 1024, ok ? (uint32_t)(bb0 + i * b_rowstep + col * 2) : G16_OOB);
                }
            }
        };

        // Fragment loads from LDS.  Every address is one of eight per-lane
        // bases plus a compile-time offset (stage, kk, im / hr):
        //  A row r = R0 + 32 im, R0 = 128 wm + lane%32: s(r) = s(R0) ^ 4(im&1),
        //  so chunk (2kk + lane/32) ^ s(r) = x ^ 2(kk ^ 2(im&1)), x = lane/32 ^ s(R0).
        //  N-contiguous B: K row kk*16 + 8(g/2) + 4hr + z (z = li/4, so k&3 = z),
        //  chunk (16wn + 4in + y) ^ 4z = 16wn + 4(in ^ z) + y.
        auto load_a = [&](int stage, int kk, u32x4_t (&af)[4]) {
#pragma unroll
            for (int im = 0; im < 4; ++im)
                af[im] = *(const u32x4_t*)(a_fb[kk ^ (2 * (im & 1))] + stage * G16_STAGE_BYTES + im * 4096);
        };
        auto load_b = [&](int stage, int kk, u32x4_t (&bfr)[4]) {
            if constexpr (B_KCONTIG) {
#pragma unroll
                for (int in = 0; in < 4; ++in)
                    bfr[in] = *(const u32x4_t*)(b_fb[kk ^ (2 * (in & 1))] + stage * G16_STAGE_BYTES + in * 4096);
            } else {
#pragma unroll
                for (int in = 0; in < 4; ++in) {
                    v4i16_t h[2];
#pragma unroll
                    for (int hr = 0; hr < 2; ++hr)
                        h[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_v4i16_t*)(b_fb[in] + stage * G16_STAGE_BYTES + kk * 8192 + hr * 2048));
                    bfr[in] = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
        };
        auto mfma_slice = [&](const u32x4_t (&af)[4], const u32x4_t (&bfr)[4]) {
#pragma unroll
            for (int im = 0; im < 4; ++im)
#pragma unroll
                for (int in = 0; in < 4; ++in)
                    acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(af[im]), as_bf16x8(bfr[in]), acc[im][in], 0, 0, 0);
        };

        // K loop.  Per K step of 64: the DMA of the next tile is issued, then
        // four 16-wide K slices run, the fragments of slice kk+1 being read
        // from LDS while the 16 MFMAs of slice kk execute.  With an
        // N-contiguous B all B fragments of the step are read before the DMA
        // is issued (the transposing reads must not be ordered after an LDS
        // DMA the compiler cannot tell apart from them).
        if (nk > 0) {
            issue_tile(0, 0);
            __builtin_amdgcn_s_waitcnt(0);     // DMA into LDS complete (vmcnt 0)
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const int st = kt & 1;
                u32x4_t af[2][4];
                if constexpr (B_KCONTIG) {
                    u32x4_t bfr[2][4];
                    load_a(st, 0, af[0]);
                    load_b(st, 0, bfr[0]);
                    if (kt + 1 < nk) issue_tile(kt + 1, st ^ 1);
#pragma unroll
                    for (int kk = 0; kk < G16_BK / 16; ++kk) {
                        if (kk + 1 < G16_BK / 16) {
                            load_a(st, kk + 1, af[(kk + 1) & 1]);
                            load_b(st, kk + 1, bfr[(kk + 1) & 1]);
                        }
                        mfma_slice(af[kk & 1], bfr[kk & 1]);
                        if (kk + 1 < G16_BK / 16) g16_interleave<8>();
                    }
                } else {
                    u32x4_t bfr[G16_BK / 16][4];
                    load_a(st, 0, af[0]);
#pragma unroll
                    for (int kk = 0; kk < G16_BK / 16; ++kk) load_b(st, kk, bfr[kk]);
                    if (kt + 1 < nk) issue_tile(kt + 1, st ^ 1);
#pragma unroll
                    for (int kk = 0; kk < G16_BK / 16; ++kk) {
                        if (kk + 1 < G16_BK / 16) load_a(st, kk + 1, af[(kk + 1) & 1]);
                        mfma_slice(af[kk & 1], bfr[kk]);
                        if (kk + 1 < G16_BK / 16) g16_interleave<4>();
                    }
                }
                // Keep every MFMA of the step ahead of the wait for the DMA.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
        }

        // ---- epilogue: + bias (binary32, once), round once, store.
        // Addresses: a wave-uniform base (this wave's 128x128 block) plus
        // 32-bit lane offsets (the host bounds 128 * sCm below 2^31).
        {
            using OutT = typename std::conditional<OUT_BF16 != 0, uint16_t, float>::type;
            const int64_t row_w = m0 + wm * 128, col_w = n0 + wn * 128;
            OutT* Cw = (OutT*)p.C + s1 * p.sC1 + s2 * p.sC2 + row_w * p.sCm + col_w;
            const int sCm = (int)p.sCm;
            const int rows_valid = (int)min<int64_t>(p.M - row_w, 128);
            const int cols_valid = (int)min<int64_t>(p.N - col_w, 128);
            // An opaque copy of the lane id keeps every epilogue value below
            // from being computed before the K loop (where it would stay live).
            int lane_e = lane;
            asm volatile("" : "+v"(lane_e));
            const int lrow = 4 * (lane_e >> 5), lcol = lane_e & 31;
            const uint16_t* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
            const bool brow = bb && p.bias_rows, bcol = bb && !p.bias_rows;
            float bv[4];
#pragma unroll
            for (int in = 0; in < 4; ++in) {
                const int cc = min(in * 32 + lcol, cols_valid - 1);
                bv[in] = bcol ? bf16_to_f32(bb[col_w + cc]) : 0.0f;
            }
#pragma unroll
            for (int im = 0; im < 4; ++im)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = im * 32 + 8 * (r >> 2) + (r & 3) + lrow;
                    if (rr < rows_valid) {
                        const float rb = brow ? bf16_to_f32(bb[row_w + rr]) : 0.0f;
#pragma unroll
                        for (int in = 0; in < 4; ++in) {
                            const int cc = in * 32 + lcol;
                            if (cc < cols_valid) {
                                float v = acc[im][in][r];
                                if (bb) v += brow ? rb : bv[in];
                                if constexpr (OUT_BF16) Cw[rr * sCm + cc] = f32_to_bf16_rne(v);
                                else                    Cw[rr * sCm + cc] = v;
                            }
                        }
                    }
                }
        }
    }
}

}  // namespace bi
