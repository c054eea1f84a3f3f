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
//   * rows past M and columns past N are read from the last valid row/column
//     (clamped addresses, never out of bounds) and never stored; the K tail
//     past K is zero-filled, which adds exact zeros;
//   * the bias (if any) is added once to the finished binary32 sum, then the
//     value is rounded once to the output dtype.
//
// Hardware mapping: 256x256 output tile per workgroup of 4 waves (2x2), each
// wave owning 128x128 = 4x4 MFMA blocks of 32x32 (256 binary32 accumulators
// per lane).  A and B tiles of 64 K-elements are staged in LDS, double
// buffered (2 x 64 KiB); each 128-byte LDS row (one M row of A, or one N
// column of B, 64 K values) holds eight 16-byte chunks placed by an XOR
// swizzle so that the 16-byte fragment reads of 8 neighbouring lanes hit
// distinct banks.  A B operand stored N-contiguous (a [K, N] weight) is
// transposed in registers on its way to LDS (8x8 blocks of bf16), so both
// operands reach the MFMA K-contiguous.  The persistent grid is min(tiles,
// compute units); workgroup w is renumbered so that the 8 XCDs (which receive
// workgroups round-robin) each work on a compact 2-D block of tiles, sharing
// their A and B panels in that XCD's L2.
#pragma once

#include "common.hpp"

namespace bi {

constexpr int G16_BM = 256;
constexpr int G16_BN = 256;
constexpr int G16_BK = 64;
constexpr int G16_THREADS = 256;
constexpr int G16_GROUP_M = 8;
constexpr int G16_STAGE_BYTES = G16_BM * G16_BK * 2;   // one operand tile: 32 KiB
constexpr int G16_LDS_BYTES = 4 * G16_STAGE_BYTES;     // {A, B} x 2 stages: 128 KiB

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

// Physical 16-byte chunk of logical chunk c in LDS row r.
__device__ __forceinline__ int g16_swz(int r) { return (r ^ (r >> 3)) & 7; }

template <bool B_KCONTIG, int OUT_BF16>
__global__ void __launch_bounds__(G16_THREADS, 1)
gemm_bf16_persistent(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[G16_LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (int)((p.K + G16_BK - 1) / G16_BK);

    const int grid = gridDim.x;
    const int w = blockIdx.x;
    const int wr = (grid % 8 == 0) ? (w % 8) * (grid / 8) + (w / 8) : w;

    for (int tile = wr; tile < p.total_tiles; tile += grid) {
        // ---- tile coordinates (scheduling only; no effect on arithmetic)
        const int s = tile / p.tiles_per_slice;
        const int t = tile - s * p.tiles_per_slice;
        const int width = G16_GROUP_M * p.tiles_n;
        const int group = t / width;
        const int first_m = group * G16_GROUP_M;
        const int gsz = min(p.tiles_m - first_m, G16_GROUP_M);
        const int pid_m = first_m + (t % width) % gsz;
        const int pid_n = (t % width) / gsz;
        const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
        const int64_t m0 = (int64_t)pid_m * G16_BM, n0 = (int64_t)pid_n * G16_BN;

        const uint16_t* Ab = p.A + s1 * p.sA1 + s2 * p.sA2;
        const uint16_t* Bb = p.B + s1 * p.sB1 + s2 * p.sB2;

        // ---- per-thread global sources for this tile: one base pointer and
        // 32-bit element offsets (the host guarantees they fit).
        // A: chunk id c = tid + 256*i -> LDS row (tid>>3) + 32*i, chunk tid&7.
        const int a_ch = tid & 7;
        const uint16_t* a_base = Ab + m0 * p.sAm + a_ch * 8;
        int a_off[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int64_t r = (tid >> 3) + 32 * i;
            r = m0 + r < p.M ? r : p.M - 1 - m0;
            a_off[i] = (int)(r * p.sAm);
        }
        // B, K-contiguous: same pattern with N columns as LDS rows.
        // B, N-contiguous: thread owns an 8(k) x 8(n) block: k = kb*8 + j, n = nb*8 + i.
        const int b_nb = tid & 31, b_kb = tid >> 5;
        const uint16_t* b_base;
        int b_off[8];
        if constexpr (B_KCONTIG) {
            b_base = Bb + n0 * p.sBn + a_ch * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int64_t c = (tid >> 3) + 32 * i;
                c = n0 + c < p.N ? c : p.N - 1 - n0;
                b_off[i] = (int)(c * p.sBn);
            }
        } else {
            int64_t c = n0 + b_nb * 8;
            c = c < p.N ? c : p.N - 8;
            b_base = Bb + c;
#pragma unroll
            for (int j = 0; j < 8; ++j) b_off[j] = (int)((b_kb * 8 + j) * p.sBk);
        }

        f32x16_t acc[4][4];
#pragma unroll
        for (int im = 0; im < 4; ++im)
#pragma unroll
            for (int in = 0; in < 4; ++in)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[im][in][r] = 0.0f;

        u32x4_t ra[8], rb[8];
        const u32x4_t zero4 = {0u, 0u, 0u, 0u};

        auto load_tile = [&](int kt) {
            const int64_t k0 = (int64_t)kt * G16_BK;
            const bool a_ok = k0 + a_ch * 8 < p.K;
            const uint16_t* a_k = a_base + k0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ra[i] = a_ok ? *(const u32x4_t*)(a_k + a_off[i]) : zero4;
            if constexpr (B_KCONTIG) {
                const uint16_t* b_k = b_base + k0;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rb[i] = a_ok ? *(const u32x4_t*)(b_k + b_off[i]) : zero4;
            } else {
                const uint16_t* b_k = b_base + k0 * p.sBk;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool ok = k0 + b_kb * 8 + j < p.K;
                    rb[j] = ok ? *(const u32x4_t*)(b_k + b_off[j]) : zero4;
                }
            }
        };

        auto store_tile = [&](int stage) {
            uint8_t* sA = smem + stage * 2 * G16_STAGE_BYTES;
            uint8_t* sB = sA + G16_STAGE_BYTES;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *(u32x4_t*)(sA + r * 128 + ((a_ch ^ g16_swz(r)) << 4)) = ra[i];
            }
            if constexpr (B_KCONTIG) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = (tid >> 3) + 32 * i;
                    *(u32x4_t*)(sB + r * 128 + ((a_ch ^ g16_swz(r)) << 4)) = rb[i];
                }
            } else {
                // 8x8 transpose: rb[j].dword[i/2] holds n = 2*(i/2), 2*(i/2)+1 of row k = j.
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    u32x4_t o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = rb[2 * q][i >> 1], hi = rb[2 * q + 1][i >> 1];
                        o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                       : ((lo & 0xffffu) | (hi << 16));
                    }
                    const int r = b_nb * 8 + i;
                    *(u32x4_t*)(sB + r * 128 + ((b_kb ^ g16_swz(r)) << 4)) = o;
                }
            }
        };

        auto compute_tile = [&](int stage) {
            const uint8_t* sA = smem + stage * 2 * G16_STAGE_BYTES;
            const uint8_t* sB = sA + G16_STAGE_BYTES;
#pragma unroll
            for (int kk = 0; kk < G16_BK / 16; ++kk) {
                const int ch = kk * 2 + (lane >> 5);
                u32x4_t af[4], bfr[4];
#pragma unroll
                for (int im = 0; im < 4; ++im) {
                    const int r = wm * 128 + im * 32 + (lane & 31);
                    af[im] = *(const u32x4_t*)(sA + r * 128 + ((ch ^ g16_swz(r)) << 4));
                }
#pragma unroll
                for (int in = 0; in < 4; ++in) {
                    const int r = wn * 128 + in * 32 + (lane & 31);
                    bfr[in] = *(const u32x4_t*)(sB + r * 128 + ((ch ^ g16_swz(r)) << 4));
                }
#pragma unroll
                for (int im = 0; im < 4; ++im)
#pragma unroll
                    for (int in = 0; in < 4; ++in)
                        acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(af[im]), as_bf16x8(bfr[in]), acc[im][in], 0, 0, 0);
            }
        };

        if (nk > 0) {
            load_tile(0);
            store_tile(0);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const bool more = kt + 1 < nk;
                if (more) load_tile(kt + 1);
                compute_tile(kt & 1);
                if (more) store_tile((kt + 1) & 1);
                __syncthreads();
            }
        }

        // ---- epilogue: + bias (binary32, once), round once, store
        void* Cb = (OUT_BF16 ? (void*)((uint16_t*)p.C + s1 * p.sC1 + s2 * p.sC2)
                             : (void*)((float*)p.C + s1 * p.sC1 + s2 * p.sC2));
        const uint16_t* bb = p.bias ? p.bias + s2 * p.sBias2 : nullptr;
        float bv[4];
#pragma unroll
        for (int in = 0; in < 4; ++in) {
            int64_t col = n0 + wn * 128 + in * 32 + (lane & 31);
            col = col < p.N ? col : p.N - 1;
            bv[in] = (bb && !p.bias_rows) ? bf16_to_f32(bb[col]) : 0.0f;
        }
#pragma unroll
        for (int im = 0; im < 4; ++im)
#pragma unroll
            for (int in = 0; in < 4; ++in) {
                const int64_t col = n0 + wn * 128 + in * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 128 + im * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < p.M && col < p.N) {
                        float v = acc[im][in][r];
                        if (bb) v += p.bias_rows ? bf16_to_f32(bb[row]) : bv[in];
                        store_out<OUT_BF16>(Cb, row * p.sCm + col, v);
                    }
                }
            }
    }
}

}  // namespace bi
