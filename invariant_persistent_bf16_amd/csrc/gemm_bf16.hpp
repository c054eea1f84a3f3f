// Persistent bfloat16 GEMM for gfx950 (CDNA4): C = A @ B (+ bias), binary32
// accumulation on the matrix cores.
//
// Batch invariance (the property of the persistent matmul in "Unmasking the
// True Culprit ...", section "Why This Achieves Batch Invariance": fixed block
// sizes, each output tile reduced inside one core, the same K order, no
// split-K) holds here by construction:
//   * one K step (32) and one MFMA instruction per dtype for every call; the
//     tile shape (chosen by the host from the shape of the product) only
//     decides which wave computes which elements;
//   * output element (i, j) is accumulated by a single chain of
//     v_mfma_f32_32x32x16_bf16 instructions, one per 16-wide K slice, K
//     ascending, starting from +0.0 (the first MFMA's literal accumulator
//     input; K = 0 runs one step of zeros); its operands are row i of A and column j
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
// accumulators per lane, held in AGPRs).  Four other tile shapes run the
// same per-element chain (G16Cfg): 128x256 (each wave 64x128), 128x128
// (each wave 64x64) and 192x256 (each wave 96x128) for products whose
// 256x256 tiles would leave compute units idle, and 256x128 (each wave
// 128x64) for N <= 128; the description
// below is of the 256x256 tile, the others scale the copy counts, LDS rows
// and fragment counts with the shape.  K advances in steps of 32 through a
// 4-stage LDS ring (4 x (16 + 16) KiB): operand tiles are copied HBM -> LDS by
// buffer_load_dwordx4 ... lds (no staging registers; a lane whose 16 bytes
// fall outside the operand gets an out-of-range offset and the hardware
// writes zeros) two to four steps ahead of their use, and the fragments of
// step k+1 are read from LDS into a second register set while the 32 MFMAs
// of step k run; the reads and copies of a step are spread evenly over its
// MFMAs.
//   * A: stages 0-1 and 2-3 form two double stages with LDS rows of 128
//     bytes (64 K values: the pair's two steps), filled by copies of 8 rows x
//     128 bytes issued at every other step, so each copy request covers whole
//     128-byte lines of A (16 rows x 64 bytes per copy ran 1-5 % slower on
//     MI355X: the addmm 3 %, the attention's P V, which streams A from HBM,
//     5 %).  The eight 16-byte chunks of
//     row r sit at chunk c ^ f2(r), f2(r) = (r >> 1) & 7, so 16 lanes reading
//     16 consecutive rows hit 16 distinct 16-byte bank groups.  Fragments
//     are ds_read_b128.  The 128x128 tile copies A one step at a time, as
//     the K-contiguous B below.
//   * a K-contiguous B, on the 256x256 and 192x256 tiles: the same 128-byte
//     rows and swizzle, in double stages that pair the steps the other way
//     (stages 1-2 and 3-0: B's stages sit in the slot order 1, 2, 3, 0),
//     filled at the even steps, so that every step issues one pair of
//     copies, of A or of B (convolution GEMM 3 % faster than with 64-byte B
//     rows).  On the other tiles: LDS rows of 64 bytes (32 K values of one N
//     column) per stage, copied one step at a time, the four 16-byte chunks
//     of row r at chunk c ^ f(r), f(r) = (r >> 2) & 3.
//   * an N-contiguous B (a [K, N] weight): LDS rows of 512 bytes (256 N values
//     of one K row), chunk c of row k at c ^ 4(k & 3).  Fragments are built by
//     two ds_read_b64_tr_b16 (gfx950's transposing LDS read: within a group of
//     16 lanes, lane t receives element t%4 of the 8 bytes addressed by lanes
//     4j + t/4, j = 0..3), giving each lane 8 consecutive K values of its N
//     column: the MFMA B operand, without a VALU transpose.
// LDS fragment reads are issued as inline assembly and waited for
// explicitly at the top of each step, so that the compiler does not order
// them behind the copies still in flight into other stages.
// The persistent grid is min(tiles, compute units); workgroup w is renumbered
// so that the 8 XCDs (which receive workgroups round-robin) each work on a
// compact 2-D block of tiles, sharing A and B panels in that XCD's L2.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bi {

constexpr int G16_BM = 256;
constexpr int G16_BN = 256;
constexpr int G16_BK = 32;
constexpr int G16_THREADS = 256;
constexpr int G16_GROUP_M = 8;
constexpr int G16_NSTAGE = 4;
constexpr uint32_t G16_OOB = 0x80000000u;                         // buffer offset that reads as zero
// Layout per tile shape: BM x BN = 256 x 256 (the tile above), 128 x 256
// (each wave 64x128) and 128 x 128 (each wave 64x64), for products whose
// 256x256 tiles leave compute units idle, 192 x 256 (each wave 96x128, for
// M a multiple of 192, such as the 1152 output channels of the patch
// convolution), or 256 x 128 (each wave 128x64, for N <= 128, which would
// fill half of a 256-wide tile).
template <int BM, int BN, bool ONE_PER_CU = true>
struct G16Cfg {
    static constexpr int WROWS = BM / 2;                        // rows of a wave's block
    static constexpr int WCOLS = BN / 2;                        // its columns
    static constexpr int IM = WROWS / 32;                       // its 32-row MFMA blocks
    static constexpr int IN = WCOLS / 32;                       // its 32-column MFMA blocks
    static constexpr int A_STAGE = BM * G16_BK * 2;             // A tile of one K step
    static constexpr int B_STAGE = BN * G16_BK * 2;             // B tile of one K step
    static constexpr int B_BASE = G16_NSTAGE * A_STAGE;         // B stages after the A stages
    static constexpr int RING = G16_NSTAGE * (A_STAGE + B_STAGE);
    static constexpr int BIAS = (4 * BM > BN ? 4 * BM : BN) * 4; // the tile's bias values, binary32 (single buffer)
    // Bias double buffered after the ring.  ONE_PER_CU: at least 81 KiB in
    // all, so that two of the kernel's workgroups never share a compute unit.
    // The grid is at most one workgroup per compute unit, and the dispatcher
    // does not promise to spread it: two 128x128 workgroups (66 KiB each) on
    // one unit would run at half speed beside an idle one.  The arithmetic
    // does not depend on it (ONE_PER_CU = false, a test-only variant, runs
    // two workgroups per unit and gives the same bits).
    static constexpr int LDS = (ONE_PER_CU && RING + BIAS < 81 * 1024) ? 81 * 1024 : RING + BIAS;
    static constexpr int NA = BM / 64;                          // A copies per wave and step (on average)
    static constexpr int NB = BN / 64;                          // B copies per wave and step
    static constexpr int NMF = 2 * IM * IN;                     // MFMAs per wave and step
    static constexpr int RB = BN * 2;                           // bytes of an N-contiguous B row in LDS
    static constexpr int LPR = RB / 16;                         // lanes per such row in one copy
};
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
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t g16_lds_addr(const void* p) {
    return (uint32_t)(size_t)((const __attribute__((address_space(3))) uint8_t*)p);
}
// Buffer descriptor of a wave-uniform base address (kept in SGPRs).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t g16_rsrc(const void* base) {
    const uint64_t v = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    void* u = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, G16_RECORDS, 0x00020000);
}
// 64 lanes x 16 bytes: lane L's bytes [base + soff + voff, +16) land at lds + 16 L.
__device__ __forceinline__ void g16_dma(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
template <int OFF>
__device__ __forceinline__ u32x4_t g16_read128(uint32_t addr) {
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ v2i32_t g16_read_tr(uint32_t addr) {
    v2i32_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// s_waitcnt with vmcnt <= V and lgkmcnt == 0 (gfx9 encoding; expcnt free).
template <int V>
__device__ __forceinline__ void g16_wait_vm_lgkm0() {
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | ((V >> 4) << 14));
}
template <int I, int N, typename F>
__device__ __forceinline__ void g16_static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        g16_static_for<I + 1, N>(f);
    }
}

// One step's MFMA operands: [kk][im] of A and [kk][in] of B.
struct G16Frags {
    u32x4_t a[2][4];
    u32x4_t b[2][4];
};

// CVEC: C allows 16-byte row stores (C aligned to 16 bytes; N, sCm, sC1, sC2
// multiples of 16 bytes' worth of elements); otherwise element stores.
// F16: binary16 operands (v_mfma_f32_32x32x16_f16, binary16 bias and 16-bit
// output) instead of bfloat16; the same tile, K order and schedule, the
// pages' fixed configuration per dtype.  OUT_BF16: 16-bit output in the
// operands' type (else binary32).
// BM x BN: tile shape, 256 x 256, 128 x 256, 256 x 128, 128 x 128 or 192 x 256 (G16Cfg); the
// per-element arithmetic is the same for all.
template <bool B_KCONTIG, int OUT_BF16, bool CVEC, bool F16 = false, int BM = 256, int BN = 256,
          bool ONE_PER_CU = true>
__global__ void __launch_bounds__(G16_THREADS, 1)
gemm_bf16_persistent(GemmParams p) {
    using C = G16Cfg<BM, BN, ONE_PER_CU>;
    constexpr int IM = C::IM, IN = C::IN;
    // A K-contiguous B is copied in pairs of K steps on the 256-wide tiles of
    // 192 or 256 rows; on the smaller tiles, where B is the larger share of a
    // step's bytes, the shallower queue of the pairs cost more than the
    // whole lines gained (128x128 tiles at M = 200, K = 4096: 37.8 -> 43.3
    // us), and B is copied one step at a time in 64-byte rows.
    constexpr bool BP = B_KCONTIG && BN == 256 && BM >= 192;
    // A is copied in pairs of K steps except on the 128x128 tile, whose
    // single round of tiles at small M waits on the queue's depth (M = 200,
    // K = 4096: 35.7 us one step at a time, 37.5 us in pairs).
    constexpr bool AP = !(BM == 128 && BN == 128);
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave index as a scalar so that LDS destinations are wave-uniform.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    // At least one K step: with K = 0 it loads only zeros (every copy is
    // out of range) and its MFMAs give the +0.0 sums of an empty product.
    const int nk = max(1, (int)((p.K + G16_BK - 1) / G16_BK));
    const int K32 = (int)p.K;   // the host bounds K below 2^30

    const int grid = gridDim.x;
    const int w = blockIdx.x;
    const int wr = (grid % 8 == 0) ? (w % 8) * (grid / 8) + (w / 8) : w;

    int ti = 0;   // tiles done by this workgroup
    for (int tile = wr; tile < p.total_tiles; tile += grid, ++ti) {
        // An opaque copy of the lane id, so that the per-lane addresses and
        // offsets below are recomputed each tile (a few VALU instructions)
        // instead of being kept live across the epilogue, where the compiler
        // would spill them and reload them before the next tile's copies.
        int lane_t = lane;
        asm volatile("" : "+v"(lane_t));
        const int tid_t = wave * 64 + lane_t;
        // ---- per-lane LDS fragment addresses
        //  A (double stage 0; the second adds 2 A_STAGE): row r = R0 + 32 im,
        //  R0 = WROWS wm + lane%32, f2(r) = f2(R0); the step's half h of the
        //  row, chunk (4h + 2kk + lane/32) ^ f2(r) = x ^ 2kk ^ 4h with
        //  x = lane/32 ^ f2(R0).
        //  K-contiguous B in pairs: the same in B's double stages (slot
        //  (s + 3) & 3 of stage s; slots 2p, 2p + 1 form double stage p); one
        //  step at a time: 64-byte rows and f(r) (stage 0; stages add B_STAGE).
        //  N-contiguous B: K row kk*16 + 8(g/2) + 4hr + z (z = li/4, k&3 = z),
        //  chunk (16wn + 4in + y) ^ 4z = 16wn + 4(in ^ z) + y.
        const uint32_t lds0 = g16_lds_addr(smem);
        uint32_t a_fb[2][2], b_fb[4];   // K-contiguous B: b_fb[2h + kk]
        {
            const int R0 = wm * C::WROWS + (lane_t & 31);
            if constexpr (AP) {
                const int x = (lane_t >> 5) ^ ((R0 >> 1) & 7);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) a_fb[h][kk] = lds0 + R0 * 128 + ((x ^ (2 * kk) ^ (4 * h)) << 4);
            } else {
                const int x = (lane_t >> 5) ^ ((R0 >> 2) & 3);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) a_fb[0][kk] = lds0 + R0 * 64 + ((x ^ (2 * kk)) << 4);
                a_fb[1][0] = a_fb[1][1] = 0;
            }
            if constexpr (BP) {
                const int N0 = wn * C::WCOLS + (lane_t & 31);
                const int xb = (lane_t >> 5) ^ ((N0 >> 1) & 7);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        b_fb[2 * h + kk] = lds0 + C::B_BASE + N0 * 128 + ((xb ^ (2 * kk) ^ (4 * h)) << 4);
            } else if constexpr (B_KCONTIG) {
                const int N0 = wn * C::WCOLS + (lane_t & 31);
                const int xb = (lane_t >> 5) ^ ((N0 >> 2) & 3);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) b_fb[kk] = lds0 + C::B_BASE + N0 * 64 + ((xb ^ (2 * kk)) << 4);
                b_fb[2] = b_fb[3] = 0;
            } else {
                const int g = lane_t >> 4, li = lane_t & 15, z = li >> 2;
                const int y = 2 * (g & 1) + ((li & 3) >> 1);
#pragma unroll
                for (int in = 0; in < IN; ++in)
                    b_fb[in] = lds0 + C::B_BASE + (8 * (g >> 1) + z) * C::RB +
                               ((((IN * wn + in) ^ z) << 2) + y) * 16 + (li & 1) * 8;
            }
        }

        // ---- tile coordinates (scheduling only; no effect on arithmetic)
        const int s = tile / p.tiles_per_slice;
        const int t = tile - s * p.tiles_per_slice;
        const int width = G16_GROUP_M * p.tiles_n;
        const int first_m = (t / width) * G16_GROUP_M;
        const int gsz = min(p.tiles_m - first_m, G16_GROUP_M);
        const int pid_m = first_m + (t % width) % gsz;
        const int pid_n = (t % width) / gsz;
        const int64_t s1 = s / p.G2, s2 = s - (s / p.G2) * p.G2;
        const int64_t m0 = (int64_t)pid_m * BM, n0 = (int64_t)pid_n * BN;
        const uint16_t* Ab = p.A + s1 * p.sA1 + s2 * p.sA2 + m0 * p.sAm;
        const uint16_t* Bb;
        if constexpr (B_KCONTIG) Bb = p.B + s1 * p.sB1 + s2 * p.sB2 + n0 * p.sBn;
        else                     Bb = p.B + s1 * p.sB1 + s2 * p.sB2 + n0;

        // ---- DMA source offsets: per-lane 32-bit byte offsets from the tile's
        // base, fixed for the tile (out-of-range rows already turned into the
        // zero-reading offset); each K step adds a uniform byte offset through
        // the instruction's scalar offset.  The host bounds every offset below 2^31.
        // A: wave w, copy j (0 .. 2NA-1) of a pair covers double-stage rows
        // (BM/4) w + 8j + lane/8; the lane writes physical chunk lane&7, i.e.
        // logical chunk (lane&7) ^ f2(row) = (lane&7) ^ (lane>>4) ^ 4(j&1)
        // (BM/4 is a multiple of 16).
        // K-contiguous B in pairs: the same as A, with BN for BM.  One step at
        // a time: copy j covers LDS rows (BN/4) w + 16j + lane/4; the lane
        // writes physical chunk lane&3, i.e. logical chunk
        // (lane&3) ^ f(row) = (lane&3) ^ ((lane>>4)&3).
        // N-contiguous B: copy j covers K rows 8w + 2j + lane/32; the lane writes
        // physical chunk lane&31 of that row, i.e. logical chunk
        // (lane&31) ^ 4(krow&3), columns clamped to the last valid 8.
        uint32_t a_off[AP ? 2 * C::NA : C::NA], b_off[BP ? 2 * C::NB : C::NB];
        const int b_u8 = ((lane_t & 3) ^ ((lane_t >> 4) & 3)) * 8;   // one-step K-contiguous B copies
        const int u8 = ((lane_t & 7) ^ (lane_t >> 4)) * 8;   // first K of a paired copy's lane chunk, even j (odd: ^ 32)
        {
            if constexpr (BP) {
                const int b_row0 = (BN / 4) * wave + (lane_t >> 3);
                const int64_t b_rows_left = p.N - n0 - b_row0;
#pragma unroll
                for (int j = 0; j < 2 * C::NB; ++j)
                    b_off[j] = b_rows_left > 8 * j ? (uint32_t)(((b_row0 + 8 * j) * (int)p.sBn + (u8 ^ (32 * (j & 1)))) * 2)
                                                   : G16_OOB;
            } else if constexpr (B_KCONTIG) {
                const int b_row0 = (BN / 4) * wave + (lane_t >> 2);
                const int64_t b_rows_left = p.N - n0 - b_row0;
#pragma unroll
                for (int j = 0; j < C::NB; ++j)
                    b_off[j] = b_rows_left > 16 * j ? (uint32_t)(((b_row0 + 16 * j) * (int)p.sBn + b_u8) * 2) : G16_OOB;
            } else {
                const int ncl = (int)min<int64_t>(p.N - 8 - n0, BN - 8);
#pragma unroll
                for (int j = 0; j < C::NB; ++j) {
                    const int krow = 8 * wave + (1024 / C::RB) * j + lane_t / C::LPR;
                    const int col = min(((lane_t % C::LPR) ^ (4 * (krow & 3))) << 3, ncl);
                    b_off[j] = (uint32_t)((krow * (int)p.sBk + col) * 2);
                }
            }
        }
        if constexpr (AP) {
            const int a_row0 = (BM / 4) * wave + (lane_t >> 3);
            const int64_t a_rows_left = p.M - m0 - a_row0;
#pragma unroll
            for (int j = 0; j < 2 * C::NA; ++j)
                a_off[j] = a_rows_left > 8 * j ? (uint32_t)(((a_row0 + 8 * j) * (int)p.sAm + (u8 ^ (32 * (j & 1)))) * 2)
                                               : G16_OOB;
        } else {
            const int a_row0 = (BM / 4) * wave + (lane_t >> 2);
            const int64_t a_rows_left = p.M - m0 - a_row0;
#pragma unroll
            for (int j = 0; j < C::NA; ++j)
                a_off[j] = a_rows_left > 16 * j ? (uint32_t)(((a_row0 + 16 * j) * (int)p.sAm + b_u8) * 2) : G16_OOB;
        }
        const int bn_krow0 = 8 * wave + lane_t / C::LPR;
        const __amdgpu_buffer_rsrc_t rsA = g16_rsrc(Ab), rsB = g16_rsrc(Bb);
        const uint32_t kstepB = B_KCONTIG ? 2u * G16_BK : (uint32_t)(2 * G16_BK * p.sBk);

        // A copy j (0 .. 2NA-1) of the K steps kt, kt+1 into the double stage
        // at stage st (even); lanes past K read zeros.
        // One step at a time (the 128x128 tile): copy j (0 .. NA-1) of step kt
        // into stage st, rows (BM/4) w + 16j + lane/4 of 64 bytes, as a
        // K-contiguous B copied one step at a time.
        auto dma_a1 = [&](int kt, int st, auto jc) {
            constexpr int j = decltype(jc)::value;
            const int kleft = K32 - kt * G16_BK;
            g16_dma(rsA, smem + st * C::A_STAGE + (wave * C::NA + j) * 1024,
                    b_u8 < kleft ? a_off[j] : G16_OOB, (uint32_t)kt * (2u * G16_BK));
        };
        auto dma_a = [&](int kt, int st, auto jc) {
            constexpr int j = decltype(jc)::value;
            const int kleft = K32 - kt * G16_BK;
            g16_dma(rsA, smem + st * C::A_STAGE + (wave * 2 * C::NA + j) * 1024,
                    (u8 ^ (32 * (j & 1))) < kleft ? a_off[j] : G16_OOB, (uint32_t)kt * (2u * G16_BK));
        };
        // B copied one step at a time: copy j (0 .. NB-1) of K step kt into stage st.
        auto dma_b = [&](int kt, int st, auto jc) {
            constexpr int j = decltype(jc)::value;
            const int kleft = K32 - kt * G16_BK;
            if constexpr (B_KCONTIG)
                g16_dma(rsB, smem + C::B_BASE + st * C::B_STAGE + (wave * C::NB + j) * 1024,
                        b_u8 < kleft ? b_off[j] : G16_OOB, (uint32_t)kt * kstepB);
            else
                g16_dma(rsB, smem + C::B_BASE + st * C::B_STAGE + (wave * C::NB + j) * 1024,
                        bn_krow0 + (1024 / C::RB) * j < kleft ? b_off[j] : G16_OOB, (uint32_t)kt * kstepB);
        };
        // K-contiguous B: copy j (0 .. 2NB-1) of the pair of K steps kt, kt+1
        // (kt odd) into B's double stage `pair`.  B's stages sit in the slot
        // order 1, 2, 3, 0, so its pairs are the stages (1, 2) and (3, 0).
        auto dma_bp = [&](int kt, int pair, auto jc) {
            constexpr int j = decltype(jc)::value;
            const int kleft = K32 - kt * G16_BK;
            g16_dma(rsB, smem + C::B_BASE + pair * 2 * C::B_STAGE + (wave * 2 * C::NB + j) * 1024,
                    (u8 ^ (32 * (j & 1))) < kleft ? b_off[j] : G16_OOB, (uint32_t)kt * kstepB);
        };
        // The prologue's pair (-1, 0): only step 0's half, from the lanes whose
        // chunk lies in the pair's second step (the others read zeros).
        auto dma_bp_first = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int uj = u8 ^ (32 * (j & 1));
            const bool ok = uj >= 32 && uj - 32 < K32 && b_off[j] != G16_OOB;
            g16_dma(rsB, smem + C::B_BASE + 2 * C::B_STAGE + (wave * 2 * C::NB + j) * 1024,
                    ok ? b_off[j] - 64u : G16_OOB, 0u);
        };
        // LDS read r of the fragments of stage ST into F: 0 .. 2IM-1 A
        // [kk = r/IM][im = r%IM]; then B (q = r - 2IM): K-contiguous [kk][in]
        // (q = kk*IN + in), N-contiguous [kk][in] half hr (q = kk*2IN + in*2 + hr).
        auto lds_read = [&](G16Frags& F, auto stc, auto rc) {
            constexpr int ST = decltype(stc)::value, r = decltype(rc)::value;
            if constexpr (r < 2 * IM) {
                constexpr int kk = r / IM, im = r % IM;
                if constexpr (AP) F.a[kk][im] = g16_read128<(ST >> 1) * 2 * C::A_STAGE + im * 4096>(a_fb[ST & 1][kk]);
                else              F.a[kk][im] = g16_read128<ST * C::A_STAGE + im * 2048>(a_fb[0][kk]);
            } else if constexpr (B_KCONTIG) {
                if constexpr (r < 2 * IM + 2 * IN) {
                    constexpr int kk = (r - 2 * IM) / IN, in = (r - 2 * IM) % IN, slot = (ST + 3) & 3;
                    if constexpr (BP)
                        F.b[kk][in] = g16_read128<(slot >> 1) * 2 * C::B_STAGE + in * 4096>(b_fb[2 * (slot & 1) + kk]);
                    else
                        F.b[kk][in] = g16_read128<ST * C::B_STAGE + in * 2048>(b_fb[kk]);
                }
            } else {
                constexpr int q = r - 2 * IM, kk = q / (2 * IN), in = (q % (2 * IN)) / 2, hr = q % 2;
                const v2i32_t h = g16_read_tr<ST * C::B_STAGE + kk * 16 * C::RB + hr * 4 * C::RB>(b_fb[in]);
                F.b[kk][in][2 * hr] = (uint32_t)h[0];
                F.b[kk][in][2 * hr + 1] = (uint32_t)h[1];
            }
        };
        // Make the fragment registers of F depend on the preceding wait.
        auto fence_frags = [&](G16Frags& F) {
            if constexpr (IM == 4)
                asm volatile("" : "+v"(F.a[0][0]), "+v"(F.a[0][1]), "+v"(F.a[0][2]), "+v"(F.a[0][3]),
                                  "+v"(F.a[1][0]), "+v"(F.a[1][1]), "+v"(F.a[1][2]), "+v"(F.a[1][3]));
            else if constexpr (IM == 3)
                asm volatile("" : "+v"(F.a[0][0]), "+v"(F.a[0][1]), "+v"(F.a[0][2]),
                                  "+v"(F.a[1][0]), "+v"(F.a[1][1]), "+v"(F.a[1][2]));
            else
                asm volatile("" : "+v"(F.a[0][0]), "+v"(F.a[0][1]), "+v"(F.a[1][0]), "+v"(F.a[1][1]));
            if constexpr (IN == 4)
                asm volatile("" : "+v"(F.b[0][0]), "+v"(F.b[0][1]), "+v"(F.b[0][2]), "+v"(F.b[0][3]),
                                  "+v"(F.b[1][0]), "+v"(F.b[1][1]), "+v"(F.b[1][2]), "+v"(F.b[1][3]));
            else
                asm volatile("" : "+v"(F.b[0][0]), "+v"(F.b[0][1]), "+v"(F.b[1][0]), "+v"(F.b[1][1]));
        };

        // Bias of the tile (by row for bias_rows, else by column): one
        // element per thread, loaded before the operand copies and written
        // to LDS only after the K loop's final wait (so no wait is spent on
        // it), in binary32: one value per column (column bias), each row's
        // value four times (row bias, so that the epilogue reads four bias
        // values per output group either way), or -0.0 without bias (x + -0.0
        // is x exactly).  Entries past M (or N) repeat the last valid one and
        // are never stored.  One buffer: the next tile writes it only after
        // its own K loop, whose barriers every wave passes after its epilogue.
        float* bias_lds = (float*)(smem + C::RING);
        uint32_t braw = 0;
        if (p.bias) {
            const int64_t b0 = p.bias_rows ? m0 : n0;
            const int nb = (int)min<int64_t>((p.bias_rows ? p.M : p.N) - b0, 256);
            braw = p.bias[s2 * p.sBias2 + b0 + min(tid_t, nb - 1)];
        }

        // Accumulators: the first K step's first MFMA of each block starts
        // from a literal +0.0 (no separate zeroing pass, no zero values kept
        // live across the tile loop).
        f32x16_t acc[IM][IN];

        G16Frags F0, F1;
        constexpr int NREAD = 2 * IM + (B_KCONTIG ? 2 : 4) * IN;

        // One K step kt (stage ST = kt % 4): wait for step kt+1's copies and
        // for the reads of step kt's fragments, barrier, then the MFMAs on
        // step kt's fragments with the step's memory instructions spread
        // between them: the LDS reads of step kt+1's fragments; at odd stages
        // A's copies of the pair kt+3, kt+4 into the double stage ST-1, ST
        // (step kt+3's half was read before the previous barrier); an
        // N-contiguous B's copies of step kt+4 into stage ST (its data now
        // lives in registers) at every stage (a K-contiguous B on the smaller
        // tiles likewise), or at even stages a paired B's pair kt+3, kt+4
        // into its stages ST-1, ST.
        // A wave's copies, in issue order: at step j the A pair (j+3, j+4) if
        // j is odd, then B's copies of step j+4, or, for a paired B, its
        // pair (j+3, j+4) if j is even.  Step kt+1's data is
        // complete once the copies issued after its last one are all that is
        // outstanding: for odd kt, B's copies of steps kt+2 and kt+3, or B's
        // pair issued at step kt-1 (2 NB copies; the A pair came at step
        // kt-2); for even kt, the A pair issued at step kt-1 and, with an
        // B copied one step at a time, B's copies of kt+2 and kt+3 (2 NA or 2 NB + 2 NA;
        // the A pair came at step kt-3).  Copies and reads past the last step are
        // harmless (zeros into an unused stage, reads of an unused stage) and
        // keep the step a single straight-line block.
        auto step = [&](int kt, auto stc, auto firstc) {
            constexpr int ST = decltype(stc)::value;
            constexpr bool FIRST = decltype(firstc)::value;
            G16Frags& cur = (ST & 1) ? F1 : F0;
            G16Frags& nxt = (ST & 1) ? F0 : F1;
            if constexpr (!AP)             g16_wait_vm_lgkm0<2 * C::NB + 2 * C::NA>();   // steps kt+2, kt+3
            else if constexpr (ST & 1)     g16_wait_vm_lgkm0<2 * C::NB>();
            else if constexpr (BP)         g16_wait_vm_lgkm0<2 * C::NA>();
            else                           g16_wait_vm_lgkm0<2 * C::NB + 2 * C::NA>();
            __builtin_amdgcn_s_barrier();
            fence_frags(cur);
            __builtin_amdgcn_sched_barrier(0);
            g16_static_for<0, C::NMF>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                constexpr int kk = i / (IM * IN), im = (i / IN) % IM, in = i % IN;
                const f32x16_t zero = {};
                const f32x16_t& c_in = (FIRST && kk == 0) ? zero : acc[im][in];
                if constexpr (F16)
                    acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        as_f16x8(cur.b[kk][in]), as_f16x8(cur.a[kk][im]), c_in, 0, 0, 0);
                else
                    acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(cur.b[kk][in]), as_bf16x8(cur.a[kk][im]), c_in, 0, 0, 0);
                // Read r after MFMA r * NMF / NREAD, copy d after
                // (2d + 1) NMF / (2 NC): at odd stages A's pair (first), at
                // even stages a paired B's pair kt+3, kt+4 (stages ST-1 and
                // ST: B's double stage 1 - ST/2), or B's copies of step kt+4
                // at every stage.
                g16_static_for<0, NREAD>([&](auto rc) {
                    constexpr int r = decltype(rc)::value;
                    if constexpr (r * C::NMF / NREAD == i)
                        lds_read(nxt, std::integral_constant<int, (ST + 1) % 4>{}, rc);
                });
                constexpr int NCA = !AP ? C::NA : (ST & 1) ? 2 * C::NA : 0;
                constexpr int NCB = BP ? ((ST & 1) ? 0 : 2 * C::NB) : C::NB;
                constexpr int NC = NCA + NCB;
                g16_static_for<0, NC>([&](auto dc) {
                    constexpr int d = decltype(dc)::value;
                    if constexpr ((2 * d + 1) * C::NMF / (2 * NC) == i) {
                        if constexpr (d < NCA && !AP) dma_a1(kt + 4, ST, dc);
                        else if constexpr (d < NCA)   dma_a(kt + 3, ST - 1, dc);
                        else if constexpr (BP)        dma_bp(kt + 3, 1 - ST / 2, std::integral_constant<int, d - NCA>{});
                        else                          dma_b(kt + 4, ST, std::integral_constant<int, d - NCA>{});
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // Prologue: the copies of steps 0..3 in the steady state's order (as
        // if issued by steps -4 .. -1), wait for step 0's, read its
        // fragments.  B one step at a time: B0, A pair (0, 1), B1, B2, A pair
        // (2, 3), B3.  Paired B: B pair (-1, 0), A pair (0, 1), B pair
        // (1, 2), A pair (2, 3).  A and B one step at a time: A0 B0, A1 B1,
        // A2 B2, A3 B3.
        if constexpr (!AP) {
            g16_static_for<0, 4>([&](auto sc) {
                constexpr int st = decltype(sc)::value;
                g16_static_for<0, C::NA>([&](auto jc) { dma_a1(st, st, jc); });
                g16_static_for<0, C::NB>([&](auto jc) { dma_b(st, st, jc); });
            });
            g16_wait_vm_lgkm0<3 * C::NB + 3 * C::NA>();
        } else if constexpr (BP) {
            g16_static_for<0, 2 * C::NB>([&](auto jc) { dma_bp_first(jc); });
            g16_static_for<0, 2 * C::NA>([&](auto jc) { dma_a(0, 0, jc); });
            g16_static_for<0, 2 * C::NB>([&](auto jc) { dma_bp(1, 0, jc); });
            g16_static_for<0, 2 * C::NA>([&](auto jc) { dma_a(2, 2, jc); });
            g16_wait_vm_lgkm0<2 * C::NB + 2 * C::NA>();
        } else {
            auto dma_b_all = [&](auto sc) {
                g16_static_for<0, C::NB>([&](auto jc) { dma_b(decltype(sc)::value, decltype(sc)::value, jc); });
            };
            dma_b_all(std::integral_constant<int, 0>{});
            g16_static_for<0, 2 * C::NA>([&](auto jc) { dma_a(0, 0, jc); });
            dma_b_all(std::integral_constant<int, 1>{});
            dma_b_all(std::integral_constant<int, 2>{});
            g16_static_for<0, 2 * C::NA>([&](auto jc) { dma_a(2, 2, jc); });
            dma_b_all(std::integral_constant<int, 3>{});
            g16_wait_vm_lgkm0<3 * C::NB + 2 * C::NA>();
        }
        __builtin_amdgcn_s_barrier();
        g16_static_for<0, NREAD>([&](auto rc) { lds_read(F0, std::integral_constant<int, 0>{}, rc); });

        using NF = std::false_type;
        step(0, std::integral_constant<int, 0>{}, std::true_type{});
        for (int kt = 1; kt < nk; kt += 4) {
            step(kt, std::integral_constant<int, 1>{}, NF{});
            if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 2>{}, NF{});
            if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 3>{}, NF{});
            if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 0>{}, NF{});
        }
        // Drain every copy (including the ones past the last step) and every
        // read before the next tile reuses the stages.  The last step's reads
        // of the next fragments are dead, but the hardware still writes their
        // registers when they return; the fences keep both fragment sets
        // allocated until after the wait, so the compiler cannot place an
        // epilogue value (an accumulator copied out of its AGPR) in one of
        // them before the late read lands there.
        g16_wait_vm_lgkm0<0>();
        fence_frags(F0);
        fence_frags(F1);
        {
            asm volatile("" : "+v"(braw));
            const float bv = p.bias ? h16_to_f32<F16>((uint16_t)braw) : -0.0f;
            if (p.bias_rows) {
                if (tid_t < BM) *(f32x4_t*)(bias_lds + 4 * tid_t) = f32x4_t{bv, bv, bv, bv};
            } else if (tid_t < BN) {
                bias_lds[tid_t] = bv;
            }
        }
        __builtin_amdgcn_s_barrier();

        // ---- epilogue: + bias (binary32, once), round once, store.
        // The MFMAs take the B fragment as their first operand, so block
        // (im, in) holds C^T: lane l, register 4g + j is C[row im*32 + l%32]
        // [col in*32 + 8g + 4(l/32) + j], four consecutive columns of one row.
        // CVEC: each wave stages its 128x128 block through its own 32 KiB of
        // the (now idle) LDS ring, 16-byte chunks of row r at chunk ^ (r mod
        // chunks per row) so that neither side conflicts, then writes whole
        // rows with 16-byte non-temporal stores (one instruction = 8 full
        // 128-byte lines for bfloat16; the output is not re-read by this
        // kernel, and keeping it out of the caches leaves them to the operand
        // panels); binary32 goes in two halves of 64 rows.  Otherwise: one
        // buffer store per element.
        // Bounds without branches: the buffer's record count ends at the last
        // valid element of this wave's block, so rows past M fall outside it,
        // and a lane whose columns are past N stores at the out-of-range
        // offset; out-of-range buffer stores are dropped.  The host bounds
        // 128 * sCm * 4 below 2^31 and, with CVEC, makes N a multiple of the
        // 16-byte chunk, so a chunk is all valid or all not.
#ifdef STUB_EPI
#pragma unroll
        for (int im = 0; im < IM; ++im)
#pragma unroll
            for (int in = 0; in < IN; ++in) asm volatile("" :: "a"(acc[im][in]));
        if (false)
#endif
        {
            using OutT = typename std::conditional<OUT_BF16 != 0, uint16_t, float>::type;
            constexpr int ESZ = (int)sizeof(OutT);
            const int64_t row_w = m0 + wm * C::WROWS, col_w = n0 + wn * C::WCOLS;
            OutT* Cw = (OutT*)p.C + s1 * p.sC1 + s2 * p.sC2 + row_w * p.sCm + col_w;
            const int sCm = (int)p.sCm;
            const int rows_valid = (int)min<int64_t>(p.M - row_w, C::WROWS);
            const int cols_valid = (int)min<int64_t>(p.N - col_w, C::WCOLS);
            // Every wave runs the epilogue; a wave with no valid row or
            // column gets an empty store range, so all its stores are dropped.
            {
                // An opaque copy of the lane id keeps every epilogue value below
                // from being computed before the K loop (where it would stay live).
                int lane_e = lane;
                asm volatile("" : "+v"(lane_e));
                const int lrow = lane_e & 31, lh = lane_e >> 5, lcol = 4 * lh;
                const uint64_t cv = (uint64_t)Cw;
                const uint32_t clo = __builtin_amdgcn_readfirstlane((uint32_t)cv);
                const uint32_t chi = __builtin_amdgcn_readfirstlane((uint32_t)(cv >> 32));
                const int nrec = __builtin_amdgcn_readfirstlane(
                    rows_valid > 0 && cols_valid > 0 ? ((rows_valid - 1) * sCm + cols_valid) * ESZ : 0);
                const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(((uint64_t)chi << 32) | clo), (short)0, nrec, 0x00020000);
                // Block (im, in), group g with its bias added once, in
                // binary32: four consecutive bias values from LDS, the
                // columns' own (column bias) or the row's value repeated
                // (row bias), or -0.0 (no bias: x + -0.0 is x exactly).
                const int bsel = p.bias_rows;
                // The bias vectors of one 32-row block, read from LDS together
                // (one wait) before the block's staging writes.
                f32x4_t bq[4 * IN];
                auto load_bias = [&](auto imc) {
                    constexpr int im = decltype(imc)::value;
                    g16_static_for<0, 4 * IN>([&](auto qc) {
                        constexpr int q = decltype(qc)::value, in = q / 4, g = q % 4;
                        const int bidx = bsel ? 4 * (wm * C::WROWS + im * 32 + lrow)
                                              : wn * C::WCOLS + in * 32 + 8 * g + lcol;
                        bq[q] = *(const f32x4_t*)(bias_lds + bidx);
                    });
                };
                auto value = [&](auto imc, auto qc) {
                    constexpr int im = decltype(imc)::value;
                    constexpr int q = decltype(qc)::value, in = q / 4, g = q % 4;
                    f32x4_t v = {acc[im][in][4 * g], acc[im][in][4 * g + 1],
                                 acc[im][in][4 * g + 2], acc[im][in][4 * g + 3]};
                    v += bq[q];
                    return v;
                };
                if constexpr (CVEC) {
                    // binary32: two passes, or one per 32-row block when the
                    // wave has an odd number of them
                    constexpr int PASSES = OUT_BF16 ? 1 : (IM % 2 == 0 ? 2 : IM);
                    constexpr int ROWB = C::WCOLS * ESZ;  // bytes of one staged row
                    constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
                    constexpr int RPP = C::WROWS / PASSES;  // rows per pass
                    constexpr int RPI = 64 / NCH;         // rows per read instruction
                    uint8_t* stg = smem + wave * (C::RING / 4);
                    static_assert(RPP * ROWB <= C::RING / 4, "a pass fits the wave's share of the ring");
                    const int t = lane_e % NCH, rsub = lane_e / NCH;
                    const bool col_ok = t * (16 / ESZ) < cols_valid;
                    g16_static_for<0, PASSES>([&](auto pc) {
                        constexpr int ps = decltype(pc)::value;
                        g16_static_for<0, IM / PASSES>([&](auto ic) {
                            constexpr int im = ps * (IM / PASSES) + decltype(ic)::value;
                            const int r = (im % (IM / PASSES)) * 32 + lrow;
                            load_bias(std::integral_constant<int, im>{});
                            g16_static_for<0, 4 * IN>([&](auto qc) {
                                constexpr int in = decltype(qc)::value / 4, g = decltype(qc)::value % 4;
                                const f32x4_t v = value(std::integral_constant<int, im>{}, qc);
                                if constexpr (OUT_BF16) {
                                    const int c = in * 4 + g;
                                    const v2u32_t w = {pack16x2<F16>(v[0], v[1]), pack16x2<F16>(v[2], v[3])};
                                    *(v2u32_t*)(stg + r * ROWB + ((c ^ (r & (NCH - 1))) << 4) + 8 * lh) = w;
                                } else {
                                    const int c = in * 8 + 2 * g + lh;
                                    *(f32x4_t*)(stg + r * ROWB + ((c ^ (r & (NCH - 1))) << 4)) = v;
                                }
                            });
                            __builtin_amdgcn_sched_barrier(0);
                        });
                        g16_static_for<0, RPP / RPI>([&](auto jc) {
                            constexpr int i = decltype(jc)::value;
                            const int r = i * RPI + rsub;
                            const u32x4_t d = *(const u32x4_t*)(stg + r * ROWB + ((t ^ (r & (NCH - 1))) << 4));
                            const uint32_t off = col_ok ? (uint32_t)((ps * RPP + r) * sCm * ESZ + t * 16) : G16_OOB;
                            __builtin_amdgcn_raw_buffer_store_b128(d, rsC, (int)off, 0, 2);
                        });
                    });
                } else {
                    g16_static_for<0, IM>([&](auto imc) {
                        constexpr int im = decltype(imc)::value;
                        const int vrow = ((im * 32 + lrow) * sCm) * ESZ;
                        load_bias(imc);
                        g16_static_for<0, 4 * IN>([&](auto qc) {
                            constexpr int in = decltype(qc)::value / 4, g = decltype(qc)::value % 4;
                            const f32x4_t v = value(imc, qc);
                            const int col = in * 32 + 8 * g + lcol;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const uint32_t off = col + j < cols_valid ? (uint32_t)(vrow + (col + j) * ESZ) : G16_OOB;
                                if constexpr (OUT_BF16)
                                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pack16x2<F16>(v[j], 0.0f), rsC,
                                                                          (int)off, 0, 0);
                                else
                                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), rsC, (int)off, 0, 0);
                            }
                        });
                    });
                }
            }
        }
        // Every wave has read its staged block (its stores consumed the reads)
        // before the next tile's copies overwrite the ring.
        if constexpr (CVEC) __builtin_amdgcn_s_barrier();
    }
}

// The kernel for a tile shape and layout (defined in gemm16_<BM>x<BN>.hip).
typedef void (*Gemm16Kern)(GemmParams);
Gemm16Kern gemm16_kernel_256x256(int f16, int kc, int out16, int cvec);
Gemm16Kern gemm16_kernel_128x256(int f16, int kc, int out16, int cvec);
Gemm16Kern gemm16_kernel_256x128(int f16, int kc, int out16, int cvec);
Gemm16Kern gemm16_kernel_128x128(int f16, int kc, int out16, int cvec);
Gemm16Kern gemm16_kernel_192x256(int f16, int kc, int out16, int cvec);
// 128x128 tiles without the 81 KiB reservation (two workgroups per compute
// unit; bfloat16 operands, vector epilogue; benchmark library only).
Gemm16Kern gemm16_kernel_128x128_shared(int kc, int out16);

}  // namespace bi
