// Benchmark / test variants (include/bi_bench.h).  They reuse the product
// kernels; what they add is a batch-size-dependent choice (split-K for the
// GEMM, split count by load for decode) or a forced launch grid.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "../../include/bi_bench.h"
#include "decode.hpp"
#include "gemm_bf16.hpp"
#include "gemm_f32.hpp"
#include "internal.hpp"
#include "softmax.hpp"

namespace bi {

// Sum of `splits` partial products in part order, then + bias, then round.
template <int OUT_BF16, int BIAS_BF16>
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t M, int64_t N,
                                     const void* __restrict__ bias, void* __restrict__ C, int64_t sCm) {
    const int64_t MN = M * N;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < MN;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = part[i];
        for (int s = 1; s < splits; ++s) v += part[s * MN + i];
        const int64_t r = i / N, c = i - (i / N) * N;
        if (bias) v += BIAS_BF16 ? bf16_to_f32(((const uint16_t*)bias)[c]) : ((const float*)bias)[c];
        store_out<OUT_BF16>(C, r * sCm + c, v);
    }
}

// Two-level merge: the `nsub` piece triples of each part are merged in piece
// order, then the parts in part order (nsub == 1: one flat merge).
template <int D, int OUT_BF16>
__global__ void decode_merge_parts_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                          int64_t BH, int parts, int nsub) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= BH * D) return;
    const int64_t bh = i / D;
    const int d = (int)(i - bh * D);
    const float* tp = ws + bh * (int64_t)parts * nsub * (2 + D);
    float Mall = -INFINITY;
    float pm[64], pl[64], po[64];
    for (int p = 0; p < parts; ++p) {
        const float* t = tp + (int64_t)p * nsub * (2 + D);
        float m = t[0];
        for (int s = 1; s < nsub; ++s) m = fmaxf(m, t[s * (2 + D)]);
        float l = 0.0f, o = 0.0f;
        for (int s = 0; s < nsub; ++s) {
            const float w = expf(t[s * (2 + D)] - m);
            l = fmaf(w, t[s * (2 + D) + 1], l);
            o = fmaf(w, t[s * (2 + D) + 2 + d], o);
        }
        pm[p] = m; pl[p] = l; po[p] = o;
        Mall = fmaxf(Mall, m);
    }
    float num = 0.0f, den = 0.0f;
    for (int p = 0; p < parts; ++p) {
        const float w = expf(pm[p] - Mall);
        num = fmaf(w, po[p], num);
        den = fmaf(w, pl[p], den);
    }
    store_out<OUT_BF16>(out, i, num / den);
}

// Split-KV decode sized by load, for the cost-of-invariance comparison: the
// KV sequence of each (b, h) is cut into `splits` parts of L = 8 TW tokens
// (the split count chosen from the batch so that the grid fills the compute
// units), each part one workgroup whose 8 waves take TW tokens each (no
// loads for tokens outside the part), and the merge runs in the same launch:
// the workgroup that finishes a (b, h) last merges its parts' triples in part
// order.  The compute units' L2 caches are not coherent with each other, so
// the triples are written and read at system scope (through to memory,
// GS_SYS = sc0 | sc1) and counted with a system-scope atomic, after the
// stores have completed; a device-scope fence would instead write back the
// whole L2 of every workgroup's XCD.  The last workgroup resets its counter
// for the next call.  Not batch invariant (the split count follows B), and
// run to run deterministic (the merge order is the part order, not the
// arrival order).
constexpr int DEC_SYS = 17;   // buffer cache policy: sc0 | sc1, system scope

template <int D, int TW, int OUT_BF16>
__global__ void __launch_bounds__(DEC_THREADS)
decode_splitkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, float* __restrict__ ws, unsigned* __restrict__ cnt,
                      void* __restrict__ out, int64_t S, int splits, float scale) {
    constexpr int L = TW * DEC_WAVES;
    const int64_t bh = blockIdx.x / splits;
    const int c = blockIdx.x - (int)(bh * splits);
    const int64_t w0 = (int64_t)c * L + (int64_t)(threadIdx.x >> 6) * TW;
    DecContigKV<D> kv;
    kv.rk = row_rsrc(k + (bh * S) * D, S * D * 2);
    kv.rv = row_rsrc(v + (bh * S) * D, S * D * 2);
    kv.lane_off = (threadIdx.x & 63) % (D / 8) * 16;
    float* tp = ws + bh * splits * (int64_t)(2 + D);
    decode_chunk_body<D, 32, DecContigKV<D>, TW, DEC_SYS>(kv, q + bh * D, tp + c * (int64_t)(2 + D), w0,
                                                          min(S, w0 + TW), scale);
    // Count this part once its triple's stores have completed; the last part merges.
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt, expcnt and lgkmcnt all zero
    __syncthreads();
    __shared__ unsigned last;
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(&cnt[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
               (unsigned)(splits - 1);
    __syncthreads();
    if (!last) return;
    const __amdgpu_buffer_rsrc_t rt = row_rsrc(tp, (int64_t)splits * (2 + D) * 4);
    auto get = [&](int i) { return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * i, 0, DEC_SYS)); };
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float M = -INFINITY;
        for (int p = 0; p < splits; ++p) M = fmaxf(M, get(p * (2 + D)));
        float num = 0.0f, den = 0.0f;
        for (int p = 0; p < splits; ++p) {
            const float w = expf(get(p * (2 + D)) - M);
            num = fmaf(w, get(p * (2 + D) + 2 + d), num);
            den = fmaf(w, get(p * (2 + D) + 1), den);
        }
        store_out<OUT_BF16>(out, bh * D + d, num / den);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&cnt[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ void read_probe_kernel(const u32x4_t* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x) {
        const u32x4_t v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// Read shape of a GEMM's A copies: a matrix of 2 KiB rows read in tiles of
// 256 rows, each tile swept in column steps of BYTES bytes per row (lanes
// BYTES/16 to a row), four steps' loads in flight per thread, a persistent
// grid over the tiles.
template <int BYTES>
__global__ void __launch_bounds__(256) row_step_probe_kernel(const u32x4_t* __restrict__ p, int64_t tiles,
                                                             uint32_t* __restrict__ sink) {
    constexpr int LPR = BYTES / 16;          // lanes per row in one step
    constexpr int PER = LPR;                 // 16-byte pieces per thread and step (256 rows x LPR / 256)
    constexpr int STEPS = 2048 / BYTES;
    const int tid = threadIdx.x;
    uint32_t acc = 0;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const u32x4_t* base = p + t * (256 * 128);   // 256 rows x 128 pieces
#pragma unroll 4
        for (int st = 0; st < STEPS; ++st) {
            u32x4_t v[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int q = tid + 256 * i, row = q / LPR, c = q % LPR;
                v[i] = __builtin_nontemporal_load(base + row * 128 + st * LPR + c);
            }
#pragma unroll
            for (int i = 0; i < PER; ++i) acc ^= v[i][0] ^ v[i][3];
        }
    }
    sink[blockIdx.x * 256 + tid] = acc;
}

// One wave: the shared xor-butterfly sum and maximum of in[0 .. 63].
__global__ void __launch_bounds__(64) wave_reduce_kernel(const float* __restrict__ in, float* __restrict__ out) {
    const int l = threadIdx.x;
    const float v = in[l];
    out[l] = wave_sum(v);
    out[64 + l] = wave_max(v);
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace bi

using namespace bi;

extern "C" {

int bi_bench_gemm_grid(int64_t G, int64_t M, int64_t N, int64_t K, const void* A, int64_t sAg,
                       int64_t sAm, int64_t sAk, const void* B, int64_t sBg, int64_t sBk,
                       int64_t sBn, const void* bias, void* C, int64_t sCg, int64_t sCm,
                       int64_t sCn, int in_dtype, int out_dtype, int grid, void* stream) {
    if (grid < 1 || grid > 65535) return BI_ERR_UNSUPPORTED;
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = G; d.G2 = 1; d.M = M; d.N = N; d.K = K;
    d.A = A; d.sA1 = sAg; d.sAm = sAm; d.sAk = sAk;
    d.B = B; d.sB1 = sBg; d.sBk = sBk; d.sBn = sBn;
    d.bias = bias; d.C = C; d.sC1 = sCg; d.sCm = sCm; d.sCn = sCn;
    d.in_dtype = in_dtype; d.out_dtype = out_dtype;
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    return gemm_launch(d, (hipStream_t)stream, grid, 0);
}

int bi_bench_gemm_tile(int64_t G, int64_t M, int64_t N, int64_t K, const void* A, int64_t sAg,
                       int64_t sAm, int64_t sAk, const void* B, int64_t sBg, int64_t sBk,
                       int64_t sBn, const void* bias, int bias_rows, void* C, int64_t sCg, int64_t sCm,
                       int64_t sCn, int in_dtype, int out_dtype, int tile_rows, void* stream) {
    if (tile_rows != 0 && tile_rows != 1 && tile_rows != 2 && tile_rows != 3 && tile_rows != 4 &&
        (tile_rows < 16 || tile_rows > 19) && tile_rows != 32 && tile_rows != 64 && tile_rows != 128)
        return BI_ERR_UNSUPPORTED;
    if (in_dtype == BI_F32 && ((tile_rows >= 1 && tile_rows <= 4) || tile_rows > 32))
        return BI_ERR_UNSUPPORTED;
    if (in_dtype != BI_F32 && tile_rows >= 16 && tile_rows <= 19) return BI_ERR_UNSUPPORTED;
    if (bias_rows != 0 && bias_rows != 1) return BI_ERR_UNSUPPORTED;
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = G; d.G2 = 1; d.M = M; d.N = N; d.K = K;
    d.A = A; d.sA1 = sAg; d.sAm = sAm; d.sAk = sAk;
    d.B = B; d.sB1 = sBg; d.sBk = sBk; d.sBn = sBn;
    d.bias = bias; d.bias_rows = bias_rows;
    d.C = C; d.sC1 = sCg; d.sCm = sCm; d.sCn = sCn;
    d.in_dtype = in_dtype; d.out_dtype = out_dtype;
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    return gemm_launch(d, (hipStream_t)stream, 0, tile_rows);
}

int bi_bench_addmm_events(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
                          const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C, int64_t sCm,
                          int64_t sCn, int in_dtype, int out_dtype, void* start_event, void* stop_event,
                          void* stream) {
    if (!start_event || !stop_event) return BI_ERR_NULL;
    GemmDesc d = mm_desc(M, N, K, A, sAm, sAk, B, sBk, sBn, bias, C, sCm, sCn, in_dtype, out_dtype);
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    const LaunchEvents ev = {(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return gemm_launch(d, (hipStream_t)stream, 0, -1, &ev);
}

int bi_bench_gemm_shared_cu(int64_t G, int64_t M, int64_t N, int64_t K, const void* A, int64_t sAg,
                            int64_t sAm, int64_t sAk, const void* B, int64_t sBg, int64_t sBk,
                            int64_t sBn, const void* bias, void* C, int64_t sCg, int64_t sCm,
                            int64_t sCn, int in_dtype, int out_dtype, int grid, void* stream) {
    if (grid < 1 || grid > 65535) return BI_ERR_UNSUPPORTED;
    if (in_dtype != BI_BF16) return BI_ERR_DTYPE;
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = G; d.G2 = 1; d.M = M; d.N = N; d.K = K;
    d.A = A; d.sA1 = sAg; d.sAm = sAm; d.sAk = sAk;
    d.B = B; d.sB1 = sBg; d.sBk = sBk; d.sBn = sBn;
    d.bias = bias; d.C = C; d.sC1 = sCg; d.sCm = sCm; d.sCn = sCn;
    d.in_dtype = in_dtype; d.out_dtype = out_dtype;
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    if (G == 0 || M == 0 || N == 0) return BI_OK;
    const int osz = out_dtype == BI_F32 ? 4 : 2, vel = 16 / osz;
    // The vector epilogue only (16-byte row stores).
    if ((uintptr_t)C % 16 || N % vel || sCm % vel || sCg % vel) return BI_ERR_LAYOUT;
    const bool kc = K == 0 || (sBk == 1 && (N == 1 || sBn % 8 == 0));
    GemmParams p;
    p.A = (const uint16_t*)A; p.B = (const uint16_t*)B; p.bias = (const uint16_t*)bias; p.C = C;
    p.M = M; p.N = N; p.K = K;
    p.sAm = sAm; p.sBk = sBk; p.sBn = sBn; p.sCm = sCm;
    p.G2 = 1;
    p.sA1 = sAg; p.sA2 = 0; p.sB1 = sBg; p.sB2 = 0; p.sC1 = sCg; p.sC2 = 0; p.sBias2 = 0; p.bias_rows = 0;
    p.tiles_m = (int)cdiv(M, 128);
    p.tiles_n = (int)cdiv(N, 128);
    p.tiles_per_slice = p.tiles_m * p.tiles_n;
    p.total_tiles = (int)(p.tiles_per_slice * G);
    hipLaunchKernelGGL(gemm16_kernel_128x128_shared(kc ? 1 : 0, out_dtype == BI_F32 ? 0 : 1), dim3(grid),
                       dim3(G16_THREADS), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_gemm_tile_rows_for(int64_t G, int64_t M, int64_t N, int64_t K, int in_dtype, int cus) {
    if (G < 1 || M < 1 || N < 1 || K < 0 || cus < 1) return BI_ERR_SHAPE;
    if (in_dtype != BI_F32 && in_dtype != BI_BF16 && in_dtype != BI_F16) return BI_ERR_DTYPE;
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = G; d.G2 = 1; d.M = M; d.N = N; d.K = K; d.in_dtype = in_dtype;
    return gemm_tile_rows(d, cus);
}

int bi_bench_gemm_tile_rows(int64_t G, int64_t M, int64_t N, int64_t K, int in_dtype) {
    if (G < 1 || M < 1 || N < 1 || K < 0) return BI_ERR_SHAPE;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    return bi_bench_gemm_tile_rows_for(G, M, N, K, in_dtype, cus);
}

int bi_bench_splitk_policy(int64_t M, int64_t N, int64_t K, int rule) {
    if (M < 1 || N < 1 || K < 1) return BI_ERR_SHAPE;
    if (rule == 1) return (M < 64 && K % (8 * 4) == 0) ? 4 : 1;
    if (rule != 0) return BI_ERR_UNSUPPORTED;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    const int64_t tiles = cdiv(M, G16_BM) * cdiv(N, G16_BN);
    int s = (int)std::max<int64_t>(1, std::min<int64_t>(16, cus / tiles));
    while (s > 1 && K % (64 * s) != 0) --s;
    return s;
}

size_t bi_bench_addmm_splitk_workspace_bytes(int64_t M, int64_t N, int splits) {
    if (M < 0 || N < 0 || splits < 1) return 0;
    return (size_t)(splits * M * N * 4);
}

int bi_bench_addmm_splitk(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
                          const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C,
                          int64_t sCm, int64_t sCn, int in_dtype, int out_dtype, int splits,
                          void* ws, size_t ws_bytes, void* stream) {
    if (splits < 1 || splits > 64) return BI_ERR_UNSUPPORTED;
    if (K % (8 * splits) != 0) return BI_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return BI_OK;
    if (!C) return BI_ERR_NULL;
    if (!ws || ws_bytes < bi_bench_addmm_splitk_workspace_bytes(M, N, splits) || ((uintptr_t)ws % 16))
        return BI_ERR_WORKSPACE;
    if (sCn != 1 || sCm < N) return BI_ERR_LAYOUT;
    const int64_t Ks = K / splits;
    const int64_t esz = in_dtype == BI_BF16 ? 2 : 4;
    // Part s is slice s of a batched product over K offsets s*Ks.
    GemmDesc d;
    std::memset(&d, 0, sizeof(d));
    d.G1 = splits; d.G2 = 1; d.M = M; d.N = N; d.K = Ks;
    d.A = A; d.sA1 = Ks * sAk; d.sAm = sAm; d.sAk = sAk;
    d.B = B; d.sB1 = Ks * sBk; d.sBk = sBk; d.sBn = sBn;
    d.C = ws; d.sC1 = M * N; d.sCm = N; d.sCn = 1;
    d.in_dtype = in_dtype; d.out_dtype = BI_F32;
    (void)esz;
    int rc = gemm_check(d);
    if (rc != BI_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    rc = gemm_launch(d, st, 0);
    if (rc != BI_OK) return rc;
    const int grid = (int)std::min<int64_t>(cdiv(M * N, 256), 65535);
    const bool ob = out_dtype == BI_BF16, bb = in_dtype == BI_BF16;
    if (ob && bb)   hipLaunchKernelGGL((splitk_reduce_kernel<1, 1>), dim3(grid), dim3(256), 0, st, (const float*)ws, splits, M, N, bias, C, sCm);
    else if (ob)    hipLaunchKernelGGL((splitk_reduce_kernel<1, 0>), dim3(grid), dim3(256), 0, st, (const float*)ws, splits, M, N, bias, C, sCm);
    else if (bb)    hipLaunchKernelGGL((splitk_reduce_kernel<0, 1>), dim3(grid), dim3(256), 0, st, (const float*)ws, splits, M, N, bias, C, sCm);
    else            hipLaunchKernelGGL((splitk_reduce_kernel<0, 0>), dim3(grid), dim3(256), 0, st, (const float*)ws, splits, M, N, bias, C, sCm);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_decode_splits_policy(int64_t B, int sms) {
    if (B < 1 || sms < 1) return BI_ERR_SHAPE;
    return (int)std::max<int64_t>(1, std::min<int64_t>(64, sms / B));
}

size_t bi_bench_decode_attn_splits_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D,
                                                   int splits) {
    if (B < 0 || H < 0 || S < 1 || D < 1 || splits < 1 || S % splits) return 0;
    const int64_t L = S / splits;
    const int64_t nsub = L > DEC_CHUNK ? cdiv(L, DEC_CHUNK) : 1;
    return (size_t)(B * H * splits * nsub * (2 + D) * 4);
}

int bi_bench_decode_attn_splits(int64_t B, int64_t H, int64_t S, int64_t D, const void* q,
                                const void* k, const void* v, void* out, float scale, void* ws,
                                size_t ws_bytes, int in_dtype, int out_dtype, int splits,
                                void* stream) {
    if (in_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (B < 0 || H < 0 || S < 1) return BI_ERR_SHAPE;
    if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
    if (splits < 1 || splits > 64 || S % splits) return BI_ERR_UNSUPPORTED;
    const int64_t L = S / splits;
    if (L % 8) return BI_ERR_UNSUPPORTED;
    if (L > DEC_CHUNK && L % DEC_CHUNK) return BI_ERR_UNSUPPORTED;
    if ((S + DEC_CHUNK) * D * 2 >= (1ll << 31)) return BI_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return BI_OK;
    if (!q || !k || !v || !out) return BI_ERR_NULL;
    if (!ws || ws_bytes < bi_bench_decode_attn_splits_workspace_bytes(B, H, S, D, splits) ||
        ((uintptr_t)ws % 16))
        return BI_ERR_WORKSPACE;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    const int piece = (int)std::min<int64_t>(L, DEC_CHUNK);
    const int nsub = (int)(L / piece);
    const int64_t BH = B * H;
    const int npieces = splits * nsub;
    hipStream_t st = (hipStream_t)stream;
    float* wsf = (float*)ws;
    const dim3 g1((unsigned)(BH * npieces)), g2((unsigned)cdiv(BH * D, 256));
    if (D == 64) {
        hipLaunchKernelGGL((decode_chunk_kernel<64>), g1, dim3(DEC_THREADS), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wsf, S, npieces, piece, scale);
        if (out_dtype == BI_BF16) hipLaunchKernelGGL((decode_merge_parts_kernel<64, 1>), g2, dim3(256), 0, st, wsf, out, BH, splits, nsub);
        else                      hipLaunchKernelGGL((decode_merge_parts_kernel<64, 0>), g2, dim3(256), 0, st, wsf, out, BH, splits, nsub);
    } else {
        hipLaunchKernelGGL((decode_chunk_kernel<128>), g1, dim3(DEC_THREADS), 0, st,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wsf, S, npieces, piece, scale);
        if (out_dtype == BI_BF16) hipLaunchKernelGGL((decode_merge_parts_kernel<128, 1>), g2, dim3(256), 0, st, wsf, out, BH, splits, nsub);
        else                      hipLaunchKernelGGL((decode_merge_parts_kernel<128, 0>), g2, dim3(256), 0, st, wsf, out, BH, splits, nsub);
    }
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_decode_splitkv_policy(int64_t B, int64_t H, int64_t S, int cus) {
    if (B < 1 || H < 1 || S < 1 || cus < 1) return BI_ERR_SHAPE;
    // the longest part (2048 down to 256 tokens, dividing S) whose grid fills the CUs
    for (int64_t L = DEC_CHUNK; L >= 256; L /= 2)
        if (S % L == 0 && (B * H * (S / L) >= cus || L == 256)) return (int)(S / L);
    return BI_ERR_UNSUPPORTED;
}

size_t bi_bench_decode_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t D, int splits) {
    if (B < 0 || H < 0 || D < 1 || splits < 1) return 0;
    // triples, then one counter per (b, h)
    return (size_t)(B * H * splits * (2 + D) * 4 + B * H * 4);
}

int bi_bench_decode_attn_splitkv(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                                 const void* v, void* out, float scale, void* ws, size_t ws_bytes, int out_dtype,
                                 int splits, void* stream) {
    if (out_dtype != BI_F32 && out_dtype != BI_BF16) return BI_ERR_DTYPE;
    if (B < 0 || H < 0 || S < 1) return BI_ERR_SHAPE;
    if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
    if (splits < 1 || S % splits) return BI_ERR_UNSUPPORTED;
    const int64_t L = S / splits;
    if (L != 256 && L != 512 && L != 1024 && L != 2048) return BI_ERR_UNSUPPORTED;
    if ((S + DEC_CHUNK) * D * 2 >= (1ll << 31)) return BI_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return BI_OK;
    if (!q || !k || !v || !out) return BI_ERR_NULL;
    if (!ws || ws_bytes < bi_bench_decode_splitkv_workspace_bytes(B, H, D, splits) || ((uintptr_t)ws % 16))
        return BI_ERR_WORKSPACE;
    if (B * H * splits > (1ll << 30)) return BI_ERR_UNSUPPORTED;
    float* wsf = (float*)ws;
    unsigned* cnt = (unsigned*)(wsf + B * H * splits * (2 + D));
    typedef void (*Kern)(const uint16_t*, const uint16_t*, const uint16_t*, float*, unsigned*, void*, int64_t, int,
                         float);
    // [D 64/128][L 256/512/1024/2048][out bf16]
    static const Kern kerns[2][4][2] = {
        {{decode_splitkv_kernel<64, 32, 0>, decode_splitkv_kernel<64, 32, 1>},
         {decode_splitkv_kernel<64, 64, 0>, decode_splitkv_kernel<64, 64, 1>},
         {decode_splitkv_kernel<64, 128, 0>, decode_splitkv_kernel<64, 128, 1>},
         {decode_splitkv_kernel<64, 256, 0>, decode_splitkv_kernel<64, 256, 1>}},
        {{decode_splitkv_kernel<128, 32, 0>, decode_splitkv_kernel<128, 32, 1>},
         {decode_splitkv_kernel<128, 64, 0>, decode_splitkv_kernel<128, 64, 1>},
         {decode_splitkv_kernel<128, 128, 0>, decode_splitkv_kernel<128, 128, 1>},
         {decode_splitkv_kernel<128, 256, 0>, decode_splitkv_kernel<128, 256, 1>}}};
    const int li = L == 256 ? 0 : L == 512 ? 1 : L == 1024 ? 2 : 3;
    hipLaunchKernelGGL(kerns[D == 128][li][out_dtype == BI_BF16], dim3((unsigned)(B * H * splits)), dim3(DEC_THREADS),
                       0, (hipStream_t)stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wsf, cnt,
                       out, S, splits, scale);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_wave_reduce(const float* in, float* out, void* stream) {
    if (!in || !out) return BI_ERR_NULL;
    hipLaunchKernelGGL(wave_reduce_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, in, out);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_read_probe(const void* p, size_t bytes, void* sink, void* stream) {
    if (!p || !sink) return BI_ERR_NULL;
    if (bytes % 16 || ((uintptr_t)p % 16)) return BI_ERR_LAYOUT;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int grid = (int)std::min<int64_t>(std::max<int64_t>(1, cdiv(n16, 256)), std::min(65536, 16 * cus));
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4_t*)p, n16, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

int bi_bench_row_step_read(const void* p, size_t bytes, int step_bytes, void* sink, void* stream) {
    if (!p || !sink) return BI_ERR_NULL;
    constexpr size_t TILE = 256 * 2048;
    if (bytes == 0 || bytes % TILE || ((uintptr_t)p % 16)) return BI_ERR_LAYOUT;
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != BI_OK) return rc;
    const int64_t tiles = (int64_t)(bytes / TILE);
    const int grid = (int)std::min<int64_t>(tiles, cus);
    const hipStream_t st = (hipStream_t)stream;
    switch (step_bytes) {
        case 64:  hipLaunchKernelGGL(row_step_probe_kernel<64>, dim3(grid), dim3(256), 0, st, (const u32x4_t*)p, tiles, (uint32_t*)sink); break;
        case 128: hipLaunchKernelGGL(row_step_probe_kernel<128>, dim3(grid), dim3(256), 0, st, (const u32x4_t*)p, tiles, (uint32_t*)sink); break;
        default: return BI_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

}  // extern "C"
