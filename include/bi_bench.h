/*
 * bi_bench.h — benchmark and test variants of the bi_* operations (libbi_bench.so).
 *
 * NOT part of the product interface.  These entry points exist to measure the
 * cost of batch invariance and to show that the invariance tests can tell a
 * batch-dependent schedule apart: they implement the batch-size-dependent
 * splits that the deterministic-inference handbook page (anrans.github.io,
 * section "根源：浮点加法的顺序") describes as the cause of batch dependence, and
 * a grid override for the invariant GEMM.  libbi_bench.so also exports every
 * bi.h entry point.  Conventions (device pointers, element strides, void*
 * stream, bi_status return codes, caller-owned workspaces) are those of bi.h.
 */
#ifndef BI_BENCH_H
#define BI_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "bi.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bi_bench_gemm_grid — the invariant GEMM of bi_bmm (with an optional column
 * bias, as bi_addmm) launched on a forced persistent grid of `grid`
 * workgroups (1 <= grid <= 65535).  Its results must equal bi_bmm's bit for
 * bit at any grid: the tile arithmetic does not depend on which workgroup
 * runs a tile.
 */
int bi_bench_gemm_grid(int64_t G, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
                       const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
                       const void* bias,
                       void* C, int64_t sCg, int64_t sCm, int64_t sCn,
                       int in_dtype, int out_dtype, int grid, void* stream);

/*
 * bi_bench_gemm_tile — the invariant GEMM of bi_bmm with the kernel forced.
 * 16-bit operands: tile_rows 0 = the persistent kernel with 256x256 tiles,
 * 1 = the persistent kernel with 128x256 tiles, 2 = with 256x128 tiles,
 * 3 = with 128x128 tiles, 4 = with 192x256 tiles, 32 / 64 / 128 = the
 * small-tile kernel with (tile_rows x 64) blocks, one wave each.
 * Binary32 operands: 0 = 64x64 tiles, 32 = 32x32 tiles, 16 = one
 * workgroup per 16x16 block with its four K chains on four waves, each
 * operand staged through LDS where its layout allows (A k-contiguous with
 * 16-byte aligned rows and K % 4 == 0; B column-contiguous with 16-byte
 * aligned k rows and N % 4 == 0), else loaded directly; 17 = the same with
 * both operands loaded directly, 18 = only B staged (where it can be), 19 =
 * only A staged (others: BI_ERR_UNSUPPORTED; 16 to 19 BI_ERR_UNSUPPORTED
 * where a 16x16 block's operands span 2^31 bytes or more).  bias (or NULL) is indexed by column (bias_rows 0, as
 * bi_addmm) or by row (1, as the convolution's output channels).  Every
 * tile_rows gives the same bits as bi_bmm / bi_addmm, which choose the kernel
 * from the shape (the choice is reported by bi_bench_gemm_tile_rows).
 */
int bi_bench_gemm_tile(int64_t G, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
                       const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
                       const void* bias, int bias_rows,
                       void* C, int64_t sCg, int64_t sCm, int64_t sCn,
                       int in_dtype, int out_dtype, int tile_rows, void* stream);

/*
 * bi_bench_addmm_events — bi_addmm (same arguments, checks, kernel choice
 * and bits) with the GEMM kernel launched through hipExtLaunchKernelGGL, so
 * that the runtime records start_event / stop_event (hipEvent_t, created
 * with timing enabled, owned by the caller) when the kernel itself starts
 * and ends: hipEventElapsedTime between them is the kernel's execution time
 * without the launch gap that events recorded around the call include.
 * M or N = 0 launches nothing and records nothing.  BI_ERR_NULL if an
 * event is NULL; otherwise bi_addmm's status.
 */
int bi_bench_addmm_events(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
                          const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C,
                          int64_t sCm, int64_t sCn, int in_dtype, int out_dtype,
                          void* start_event, void* stop_event, void* stream);

/*
 * bi_bench_gemm_shared_cu — the invariant GEMM of bi_bmm (bfloat16 operands,
 * optional column bias as bi_addmm) on the persistent kernel with 128x128
 * tiles compiled without its LDS reservation (66 KiB per workgroup instead of
 * 81), launched on `grid` workgroups (1 <= grid <= 65535): with a grid above
 * the compute-unit count two of its workgroups share a compute unit.  Output
 * layouts that allow 16-byte row stores only (else BI_ERR_LAYOUT).  Its
 * results must equal bi_bmm's bit for bit.
 */
int bi_bench_gemm_shared_cu(int64_t G, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
                            const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
                            const void* bias,
                            void* C, int64_t sCg, int64_t sCm, int64_t sCn,
                            int in_dtype, int out_dtype, int grid, void* stream);

/*
 * bi_bench_gemm_tile_rows — the tile_rows that bi_bmm (G slices) or
 * bi_addmm / bi_mm (G = 1) pick for an M x N x K product on the current
 * device: 0, 1, 2, 3, 4, 32, 64 or 128 for 16-bit operands, 0, 32 or 16
 * for binary32.  Negative bi_status on a bad shape or without a gfx950 device.
 */
int bi_bench_gemm_tile_rows(int64_t G, int64_t M, int64_t N, int64_t K, int in_dtype);

/*
 * bi_bench_gemm_tile_rows_for — the same choice for a device with `cus`
 * compute units (host arithmetic only: callable without a GPU).
 * BI_ERR_SHAPE on a bad shape or cus < 1, BI_ERR_DTYPE on an unknown dtype.
 */
int bi_bench_gemm_tile_rows_for(int64_t G, int64_t M, int64_t N, int64_t K, int in_dtype, int cus);

/*
 * bi_bench_splitk_policy — the number of K splits a batch-size-tuned GEMM
 * would pick for an M x N x K product.
 *   rule 0: fill the compute units: splits = clamp(CUs / tiles, 1, 16),
 *           tiles = ceil(M/256) * ceil(N/256), reduced until K splits evenly
 *           into multiples of 64 (needs a current device);
 *   rule 1: the handbook's simulation: 4 if M < 64 else 1.
 * Returns the split count (>= 1) or a negative bi_status.
 */
int bi_bench_splitk_policy(int64_t M, int64_t N, int64_t K, int rule);

/* Workspace of bi_bench_addmm_splitk: splits * M * N binary32 partial sums. */
size_t bi_bench_addmm_splitk_workspace_bytes(int64_t M, int64_t N, int splits);

/*
 * bi_bench_addmm_splitk — C = A @ B + bias with K cut into `splits` equal
 * parts (K % (8 * splits) == 0): each part is an independent invariant GEMM
 * into ws, then the parts are added in part order and the bias is added.
 * Layout rules: those of bi_addmm.  A different split count gives different
 * bits: this is the batch-dependent schedule the invariant path forbids.
 */
int bi_bench_addmm_splitk(int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t sAm, int64_t sAk,
                          const void* B, int64_t sBk, int64_t sBn,
                          const void* bias,
                          void* C, int64_t sCm, int64_t sCn,
                          int in_dtype, int out_dtype, int splits,
                          void* ws, size_t ws_bytes, void* stream);

/* The handbook's load-based split count: max(1, min(64, sms / B)). */
int bi_bench_decode_splits_policy(int64_t B, int sms);

size_t bi_bench_decode_attn_splits_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D,
                                                   int splits);

/*
 * bi_bench_decode_attn_splits — decode attention with the KV sequence cut
 * into `splits` equal parts (S % splits == 0, S / splits a multiple of 8)
 * instead of fixed 2048-token chunks.  Parts longer than 2048 tokens are
 * computed as 2048-token pieces merged inside the part, then the parts are
 * merged in order.  Arguments as bi_decode_attn.
 */
int bi_bench_decode_attn_splits(int64_t B, int64_t H, int64_t S, int64_t D,
                                const void* q, const void* k, const void* v, void* out,
                                float scale, void* ws, size_t ws_bytes,
                                int in_dtype, int out_dtype, int splits, void* stream);

/*
 * bi_bench_decode_attn_splitkv — decode attention (bfloat16 q, K, V as in
 * bi_decode_attn, contiguous) split by load, as a fair batch-size-tuned
 * competitor of the fixed 2048-token chunks: each (b, h) is cut into
 * `splits` parts of L = S / splits tokens (L in {256, 512, 1024, 2048}, else
 * BI_ERR_UNSUPPORTED), one workgroup per part with its 8 waves taking L / 8
 * tokens each, and the parts' triples are merged in part order in the same
 * launch by the workgroup that finishes a (b, h) last.  NOT batch
 * invariant when the split count follows B (bi_bench_decode_splitkv_policy).
 * ws: bi_bench_decode_splitkv_workspace_bytes(B, H, D, splits) bytes,
 * 16-byte aligned, ZEROED by the caller before its first use (the last
 * B * H words are counters that every call leaves at zero again).  Calls
 * that share a workspace must not overlap.  bi_bench_decode_splitkv_policy
 * gives the split count S / L for the longest L in {2048, 1024, 512, 256}
 * dividing S whose grid of B * H * S / L workgroups fills `cus` compute units
 * (L = 256 if none does; BI_ERR_UNSUPPORTED if 256 does not divide S).
 */
int bi_bench_decode_splitkv_policy(int64_t B, int64_t H, int64_t S, int cus);
size_t bi_bench_decode_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t D, int splits);
int bi_bench_decode_attn_splitkv(int64_t B, int64_t H, int64_t S, int64_t D, const void* q, const void* k,
                                 const void* v, void* out, float scale, void* ws, size_t ws_bytes, int out_dtype,
                                 int splits, void* stream);

/*
 * bi_bench_read_probe — streams `bytes` (a multiple of 16) from `p` with
 * 16-byte loads and writes one reduction word per workgroup to `sink`
 * (at least 4 * 65536 bytes), to measure the achievable HBM read rate.
 */
int bi_bench_read_probe(const void* p, size_t bytes, void* sink, void* stream);

/*
 * bi_bench_row_step_read — reads `bytes` (a non-zero multiple of 512 KiB,
 * `p` 16-byte aligned) as a matrix of 2 KiB rows, in tiles of 256 rows, each
 * tile swept in column steps of `step_bytes` (64 or 128) per row: the
 * request shape of a GEMM's operand copies of one or two K steps.  One
 * workgroup per CU (at most one per tile) loops over the tiles; each writes
 * 256 reduction words to `sink` (at least 1024 * CUs bytes).  Errors:
 * BI_ERR_NULL, BI_ERR_LAYOUT, BI_ERR_UNSUPPORTED (other step sizes).
 */
int bi_bench_row_step_read(const void* p, size_t bytes, int step_bytes, void* sink, void* stream);

/*
 * bi_bench_wave_reduce — one wave of 64 lanes: lane l holds in[l] (binary32,
 * 64 values) and writes the library's wave-wide xor-butterfly sum to out[l]
 * and maximum to out[64 + l] (out: 128 values).  Exposes the reduction the
 * softmax, row operations and attention probabilities share, so that a test
 * can pin its order (offsets 32, 16, ..., 1) bit for bit.
 */
int bi_bench_wave_reduce(const float* in, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_BENCH_H */
