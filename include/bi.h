/*
 * bi.h — batch-invariant dense contractions for AMD Instinct MI355X (gfx950).
 *
 * Every entry point computes each output row with a reduction order fixed by
 * the operation's own shape parameters that do not count requests (K, the
 * kernel size, the sequence length) and never by the batch dimension (M, G,
 * N of the convolution, B of decode): the same request gives the same bits
 * whether it is computed alone or inside any batch.  The method follows the
 * persistent matmul of "Unmasking the True Culprit: Why Temperature=0 Doesn't
 * Mean Deterministic LLM Inference" (section "Technical Deep Dive: Batch
 * Invariant Kernels": a reduction order fixed per dtype, float32 tile
 * accumulation, ascending K loop, no split-K; here the order is fixed by the
 * matrix instruction and the K step, while the output tile may be chosen
 * from the shape since it never changes an element's order), the per-sample
 * Conv2d and
 * batched matmul of "Batch-Invariant Kernel Design: Conv2d and Attention BMM"
 * (sections "Kernel 1: Conv2d" and "Kernel 2: Attention BMM"), and the
 * fixed-length split-KV decoding of the deterministic-inference handbook
 * page (anrans.github.io, section "根源：浮点加法的顺序" and the list of
 * batch-invariant rules after it).
 *
 * Conventions shared by every call
 *   - Plain C ABI; all data pointers are DEVICE pointers; all strides are
 *     int64 ELEMENT strides.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  Work is enqueued on that stream and the
 *     library never synchronises.
 *   - Ownership: the caller owns every buffer, outputs and workspaces
 *     included.  The library allocates no device memory and keeps no mutable
 *     global state (it caches the read-only compute-unit count per device),
 *     apart from the per-thread timing events of bi_set_launch_events.
 *   - Dtypes: BI_F32 = IEEE binary32, BI_BF16 = bfloat16, BI_F16 = IEEE
 *     binary16 (the matmul family and the convolution only).  Accumulation is
 *     always binary32.  16-bit outputs are the binary32 result rounded to
 *     nearest-even, bit for bit the same as rounding the BI_F32 output.
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     a negative bi_status is returned and nothing runs.  A failed launch
 *     returns BI_ERR_LAUNCH.  Faults inside a kernel surface at the caller's
 *     next synchronisation.  No exception crosses the ABI.
 *   - Outputs must not overlap inputs.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BI_F32 = 0, BI_BF16 = 1, BI_F16 = 2 } bi_dtype;

typedef enum {
    BI_OK = 0,
    BI_ERR_NULL = -1,        /* a required pointer is NULL */
    BI_ERR_SHAPE = -2,       /* negative or inconsistent sizes */
    BI_ERR_DTYPE = -3,       /* dtype code not accepted by this entry point */
    BI_ERR_LAYOUT = -4,      /* strides / alignment the kernels do not take */
    BI_ERR_UNSUPPORTED = -5, /* valid request outside what is implemented */
    BI_ERR_WORKSPACE = -6,   /* workspace NULL, too small or misaligned */
    BI_ERR_LAUNCH = -7,      /* the HIP runtime refused a launch or query */
    BI_ERR_DEVICE = -8,      /* no usable gfx950 device is current */
    BI_ERR_SCRATCH = -9      /* more than a no-allocation entry point's static scratch */
} bi_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* bi_status_string(int status);

/*
 * bi_mm — C[M,N] = A[M,K] @ B[K,N].
 * Source: "Unmasking the True Culprit ..." section "Technical Deep Dive:
 * Batch Invariant Kernels" (persistent matmul kernel and its host wrapper).
 *
 * A: element (i,k) at A[i*sAm + k*sAk]; B: (k,j) at B[k*sBk + j*sBn];
 * C: (i,j) at C[i*sCm + j*sCn].  in_dtype is the dtype of A and B,
 * out_dtype the dtype of C: BI_F32, or the 16-bit in_dtype (BI_BF16 is also
 * accepted for BI_F32 operands).  BI_F16 operands run the bfloat16 kernel's
 * tile, K order and schedule on the binary16 matrix-core instruction: one
 * fixed configuration per dtype, as the source's per-dtype table (whose fp16
 * entry is a wider tile for its hardware).
 * Reduction: k ascending in fixed steps of the dtype's K tile; each output
 * tile is owned by one workgroup from the first k to the last (no split-K,
 * no atomics).  Row i of C depends only on row i of A, B, K and the dtypes.
 * Layout accepted:
 *   BI_BF16, BI_F16: sAk == 1, sAm % 8 == 0, A 16-byte aligned, K % 8 == 0;
 *            B either K-contiguous (sBk == 1, sBn % 8 == 0) or N-contiguous
 *            (sBn == 1, sBk % 8 == 0, N % 8 == 0), 16-byte aligned;
 *            C with sCn == 1.
 *   BI_F32:  any non-negative strides; C with sCn == 1.
 * M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 */
int bi_mm(int64_t M, int64_t N, int64_t K,
          const void* A, int64_t sAm, int64_t sAk,
          const void* B, int64_t sBk, int64_t sBn,
          void* C, int64_t sCm, int64_t sCn,
          int in_dtype, int out_dtype, void* stream);

/*
 * bi_addmm — C = A @ B + bias, bias [N] of in_dtype broadcast over rows
 * (beta = alpha = 1, the only form the method registers).  The bias is
 * widened to binary32 and added once, after the last K step, then the sum is
 * rounded once to out_dtype.  bias == NULL gives bi_mm.
 * Source: as bi_mm; the wrapper's bias argument and the addmm override in
 * "Integration with PyTorch: The torch.Library Approach".
 * Layout rules: as bi_mm; bias is contiguous and aligned to its element.
 */
int bi_addmm(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t sAm, int64_t sAk,
             const void* B, int64_t sBk, int64_t sBn,
             const void* bias,
             void* C, int64_t sCm, int64_t sCn,
             int in_dtype, int out_dtype, void* stream);

/*
 * bi_bmm — C[g] = A[g] @ B[g] for g in [0, G).
 * Source: "Batch-Invariant Kernel Design: Conv2d and Attention BMM", section
 * "Kernel 2: Attention BMM".  Slice g is a product of its own: its operands
 * start g slice strides into A, B and C, and its K sum runs in the order any
 * other slice uses, so G never enters its arithmetic.  Slice g of the result
 * is bit-identical to bi_mm on A[g], B[g] alone.
 * Element strides sAg, sBg, sCg step between slices (0 broadcasts an operand).
 * Layout rules per slice: as bi_mm, and for 16-bit dtypes sAg % 8 == sBg % 8 == 0.
 */
int bi_bmm(int64_t G, int64_t M, int64_t N, int64_t K,
           const void* A, int64_t sAg, int64_t sAm, int64_t sAk,
           const void* B, int64_t sBg, int64_t sBk, int64_t sBn,
           void* C, int64_t sCg, int64_t sCm, int64_t sCn,
           int in_dtype, int out_dtype, void* stream);

/*
 * bi_conv2d — non-transposed 2-D convolution, NCHW.
 * Source: "Batch-Invariant VLAs", section "Replacing nn.Conv2d" (per-sample
 * unfold, flattened-kernel product, bias), and "Batch-Invariant Kernel
 * Design ...", section "Kernel 1: Conv2d" (stride, padding, dilation,
 * groups).  Lowered to an explicit unfold into the workspace, laid out
 * [n][g][location][k] with k = ci*Kh*Kw + kh*Kw + kw zero-padded to a
 * multiple of 8, followed by the batched GEMM above with one slice per
 * (sample, group): y[n, g*Cout/G + c, :] = Wg[c, :] @ U[n, g] + bias.
 *
 * x [N, Cin, H, W] contiguous; w [Cout, Cin/groups, Kh, Kw] contiguous;
 * bias [Cout] or NULL; y [N, Cout, OH, OW] contiguous with
 * OH = (H + 2*ph - dh*(Kh-1) - 1)/sh + 1 (and OW likewise).
 * x, w, bias are in_dtype (BI_BF16, BI_F16 or BI_F32); y is out_dtype (as
 * bi_mm).
 * ws: device workspace of at least bi_conv2d_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller, contents undefined on return.
 * Errors: BI_ERR_SHAPE if Cin or Cout is not divisible by groups or the
 * output would be empty; BI_ERR_WORKSPACE if ws is too small.
 */
size_t bi_conv2d_workspace_bytes(int64_t N, int64_t Cin, int64_t H, int64_t W,
                                 int64_t Cout, int64_t Kh, int64_t Kw,
                                 int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                                 int64_t dh, int64_t dw, int64_t groups, int in_dtype);
int bi_conv2d(int64_t N, int64_t Cin, int64_t H, int64_t W, const void* x,
              int64_t Cout, int64_t Kh, int64_t Kw, const void* w, const void* bias,
              int64_t sh, int64_t sw, int64_t ph, int64_t pw,
              int64_t dh, int64_t dw, int64_t groups,
              void* y, void* ws, size_t ws_bytes,
              int in_dtype, int out_dtype, void* stream);

/*
 * bi_decode_attn — single-query attention per (b, h) over a KV cache,
 * split into fixed-length chunks of bi_decode_chunk_tokens() tokens counted
 * from position 0 (the last chunk may be shorter).
 * Source: the deterministic-inference handbook page, section
 * "根源：浮点加法的顺序" (flash-decoding experiment: per-chunk max, sum of
 * exponentials and exp-weighted V sum, merged by the log-sum-exp rule) and
 * its rule that split-KV must cut by a fixed length (2048 tokens for decode)
 * rather than a fixed number of parts.
 *
 *   s_t = scale * (q . k_t);  per chunk c: m_c = max s_t, l_c = sum e^{s_t-m_c},
 *   o_c = sum e^{s_t-m_c} v_t;  out = sum_c e^{m_c-M} o_c / sum_c e^{m_c-M} l_c,
 *   M = max_c m_c, chunks merged in ascending order.
 *
 * q [B, H, D], k and v [B, H, S, D], out [B, H, D], all contiguous.
 * in_dtype must be BI_BF16; out_dtype BI_F32 or BI_BF16.  D must be 64 or 128.
 * ws: at least bi_decode_attn_workspace_bytes(B, H, S, D) bytes, 16-byte
 * aligned; receives the per-chunk triples [B, H, nchunk, 2 + D] (binary32:
 * m, l, o[D]) and is owned by the caller.
 * BI_ERR_UNSUPPORTED when (S + 2048) * D * 2 >= 2^31 (one (b, h) row of K or
 * V is addressed with 32-bit byte offsets), or D is not 64 or 128.
 */
size_t bi_decode_attn_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D);
int bi_decode_attn(int64_t B, int64_t H, int64_t S, int64_t D,
                   const void* q, const void* k, const void* v, void* out,
                   float scale, void* ws, size_t ws_bytes,
                   int in_dtype, int out_dtype, void* stream);

/*
 * bi_decode_attn_noalloc — bi_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it).
 * Same arguments, layouts, kernels and bits as bi_decode_attn; the chunk
 * triples go to a static device array of BI_DECODE_SCRATCH_BYTES per GPU
 * (held from the library's first use on that GPU until the process ends).
 * The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine.  Its first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress).
 * Errors: those of bi_decode_attn except BI_ERR_WORKSPACE, and
 * BI_ERR_SCRATCH when bi_decode_attn_workspace_bytes(B, H, S, D) exceeds
 * BI_DECODE_SCRATCH_BYTES, i.e. B * H * ceil(S / 2048) above 127100 chunks
 * at D = 64 or 64527 at D = 128 (B = 256, H = 32, S = 8192 is 32768).
 * Calls on one GPU share its array: two calls whose kernels overlap on that
 * GPU (different streams, or different host threads without ordering) race
 * and may return wrong results; calls ordered on one stream are safe.
 */
#define BI_DECODE_SCRATCH_BYTES (32u << 20)
int bi_decode_attn_noalloc(int64_t B, int64_t H, int64_t S, int64_t D,
                           const void* q, const void* k, const void* v, void* out,
                           float scale, int in_dtype, int out_dtype, void* stream);

/* The fixed KV chunk length of bi_decode_attn (2048, the handbook's decode split). */
int bi_decode_chunk_tokens(void);

/*
 * bi_decode_attn_paged — bi_decode_attn for a batch of requests of their own
 * lengths whose K and V live in a paged cache.
 * Source: the deterministic-inference handbook page, sections "与 batch 无关：
 * 固定切分" (fixed-length KV split, chunk boundaries at absolute token
 * positions) and "框架里的开关" (chunked prefill and the prefix cache must
 * leave a request's results unchanged), applied to the flash-decoding
 * experiment of section "根源：浮点加法的顺序".
 *
 * Request b attends over its first len_b = seq_lens[b] tokens; token t of it
 * is row t % page_size of page block_table[b * max_pages + t / page_size].
 * The chunks are [2048c, 2048c + 2048) ∩ [0, len_b) and the arithmetic is that
 * of bi_decode_attn, so request b's output has the bits bi_decode_attn gives
 * for B = 1, S = len_b on the same values, whatever the other requests, their
 * lengths, max_pages, max_seq_len or where its pages are placed.
 *
 * q [B, H, D] contiguous; k_cache, v_cache [num_pages, H, page_size, D]
 * contiguous (one page holds page_size tokens of every head);
 * block_table [B, max_pages] int32 contiguous (device memory; entries past a
 * request's ceil(len_b / page_size) pages are not read); seq_lens [B] int32
 * (device memory); out [B, H, D].  page_size must be a power of two with
 * max_seq_len <= max_pages * page_size.  max_seq_len (host) bounds every
 * len_b and sizes the grid and ws: a length outside [0, max_seq_len] is
 * clamped to it, a page id outside [0, num_pages) reads page 0 (no access
 * leaves the caches; the result is then meaningless).  len_b = 0 gives NaN.
 * in_dtype must be BI_BF16; out_dtype BI_F32 or BI_BF16; D 64 or 128.
 * ws: at least bi_decode_attn_paged_workspace_bytes(B, H, max_seq_len, D)
 * bytes, 16-byte aligned, owned by the caller.
 * BI_ERR_UNSUPPORTED when max_seq_len + 2048 >= 2^31 or page_size * D * 2
 * >= 2^31 (32-bit token and in-page offsets).
 */
size_t bi_decode_attn_paged_workspace_bytes(int64_t B, int64_t H, int64_t max_seq_len, int64_t D);
int bi_decode_attn_paged(int64_t B, int64_t H, int64_t D, const void* q,
                         const void* k_cache, const void* v_cache,
                         int64_t num_pages, int64_t page_size,
                         const int32_t* block_table, int64_t max_pages,
                         const int32_t* seq_lens, int64_t max_seq_len,
                         void* out, float scale, void* ws, size_t ws_bytes,
                         int in_dtype, int out_dtype, void* stream);

/*
 * bi_prefill_attn_paged — causal attention of a batch of prefill chunks over
 * a paged KV cache, the KV split at a fixed length of 4096 tokens.
 * Source: the deterministic-inference handbook page, section "与 batch 无关：
 * 固定切分" (attention splits KV by a fixed length, 4096 tokens for prefill;
 * a request's KV and attention must not depend on how its prompt was cut into
 * prefill chunks or whether its prefix came from the cache), with the
 * per-chunk triple and log-sum-exp merge of section "根源：浮点加法的顺序".
 *
 * Request b owns query rows cu_q[b] .. cu_q[b+1]-1 of q [total_q, H, D]
 * (contiguous); row cu_q[b] + j is at position pos = q_pos0[b] + j and
 * attends to the request's keys 0 .. pos, key t stored at row t % page_size
 * of page block_table[b * max_pages + t / page_size] of k_cache and v_cache
 * [num_pages, H, page_size, D] (the caller has written the chunk's own keys
 * and values there).  With x_t = (q . k_t) * fl(scale * log2 e) in binary32,
 * each 4096-token chunk c of keys gives m_c = max x_t, l_c = sum 2^(x_t - m_c),
 * o_c = sum 2^(x_t - m_c) v_t, merged in ascending c:
 *   out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c.
 * A query's bits depend only on its position and the keys: the same prompt
 * prefilled in one call or in chunks (each with its q_pos0), alone or in a
 * batch, gives the same bits per query.
 *
 * cu_q [B+1], q_pos0 [B], block_table [B, max_pages]: int32 device memory.
 * max_q and max_kv_len (host) size the grid: every request has at most max_q
 * queries and q_pos0[b] + (its query count) <= max_kv_len <= max_pages *
 * page_size; device values outside these bounds are clamped (no access
 * leaves the buffers; the result is then meaningless), a page id outside
 * [0, num_pages) reads page 0.  out [total_q, H, D], 16-byte aligned.
 * in_dtype BI_BF16; out_dtype BI_F32 or BI_BF16; D must be 128; page_size a
 * power of two.  ws: bi_prefill_attn_paged_workspace_bytes(total_q, H,
 * max_kv_len, D) bytes, 16-byte aligned, owned by the caller (0 bytes, and ws
 * may be null, when max_kv_len <= 4096).
 */
size_t bi_prefill_attn_paged_workspace_bytes(int64_t total_q, int64_t H, int64_t max_kv_len, int64_t D);
int bi_prefill_attn_paged(int64_t B, int64_t H, int64_t D, const void* q, int64_t total_q,
                          const int32_t* cu_q, const int32_t* q_pos0, int64_t max_q,
                          const void* k_cache, const void* v_cache,
                          int64_t num_pages, int64_t page_size,
                          const int32_t* block_table, int64_t max_pages, int64_t max_kv_len,
                          void* out, float scale, void* ws, size_t ws_bytes,
                          int in_dtype, int out_dtype, void* stream);

/*
 * bi_softmax_rows — P[r, :] = softmax(scale * S[r, :]) for each row, in
 * binary32: max, exponentials, their sum and the division, with one
 * wave per row and a reduction tree fixed by `cols` alone (the
 * row-per-program reduction of "Unmasking the True Culprit ...", section
 * "Beyond Matrix Multiplication").  It is the glue between the two batched
 * products of attention (S = Q @ K^T, P = softmax(scale * S), O = P @ V).
 * S: binary32 with row stride ldS (unit column stride), 4-byte aligned;
 * P: out_dtype (BI_F32 or BI_BF16) with row stride ldP, element aligned.
 * Rows that are 16-byte aligned (8-byte for a bfloat16 P) with cols, ldS
 * and ldP multiples of 4 are read and written with vector accesses; the
 * result bits are the same either way.  rows == 0 or cols == 0: nothing.
 * Errors: BI_ERR_DTYPE, BI_ERR_SHAPE (negative sizes), BI_ERR_NULL,
 * BI_ERR_LAYOUT (ld < cols with rows > 1, misaligned), BI_ERR_UNSUPPORTED
 * (cols > 2^24), BI_ERR_DEVICE.
 */
int bi_softmax_rows(int64_t rows, int64_t cols, const void* S, int64_t ldS, float scale,
                    void* P, int64_t ldP, int out_dtype, void* stream);

/*
 * bi_attention_probs — P[g, t, :] = softmax(scale * Q[g, t, :] @ K[g]^T) in
 * bfloat16, for g < G, t < T, over Tk keys, with the bits of the two-stage
 * path: bi_bmm(Q, K^T) into binary32 S, then bi_softmax_rows(S, scale) to
 * bfloat16 P ("Batch-Invariant Kernel Design: Conv2d and Attention BMM",
 * section "Kernel 2: Attention BMM"; the softmax of "Unmasking the True
 * Culprit ...", section "Beyond Matrix Multiplication").  S is not written
 * to memory: a workgroup keeps a slice's keys in registers and a block of 32
 * query rows' scores in LDS.  Q: bfloat16 (g, t, d) at Q[g*sQg + t*sQt + d];
 * K: (g, j, d) at K[g*sKg + j*sKt + d] (d contiguous, rows 16-byte aligned:
 * Q, K 16-byte aligned and their strides multiples of 8); P: bfloat16 (g, t,
 * j) at P[g*sPg + t*sPt + j], 8-byte aligned, strides multiples of 4.
 * D in {64, 128}, Tk in {256, 512, 768, 1024} (else BI_ERR_UNSUPPORTED).
 * G == 0 or T == 0: nothing.  Errors before any launch: BI_ERR_SHAPE
 * (negative sizes), BI_ERR_NULL, BI_ERR_LAYOUT, BI_ERR_UNSUPPORTED,
 * BI_ERR_DEVICE.
 */
int bi_attention_probs(int64_t G, int64_t T, int64_t Tk, int64_t D, const void* Q, int64_t sQg,
                       int64_t sQt, const void* K, int64_t sKg, int64_t sKt, float scale, void* P,
                       int64_t sPg, int64_t sPt, void* stream);

/*
 * Row operations beside the matmul, each row reduced by one wave (one
 * workgroup for rows longer than 4096) in an order fixed by `cols` alone, never
 * by the number of rows ("Unmasking the True Culprit ...", section "Beyond
 * Matrix Multiplication"; the deterministic-inference handbook page, section
 * "与 batch 无关：固定切分").  Row r of x is x[r * ldx + j] (unit column stride),
 * in_dtype BI_F32 or BI_BF16 (widened exactly); arithmetic in binary32; the
 * output is out_dtype, bfloat16 by round-to-nearest-even of the binary32
 * result.  Rows that are 16-byte (binary32) or 8-byte (bfloat16) aligned with
 * cols and the leading dimensions multiples of 4 use vector accesses; the
 * bits are the same either way.  rows == 0 (or cols == 0 where allowed): no
 * work.  Errors before any launch: BI_ERR_DTYPE, BI_ERR_SHAPE (negative
 * sizes), BI_ERR_NULL, BI_ERR_LAYOUT (ld < cols with rows > 1, an element
 * misaligned), BI_ERR_UNSUPPORTED (cols > 2^24), BI_ERR_DEVICE.
 */

/*
 * bi_rms_norm — y[r, j] = (x[r, j] * s_r) * w[j],
 * s_r = 1 / sqrt(sum_i x[r, i]^2 / cols + eps) (section "Batch-Invariant
 * RMSNorm": the squares summed in a fixed order, divided by cols, then the
 * reciprocal square root; eps >= 0, finite, else BI_ERR_SHAPE).  w: [cols],
 * in_dtype, 4-byte (binary32) or 2-byte aligned.  y: [rows, cols] with ldy.
 */
int bi_rms_norm(int64_t rows, int64_t cols, const void* x, int64_t ldx, const void* w, float eps,
                void* y, int64_t ldy, int in_dtype, int out_dtype, void* stream);

/*
 * bi_log_softmax_rows — y[r, j] = (x[r, j] - m_r) - log(sum_i exp(x[r, i] - m_r)),
 * m_r = max_i x[r, i] (section "Log-Softmax with Fixed Reduction Strategy").
 * exp is the hardware base-2 exponential of (x - m) * log2(e); log and the
 * sums are binary32.  y: [rows, cols] with ldy.
 */
int bi_log_softmax_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* y, int64_t ldy,
                        int in_dtype, int out_dtype, void* stream);

/*
 * bi_mean_rows — y[r] = sum_j x[r, j] / cols (the overridden mean over the
 * last dimension in the first page's operator list; the handbook's "求均值").
 * y: [rows] contiguous.  cols == 0 with rows > 0: BI_ERR_SHAPE.
 */
int bi_mean_rows(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* y, int in_dtype,
                 int out_dtype, void* stream);

/*
 * bi_set_launch_events — attach timing events to the library's own kernels.
 * For callers that time the entry points' kernels without a profiler (events
 * recorded around a call also time the event packets and the launch gaps).
 *
 * start, stop: hipEvent_t values passed as void*, created with timing
 * enabled and recorded at least once; the caller owns them.  After the call,
 * the first kernel that any entry point launches from this host thread
 * records start when it begins, and every kernel launched from this thread
 * records stop when it ends, so once the calls complete, the elapsed time
 * between the events is the time from the first kernel's start to the last
 * one's end.  stop == NULL clears the setting (start is then ignored); a new
 * call restarts it.  Entry points that launch no kernel (empty shapes,
 * argument errors) leave the events untouched.  Returns BI_OK.
 */
int bi_set_launch_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
