"""GPU tests of the small-tile 16-bit GEMM (through the C ABI).

The library computes a 16-bit product either with the persistent 256x256
kernel or, where those tiles would leave most compute units idle, with
one-wave (32, 64 or 128) x 64 blocks, or with 128x256, 128x128 or 192x256
persistent tiles; the choice is a function of the shape.
Both must give the same bits for every element.  Here each forced tile size is
compared bit for bit with the persistent kernel on ragged shapes (M, N, K
tails, one row, K = 8), both B layouts, column bias (addmm) and row bias (the
convolution's output channels), binary32 and 16-bit outputs, bfloat16 and
binary16 operands, batched slices and padded output rows; the small-tile
results are also checked against the fp64 oracle.  The automatic choice is
checked on the shapes it is for: the batch-1 linear of the addmm workload and
the batch-1 SigLIP patch convolution.  Binary32 products have kernels of
their own (64x64 and 32x32 tiles, 16x16 blocks with one K chain per wave; the
same 16x16x4 MFMA chains per element), compared the same way.
"""
import pytest
import torch

import oracle
import synth
from helpers import assert_bf16_is_rne_of, assert_parity, bitwise_equal, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi, bi_bench
DEV = "cuda"
TILES = (1, 2, 3, 4, 32, 64, 128)   # 1 / 2 / 3 / 4: the persistent kernel with 128x256 / 256x128 / 128x128 / 192x256 tiles


def _operands(G, M, N, K, b_layout, dtype, seed):
    A = synth.randn((G, M, K), seed=seed, dtype=dtype)
    if b_layout == "n_contig":
        B = synth.randn((G, K, N), seed=seed + 1, dtype=dtype, scale=0.05)
    else:
        B = synth.randn((G, N, K), seed=seed + 1, dtype=dtype, scale=0.05).transpose(1, 2)
    return A, B


@pytest.mark.parametrize("G,M,N,K", [(1, 1, 40, 8), (1, 7, 264, 72), (1, 33, 96, 600), (2, 65, 136, 1000),
                                     (1, 130, 296, 4104), (3, 200, 32, 264), (1, 300, 520, 584)])
@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_small_tiles_equal_persistent_bf16(G, M, N, K, b_layout):
    A, B = _operands(G, M, N, K, b_layout, torch.bfloat16, seed=M + N + K)
    bias = synth.randn((N,), seed=K, dtype=torch.bfloat16, scale=0.02)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    for od in (bi.BI_F32, bi.BI_BF16):
        ref = bi_bench.gemm_tile(Ad, Bd, 0, bias=bd, out_dtype=od)
        outs = {t: bi_bench.gemm_tile(Ad, Bd, t, bias=bd, out_dtype=od) for t in TILES}
        torch.cuda.synchronize()
        for t, o in outs.items():
            assert bitwise_equal(o, ref), f"tile rows {t} differ from the persistent kernel (out {od})"
        if od == bi.BI_F32:
            f32 = outs[32]
        else:
            assert_bf16_is_rne_of(outs[32], f32, "small tile bf16 out")
    for g in range(G):
        assert_parity(to64(f32[g]), oracle.mm(A[g], B[g], bias), f"small tile {G}x{M}x{N}x{K} slice {g}")


@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_small_tiles_row_bias_and_no_bias(b_layout):
    # Row bias (one value per output row, as the convolution's channels) and no bias.
    G, M, N, K = 2, 100, 72, 592
    A, B = _operands(G, M, N, K, b_layout, torch.bfloat16, seed=11)
    rb = synth.randn((M,), seed=12, dtype=torch.bfloat16, scale=0.1)
    Ad, Bd, rbd = A.to(DEV), B.to(DEV), rb.to(DEV)
    for bias, rows in ((rbd, True), (None, False)):
        ref = bi_bench.gemm_tile(Ad, Bd, 0, bias=bias, bias_rows=rows, out_dtype=bi.BI_F32)
        outs = [bi_bench.gemm_tile(Ad, Bd, t, bias=bias, bias_rows=rows, out_dtype=bi.BI_F32) for t in TILES]
        torch.cuda.synchronize()
        for o in outs:
            assert bitwise_equal(o, ref), f"bias_rows={rows} differs from the persistent kernel"
        for g in range(G):
            want = oracle.mm(A[g], B[g])
            if bias is not None:
                want = want + rb.double().numpy()[:, None]
            assert_parity(to64(outs[0][g]), want, f"bias_rows={rows} slice {g}")


@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_small_tiles_equal_persistent_f16(b_layout):
    G, M, N, K = 1, 45, 200, 328
    A, B = _operands(G, M, N, K, b_layout, torch.float16, seed=21)
    bias = synth.randn((N,), seed=22, dtype=torch.float16, scale=0.02)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    for od in (bi.BI_F32, bi.BI_F16):
        ref = bi_bench.gemm_tile(Ad, Bd, 0, bias=bd, out_dtype=od)
        outs = [bi_bench.gemm_tile(Ad, Bd, t, bias=bd, out_dtype=od) for t in TILES]
        torch.cuda.synchronize()
        for o in outs:
            assert bitwise_equal(o, ref), f"binary16 small tile differs (out {od})"
    assert_parity(to64(bi_bench.gemm_tile(Ad, Bd, 32, bias=bd, out_dtype=bi.BI_F32)[0]),
                  oracle.mm(A[0], B[0], bias), "binary16 small tile")


def test_small_tiles_element_epilogue():
    # Outputs that allow no 4-wide stores (N % 4 != 0, written into a view
    # with padded rows) go through element stores: same bits.
    M, N, K = 37, 301, 136
    A = synth.randn((M, K), seed=31, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((N, K), seed=32, dtype=torch.bfloat16, scale=0.05).t().to(DEV)
    bias = synth.randn((N,), seed=33, dtype=torch.bfloat16).to(DEV)
    for od, tdt in ((bi.BI_F32, torch.float32), (bi.BI_BF16, torch.bfloat16)):
        big = torch.full((M, N + 3), 7.0, dtype=tdt, device=DEV)
        ref = bi_bench.gemm_tile(A, B, 0, bias=bias, out_dtype=od)
        for t in (1, 2, 3, 4, 32):
            big.fill_(7.0)
            out = bi_bench.gemm_tile(A, B, t, bias=bias, out_dtype=od, out=big[:, :N])
            torch.cuda.synchronize()
            assert bitwise_equal(out, ref), f"element epilogue changes the bits (tile {t})"
            assert torch.all(big[:, N:] == 7.0), f"a store landed past N (tile {t})"


def test_small_tile_k_zero():
    A = torch.empty(5, 0, dtype=torch.bfloat16, device=DEV)
    B = torch.empty(0, 40, dtype=torch.bfloat16, device=DEV)
    bias = synth.randn((40,), seed=41, dtype=torch.bfloat16).to(DEV)
    out = bi_bench.gemm_tile(A, B, 32, bias=bias, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert torch.equal(out, bias.float().expand(5, 40))


def test_auto_choice_on_batch1_linear_and_conv():
    # The shapes the small tile is for pick it, the large batch does not, and
    # every choice gives row 0 (sample 0) the same bits.
    assert bi_bench.gemm_tile_rows(1, 1, 14336, 4096) == 32
    assert bi_bench.gemm_tile_rows(1, 64, 14336, 4096) == 64
    assert bi_bench.gemm_tile_rows(1, 200, 14336, 4096) == 3      # 128x128 persistent tiles
    assert bi_bench.gemm_tile_rows(1, 512, 14336, 4096) == 1      # 128x256
    assert bi_bench.gemm_tile_rows(1, 8192, 14336, 4096) == 0
    assert bi_bench.gemm_tile_rows(1, 1152, 256, 592) == 32      # conv, one image
    assert bi_bench.gemm_tile_rows(4, 1152, 256, 592) == 3       # conv, 4 images
    assert bi_bench.gemm_tile_rows(1, 768, 14336, 4096) == 4      # 192x256, one round
    assert bi_bench.gemm_tile_rows(32, 1152, 256, 592) == 4      # conv, 32 images: 192x256
    assert bi_bench.gemm_tile_rows(48, 1152, 256, 592) == 0      # conv, 48 images
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(DEV), bias.to(DEV)
    X = synth.addmm_batch(x0, 200, device=DEV)
    auto = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
    forced = bi_bench.gemm_tile(X, Wd, 0, bias=bd, out_dtype=bi.BI_F32)
    one = bi.bi_addmm(bd, X[:1].contiguous(), Wd, out_dtype=bi.BI_F32)
    torch.cuda.synchronize()
    assert bitwise_equal(auto, forced), "the automatic choice changes the bits"
    assert bitwise_equal(one[0], forced[0]), "row 0 alone differs from row 0 in the batch"


@pytest.mark.parametrize("G,M,N,K", [(1, 1, 40, 4), (1, 37, 100, 130), (2, 70, 33, 512), (1, 200, 256, 4096),
                                     (1, 512, 512, 66), (2, 21, 47, 772), (1, 5, 30, 1284)])
@pytest.mark.parametrize("layout", ["plain", "transposed"])
def test_f32_tiles_same_bits(G, M, N, K, layout):
    # Binary32: 32x32 tiles (16x16 MFMA blocks, four K chains per wave) and
    # 16x16 blocks with the four chains on four waves (each operand staged
    # through LDS in stages of 256 k where its layout allows -- 1 to 16
    # stages here, ragged last stage -- or loaded directly, in all four
    # combinations), against 64x64 tiles, with the K
    # tail (K % 32 != 0, K % 4 != 0), ragged M and N, transposed views,
    # column and row bias, binary32 and bfloat16 outputs.
    A = synth.randn((G, M, K), seed=M + K, dtype=torch.float32)
    if layout == "plain":
        B = synth.randn((G, K, N), seed=N + K, dtype=torch.float32, scale=0.05)
    else:
        A = synth.randn((G, K, M), seed=M + K, dtype=torch.float32).transpose(1, 2)
        B = synth.randn((G, N, K), seed=N + K, dtype=torch.float32, scale=0.05).transpose(1, 2)
    cb = synth.randn((N,), seed=3, dtype=torch.float32, scale=0.02)
    rb = synth.randn((M,), seed=4, dtype=torch.float32, scale=0.02)
    Ad, Bd, cbd, rbd = A.to(DEV), B.to(DEV), cb.to(DEV), rb.to(DEV)
    for bias, rows in ((cbd, False), (rbd, True), (None, False)):
        for od in (bi.BI_F32, bi.BI_BF16):
            big = bi_bench.gemm_tile(Ad, Bd, 0, bias=bias, bias_rows=rows, out_dtype=od)
            small = bi_bench.gemm_tile(Ad, Bd, 32, bias=bias, bias_rows=rows, out_dtype=od)
            torch.cuda.synchronize()
            assert bitwise_equal(small, big), f"fp32 32x32 tiles differ (bias_rows={rows}, out {od})"
            for t in (16, 17, 18, 19):
                split = bi_bench.gemm_tile(Ad, Bd, t, bias=bias, bias_rows=rows, out_dtype=od)
                torch.cuda.synchronize()
                assert bitwise_equal(split, big), f"fp32 split chains {t} differ (bias_rows={rows}, out {od})"
    for t in (32, 16, 17, 18, 19):
        out = bi_bench.gemm_tile(Ad, Bd, t, bias=cbd, out_dtype=bi.BI_F32)
        torch.cuda.synchronize()
        for g in range(G):
            assert_parity(to64(out[g]), oracle.mm(A[g], B[g], cb), f"fp32 kernel {t} slice {g}")
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert bi_bench.gemm_tile_rows(G, M, N, K, bi.BI_F32) == (32 if M == 512 else 16)
