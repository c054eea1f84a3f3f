"""GPU parity and invariance of bi_mm / bi_addmm / bi_bmm (through the C ABI).

Parity: binary32 outputs against the fp64 oracle on the same seeded inputs,
at sizes spanning several 256x256 tiles with ragged M/N tails, and at the
full addmm shape (K=4096, N=14336) on sampled rows.  Invariance: row 0 is bit
for bit the same at every batch size; slices of a batched product equal the
plain product; repeated calls are identical.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_bf16_is_rne_of, assert_bf16_rounding, assert_parity,
                     assert_within_dot_bound, bitwise_equal, to64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------- bf16
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (70, 264, 512), (300, 520, 584), (513, 256, 64),
                                   (257, 1000, 136)])
@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_bf16_addmm_parity_ragged(M, N, K, b_layout):
    A = synth.randn((M, K), seed=M + 1, dtype=torch.bfloat16)
    if b_layout == "n_contig":
        B = synth.randn((K, N), seed=N + 2, dtype=torch.bfloat16, scale=0.05)
    else:
        B = synth.randn((N, K), seed=N + 2, dtype=torch.bfloat16, scale=0.05).t()
    bias = synth.randn((N,), seed=K + 3, dtype=torch.bfloat16, scale=0.02)
    ref = oracle.mm(A, B, bias)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    C32 = bi.bi_addmm(bd, Ad, Bd, out_dtype=bi.BI_F32)
    C16 = bi.bi_addmm(bd, Ad, Bd, out_dtype=bi.BI_BF16)
    Cmm = bi.bi_mm(Ad, Bd, out_dtype=bi.BI_F32)
    _sync()
    assert_parity(to64(C32), ref, f"addmm {M}x{N}x{K} {b_layout}")
    assert_parity(to64(Cmm), oracle.mm(A, B), f"mm {M}x{N}x{K} {b_layout}")
    assert_bf16_is_rne_of(C16, C32, "addmm bf16 out")
    assert_bf16_rounding(C16, ref, "addmm bf16 out")


@pytest.mark.parametrize("case", ["n_mod8_is_4", "n_odd_kcontig", "padded_ldc", "misaligned_c"])
def test_bf16_epilogue_paths_same_bits(case):
    # The output layout picks the epilogue (16-byte row stores staged through
    # LDS, or element stores): values must not depend on it, and both must
    # match the oracle, including the ragged row and column tails.
    M, N, K = {"n_mod8_is_4": (300, 260, 192), "n_odd_kcontig": (129, 301, 136),
               "padded_ldc": (200, 256, 72), "misaligned_c": (77, 264, 64)}[case]
    A = synth.randn((M, K), seed=M, dtype=torch.bfloat16)
    if N % 8:   # an N-contiguous B needs N % 8 == 0
        B = synth.randn((N, K), seed=N, dtype=torch.bfloat16, scale=0.1).t()
    else:
        B = synth.randn((K, N), seed=N, dtype=torch.bfloat16, scale=0.1)
    bias = synth.randn((N,), seed=K, dtype=torch.bfloat16, scale=0.1)
    ref = oracle.mm(A, B, bias)
    Ad, Bd, bd = A.to(DEV), B.to(DEV), bias.to(DEV)
    outs = {}
    for od, tdt in ((bi.BI_F32, torch.float32), (bi.BI_BF16, torch.bfloat16)):
        plain = bi.bi_addmm(bd, Ad, Bd, out_dtype=od)
        if case == "padded_ldc":
            buf = torch.full((M, N + 4), 7.0, dtype=tdt, device=DEV)
            odd = buf[:, :N]
        elif case == "misaligned_c":
            buf = torch.full((M * N + 1,), 7.0, dtype=tdt, device=DEV)
            odd = buf[1:].view(M, N)
        else:
            buf, odd = None, torch.empty((M, N), dtype=tdt, device=DEV)
        bi.bi_addmm(bd, Ad, Bd, out=odd, out_dtype=od)
        _sync()
        assert bitwise_equal(plain, odd), f"{case}: epilogue path changed the bits ({tdt})"
        if case == "padded_ldc":
            assert torch.all(buf[:, N:] == 7.0), "padding columns were written"
        if case == "misaligned_c":
            assert buf[0].item() == 7.0, "element before C was written"
        outs[od] = plain
    assert_parity(to64(outs[bi.BI_F32]), ref, f"epilogue {case}")
    assert_bf16_is_rne_of(outs[bi.BI_BF16], outs[bi.BI_F32], f"epilogue {case} bf16")


def test_bf16_layouts_give_identical_bits():
    # The two B layouts feed the same MFMA chain: results must match bit for bit.
    M, N, K = 130, 264, 320
    A = synth.randn((M, K), seed=5, dtype=torch.bfloat16).to(DEV)
    Bn = synth.randn((K, N), seed=6, dtype=torch.bfloat16).to(DEV)
    Bk = Bn.t().contiguous().t()
    assert Bk.stride(0) == 1
    c1 = bi.bi_mm(A, Bn, out_dtype=bi.BI_F32)
    c2 = bi.bi_mm(A, Bk, out_dtype=bi.BI_F32)
    _sync()
    assert bitwise_equal(c1, c2)


def test_bf16_closed_forms_exact():
    M, N, K = 100, 272, 640
    A = synth.randn((M, K), seed=7, dtype=torch.bfloat16)
    eye = torch.eye(K, dtype=torch.bfloat16)
    got = bi.bi_mm(A.to(DEV), eye[:, :N].contiguous().to(DEV), out_dtype=bi.BI_F32)
    ones = bi.bi_addmm(torch.full((N,), 0.5, dtype=torch.bfloat16, device=DEV),
                       torch.ones(M, K, dtype=torch.bfloat16, device=DEV),
                       torch.ones(K, N, dtype=torch.bfloat16, device=DEV), out_dtype=bi.BI_F32)
    _sync()
    assert torch.equal(got.cpu(), A[:, :N].float())
    assert torch.all(ones == K + 0.5)


@pytest.mark.parametrize("b_layout", ["n_contig", "k_contig"])
def test_bf16_small_integers_bitwise_equal_oracle(b_layout):
    M, N, K = 260, 304, 1024
    A = synth.randint((M, K), -4, 4, seed=8, dtype=torch.bfloat16)
    B = synth.randint((K, N), -4, 4, seed=9, dtype=torch.bfloat16)
    if b_layout == "k_contig":
        B = B.t().contiguous().t()
    bias = synth.randint((N,), -50, 50, seed=10, dtype=torch.bfloat16)
    got = bi.bi_addmm(bias.to(DEV), A.to(DEV), B.to(DEV), out_dtype=bi.BI_F32)
    _sync()
    assert np.array_equal(to64(got), oracle.mm(A, B, bias))


def test_bf16_k_zero_and_empty():
    A = torch.empty(5, 0, dtype=torch.bfloat16, device=DEV)
    B = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    bias = torch.full((16,), 2.0, dtype=torch.bfloat16, device=DEV)
    C = bi.bi_addmm(bias, A, B, out_dtype=bi.BI_F32)
    E = bi.bi_mm(torch.empty(0, 8, dtype=torch.bfloat16, device=DEV),
                 torch.empty(8, 16, dtype=torch.bfloat16, device=DEV))
    _sync()
    assert torch.all(C == 2.0) and E.shape == (0, 16)


def test_addmm_full_shape_row0_invariant_and_sampled_parity():
    """The addmm workload: X [M, 4096], W [4096, 14336], bias; row 0 bitwise
    equal for M in {1, 63, 64, 200, 2048, 8192}; sampled rows of M=8192 and
    all of M=63 against the oracle."""
    W, bias, x0 = synth.addmm_shared()
    Wd, bd = W.to(DEV), bias.to(DEV)
    row0_16, row0_32 = {}, {}
    for M in (1, 63, 64, 200, 2048, 8192):
        X = synth.addmm_batch(x0, M, device=DEV)
        C16 = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_BF16)
        C32 = bi.bi_addmm(bd, X, Wd, out_dtype=bi.BI_F32)
        _sync()
        row0_16[M], row0_32[M] = C16[0].clone(), C32[0].clone()
        if M == 8192:
            rows = [0, 1, 255, 256, 4097, 8191]
            Xs = X[rows].cpu()
            ref = oracle.mm(Xs, W, bias)
            assert_parity(to64(C32[rows]), ref, "addmm M=8192 sampled rows")
            assert_bf16_rounding(C16[rows], ref, "addmm M=8192 bf16 rows")
            assert_bf16_is_rne_of(C16, C32, "addmm M=8192")
        if M == 63:
            ref = oracle.mm(X.cpu(), W, bias)
            assert_parity(to64(C32), ref, "addmm M=63")
        del X, C16, C32
    for M in row0_16:
        assert bitwise_equal(row0_16[M], row0_16[1]), f"row 0 (bf16 out) differs at M={M}"
        assert bitwise_equal(row0_32[M], row0_32[1]), f"row 0 (fp32 out) differs at M={M}"


def test_repeat_determinism_1000():
    # The run-to-run check of the temperature-determinism page: 2048^2 bf16, 1000 calls.
    A = synth.randn((2048, 2048), seed=11, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((2048, 2048), seed=12, dtype=torch.bfloat16).to(DEV)
    ref = bi.bi_mm(A, B)
    out = torch.empty_like(ref)
    diff = torch.zeros((), dtype=torch.float32, device=DEV)
    for _ in range(1000):
        bi.bi_mm(A, B, out=out)
        diff = torch.maximum(diff, (out.float() - ref.float()).abs().max())
    _sync()
    assert diff.item() == 0.0


def test_linspace_batch_dependence_shape():
    # The batch-dependence demo of the temperature-determinism page, with a
    # bf16 operand: mm(a[:1], b) must equal mm(a, b)[:1] exactly.
    Bsz, D = 2048, 4096
    a = torch.linspace(-100, 100, Bsz * D).reshape(Bsz, D).to(torch.bfloat16).to(DEV)
    b = torch.linspace(-100, 100, D * D).reshape(D, D).to(torch.bfloat16).to(DEV)
    o1 = bi.bi_mm(a[:1], b, out_dtype=bi.BI_F32)
    o2 = bi.bi_mm(a, b, out_dtype=bi.BI_F32)
    _sync()
    assert bitwise_equal(o1[0], o2[0])
    # The sums cancel almost completely (row 0 of a is ~-100 throughout, each
    # column of b runs from -100 to 100), so the relative error of the result
    # is unbounded; the binary32 dot-product bound gamma_K * sum |a||b| holds.
    a0, bc = a[:1].cpu(), b.cpu()
    ref = oracle.mm(a0, bc)
    mag = oracle.mm(a0.abs(), bc.abs())
    assert_within_dot_bound(to64(o1), ref, mag, K=D)


# ------------------------------------------------------------------- bmm
def test_bmm_slices_equal_mm_and_parity():
    G, M, N, K = 5, 300, 264, 136
    A = synth.randn((G, M, K), seed=13, dtype=torch.bfloat16)
    B = synth.randn((G, N, K), seed=14, dtype=torch.bfloat16).transpose(1, 2)   # K-contiguous
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = bi.bi_bmm(Ad, Bd, out_dtype=bi.BI_F32)
    per = [bi.bi_mm(Ad[g], Bd[g], out_dtype=bi.BI_F32) for g in range(G)]
    _sync()
    for g in range(G):
        assert bitwise_equal(C[g], per[g]), f"slice {g} differs from bi_mm"
    assert_parity(to64(C), oracle.bmm(A, B), "bmm")


def test_bmm_broadcast_operand():
    G, M, N, K = 3, 64, 256, 64
    A = synth.randn((M, K), seed=15, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((G, K, N), seed=16, dtype=torch.bfloat16).to(DEV)
    C = bi.bi_bmm(A.unsqueeze(0).expand(G, M, K), B, out_dtype=bi.BI_F32)
    _sync()
    for g in range(G):
        assert bitwise_equal(C[g], bi.bi_mm(A, B[g], out_dtype=bi.BI_F32))


# ------------------------------------------------------------------ fp32
def test_mm_fp32_row0_invariant_and_parity():
    """The mm workload: W randn [4096, 256] fp32, X rows randn, row 0 shared
    across M in {1, 8, 63, 64, 200}."""
    W, X = synth.mm_inputs()
    Wd = W.to(DEV)
    outs = {}
    for M, Xm in X.items():
        C = bi.bi_mm(Xm.to(DEV), Wd)
        _sync()
        outs[M] = C
        assert_parity(to64(C), oracle.mm(Xm, W), f"mm fp32 M={M}")
    for M in outs:
        assert bitwise_equal(outs[M][0], outs[1][0]), f"row 0 differs at M={M}"


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (4, 256, 281), (65, 130, 47), (200, 64, 4096)])
def test_fp32_mm_parity_strided(M, N, K):
    A = synth.randn((K, M), seed=17, dtype=torch.float32).t()       # M-contiguous view
    B = synth.randn((K, N), seed=18, dtype=torch.float32)
    bias = synth.randn((N,), seed=19, dtype=torch.float32)
    C = bi.bi_addmm(bias.to(DEV), A.to(DEV), B.to(DEV))
    _sync()
    assert_parity(to64(C), oracle.mm(A, B, bias), f"fp32 addmm {M}x{N}x{K}")


def test_fp32_bmm_profiler_shape():
    # The attention-weights @ values shape of the VLA page's profiler table:
    # [32, 8, 4, 281] @ [32, 8, 281, 256] in binary32, flattened to 256 slices.
    A = synth.randn((256, 4, 281), seed=20)
    B = synth.randn((256, 281, 256), seed=21)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = bi.bi_bmm(Ad, Bd)
    C8 = bi.bi_bmm(Ad[:8], Bd[:8])
    _sync()
    assert bitwise_equal(C[:8], C8)
    assert_parity(to64(C[:16]), oracle.bmm(A[:16], B[:16]), "fp32 bmm 4x281x256")
