"""The shape-only kernel choice of the 16-bit and binary32 GEMM, on the host.

bi_bench_gemm_tile_rows_for evaluates the library's choice for a device with
a given number of compute units without touching a GPU.  Every candidate
kernel computes each element with the same instruction chain (the GPU tests
compare them bit for bit), so the choice only affects speed; these checks pin
it on the shapes it was fitted to on a 256-CU MI355X (the addmm with K = 4096,
N = 14336 at batch sizes 1 to 8192, the patch convolution's GEMM at 1 to 48
images, the attention products) and check that it only ever returns a kernel
that exists for the operand type.
"""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "invariant_persistent_bf16_amd", "libbi_bench.so")
F32, BF16, F16 = 0, 1, 2
SHAPE, DTYPE = -2, -3
i64 = ctypes.c_int64


@pytest.fixture(scope="module")
def choose():
    if not os.path.exists(LIB):
        pytest.skip("libbi_bench.so not built")
    L = ctypes.CDLL(LIB)
    f = L.bi_bench_gemm_tile_rows_for
    f.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    f.restype = ctypes.c_int
    return lambda G, M, N, K, dt=BF16, cus=256: f(G, M, N, K, dt, cus)


# 0 = 256x256, 1 = 128x256, 2 = 256x128, 3 = 128x128, 4 = 192x256 persistent
# tiles; 32 / 64 / 128 = one-wave small tiles of that many rows (binary32:
# 32 = 32x32 tiles, 16 = 16x16 blocks with one K chain per wave).  Each entry
# is the fastest kernel measured for the shape (graph replay, same box).
ADDMM = {1: 32, 16: 32, 32: 32, 64: 64, 96: 3, 128: 3, 200: 3, 256: 3, 384: 1, 512: 1,
         576: 4, 768: 4, 1024: 0, 1152: 1, 1536: 1, 2048: 0, 8192: 0}
CONV = {1: 32, 4: 3, 8: 3, 16: 1, 24: 1, 32: 4, 48: 0}


@pytest.mark.parametrize("M,want", sorted(ADDMM.items()))
def test_addmm_batch_sizes(choose, M, want):
    assert choose(1, M, 14336, 4096) == want
    assert choose(1, M, 14336, 4096, F16) == want      # binary16 takes the same kernels


@pytest.mark.parametrize("B,want", sorted(CONV.items()))
def test_patch_conv_gemm(choose, B, want):
    assert choose(B, 1152, 256, 592) == want


def test_attention_products_and_binary32(choose):
    assert choose(256, 1024, 1024, 128) == 0     # Q K^T
    assert choose(256, 1024, 128, 1024) == 2     # P V: N = 128 fills half of a 256-wide tile
    assert choose(1, 200, 256, 4096, F32) == 16  # binary32: one chain per wave on 16x16 blocks
    assert choose(1, 512, 512, 66, F32) == 32    # binary32: 32x32 tiles, four chains per wave
    assert choose(1, 4096, 4096, 1024, F32) == 0


def test_only_existing_kernels(choose):
    allowed16, allowed32 = {0, 1, 2, 3, 4, 32, 64, 128}, {0, 16, 32}
    for cus in (80, 256, 304):
        for G in (1, 3, 64):
            for M in (1, 7, 100, 1000, 5000):
                for N in (8, 128, 129, 1000, 14336):
                    for K in (0, 8, 600, 4096):
                        assert choose(G, M, N, K, BF16, cus) in allowed16
                        assert choose(G, M, N, K, F32, cus) in allowed32
                        r = choose(G, M, N, K, BF16, cus)
                        if r == 2:
                            assert N <= 128                # the 256x128 tile only for narrow N


def test_errors(choose):
    assert choose(1, 0, 8, 8) == SHAPE
    assert choose(0, 8, 8, 8) == SHAPE
    assert choose(1, 8, 8, -1) == SHAPE
    assert choose(1, 8, 8, 8, BF16, 0) == SHAPE
    assert choose(1, 8, 8, 8, 7) == DTYPE
