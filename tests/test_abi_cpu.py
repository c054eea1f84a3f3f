"""C-ABI checks that need no GPU: the built libraries load, export every
function their headers declare, and reject bad arguments on the host with the
documented status code before touching a device (no compute call is made).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "invariant_persistent_bf16_amd")
HEADERS = {"bi.h": "libbi.so", "bi_bench.h": "libbi_bench.so"}

OK, NULL, SHAPE, DTYPE, LAYOUT, UNSUP, WS = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
P = 0x10000          # a fake, 64 KiB-aligned "device" pointer: never dereferenced
i64 = ctypes.c_int64


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_\w+)\s*\(", text)))


def load(name):
    path = os.path.join(PKG, name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not built")
    return ctypes.CDLL(path)


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_library_exports_every_declared_symbol(header):
    if not os.path.exists(os.path.join(ROOT, "include", header)):
        pytest.skip(f"{header} absent")
    lib = load(HEADERS[header])
    names = declared(header)
    assert names, "no declarations found"
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"{HEADERS[header]} lacks {missing}"


@pytest.fixture(scope="module")
def bi():
    L = load("libbi.so")
    vp = ctypes.c_void_p
    L.bi_mm.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, ctypes.c_int,
                        ctypes.c_int, vp]
    L.bi_addmm.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp, i64, i64,
                           ctypes.c_int, ctypes.c_int, vp]
    L.bi_bmm.argtypes = [i64, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64,
                         i64, ctypes.c_int, ctypes.c_int, vp]
    L.bi_conv2d_workspace_bytes.restype = ctypes.c_size_t
    L.bi_conv2d_workspace_bytes.argtypes = [i64] * 14 + [ctypes.c_int]
    L.bi_conv2d.argtypes = [i64, i64, i64, i64, vp, i64, i64, i64, vp, vp] + [i64] * 7 + \
        [vp, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
    L.bi_decode_attn_workspace_bytes.restype = ctypes.c_size_t
    L.bi_decode_attn_workspace_bytes.argtypes = [i64] * 4
    L.bi_decode_attn.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_float, vp,
                                 ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
    L.bi_decode_attn_paged_workspace_bytes.restype = ctypes.c_size_t
    L.bi_decode_attn_paged_workspace_bytes.argtypes = [i64] * 4
    L.bi_decode_attn_paged.argtypes = [i64, i64, i64, vp, vp, vp, i64, i64, vp, i64, vp, i64, vp,
                                       ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
    L.bi_prefill_attn_paged_workspace_bytes.restype = ctypes.c_size_t
    L.bi_prefill_attn_paged_workspace_bytes.argtypes = [i64] * 4
    L.bi_prefill_attn_paged.argtypes = [i64, i64, i64, vp, i64, vp, vp, i64, vp, vp, i64, i64, vp, i64, i64, vp,
                                        ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
    L.bi_softmax_rows.argtypes = [i64, i64, vp, i64, ctypes.c_float, vp, i64, ctypes.c_int, vp]
    L.bi_attention_probs.argtypes = [i64, i64, i64, i64, vp, i64, i64, vp, i64, i64, ctypes.c_float, vp,
                                     i64, i64, vp]
    L.bi_rms_norm.argtypes = [i64, i64, vp, i64, vp, ctypes.c_float, vp, i64, ctypes.c_int, ctypes.c_int, vp]
    L.bi_log_softmax_rows.argtypes = [i64, i64, vp, i64, vp, i64, ctypes.c_int, ctypes.c_int, vp]
    L.bi_mean_rows.argtypes = [i64, i64, vp, i64, vp, ctypes.c_int, ctypes.c_int, vp]
    L.bi_status_string.restype = ctypes.c_char_p
    return L


def mm(L, M=64, N=64, K=64, A=P, sAm=64, sAk=1, B=P, sBk=64, sBn=1, C=P, sCm=64, sCn=1,
       ind=BF16, outd=F32):
    return L.bi_mm(M, N, K, A, sAm, sAk, B, sBk, sBn, C, sCm, sCn, ind, outd, None)


def test_status_strings(bi):
    for code in (OK, NULL, SHAPE, DTYPE, LAYOUT, UNSUP, WS, -7, -8, 12345):
        assert bi.bi_status_string(code)
    assert bi.bi_status_string(LAYOUT).startswith(b"BI_ERR_LAYOUT")


def test_gemm_validation(bi):
    assert mm(bi, ind=7) == DTYPE
    assert mm(bi, outd=2) == DTYPE
    assert mm(bi, M=-1) == SHAPE
    assert mm(bi, C=None) == NULL
    assert mm(bi, A=None) == NULL
    assert mm(bi, sAk=2) == LAYOUT                 # bf16 A must be K-contiguous
    assert mm(bi, sAm=60) == LAYOUT                # 16-byte rows
    assert mm(bi, A=P + 2) == LAYOUT               # 16-byte aligned
    assert mm(bi, K=60, sAm=64) == LAYOUT          # K % 8
    assert mm(bi, sBk=2, sBn=3) == LAYOUT          # B neither K- nor N-contiguous
    assert mm(bi, N=60, sBk=64, sBn=1, sCm=64) == LAYOUT   # N-contiguous B needs N % 8
    assert mm(bi, sCn=2) == LAYOUT
    assert mm(bi, sAm=-64) == LAYOUT
    assert mm(bi, sAm=1 << 24) == UNSUP            # 32-bit in-tile offsets
    assert mm(bi, ind=F32, A=P + 2) == LAYOUT      # fp32 needs 4-byte alignment
    # Empty problems are no-ops that never reach the device.
    assert mm(bi, M=0) == OK
    assert mm(bi, N=0) == OK
    assert bi.bi_bmm(0, 4, 4, 8, P, 0, 8, 1, P, 0, 4, 1, P, 0, 4, 1, BF16, F32, None) == OK
    assert bi.bi_bmm(-1, 4, 4, 8, P, 0, 8, 1, P, 0, 4, 1, P, 0, 4, 1, BF16, F32, None) == SHAPE
    assert bi.bi_bmm(2, 4, 8, 8, P, 4, 8, 1, P, 0, 8, 1, P, 0, 8, 1, BF16, F32, None) == LAYOUT
    assert bi.bi_addmm(4, 8, 8, P, 8, 1, P, 8, 1, P + 1, P, 8, 1, BF16, F32, None) == LAYOUT


def siglip_ws(bi, N=32):
    return bi.bi_conv2d_workspace_bytes(N, 3, 224, 224, 1152, 14, 14, 14, 14, 0, 0, 1, 1, 1, BF16)


def test_conv_workspace_size_and_validation(bi):
    # packed weight 1152 x 592 bf16 (256-byte rounded) + unfold 32 x 256 x 592 bf16
    assert siglip_ws(bi) == 1152 * 592 * 2 + 32 * 256 * 592 * 2
    assert siglip_ws(bi, N=1) == 1152 * 592 * 2 + 256 * 592 * 2
    assert bi.bi_conv2d_workspace_bytes(1, 3, 8, 8, 4, 3, 3, 1, 1, 0, 0, 1, 1, 2, BF16) == 0

    def conv(**kw):
        a = dict(N=2, Cin=3, H=28, W=28, x=P, Cout=4, Kh=14, Kw=14, w=P, bias=None, sh=14, sw=14,
                 ph=0, pw=0, dh=1, dw=1, groups=1, y=P, ws=P, ws_bytes=1 << 20, ind=BF16, outd=F32)
        a.update(kw)
        return bi.bi_conv2d(*a.values(), None)

    assert conv(groups=2) == SHAPE            # Cin % groups
    assert conv(sh=0) == SHAPE
    assert conv(H=5) == SHAPE                 # empty output
    assert conv(ind=3) == DTYPE
    assert conv(outd=3) == DTYPE
    assert conv(x=None) == NULL
    assert conv(ws=None) == WS
    assert conv(ws_bytes=100) == WS
    assert conv(ws=P + 16) == WS              # 256-byte aligned workspace
    assert conv(N=0) == OK


def test_decode_workspace_size_and_validation(bi):
    assert bi.bi_decode_attn_workspace_bytes(256, 32, 8192, 64) == 256 * 32 * 4 * 66 * 4
    assert bi.bi_decode_attn_workspace_bytes(1, 1, 2049, 128) == 2 * 130 * 4

    def dec(**kw):
        a = dict(B=2, H=2, S=4096, D=64, q=P, k=P, v=P, out=P, scale=0.125, ws=P, ws_bytes=1 << 20,
                 ind=BF16, outd=F32)
        a.update(kw)
        return bi.bi_decode_attn(*a.values(), None)

    assert dec(ind=F32) == DTYPE
    assert dec(outd=9) == DTYPE
    assert dec(S=0) == SHAPE
    assert dec(D=96) == UNSUP
    assert dec(k=None) == NULL
    assert dec(ws=None) == WS
    assert dec(ws_bytes=8) == WS
    assert dec(q=P + 8) == LAYOUT
    assert dec(B=0) == OK


def test_paged_decode_workspace_size_and_validation(bi):
    assert bi.bi_decode_attn_paged_workspace_bytes(256, 32, 8192, 64) == 256 * 32 * 4 * 66 * 4
    assert bi.bi_decode_attn_paged_workspace_bytes(3, 2, 2049, 128) == 3 * 2 * 2 * 130 * 4
    assert bi.bi_decode_attn_paged_workspace_bytes(3, 2, 0, 128) == 0

    def dec(**kw):
        a = dict(B=2, H=2, D=64, q=P, kc=P, vc=P, num_pages=64, page=16, bt=P, max_pages=32, sl=P,
                 max_seq=512, out=P, scale=0.125, ws=P, ws_bytes=1 << 20, ind=BF16, outd=F32)
        a.update(kw)
        return bi.bi_decode_attn_paged(*a.values(), None)

    assert dec(ind=F32) == DTYPE and dec(outd=7) == DTYPE
    assert dec(page=12) == SHAPE and dec(page=0) == SHAPE        # page size a power of two
    assert dec(max_seq=513) == SHAPE                             # beyond max_pages * page
    assert dec(max_seq=0) == SHAPE and dec(num_pages=0) == SHAPE and dec(B=-1) == SHAPE
    assert dec(D=96) == UNSUP
    assert dec(max_seq=(1 << 31) - 100, max_pages=1 << 27) == UNSUP
    assert dec(bt=None) == NULL and dec(sl=None) == NULL and dec(vc=None) == NULL
    assert dec(ws=None) == WS and dec(ws_bytes=100) == WS
    assert dec(kc=P + 8) == LAYOUT and dec(bt=P + 2) == LAYOUT
    assert dec(B=0) == OK and dec(H=0) == OK


def test_prefill_workspace_size_and_validation(bi):
    assert bi.bi_prefill_attn_paged_workspace_bytes(1000, 8, 4096, 128) == 0       # one chunk: none
    assert bi.bi_prefill_attn_paged_workspace_bytes(1000, 8, 4097, 128) == 2 * 8 * 132 * 1000 * 4

    def pf(**kw):
        a = dict(B=2, H=2, D=128, q=P, total_q=64, cu=P, p0=P, max_q=32, kc=P, vc=P, num_pages=64,
                 page=16, bt=P, max_pages=32, max_kv=512, out=P, scale=0.1, ws=P, ws_bytes=0,
                 ind=BF16, outd=F32)
        a.update(kw)
        return bi.bi_prefill_attn_paged(*a.values(), None)

    assert pf(ind=F32) == DTYPE and pf(outd=3) == DTYPE
    assert pf(page=24) == SHAPE and pf(max_kv=513) == SHAPE and pf(max_q=0) == SHAPE
    assert pf(total_q=-1) == SHAPE and pf(num_pages=0) == SHAPE
    assert pf(D=64) == UNSUP
    assert pf(cu=None) == NULL and pf(bt=None) == NULL and pf(out=None) == NULL
    assert pf(out=P + 8) == LAYOUT and pf(q=P + 4) == LAYOUT and pf(p0=P + 2) == LAYOUT
    assert pf(max_kv=5000, max_pages=400) == WS                       # two chunks need ws
    assert pf(max_kv=5000, max_pages=400, ws=P + 8, ws_bytes=1 << 20) == WS    # 16-byte aligned ws
    assert pf(B=0) == OK and pf(total_q=0) == OK


def test_softmax_validation(bi):
    assert bi.bi_softmax_rows(4, 8, P, 8, 1.0, P, 8, 5, None) == DTYPE
    assert bi.bi_softmax_rows(-1, 8, P, 8, 1.0, P, 8, BF16, None) == SHAPE
    assert bi.bi_softmax_rows(4, 8, None, 8, 1.0, P, 8, BF16, None) == NULL
    assert bi.bi_softmax_rows(4, 8, P, 4, 1.0, P, 8, BF16, None) == LAYOUT
    assert bi.bi_softmax_rows(0, 8, P, 8, 1.0, P, 8, BF16, None) == OK


def test_attention_probs_validation(bi):
    def ap(G=2, T=64, Tk=1024, D=128, Q=P, sQg=64 * 128, sQt=128, K=P, sKg=1024 * 128, sKt=128,
           Pp=P, sPg=64 * 1024, sPt=1024):
        return bi.bi_attention_probs(G, T, Tk, D, Q, sQg, sQt, K, sKg, sKt, 0.125, Pp, sPg, sPt, None)
    assert ap(T=-1) == SHAPE
    assert ap(D=96) == UNSUP and ap(Tk=1000) == UNSUP and ap(Tk=2048) == UNSUP
    assert ap(G=0) == OK and ap(T=0) == OK
    assert ap(Q=None) == NULL and ap(Pp=None) == NULL
    assert ap(Q=P + 8) == LAYOUT            # Q rows not 16-byte aligned
    assert ap(sKt=132) == LAYOUT            # K row stride not a multiple of 8 elements
    assert ap(sPt=1022) == LAYOUT           # P row stride not a multiple of 4
    assert ap(sQt=64) == LAYOUT             # rows overlap: stride below D


def test_row_ops_validation(bi):
    rms = lambda rows=4, cols=8, x=P, ldx=8, w=P, eps=1e-6, y=P, ldy=8, i=BF16, o=BF16: \
        bi.bi_rms_norm(rows, cols, x, ldx, w, eps, y, ldy, i, o, None)
    assert rms(i=3) == DTYPE and rms(o=9) == DTYPE
    assert rms(rows=-1) == SHAPE and rms(cols=-2) == SHAPE
    assert rms(x=None) == NULL and rms(w=None) == NULL and rms(y=None) == NULL
    assert rms(ldx=4) == LAYOUT and rms(ldy=7) == LAYOUT and rms(x=P + 1) == LAYOUT
    assert rms(w=P + 1) == LAYOUT
    assert rms(eps=-1.0) == SHAPE and rms(eps=float("nan")) == SHAPE
    assert rms(cols=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1) == UNSUP
    assert rms(rows=0) == OK and rms(cols=0) == OK
    lsm = lambda rows=4, cols=8, x=P, ldx=8, y=P, ldy=8, i=F32, o=F32: \
        bi.bi_log_softmax_rows(rows, cols, x, ldx, y, ldy, i, o, None)
    assert lsm(i=2) == DTYPE and lsm(rows=-3) == SHAPE and lsm(y=None) == NULL
    assert lsm(ldx=7) == LAYOUT and lsm(y=P + 2) == LAYOUT and lsm(rows=0) == OK
    mean = lambda rows=4, cols=8, x=P, ldx=8, y=P, i=BF16, o=F32: bi.bi_mean_rows(rows, cols, x, ldx, y, i, o, None)
    assert mean(o=5) == DTYPE and mean(cols=0) == SHAPE and mean(x=None) == NULL
    assert mean(ldx=3) == LAYOUT and mean(rows=0) == OK and mean(rows=0, cols=0) == OK
