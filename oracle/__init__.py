"""Reference oracle (test infrastructure only).

ctypes front end of ``oracle.c``: the plain fp64 CPU statement of every
operation on the batch-invariant contraction path.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg import this package; the product
library and its binding never do.  Inputs are CPU torch tensors (float32 or
bfloat16, any strides); results are float64 numpy arrays.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F16 = 0, 1, 2
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.oracle_bf16_rne.restype = ctypes.c_double
        _lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
        _lib.oracle_widen.restype = ctypes.c_double
        _lib.oracle_widen.argtypes = [_vp, ctypes.c_int, _i64]
        _lib.oracle_conv_out.restype = _i64
        _lib.oracle_conv_out.argtypes = [_i64] * 5
    return _lib


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"oracle takes float32, bfloat16 or float16 tensors, got {t.dtype}")


def _cpu(t):
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    return t


def _ptr(t):
    return _vp(_cpu(t).data_ptr()) if t is not None else _vp(0)


def _idx(sel):
    if sel is None:
        return None, _vp(0), 0
    arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    return arr, _vp(arr.ctypes.data), len(arr)


def _out(shape):
    o = np.zeros(shape, dtype=np.float64)
    return o, o.ctypes.data_as(_dp)


def set_threads(n=0):
    """Threads of the oracle's parallel loops (n < 1: unchanged); returns the
    count in force.  Timing only: no result depends on it."""
    return int(_load().oracle_set_threads(ctypes.c_int(int(n))))


def bf16_rne(x):
    """Nearest bfloat16 value of a double, ties to even (single rounding)."""
    return _load().oracle_bf16_rne(float(x))


def bf16_rne_array(a):
    """Nearest bfloat16 values of a float64 array, ties to even."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    out = np.empty_like(a)
    _load().oracle_bf16_rne_array(a.ctypes.data_as(_dp), out.ctypes.data_as(_dp), _i64(a.size))
    return out


def widen(t, i):
    """Exact value of element i of a float32 / bfloat16 / float16 tensor."""
    return _load().oracle_widen(_ptr(t), _dt(t), i)


def conv_out(n, k, s, p, d):
    return _load().oracle_conv_out(n, k, s, p, d)


def mm(A, B, bias=None, rows=None):
    """C = A @ B (+ bias) in fp64; rows selects output rows of A."""
    lib = _load()
    M, K = A.shape
    K2, N = B.shape
    assert K == K2 and A.dtype == B.dtype and (bias is None or bias.dtype == A.dtype)
    keep, rp, nr = _idx(rows)
    out, op = _out((nr if rows is not None else M, N))
    lib.oracle_mm(_i64(M), _i64(N), _i64(K), _ptr(A), _i64(A.stride(0)), _i64(A.stride(1)),
                  _ptr(B), _i64(B.stride(0)), _i64(B.stride(1)), _ptr(bias), ctypes.c_int(_dt(A)),
                  rp, _i64(nr), op)
    return out


def bmm(A, B, slices=None):
    lib = _load()
    G, M, K = A.shape
    G2, K2, N = B.shape
    assert G == G2 and K == K2 and A.dtype == B.dtype
    keep, sp, ns = _idx(slices)
    out, op = _out((ns if slices is not None else G, M, N))
    lib.oracle_bmm(_i64(G), _i64(M), _i64(N), _i64(K),
                   _ptr(A), _i64(A.stride(0)), _i64(A.stride(1)), _i64(A.stride(2)),
                   _ptr(B), _i64(B.stride(0)), _i64(B.stride(1)), _i64(B.stride(2)),
                   ctypes.c_int(_dt(A)), sp, _i64(ns), op)
    return out


def _conv(fn, x, w, bias, stride, padding, dilation, groups, samples):
    lib = _load()
    x = x.contiguous()
    w = w.contiguous()
    N, Cin, H, W = x.shape
    Cout, cig, Kh, Kw = w.shape
    assert cig * groups == Cin and Cout % groups == 0
    sh, sw = stride
    ph, pw = padding
    dh, dw = dilation
    OH, OW = conv_out(H, Kh, sh, ph, dh), conv_out(W, Kw, sw, pw, dw)
    keep, sp, ns = _idx(samples)
    out, op = _out((ns if samples is not None else N, Cout, OH, OW))
    fn(_i64(N), _i64(Cin), _i64(H), _i64(W), _ptr(x), _i64(Cout), _i64(Kh), _i64(Kw), _ptr(w),
       _ptr(bias), _i64(sh), _i64(sw), _i64(ph), _i64(pw), _i64(dh), _i64(dw), _i64(groups),
       ctypes.c_int(_dt(x)), sp, _i64(ns), op)
    return out


def conv2d_direct(x, w, bias=None, stride=(1, 1), padding=(0, 0), dilation=(1, 1), groups=1,
                  samples=None):
    """Direct seven-loop convolution in fp64 (NCHW in, [n, Cout, OH, OW] out)."""
    return _conv(_load().oracle_conv2d_direct, x, w, bias, stride, padding, dilation, groups, samples)


def conv2d_unfold(x, w, bias=None, stride=(1, 1), padding=(0, 0), dilation=(1, 1), groups=1,
                  samples=None):
    """Unfold-matrix formulation of the same convolution (cross-check)."""
    return _conv(_load().oracle_conv2d_unfold, x, w, bias, stride, padding, dilation, groups, samples)


def softmax_rows(S, scale):
    """Row softmax of scale * S (S a float32 matrix, any row stride)."""
    lib = _load()
    assert S.dtype == torch.float32 and S.stride(1) == 1
    rows, cols = S.shape
    out, op = _out((rows, cols))
    lib.oracle_softmax_rows(_i64(rows), _i64(cols), _ptr(S), _i64(S.stride(0)),
                            ctypes.c_double(scale), op)
    return out


def _rows_in(x):
    assert x.dtype in (torch.float32, torch.bfloat16) and x.dim() == 2 and x.stride(1) == 1
    return BF16 if x.dtype == torch.bfloat16 else F32


def rms_norm(x, w, eps):
    """RMSNorm of each row of x [rows, cols] with weight w [cols] (same dtype)."""
    lib = _load()
    dt = _rows_in(x)
    assert w.dtype == x.dtype and w.dim() == 1 and w.shape[0] == x.shape[1]
    w = w.contiguous()
    rows, cols = x.shape
    out, op = _out((rows, cols))
    lib.oracle_rms_norm(_i64(rows), _i64(cols), _ptr(x), _i64(x.stride(0)), dt, _ptr(w),
                        ctypes.c_double(eps), op)
    return out


def log_softmax_rows(x):
    """log-softmax of each row of x [rows, cols]."""
    lib = _load()
    dt = _rows_in(x)
    rows, cols = x.shape
    out, op = _out((rows, cols))
    lib.oracle_log_softmax_rows(_i64(rows), _i64(cols), _ptr(x), _i64(x.stride(0)), dt, op)
    return out


def mean_rows(x):
    """Mean of each row of x [rows, cols]."""
    lib = _load()
    dt = _rows_in(x)
    rows, cols = x.shape
    out, op = _out((rows,))
    lib.oracle_mean_rows(_i64(rows), _i64(cols), _ptr(x), _i64(x.stride(0)), dt, op)
    return out


def attention(Q, K, V, scale, p_bf16=False, slices=None):
    """softmax(scale * Q K^T) V per batch element; Q, K, V [G, T, D]."""
    lib = _load()
    Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
    G, T, D = Q.shape
    keep, sp, ns = _idx(slices)
    out, op = _out((ns if slices is not None else G, T, D))
    lib.oracle_attention(_i64(G), _i64(T), _i64(D), _ptr(Q), _ptr(K), _ptr(V),
                         ctypes.c_double(scale), ctypes.c_int(_dt(Q)), ctypes.c_int(int(p_bf16)),
                         sp, _i64(ns), op)
    return out


def decode(q, k, v, scale, reqs=None):
    """Unsplit single-query attention; q [B,H,D], k, v [B,H,S,D]."""
    lib = _load()
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    B, H, S, D = k.shape
    keep, rp, nr = _idx(reqs)
    out, op = _out((nr if reqs is not None else B, H, D))
    lib.oracle_decode(_i64(B), _i64(H), _i64(S), _i64(D), _ptr(q), _ptr(k), _ptr(v),
                      ctypes.c_double(scale), ctypes.c_int(_dt(q)), rp, _i64(nr), op)
    return out


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale):
    """Decode over a paged cache: q [B,H,D], caches [num_pages,H,P,D],
    block_table [B, max_pages] int32, seq_lens [B] int32."""
    lib = _load()
    q, k_cache, v_cache = q.contiguous(), k_cache.contiguous(), v_cache.contiguous()
    bt = block_table.contiguous().to(torch.int32)
    sl = seq_lens.contiguous().to(torch.int32)
    B, H, D = q.shape
    P = k_cache.shape[2]
    out, op = _out((B, H, D))
    lib.oracle_decode_paged(_i64(B), _i64(H), _i64(D), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                            _i64(bt.shape[1]), _ptr(sl), _i64(P), ctypes.c_double(scale),
                            ctypes.c_int(_dt(q)), op)
    return out


def prefill_paged(q, cu_q, q_pos0, k_cache, v_cache, block_table, scale):
    """Causal prefill over a paged cache: q [total_q, H, D] (request b's rows
    cu_q[b] .. cu_q[b+1]-1, the first at absolute position q_pos0[b]), caches
    [num_pages, H, P, D], block_table [B, max_pages] int32."""
    lib = _load()
    q, k_cache, v_cache = q.contiguous(), k_cache.contiguous(), v_cache.contiguous()
    cu = torch.as_tensor(cu_q).contiguous().to(torch.int32)
    p0 = torch.as_tensor(q_pos0).contiguous().to(torch.int32)
    bt = block_table.contiguous().to(torch.int32)
    T, H, D = q.shape
    B = p0.shape[0]
    assert cu.shape[0] == B + 1 and int(cu[-1]) == T
    P = k_cache.shape[2]
    out, op = _out((T, H, D))
    lib.oracle_prefill_paged(_i64(B), _i64(H), _i64(D), _ptr(q), _ptr(cu), _ptr(p0), _ptr(k_cache),
                             _ptr(v_cache), _ptr(bt), _i64(bt.shape[1]), _i64(P), ctypes.c_double(scale),
                             ctypes.c_int(_dt(q)), op)
    return out


def decode_chunked(q, k, v, scale, chunk=2048, reqs=None, triples=False):
    """Fixed-length-chunk flash decoding with an ascending-order LSE merge."""
    lib = _load()
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    B, H, S, D = k.shape
    nc = (S + chunk - 1) // chunk
    keep, rp, nr = _idx(reqs)
    n = nr if reqs is not None else B
    out, op = _out((n, H, D))
    trip, tp = _out((n, H, nc, 2 + D)) if triples else (None, ctypes.cast(0, _dp))
    lib.oracle_decode_chunked(_i64(B), _i64(H), _i64(S), _i64(D), _ptr(q), _ptr(k), _ptr(v),
                              ctypes.c_double(scale), ctypes.c_int(_dt(q)), _i64(chunk), rp,
                              _i64(nr), op, tp)
    return (out, trip) if triples else out


def sim_splitk_gemm_f32(X, W, splits):
    """Binary32 split-K product of the handbook's experiment (negative control)."""
    lib = _load()
    X = X.contiguous().float()
    W = W.contiguous().float()
    M, K = X.shape
    N = W.shape[1]
    out = torch.empty(M, N, dtype=torch.float32)
    lib.sim_splitk_gemm_f32(_i64(M), _i64(N), _i64(K), _ptr(X), _ptr(W), _i64(splits), _ptr(out))
    return out


def sim_decode_splits_f32(q, K, V, scale, splits):
    """Binary32 flash decoding with a given part count (negative control)."""
    lib = _load()
    q, K, V = q.contiguous().float(), K.contiguous().float(), V.contiguous().float()
    S, D = K.shape
    out = torch.empty(D, dtype=torch.float32)
    lib.sim_decode_splits_f32(_i64(S), _i64(D), _ptr(q), _ptr(K), _ptr(V), ctypes.c_float(scale),
                              _i64(splits), _ptr(out))
    return out
