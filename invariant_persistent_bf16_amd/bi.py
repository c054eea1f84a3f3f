"""Python binding of libbi.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes device
torch tensors; torch supplies device memory and the current HIP stream, and
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or refuses a call, an exception says so.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi.so")

BI_F32, BI_BF16, BI_F16 = 0, 1, 2
_i64, _vp, _int, _f32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "bi_status_string": (ctypes.c_char_p, [_int]),
    "bi_set_launch_events": (_int, [_vp, _vp]),
    "bi_mm": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _int, _vp]),
    "bi_addmm": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _i64,
                        _int, _int, _vp]),
    "bi_bmm": (_int, [_i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64,
                      _i64, _i64, _int, _int, _vp]),
    "bi_conv2d_workspace_bytes": (_sz, [_i64] * 14 + [_int]),
    "bi_conv2d": (_int, [_i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _vp] + [_i64] * 7 +
                  [_vp, _vp, _sz, _int, _int, _vp]),
    "bi_decode_attn_workspace_bytes": (_sz, [_i64] * 4),
    "bi_decode_attn": (_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _vp, _sz, _int, _int, _vp]),
    "bi_decode_attn_noalloc": (_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _int, _int, _vp]),
    "bi_decode_chunk_tokens": (_int, []),
    "bi_decode_attn_paged_workspace_bytes": (_sz, [_i64] * 4),
    "bi_decode_attn_paged": (_int, [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                    _f32, _vp, _sz, _int, _int, _vp]),
    "bi_prefill_attn_paged_workspace_bytes": (_sz, [_i64] * 4),
    "bi_prefill_attn_paged": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _i64,
                                     _i64, _vp, _f32, _vp, _sz, _int, _int, _vp]),
    "bi_softmax_rows": (_int, [_i64, _i64, _vp, _i64, _f32, _vp, _i64, _int, _vp]),
    "bi_attention_probs": (_int, [_i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _f32, _vp,
                                  _i64, _i64, _vp]),
    "bi_rms_norm": (_int, [_i64, _i64, _vp, _i64, _vp, _f32, _vp, _i64, _int, _int, _vp]),
    "bi_log_softmax_rows": (_int, [_i64, _i64, _vp, _i64, _vp, _i64, _int, _int, _vp]),
    "bi_mean_rows": (_int, [_i64, _i64, _vp, _i64, _vp, _int, _int, _vp]),
}

_lib = None


class BIError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib():
    """The loaded libbi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().bi_status_string(int(status)).decode()


def bi_status_string(status):
    return status_string(status)


def _dt(t):
    if t.dtype == torch.float32:
        return BI_F32
    if t.dtype == torch.bfloat16:
        return BI_BF16
    if t.dtype == torch.float16:
        return BI_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tdt(code):
    return {BI_F32: torch.float32, BI_BF16: torch.bfloat16, BI_F16: torch.float16}[code]


def _p(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise BIError(fn, rc)


def _empty(shape, dtype, device, stream):
    """A new device tensor owned by the stream the kernels run on.  torch's
    caching allocator hands a freed block only to later allocations on the
    stream that owns it; a workspace allocated on another stream than the
    kernel's could be reused there while the kernel still reads it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _out(shape, out_dtype, device, out, stream=None):
    if out is not None:
        return out
    return _empty(shape, _tdt(out_dtype), device, stream)


def bi_mm(A, B, out=None, out_dtype=None, stream=None):
    """C = A @ B (A [M, K], B [K, N]; strided views allowed as the header states)."""
    M, K = A.shape
    N = B.shape[1]
    od = _dt(A) if out_dtype is None else out_dtype
    C = _out((M, N), od, A.device, out, stream)
    _check("bi_mm", lib().bi_mm(M, N, K, _p(A), A.stride(0), A.stride(1), _p(B), B.stride(0),
                                B.stride(1), _p(C), C.stride(0), C.stride(1), _dt(A), _dt(C),
                                _stream(stream)))
    return C


def bi_addmm(bias, A, B, out=None, out_dtype=None, stream=None):
    """C = A @ B + bias (bias [N])."""
    M, K = A.shape
    N = B.shape[1]
    od = _dt(A) if out_dtype is None else out_dtype
    C = _out((M, N), od, A.device, out, stream)
    _check("bi_addmm", lib().bi_addmm(M, N, K, _p(A), A.stride(0), A.stride(1), _p(B), B.stride(0),
                                      B.stride(1), _p(bias), _p(C), C.stride(0), C.stride(1),
                                      _dt(A), _dt(C), _stream(stream)))
    return C


def bi_bmm(A, B, out=None, out_dtype=None, stream=None):
    """C[g] = A[g] @ B[g] (A [G, M, K], B [G, K, N])."""
    G, M, K = A.shape
    N = B.shape[2]
    od = _dt(A) if out_dtype is None else out_dtype
    C = _out((G, M, N), od, A.device, out, stream)
    _check("bi_bmm", lib().bi_bmm(G, M, N, K, _p(A), A.stride(0), A.stride(1), A.stride(2),
                                  _p(B), B.stride(0), B.stride(1), B.stride(2),
                                  _p(C), C.stride(0), C.stride(1), C.stride(2),
                                  _dt(A), _dt(C), _stream(stream)))
    return C


def conv_out_hw(H, W, Kh, Kw, stride, padding, dilation):
    oh = (H + 2 * padding[0] - dilation[0] * (Kh - 1) - 1) // stride[0] + 1
    ow = (W + 2 * padding[1] - dilation[1] * (Kw - 1) - 1) // stride[1] + 1
    return oh, ow


def bi_conv2d_workspace_bytes(x_shape, w_shape, stride=(1, 1), padding=(0, 0), dilation=(1, 1),
                              groups=1, in_dtype=BI_BF16):
    N, Cin, H, W = x_shape
    Cout, _, Kh, Kw = w_shape
    return lib().bi_conv2d_workspace_bytes(N, Cin, H, W, Cout, Kh, Kw, stride[0], stride[1],
                                           padding[0], padding[1], dilation[0], dilation[1],
                                           groups, in_dtype)


def bi_conv2d(x, w, bias=None, stride=(1, 1), padding=(0, 0), dilation=(1, 1), groups=1,
              out=None, out_dtype=None, workspace=None, stream=None):
    """y = conv2d(x, w, bias) in NCHW via unfold + batched GEMM."""
    N, Cin, H, W = x.shape
    Cout, _, Kh, Kw = w.shape
    OH, OW = conv_out_hw(H, W, Kh, Kw, stride, padding, dilation)
    od = _dt(x) if out_dtype is None else out_dtype
    y = _out((N, Cout, OH, OW), od, x.device, out, stream)
    need = bi_conv2d_workspace_bytes(x.shape, w.shape, stride, padding, dilation, groups, _dt(x))
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, x.device, stream)
    _check("bi_conv2d", lib().bi_conv2d(N, Cin, H, W, _p(x), Cout, Kh, Kw, _p(w), _p(bias),
                                        stride[0], stride[1], padding[0], padding[1], dilation[0],
                                        dilation[1], groups, _p(y), _p(workspace),
                                        workspace.numel() * workspace.element_size(), _dt(x), _dt(y),
                                        _stream(stream)))
    return y


def bi_decode_chunk_tokens():
    return lib().bi_decode_chunk_tokens()


def bi_decode_attn_workspace_bytes(B, H, S, D):
    return lib().bi_decode_attn_workspace_bytes(B, H, S, D)


def bi_decode_attn(q, k, v, scale, out=None, out_dtype=BI_F32, workspace=None, stream=None):
    """Fixed-chunk split-KV decode attention: q [B,H,D], k, v [B,H,S,D] -> out [B,H,D]."""
    B, H, S, D = k.shape
    o = _out((B, H, D), out_dtype, q.device, out, stream)
    need = bi_decode_attn_workspace_bytes(B, H, S, D)
    if workspace is None:
        workspace = _empty(max(need // 4, 1), torch.float32, q.device, stream)
    _check("bi_decode_attn", lib().bi_decode_attn(B, H, S, D, _p(q), _p(k), _p(v), _p(o),
                                                  float(scale), _p(workspace),
                                                  workspace.numel() * workspace.element_size(),
                                                  _dt(q), _dt(o), _stream(stream)))
    return o


def bi_decode_attn_noalloc(q, k, v, scale, out, stream=None):
    """bi_decode_attn with the chunk triples in the library's static scratch
    (the call allocates nothing; out [B, H, D] fp32 or bf16 is the caller's)."""
    B, H, S, D = k.shape
    _check("bi_decode_attn_noalloc", lib().bi_decode_attn_noalloc(B, H, S, D, _p(q), _p(k), _p(v), _p(out),
                                                                  float(scale), _dt(q), _dt(out),
                                                                  _stream(stream)))
    return out


def bi_decode_attn_paged_workspace_bytes(B, H, max_seq_len, D):
    return lib().bi_decode_attn_paged_workspace_bytes(B, H, max_seq_len, D)


def bi_decode_attn_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale, out=None,
                         out_dtype=BI_F32, workspace=None, stream=None):
    """Split-KV decode over a paged cache: q [B,H,D], k_cache, v_cache [num_pages,H,P,D],
    block_table [B, max_pages] int32, seq_lens [B] int32 (both on the device) -> out [B,H,D]."""
    B, H, D = q.shape
    num_pages, _, P, _ = k_cache.shape
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    o = _out((B, H, D), out_dtype, q.device, out, stream)
    need = bi_decode_attn_paged_workspace_bytes(B, H, max_seq_len, D)
    if workspace is None:
        workspace = _empty(max(need // 4, 1), torch.float32, q.device, stream)
    _check("bi_decode_attn_paged", lib().bi_decode_attn_paged(
        B, H, D, _p(q), _p(k_cache), _p(v_cache), num_pages, P, _p(block_table), block_table.shape[1],
        _p(seq_lens), int(max_seq_len), _p(o), float(scale), _p(workspace),
        workspace.numel() * workspace.element_size(), _dt(q), _dt(o), _stream(stream)))
    return o


def bi_prefill_attn_paged_workspace_bytes(total_q, H, max_kv_len, D):
    return lib().bi_prefill_attn_paged_workspace_bytes(total_q, H, max_kv_len, D)


def bi_prefill_attn_paged(q, cu_q, q_pos0, max_q, k_cache, v_cache, block_table, max_kv_len, scale,
                          out=None, out_dtype=BI_F32, workspace=None, stream=None):
    """Causal prefill attention over a paged cache, KV split at 4096 tokens:
    q [total_q, H, D]; cu_q [B+1], q_pos0 [B], block_table [B, max_pages] int32 on
    the device; caches [num_pages, H, P, D] -> out [total_q, H, D]."""
    T, H, D = q.shape
    B = q_pos0.shape[0]
    num_pages, _, P, _ = k_cache.shape
    for t in (cu_q, q_pos0, block_table):
        if t.dtype != torch.int32:
            raise TypeError("cu_q, q_pos0 and block_table must be int32")
    o = _out((T, H, D), out_dtype, q.device, out, stream)
    need = bi_prefill_attn_paged_workspace_bytes(T, H, max_kv_len, D)
    if workspace is None and need > 0:
        workspace = _empty(need // 4, torch.float32, q.device, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bi_prefill_attn_paged", lib().bi_prefill_attn_paged(
        B, H, D, _p(q), T, _p(cu_q), _p(q_pos0), int(max_q), _p(k_cache), _p(v_cache), num_pages, P,
        _p(block_table), block_table.shape[1], int(max_kv_len), _p(o), float(scale), _p(workspace), wsz,
        _dt(q), _dt(o), _stream(stream)))
    return o


def bi_softmax_rows(S, scale, out=None, out_dtype=BI_BF16, stream=None):
    """P = softmax(scale * S) row-wise; S a float32 matrix [rows, cols]."""
    rows, cols = S.shape
    P = _out((rows, cols), out_dtype, S.device, out, stream)
    _check("bi_softmax_rows", lib().bi_softmax_rows(rows, cols, _p(S), S.stride(0), float(scale), _p(P),
                                                    P.stride(0), _dt(P), _stream(stream)))
    return P


def bi_rms_norm(x, w, eps=1e-6, out=None, out_dtype=None, stream=None):
    """y = RMSNorm(x) * w over the last dimension of x [rows, cols]."""
    rows, cols = x.shape
    od = _dt(x) if out_dtype is None else out_dtype
    y = _out((rows, cols), od, x.device, out, stream)
    _check("bi_rms_norm", lib().bi_rms_norm(rows, cols, _p(x), x.stride(0), _p(w), float(eps), _p(y),
                                            y.stride(0), _dt(x), _dt(y), _stream(stream)))
    return y


def bi_log_softmax_rows(x, out=None, out_dtype=None, stream=None):
    """log-softmax over the last dimension of x [rows, cols]."""
    rows, cols = x.shape
    od = _dt(x) if out_dtype is None else out_dtype
    y = _out((rows, cols), od, x.device, out, stream)
    _check("bi_log_softmax_rows", lib().bi_log_softmax_rows(rows, cols, _p(x), x.stride(0), _p(y), y.stride(0),
                                                            _dt(x), _dt(y), _stream(stream)))
    return y


def bi_mean_rows(x, out=None, out_dtype=BI_F32, stream=None):
    """Mean over the last dimension of x [rows, cols] -> [rows]."""
    rows, cols = x.shape
    y = _out((rows,), out_dtype, x.device, out, stream)
    _check("bi_mean_rows", lib().bi_mean_rows(rows, cols, _p(x), x.stride(0), _p(y), _dt(x), _dt(y),
                                              _stream(stream)))
    return y


def bi_attention_probs(Q, K, scale, out=None, stream=None):
    """P = softmax(scale * Q @ K^T) in bfloat16 (Q [G, T, D], K [G, Tk, D]),
    with the bits of bi_bmm + bi_softmax_rows, without writing S."""
    G, T, D = Q.shape
    Tk = K.shape[1]
    P = _out((G, T, Tk), BI_BF16, Q.device, out, stream)
    _check("bi_attention_probs", lib().bi_attention_probs(
        G, T, Tk, D, _p(Q), Q.stride(0), Q.stride(1), _p(K), K.stride(0), K.stride(1), float(scale),
        _p(P), P.stride(0), P.stride(1), _stream(stream)))
    return P


def attention(Q, K, V, scale, S_buf=None, P_buf=None, out=None, stream=None):
    """Attention of flattened [G, T, D] operands.  With S_buf, three launches:
    S = bi_bmm(Q, K^T) (fp32, into S_buf), P = bi_softmax_rows(S, scale)
    (bf16), O = bi_bmm(P, V) (fp32).  Without: P = bi_attention_probs(Q, K,
    scale) (the same P bits, S never written), then O = bi_bmm(P, V)."""
    G, T, D = Q.shape
    if S_buf is None and Q.dtype == torch.bfloat16:
        P = bi_attention_probs(Q, K, scale, out=P_buf, stream=stream)
        return bi_bmm(P, V, out=out, out_dtype=BI_F32, stream=stream)
    S = bi_bmm(Q, K.transpose(1, 2), out=S_buf, out_dtype=BI_F32, stream=stream)
    P = bi_softmax_rows(S.view(G * T, T), scale, out=None if P_buf is None else P_buf.view(G * T, T),
                        out_dtype=_dt(Q), stream=stream)
    return bi_bmm(P.view(G, T, T), V, out=out, out_dtype=BI_F32, stream=stream)


def bi_set_launch_events(start, stop):
    """Attach torch.cuda.Event objects (enable_timing=True, each recorded once
    before) to the library's kernels launched from this thread: start at the
    first kernel's start, stop at the last kernel's end.  (None, None) clears."""
    if stop is None:
        lib().bi_set_launch_events(None, None)
        return
    if not start.cuda_event or not stop.cuda_event:
        raise ValueError("record both events once before timing with them")
    lib().bi_set_launch_events(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event))
