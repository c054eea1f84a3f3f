"""ctypes binding of libbi_bench.so (benchmark / test variants, include/bi_bench.h).

Marshalling only, like bi.py.  Not part of the product path: these calls
exist to measure the cost of batch invariance and to show that the tests
detect a batch-dependent reduction order.
"""
import ctypes
import os

import torch

from . import bi as _bi

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi_bench.so")
_i64, _vp, _int, _f32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "bi_bench_gemm_grid": (_int, [_i64] * 4 + [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _vp,
                                             _i64, _i64, _i64, _int, _int, _int, _vp]),
    "bi_bench_gemm_tile": (_int, [_i64] * 4 + [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _int, _vp,
                                             _i64, _i64, _i64, _int, _int, _int, _vp]),
    "bi_bench_gemm_shared_cu": (_int, [_i64] * 4 + [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _vp,
                                                  _i64, _i64, _i64, _int, _int, _int, _vp]),
    "bi_bench_gemm_tile_rows": (_int, [_i64, _i64, _i64, _i64, _int]),
    "bi_bench_gemm_tile_rows_for": (_int, [_i64, _i64, _i64, _i64, _int, _int]),
    "bi_bench_splitk_policy": (_int, [_i64, _i64, _i64, _int]),
    "bi_bench_addmm_splitk_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "bi_bench_addmm_splitk": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64,
                                     _i64, _int, _int, _int, _vp, _sz, _vp]),
    "bi_bench_decode_splits_policy": (_int, [_i64, _int]),
    "bi_bench_decode_attn_splits_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "bi_bench_decode_attn_splits": (_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _vp, _sz,
                                           _int, _int, _int, _vp]),
    "bi_bench_read_probe": (_int, [_vp, _sz, _vp, _vp]),
    "bi_bench_row_step_read": (_int, [_vp, _sz, _int, _vp, _vp]),
    "bi_bench_wave_reduce": (_int, [_vp, _vp, _vp]),
    "bi_bench_decode_splitkv_policy": (_int, [_i64, _i64, _i64, _int]),
    "bi_bench_decode_splitkv_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "bi_bench_decode_attn_splitkv": (_int, [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _vp, _sz, _int,
                                            _int, _vp]),
    "bi_bench_addmm_events": (_int, [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64,
                                     _i64, _int, _int, _vp, _vp, _vp]),
}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


_p, _dt, _stream, _check, _empty = _bi._p, _bi._dt, _bi._stream, _bi._check, _bi._empty


def gemm_grid(A, B, grid, bias=None, out=None, out_dtype=None, stream=None):
    """The invariant batched GEMM (A [G,M,K] or [M,K]) on a forced grid."""
    squeeze = A.dim() == 2
    if squeeze:
        A, B = A.unsqueeze(0), B.unsqueeze(0)
    G, M, K = A.shape
    N = B.shape[2]
    od = _dt(A) if out_dtype is None else out_dtype
    C = out if out is not None else _empty((G, M, N), _bi._tdt(od), A.device, stream)
    if C.dim() == 2:
        C = C.unsqueeze(0)
    _check("bi_bench_gemm_grid", lib().bi_bench_gemm_grid(
        G, M, N, K, _p(A), A.stride(0), A.stride(1), A.stride(2), _p(B), B.stride(0), B.stride(1),
        B.stride(2), _p(bias), _p(C), C.stride(0), C.stride(1), C.stride(2), _dt(A), _dt(C), grid,
        _stream(stream)))
    return C[0] if squeeze else C


def gemm_shared_cu(A, B, grid, bias=None, out=None, out_dtype=None, stream=None):
    """The invariant batched bf16 GEMM on the 128x128-tile kernel without its
    LDS reservation, on a forced grid (two workgroups may share a CU)."""
    squeeze = A.dim() == 2
    if squeeze:
        A, B = A.unsqueeze(0), B.unsqueeze(0)
    G, M, K = A.shape
    N = B.shape[2]
    od = _dt(A) if out_dtype is None else out_dtype
    C = out if out is not None else _empty((G, M, N), _bi._tdt(od), A.device, stream)
    if C.dim() == 2:
        C = C.unsqueeze(0)
    _check("bi_bench_gemm_shared_cu", lib().bi_bench_gemm_shared_cu(
        G, M, N, K, _p(A), A.stride(0), A.stride(1), A.stride(2), _p(B), B.stride(0), B.stride(1),
        B.stride(2), _p(bias), _p(C), C.stride(0), C.stride(1), C.stride(2), _dt(A), _dt(C), grid,
        _stream(stream)))
    return C[0] if squeeze else C


def gemm_tile(A, B, tile_rows, bias=None, bias_rows=False, out=None, out_dtype=None, stream=None):
    """The invariant 16-bit batched GEMM (A [G,M,K] or [M,K]) with the kernel
    forced: tile_rows 0 / 1 / 2 / 3 / 4 = persistent 256x256 / 128x256 / 256x128 /
    128x128 / 192x256, 32 / 64 / 128 = small tile (binary32: 0 = 64x64 tiles,
    32 = 32x32 tiles, 16 = 16x16 blocks with one K chain per wave)."""
    squeeze = A.dim() == 2
    if squeeze:
        A, B = A.unsqueeze(0), B.unsqueeze(0)
    G, M, K = A.shape
    N = B.shape[2]
    od = _dt(A) if out_dtype is None else out_dtype
    C = out if out is not None else _empty((G, M, N), _bi._tdt(od), A.device, stream)
    if C.dim() == 2:
        C = C.unsqueeze(0)
    _check("bi_bench_gemm_tile", lib().bi_bench_gemm_tile(
        G, M, N, K, _p(A), A.stride(0), A.stride(1), A.stride(2), _p(B), B.stride(0), B.stride(1),
        B.stride(2), _p(bias), int(bias_rows), _p(C), C.stride(0), C.stride(1), C.stride(2), _dt(A), _dt(C),
        tile_rows, _stream(stream)))
    return C[0] if squeeze else C


def gemm_tile_rows(G, M, N, K, in_dtype=_bi.BI_BF16):
    """The kernel bi_bmm / bi_addmm pick for the shape: 0..4 (persistent tile shapes) or 32 / 64 / 128."""
    r = lib().bi_bench_gemm_tile_rows(G, M, N, K, in_dtype)
    if r < 0:
        raise RuntimeError(f"bi_bench_gemm_tile_rows: {_bi.lib().bi_status_string(r).decode()}")
    return r


def gemm_tile_rows_for(G, M, N, K, cus, in_dtype=_bi.BI_BF16):
    """The same choice for a device with `cus` compute units (no GPU needed)."""
    r = lib().bi_bench_gemm_tile_rows_for(G, M, N, K, in_dtype, cus)
    if r < 0:
        raise RuntimeError(f"bi_bench_gemm_tile_rows_for: {_bi.lib().bi_status_string(r).decode()}")
    return r


def splitk_policy(M, N, K, rule=0):
    r = lib().bi_bench_splitk_policy(M, N, K, rule)
    if r < 0:
        raise _bi.BIError("bi_bench_splitk_policy", r)
    return r


def addmm_splitk(bias, A, B, splits, out=None, out_dtype=None, workspace=None, stream=None):
    M, K = A.shape
    N = B.shape[1]
    od = _dt(A) if out_dtype is None else out_dtype
    C = out if out is not None else _empty((M, N), _bi._tdt(od), A.device, stream)
    need = lib().bi_bench_addmm_splitk_workspace_bytes(M, N, splits)
    if workspace is None:
        workspace = _empty(max(need // 4, 1), torch.float32, A.device, stream)
    _check("bi_bench_addmm_splitk", lib().bi_bench_addmm_splitk(
        M, N, K, _p(A), A.stride(0), A.stride(1), _p(B), B.stride(0), B.stride(1), _p(bias), _p(C),
        C.stride(0), C.stride(1), _dt(A), _dt(C), splits, _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return C


def decode_splits_policy(B, sms):
    return lib().bi_bench_decode_splits_policy(B, sms)


def decode_attn_splits(q, k, v, scale, splits, out=None, out_dtype=_bi.BI_F32, workspace=None,
                       stream=None):
    B, H, S, D = k.shape
    o = out if out is not None else _empty((B, H, D), _bi._tdt(out_dtype), q.device, stream)
    need = lib().bi_bench_decode_attn_splits_workspace_bytes(B, H, S, D, splits)
    if workspace is None:
        workspace = _empty(max(need // 4, 1), torch.float32, q.device, stream)
    _check("bi_bench_decode_attn_splits", lib().bi_bench_decode_attn_splits(
        B, H, S, D, _p(q), _p(k), _p(v), _p(o), float(scale), _p(workspace),
        workspace.numel() * workspace.element_size(), _dt(q), _dt(o), splits, _stream(stream)))
    return o


def read_probe(buf, sink, stream=None):
    _check("bi_bench_read_probe", lib().bi_bench_read_probe(
        _p(buf), buf.numel() * buf.element_size(), _p(sink), _stream(stream)))


def row_step_read(buf, step_bytes, sink, stream=None):
    """Read buf (a multiple of 512 KiB) as 2 KiB rows in tiles of 256, step_bytes (64 or 128) per row and step."""
    _check("bi_bench_row_step_read", lib().bi_bench_row_step_read(
        _p(buf), buf.numel() * buf.element_size(), int(step_bytes), _p(sink), _stream(stream)))


def addmm_events(bias, A, B, start, stop, out=None, out_dtype=None, stream=None):
    """bi_addmm's product with the GEMM kernel launched so that the runtime
    records `start` / `stop` (torch.cuda.Event, enable_timing=True, each
    recorded once before so that it exists) at the start and the end of the
    kernel's own execution."""
    M, K = A.shape
    N = B.shape[1]
    od = _dt(A) if out_dtype is None else out_dtype
    C = out if out is not None else _empty((M, N), _bi._tdt(od), A.device, stream)
    if not start.cuda_event or not stop.cuda_event:
        raise ValueError("record both events once before timing with them")
    _check("bi_bench_addmm_events", lib().bi_bench_addmm_events(
        M, N, K, _p(A), A.stride(0), A.stride(1), _p(B), B.stride(0), B.stride(1), _p(bias), _p(C),
        C.stride(0), C.stride(1), _dt(A), _dt(C), ctypes.c_void_p(start.cuda_event),
        ctypes.c_void_p(stop.cuda_event), _stream(stream)))
    return C


def decode_splitkv_policy(B, H, S, cus):
    return lib().bi_bench_decode_splitkv_policy(B, H, S, cus)


def decode_splitkv_workspace(B, H, D, splits, device):
    """A zeroed workspace for decode_attn_splitkv (its counters start at zero)."""
    n = lib().bi_bench_decode_splitkv_workspace_bytes(B, H, D, splits)
    return torch.zeros((n + 3) // 4, dtype=torch.float32, device=device)


def decode_attn_splitkv(q, k, v, scale, splits, workspace, out=None, out_dtype=_bi.BI_F32, stream=None):
    """Decode split by load into `splits` parts, merged in the same launch
    (q [B, H, D], K, V [B, H, S, D] contiguous bfloat16)."""
    B, H, D = q.shape
    S = k.shape[2]
    o = out if out is not None else _empty((B, H, D), _bi._tdt(out_dtype), q.device, stream)
    _check("bi_bench_decode_attn_splitkv", lib().bi_bench_decode_attn_splitkv(
        B, H, S, D, _p(q), _p(k), _p(v), _p(o), float(scale), _p(workspace), workspace.numel() * 4,
        _dt(o), splits, _stream(stream)))
    return o


def wave_reduce(x, stream=None):
    """The library's wave-wide xor-butterfly sum and maximum of x (64 binary32
    values on the device): returns (sum per lane, max per lane)."""
    assert x.dtype == torch.float32 and x.numel() == 64 and x.is_contiguous()
    out = _empty((128,), torch.float32, x.device, stream)
    _check("bi_bench_wave_reduce", lib().bi_bench_wave_reduce(_p(x), _p(out), _stream(stream)))
    return out[:64], out[64:]
