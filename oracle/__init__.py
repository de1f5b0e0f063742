"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg
may import this package.  It wraps oracle/libdsa_oracle.so (plain C, fp64, see
dsa_oracle.h) with numpy in/out and shares nothing with the GPU library.

Parity status of each function is recorded in the test-suite pins
(tests/test_oracle_*.py): all three stages are pinned; the config readings
(causal bound, value width, distributions) are recorded decisions, not pins.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib(path=None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(L):
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    L.dsa_oracle_e4m3fn_value.restype = f64
    L.dsa_oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
    L.dsa_oracle_bf16_value.restype = f64
    L.dsa_oracle_bf16_value.argtypes = [ctypes.c_uint16]
    L.dsa_oracle_indexer_logits.restype = ctypes.c_int
    L.dsa_oracle_indexer_logits.argtypes = [P, P, P, P, P, P, P, i64, i64, i64,
                                            i32, i32, P, i64, P, P]
    L.dsa_oracle_topk.restype = ctypes.c_int
    L.dsa_oracle_topk.argtypes = [P, P, P, i64, i64, i64, i32, P, i64, P]
    L.dsa_oracle_sparse_attn.restype = ctypes.c_int
    L.dsa_oracle_sparse_attn.argtypes = [P, P, i32, P, P, P, i64, i64, i64,
                                         i32, i32, i32, i32, f64, P, i64, P]
    L.dsa_oracle_sparse_attn_ex.restype = ctypes.c_int
    L.dsa_oracle_sparse_attn_ex.argtypes = [P, i32, P, P, i32, P, P, P, i64, i64, i64,
                                            i32, i32, i32, i32, f64, P, i64, P, P]
    L.dsa_oracle_sparse_attn_bwd.restype = ctypes.c_int
    L.dsa_oracle_sparse_attn_bwd.argtypes = [P, P, P, P, P, i64, i64, i64, i32, i32, i32,
                                             i32, f64, P, i64, P, P, P, P, P, P]
    L.dsa_oracle_num_threads.restype = ctypes.c_int
    return L


def _np(x, dtype):
    """numpy view of a numpy array or CPU torch tensor, C-contiguous."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().cpu().contiguous()
        if x.dtype in (torch.float8_e4m3fn,):
            x = x.view(torch.uint8)
        elif x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        x = x.numpy()
    x = np.ascontiguousarray(x)
    if x.dtype != np.dtype(dtype):
        if x.dtype.itemsize == np.dtype(dtype).itemsize and x.dtype.kind in "iu" \
                and np.dtype(dtype).kind in "iu":
            x = x.view(dtype)
        else:
            x = x.astype(dtype)
    return x


def _is_fp8(x):
    """True for e4m3fn codes: a torch float8_e4m3fn tensor or 8-bit integers."""
    if hasattr(x, "detach"):
        import torch
        return x.dtype in (torch.float8_e4m3fn, torch.uint8, torch.int8)
    return np.asarray(x).dtype.itemsize == 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, int(r.size)


def e4m3fn_value(code):
    return lib().dsa_oracle_e4m3fn_value(int(code))


def bf16_value(bits):
    return lib().dsa_oracle_bf16_value(int(bits) & 0xFFFF)


def num_threads():
    return lib().dsa_oracle_num_threads()


def indexer_logits(q, q_scale, k, k_scale, w, ks, ke, rows=None, with_terms=False):
    """logits [n_rows, N] fp32 (NaN outside each row's window) and, if asked,
    terms [n_rows, N] fp64 = sum of |terms| for the tolerance.

    q [B,M,H,D] / k [B,N,D] are e4m3fn codes (uint8 or torch float8_e4m3fn)."""
    q8 = _np(q, np.uint8)
    k8 = _np(k, np.uint8)
    B, M, H, D = q8.shape
    N = k8.shape[1]
    assert k8.shape == (B, N, D)
    qs = _np(q_scale, np.float32)
    ksc = _np(k_scale, np.float32)
    w32 = _np(w, np.float32)
    ks32 = _np(ks, np.int32)
    ke32 = _np(ke, np.int32)
    assert ksc.size == B * N and w32.size == B * M * H
    assert ks32.size == B * M and ke32.size == B * M
    assert qs is None or qs.size == B * M * H
    r, n = _rows(rows)
    n_out = n if r is not None else B * M
    out = np.empty((n_out, N), np.float32)
    terms = np.empty((n_out, N), np.float64) if with_terms else None
    rc = lib().dsa_oracle_indexer_logits(_ptr(q8), _ptr(qs), _ptr(k8), _ptr(ksc),
                                         _ptr(w32), _ptr(ks32), _ptr(ke32), B, M, N,
                                         H, D, _ptr(r), n, _ptr(out), _ptr(terms))
    if rc != 0:
        raise ValueError("oracle indexer: invalid argument")
    return (out, terms) if with_terms else out


def topk(logits_rows, ks, ke, B, M, N, K, rows=None):
    """Exact top-k of each listed row; logits_rows is [n_rows, N] fp32."""
    lg = _np(logits_rows, np.float32)
    ks32 = _np(ks, np.int32)
    ke32 = _np(ke, np.int32)
    r, n = _rows(rows)
    n_out = n if r is not None else B * M
    assert lg.shape == (n_out, N), (lg.shape, n_out, N)
    out = np.empty((n_out, K), np.int32)
    rc = lib().dsa_oracle_topk(_ptr(lg), _ptr(ks32), _ptr(ke32), B, M, N, K,
                               _ptr(r), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle topk: invalid argument")
    return out


def sparse_attn(q, kv, attn_sink, topk_idxs, sm_scale, dv, kv_scale=None, rows=None,
                q_scale=None, q_fp8=None, with_terms=False):
    """o [n_rows, Hq, Dv] fp64.  q [B,M,Hq,Dqk]: bf16, or e4m3fn codes (uint8
    or torch float8_e4m3fn; q_fp8 may say so explicitly) with q_scale
    [B,M,Hq] (None = 1); kv [B,N,Dqk] bf16, or e4m3fn codes with kv_scale
    [B,N].  with_terms: (o, terms), terms[..., c] = sum_j p_j |v_jc|."""
    if q_fp8 is None:
        q_fp8 = _is_fp8(q)
    if q_scale is not None and not q_fp8:
        raise ValueError("oracle sparse_attn: q_scale needs an fp8 q")
    qn = _np(q, np.uint8 if q_fp8 else np.uint16)
    B, M, Hq, Dqk = qn.shape
    fp8 = kv_scale is not None
    kvn = _np(kv, np.uint8 if fp8 else np.uint16)
    N = kvn.shape[1]
    assert kvn.shape == (B, N, Dqk)
    idx = _np(topk_idxs, np.int32)
    K = idx.shape[-1]
    assert idx.size == B * M * K
    sink = _np(attn_sink, np.float32)
    kvs = _np(kv_scale, np.float32)
    qs = _np(q_scale, np.float32)
    if qs is not None:
        assert qs.size == B * M * Hq
    r, n = _rows(rows)
    n_out = n if r is not None else B * M
    out = np.empty((n_out, Hq, dv), np.float64)
    terms = np.empty((n_out, Hq, dv), np.float64) if with_terms else None
    rc = lib().dsa_oracle_sparse_attn_ex(_ptr(qn), int(bool(q_fp8)), _ptr(qs), _ptr(kvn),
                                         int(fp8), _ptr(kvs), _ptr(sink), _ptr(idx), B, M,
                                         N, Hq, Dqk, dv, K, float(sm_scale), _ptr(r), n,
                                         _ptr(out), _ptr(terms))
    if rc != 0:
        raise ValueError("oracle sparse_attn: invalid argument")
    return (out, terms) if with_terms else out


def sparse_attn_bwd(q, kv, attn_sink, topk_idxs, dO, sm_scale, dv, rows=None,
                    with_terms=False):
    """(dq [n_rows, Hq, Dqk], dkv [B, N, Dqk], dsink [Hq] or None), fp64, of
    the bf16 sparse attention; dkv and dsink hold the listed rows'
    contributions.  with_terms: also (tdq, tdkv, tdsink or None), sums of
    |terms|."""
    q16 = _np(q, np.uint16)
    B, M, Hq, Dqk = q16.shape
    kvn = _np(kv, np.uint16)
    N = kvn.shape[1]
    assert kvn.shape == (B, N, Dqk)
    idx = _np(topk_idxs, np.int32)
    K = idx.shape[-1]
    assert idx.size == B * M * K
    g16 = _np(dO, np.uint16)
    assert g16.size == B * M * Hq * dv
    sink = _np(attn_sink, np.float32)
    r, n = _rows(rows)
    n_out = n if r is not None else B * M
    dq = np.empty((n_out, Hq, Dqk), np.float64)
    dkv = np.empty((B, N, Dqk), np.float64)
    dsink = np.empty(Hq, np.float64) if sink is not None else None
    tdq = np.empty_like(dq) if with_terms else None
    tdkv = np.empty_like(dkv) if with_terms else None
    tds = np.empty(Hq, np.float64) if (with_terms and sink is not None) else None
    rc = lib().dsa_oracle_sparse_attn_bwd(_ptr(q16), _ptr(kvn), _ptr(sink), _ptr(idx),
                                          _ptr(g16), B, M, N, Hq, Dqk, dv, K,
                                          float(sm_scale), _ptr(r), n, _ptr(dq), _ptr(dkv),
                                          _ptr(dsink), _ptr(tdq), _ptr(tdkv), _ptr(tds))
    if rc != 0:
        raise ValueError("oracle sparse_attn_bwd: invalid argument")
    if with_terms:
        return dq, dkv, dsink, tdq, tdkv, tds
    return dq, dkv, dsink
