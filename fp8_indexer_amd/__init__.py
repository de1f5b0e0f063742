"""fp8_indexer_amd -- Python binding of libdsa, the DSA hot path on MI355X.

Thin ctypes marshalling over the C ABI in include/dsa.h: torch tensors are
used for device memory and the current HIP stream only; every step of the
path runs in libdsa's HIP kernels.  There is no fallback: if libdsa.so is not
built, every call raises.

    logits = indexer_logits(q8, q_scale, k8, k_scale, w, ks, ke)
    idx    = topk(logits, ks, ke, K)
    o      = sparse_attn_fwd(q, kv, attn_sink, idx, sm_scale, dv)
    logits, idx, o = prefill(...)
"""
import ctypes
import os

import torch

__all__ = ["DSAError", "lib", "version", "indexer_logits", "topk", "sparse_attn_fwd",
           "prefill", "KV_BF16", "KV_FP8_E4M3FN", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")
KV_BF16, KV_FP8_E4M3FN = 0, 1
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_VALUE", 2: "DSA_ERR_NOT_SUPPORTED",
           3: "DSA_ERR_LAUNCH"}
EXPORTS = ("dsa_indexer_logits", "dsa_topk", "dsa_sparse_attn_fwd", "dsa_prefill",
           "dsa_status_string", "dsa_version")


class DSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class PrefillArgs(ctypes.Structure):
    """Mirror of dsa_prefill_args (include/dsa.h)."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seq_q", ctypes.c_int64), ("seq_kv", ctypes.c_int64),
        ("index_q", ctypes.c_void_p), ("index_q_scale", ctypes.c_void_p),
        ("index_k", ctypes.c_void_p), ("index_k_scale", ctypes.c_void_p),
        ("index_weights", ctypes.c_void_p), ("ks", ctypes.c_void_p), ("ke", ctypes.c_void_p),
        ("index_heads", ctypes.c_int32), ("index_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_dtype", ctypes.c_int),
        ("kv_scale", ctypes.c_void_p), ("attn_sink", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("heads", ctypes.c_int32), ("dqk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("logits", ctypes.c_void_p), ("topk_idxs", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded libdsa (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m fp8_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.dsa_indexer_logits.restype = ctypes.c_int
        L.dsa_indexer_logits.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32, P]
        L.dsa_topk.restype = ctypes.c_int
        L.dsa_topk.argtypes = [P, P, P, P, i64, i64, i64, i32, P]
        L.dsa_sparse_attn_fwd.restype = ctypes.c_int
        L.dsa_sparse_attn_fwd.argtypes = [P, P, ctypes.c_int, P, P, P, P, i64, i64, i64, i32,
                                          i32, i32, i32, ctypes.c_float, P]
        L.dsa_prefill.restype = ctypes.c_int
        L.dsa_prefill.argtypes = [ctypes.POINTER(PrefillArgs), P]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [ctypes.c_int]
        L.dsa_version.restype = ctypes.c_int
        _lib = L
    return _lib


def version():
    return lib().dsa_version()


def _check(fn, st):
    if st != 0:
        raise DSAError(fn, st, lib().dsa_status_string(st).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def indexer_logits(q, q_scale, k, k_scale, weights, ks, ke, logits=None):
    """logits [B,M,N] fp32 (entries outside each row's window are untouched)."""
    _dev(q, "q", _FP8)
    _dev(k, "k", _FP8)
    _dev(q_scale, "q_scale", (torch.float32,))
    _dev(k_scale, "k_scale", (torch.float32,))
    _dev(weights, "weights", (torch.float32,))
    _dev(ks, "ks", (torch.int32,))
    _dev(ke, "ke", (torch.int32,))
    B, M, H, D = q.shape
    N = k.shape[1]
    if logits is None:
        logits = torch.empty((B, M, N), dtype=torch.float32, device=q.device)
    _dev(logits, "logits", (torch.float32,))
    _check("dsa_indexer_logits", lib().dsa_indexer_logits(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(weights), _ptr(ks), _ptr(ke),
        _ptr(logits), B, M, N, H, D, _stream(q)))
    return logits


def topk(logits, ks, ke, K, out=None):
    """topk_idxs [B,M,K] int32: ascending selected indices, then -1."""
    _dev(logits, "logits", (torch.float32,))
    _dev(ks, "ks", (torch.int32,))
    _dev(ke, "ke", (torch.int32,))
    B, M, N = logits.shape
    if out is None:
        out = torch.empty((B, M, K), dtype=torch.int32, device=logits.device)
    _dev(out, "out", (torch.int32,))
    _check("dsa_topk", lib().dsa_topk(_ptr(logits), _ptr(ks), _ptr(ke), _ptr(out), B, M, N,
                                      K, _stream(logits)))
    return out


def sparse_attn_fwd(q, kv, attn_sink, topk_idxs, sm_scale=0.0, dv=None, kv_scale=None, out=None):
    """o [B,M,Hq,Dv] bf16.  kv is bf16, or e4m3fn codes with kv_scale [B,N]."""
    _dev(q, "q", (torch.bfloat16,))
    fp8 = kv_scale is not None
    _dev(kv, "kv", _FP8 if fp8 else (torch.bfloat16,))
    _dev(kv_scale, "kv_scale", (torch.float32,))
    _dev(attn_sink, "attn_sink", (torch.float32,))
    _dev(topk_idxs, "topk_idxs", (torch.int32,))
    B, M, Hq, Dqk = q.shape
    N = kv.shape[1]
    K = topk_idxs.shape[-1]
    dv = Dqk if dv is None else dv
    if out is None:
        out = torch.empty((B, M, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,))
    _check("dsa_sparse_attn_fwd", lib().dsa_sparse_attn_fwd(
        _ptr(q), _ptr(kv), KV_FP8_E4M3FN if fp8 else KV_BF16, _ptr(kv_scale), _ptr(attn_sink),
        _ptr(topk_idxs), _ptr(out), B, M, N, Hq, Dqk, dv, K, float(sm_scale), _stream(q)))
    return out


def prefill(index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q, kv,
            attn_sink, sm_scale=0.0, dv=None, kv_scale=None, logits=None, topk_idxs=None,
            out=None):
    """The whole path on the current stream; returns (logits, topk_idxs, o)."""
    for t, n, d in ((index_q, "index_q", _FP8), (index_k, "index_k", _FP8),
                    (index_q_scale, "index_q_scale", (torch.float32,)),
                    (index_k_scale, "index_k_scale", (torch.float32,)),
                    (index_weights, "index_weights", (torch.float32,)),
                    (ks, "ks", (torch.int32,)), (ke, "ke", (torch.int32,)),
                    (q, "q", (torch.bfloat16,)), (attn_sink, "attn_sink", (torch.float32,)),
                    (kv_scale, "kv_scale", (torch.float32,))):
        _dev(t, n, d)
    fp8 = kv_scale is not None
    _dev(kv, "kv", _FP8 if fp8 else (torch.bfloat16,))
    B, M, H, D = index_q.shape
    N = index_k.shape[1]
    _, _, Hq, Dqk = q.shape
    dv = Dqk if dv is None else dv
    dev = q.device
    if logits is None:
        logits = torch.empty((B, M, N), dtype=torch.float32, device=dev)
    if topk_idxs is None:
        topk_idxs = torch.empty((B, M, K), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, M, Hq, dv), dtype=torch.bfloat16, device=dev)
    _dev(logits, "logits", (torch.float32,))
    _dev(topk_idxs, "topk_idxs", (torch.int32,))
    _dev(out, "out", (torch.bfloat16,))
    a = PrefillArgs(
        batch=B, seq_q=M, seq_kv=N, index_q=index_q.data_ptr(),
        index_q_scale=index_q_scale.data_ptr() if index_q_scale is not None else None,
        index_k=index_k.data_ptr(), index_k_scale=index_k_scale.data_ptr(),
        index_weights=index_weights.data_ptr(), ks=ks.data_ptr(), ke=ke.data_ptr(),
        index_heads=H, index_dim=D, topk=K, q=q.data_ptr(), kv=kv.data_ptr(),
        kv_dtype=KV_FP8_E4M3FN if fp8 else KV_BF16,
        kv_scale=kv_scale.data_ptr() if fp8 else None,
        attn_sink=attn_sink.data_ptr() if attn_sink is not None else None,
        o=out.data_ptr(), heads=Hq, dqk=Dqk, dv=dv, sm_scale=float(sm_scale),
        logits=logits.data_ptr(), topk_idxs=topk_idxs.data_ptr())
    _check("dsa_prefill", lib().dsa_prefill(ctypes.byref(a), _stream(q)))
    return logits, topk_idxs, out
