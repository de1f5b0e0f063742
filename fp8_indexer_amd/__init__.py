"""fp8_indexer_amd -- Python binding of libdsa, the DSA hot path on MI355X.

Thin ctypes marshalling over the C ABI in include/dsa.h: torch tensors are
used for device memory and the current HIP stream only; every step of the
path runs in libdsa's HIP kernels.  There is no fallback: if libdsa.so is not
built, every call raises.

    logits = indexer_logits(q8, q_scale, k8, k_scale, w, ks, ke)
    idx    = topk(logits, ks, ke, K)
    o      = sparse_attn_fwd(q, kv, attn_sink, idx, sm_scale, dv)
    logits, idx, o = prefill(...)

Shapes, dtypes, contiguity and devices of every tensor are checked here
before the C call (the C ABI sees pointers only and cannot): a mismatch
raises ValueError (shape) or TypeError (dtype, device).

`workspace` (top-k, attention, prefill): "auto" (default) takes the device
scratch the call's fastest path needs from torch's caching allocator on the
current stream; None runs the paths that need no scratch; a contiguous
uint8 CUDA tensor is used as given.
"""
import ctypes
import os

import torch

__all__ = ["DSAError", "lib", "version", "indexer_logits", "indexer_topk",
           "indexer_topk_workspace_size", "topk", "sparse_attn_fwd", "sparse_attn_bwd",
           "prefill", "topk_workspace_size", "sparse_attn_workspace_size",
           "prefill_workspace_size", "prefill_noalloc", "sparse_attn_fwd_fp8",
           "sparse_attn_fp8_workspace_size", "attn_fp8_supported", "KV_BF16", "KV_FP8_E4M3FN",
           "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")
KV_BF16, KV_FP8_E4M3FN = 0, 1
EXPORTS = ("dsa_indexer_logits", "dsa_indexer_topk", "dsa_indexer_topk_workspace_size",
           "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_attn_fwd",
           "dsa_sparse_attn_workspace_size", "dsa_prefill", "dsa_prefill_workspace_size",
           "dsa_prefill_noalloc", "dsa_sparse_attn_bwd", "dsa_sparse_attn_fwd_fp8",
           "dsa_sparse_attn_fp8_workspace_size", "dsa_status_string", "dsa_version")
NOALLOC_SCRATCH_BYTES = 48 << 20  # DSA_NOALLOC_SCRATCH_BYTES


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
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib():
    """The loaded libdsa (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m fp8_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        psz = ctypes.POINTER(ctypes.c_size_t)
        L.dsa_indexer_logits.restype = ctypes.c_int
        L.dsa_indexer_logits.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32, P]
        L.dsa_indexer_topk_workspace_size.restype = ctypes.c_int
        L.dsa_indexer_topk_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i64, psz]
        L.dsa_indexer_topk.restype = ctypes.c_int
        L.dsa_indexer_topk.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32, i32, i64,
                                       P, sz, P]
        L.dsa_topk_workspace_size.restype = ctypes.c_int
        L.dsa_topk_workspace_size.argtypes = [i64, i64, i64, i32, psz]
        L.dsa_topk.restype = ctypes.c_int
        L.dsa_topk.argtypes = [P, P, P, P, i64, i64, i64, i32, P, sz, P]
        L.dsa_sparse_attn_workspace_size.restype = ctypes.c_int
        L.dsa_sparse_attn_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32, psz]
        L.dsa_sparse_attn_fwd.restype = ctypes.c_int
        L.dsa_sparse_attn_fwd.argtypes = [P, P, ctypes.c_int, P, P, P, P, i64, i64, i64, i32,
                                          i32, i32, i32, ctypes.c_float, P, sz, P]
        L.dsa_sparse_attn_fp8_workspace_size.restype = ctypes.c_int
        L.dsa_sparse_attn_fp8_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32, psz]
        L.dsa_sparse_attn_fwd_fp8.restype = ctypes.c_int
        L.dsa_sparse_attn_fwd_fp8.argtypes = [P, P, P, P, P, P, P, i64, i64, i64, i32, i32, i32,
                                              i32, ctypes.c_float, P, sz, P]
        L.dsa_sparse_attn_bwd.restype = ctypes.c_int
        L.dsa_sparse_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32,
                                          i32, i32, ctypes.c_float, P]
        L.dsa_prefill_workspace_size.restype = ctypes.c_int
        L.dsa_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs), psz]
        L.dsa_prefill.restype = ctypes.c_int
        L.dsa_prefill.argtypes = [ctypes.POINTER(PrefillArgs), P]
        L.dsa_prefill_noalloc.restype = ctypes.c_int
        L.dsa_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), P]
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


_FP8 = (torch.float8_e4m3fn, torch.uint8)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_BF16 = (torch.bfloat16,)


def _tensor(t, name, dtypes, shape):
    """dtype, contiguity and shape of one argument (None passes)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rank(t, name, n):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != n:
        raise ValueError(f"{name}: expected {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _same_device(ref, *ts):
    """Every given tensor is a CUDA (HIP) tensor on ref's device."""
    if not ref.is_cuda:
        raise TypeError("tensors must be CUDA (HIP) tensors")
    for t in ts:
        if t is not None and t.device != ref.device:
            raise TypeError(f"all tensors must be on {ref.device}, found one on {t.device}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(workspace, nbytes, device):
    """(pointer, size) of the scratch to pass: see the module docstring."""
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        if nbytes == 0:
            return None, 0, None
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return ctypes.c_void_p(buf.data_ptr()), nbytes, buf
    _tensor(workspace, "workspace", (torch.uint8,), (workspace.numel(),))
    if workspace.device != device:
        raise TypeError(f"workspace must be on {device}")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), workspace


def topk_workspace_size(B, M, N, K):
    """Bytes of scratch dsa_topk's fastest path needs (0: none)."""
    n = ctypes.c_size_t(0)
    _check("dsa_topk_workspace_size", lib().dsa_topk_workspace_size(B, M, N, K, ctypes.byref(n)))
    return n.value


def sparse_attn_workspace_size(B, M, Hq, Dqk, Dv, K):
    """Bytes of scratch dsa_sparse_attn_fwd's fastest path needs on the
    current device (0: none)."""
    n = ctypes.c_size_t(0)
    _check("dsa_sparse_attn_workspace_size",
           lib().dsa_sparse_attn_workspace_size(B, M, Hq, Dqk, Dv, K, ctypes.byref(n)))
    return n.value


def sparse_attn_fp8_workspace_size(B, M, Hq, Dqk, Dv, K):
    """Bytes of scratch dsa_sparse_attn_fwd_fp8's fastest path needs on the
    current device (0: none)."""
    n = ctypes.c_size_t(0)
    _check("dsa_sparse_attn_fp8_workspace_size",
           lib().dsa_sparse_attn_fp8_workspace_size(B, M, Hq, Dqk, Dv, K, ctypes.byref(n)))
    return n.value


def attn_fp8_supported(Hq, Dqk, Dv):
    """Whether dsa_sparse_attn_fwd_fp8 supports these head and width sizes
    (asked of the library: its workspace-size query validates the shape)."""
    n = ctypes.c_size_t(0)
    rc = lib().dsa_sparse_attn_fp8_workspace_size(1, 1, Hq, Dqk, Dv, 1, ctypes.byref(n))
    return rc == 0


def indexer_logits(q, q_scale, k, k_scale, weights, ks, ke, logits=None):
    """logits [B,M,N] fp32 (entries outside each row's window are untouched)."""
    B, M, H, D = _rank(q, "q", 4)
    N = _rank(k, "k", 3)[1]
    _tensor(q, "q", _FP8, (B, M, H, D))
    _tensor(k, "k", _FP8, (B, N, D))
    _tensor(q_scale, "q_scale", _F32, (B, M, H))
    _tensor(k_scale, "k_scale", _F32, (B, N))
    _tensor(weights, "weights", _F32, (B, M, H))
    _tensor(ks, "ks", _I32, (B, M))
    _tensor(ke, "ke", _I32, (B, M))
    _tensor(logits, "logits", _F32, (B, M, N))
    _same_device(q, q_scale, k, k_scale, weights, ks, ke, logits)
    if logits is None:
        logits = torch.empty((B, M, N), dtype=torch.float32, device=q.device)
    _check("dsa_indexer_logits", lib().dsa_indexer_logits(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(weights), _ptr(ks), _ptr(ke),
        _ptr(logits), B, M, N, H, D, _stream(q)))
    return logits


def indexer_topk_workspace_size(B, M, N, H, D, K, slab_rows=0):
    """Bytes of scratch dsa_indexer_topk needs (a slab's logits + top-k)."""
    n = ctypes.c_size_t(0)
    _check("dsa_indexer_topk_workspace_size", lib().dsa_indexer_topk_workspace_size(
        B, M, N, H, D, K, slab_rows, ctypes.byref(n)))
    return n.value


def indexer_topk(q, q_scale, k, k_scale, weights, ks, ke, K, out=None, slab_rows=0,
                 workspace="auto"):
    """topk_idxs [B,M,K] int32 of the indexer scores, without a [B,M,N]
    logits buffer (rows are scored and selected in workspace slabs)."""
    B, M, H, D = _rank(q, "q", 4)
    N = _rank(k, "k", 3)[1]
    _tensor(q, "q", _FP8, (B, M, H, D))
    _tensor(k, "k", _FP8, (B, N, D))
    _tensor(q_scale, "q_scale", _F32, (B, M, H))
    _tensor(k_scale, "k_scale", _F32, (B, N))
    _tensor(weights, "weights", _F32, (B, M, H))
    _tensor(ks, "ks", _I32, (B, M))
    _tensor(ke, "ke", _I32, (B, M))
    _tensor(out, "out", _I32, (B, M, K))
    _same_device(q, q_scale, k, k_scale, weights, ks, ke, out)
    if out is None:
        out = torch.empty((B, M, K), dtype=torch.int32, device=q.device)
    need = (indexer_topk_workspace_size(B, M, N, H, D, K, slab_rows)
            if isinstance(workspace, str) else 0)
    wp, wn, _keep = _workspace(workspace, need, q.device)
    _check("dsa_indexer_topk", lib().dsa_indexer_topk(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(weights), _ptr(ks), _ptr(ke),
        _ptr(out), B, M, N, H, D, K, slab_rows, wp, wn, _stream(q)))
    return out


def topk(logits, ks, ke, K, out=None, workspace="auto"):
    """topk_idxs [B,M,K] int32: ascending selected indices, then -1."""
    B, M, N = _rank(logits, "logits", 3)
    _tensor(logits, "logits", _F32, (B, M, N))
    _tensor(ks, "ks", _I32, (B, M))
    _tensor(ke, "ke", _I32, (B, M))
    _tensor(out, "out", _I32, (B, M, K))
    _same_device(logits, ks, ke, out)
    if out is None:
        out = torch.empty((B, M, K), dtype=torch.int32, device=logits.device)
    need = topk_workspace_size(B, M, N, K) if isinstance(workspace, str) else 0
    wp, wn, _keep = _workspace(workspace, need, logits.device)
    _check("dsa_topk", lib().dsa_topk(_ptr(logits), _ptr(ks), _ptr(ke), _ptr(out), B, M, N, K,
                                      wp, wn, _stream(logits)))
    return out


def sparse_attn_fwd(q, kv, attn_sink, topk_idxs, sm_scale=0.0, dv=None, kv_scale=None, out=None,
                    workspace="auto"):
    """o [B,M,Hq,Dv] bf16.  kv is bf16, or e4m3fn codes with kv_scale [B,N]."""
    B, M, Hq, Dqk = _rank(q, "q", 4)
    N = _rank(kv, "kv", 3)[1]
    K = _rank(topk_idxs, "topk_idxs", 3)[2]
    fp8 = kv_scale is not None
    dv = Dqk if dv is None else dv
    _tensor(q, "q", _BF16, (B, M, Hq, Dqk))
    _tensor(kv, "kv", _FP8 if fp8 else _BF16, (B, N, Dqk))
    _tensor(kv_scale, "kv_scale", _F32, (B, N))
    _tensor(attn_sink, "attn_sink", _F32, (Hq,))
    _tensor(topk_idxs, "topk_idxs", _I32, (B, M, K))
    _tensor(out, "out", _BF16, (B, M, Hq, dv))
    _same_device(q, kv, kv_scale, attn_sink, topk_idxs, out)
    if out is None:
        out = torch.empty((B, M, Hq, dv), dtype=torch.bfloat16, device=q.device)
    with torch.cuda.device(q.device):  # the split count follows the device's CU count
        need = (sparse_attn_workspace_size(B, M, Hq, Dqk, dv, K) if isinstance(workspace, str)
                else 0)
        wp, wn, _keep = _workspace(workspace, need, q.device)
        _check("dsa_sparse_attn_fwd", lib().dsa_sparse_attn_fwd(
            _ptr(q), _ptr(kv), KV_FP8_E4M3FN if fp8 else KV_BF16, _ptr(kv_scale),
            _ptr(attn_sink), _ptr(topk_idxs), _ptr(out), B, M, N, Hq, Dqk, dv, K,
            float(sm_scale), wp, wn, _stream(q)))
    return out


def sparse_attn_fwd_fp8(q, q_scale, kv, kv_scale, attn_sink, topk_idxs, sm_scale=0.0, dv=512,
                        out=None, workspace="auto"):
    """o [B,M,Hq,Dv] bf16 of the full-FP8 attention: q [B,M,Hq,Dqk] and kv
    [B,N,Dqk] e4m3fn codes with q_scale [B,M,Hq] (or None) and kv_scale
    [B,N]."""
    B, M, Hq, Dqk = _rank(q, "q", 4)
    N = _rank(kv, "kv", 3)[1]
    K = _rank(topk_idxs, "topk_idxs", 3)[2]
    _tensor(q, "q", _FP8, (B, M, Hq, Dqk))
    _tensor(q_scale, "q_scale", _F32, (B, M, Hq))
    _tensor(kv, "kv", _FP8, (B, N, Dqk))
    if kv_scale is None:
        raise ValueError("kv_scale is required")
    _tensor(kv_scale, "kv_scale", _F32, (B, N))
    _tensor(attn_sink, "attn_sink", _F32, (Hq,))
    _tensor(topk_idxs, "topk_idxs", _I32, (B, M, K))
    _tensor(out, "out", _BF16, (B, M, Hq, dv))
    _same_device(q, q_scale, kv, kv_scale, attn_sink, topk_idxs, out)
    if out is None:
        out = torch.empty((B, M, Hq, dv), dtype=torch.bfloat16, device=q.device)
    with torch.cuda.device(q.device):
        need = (sparse_attn_fp8_workspace_size(B, M, Hq, Dqk, dv, K)
                if isinstance(workspace, str) else 0)
        wp, wn, _keep = _workspace(workspace, need, q.device)
        _check("dsa_sparse_attn_fwd_fp8", lib().dsa_sparse_attn_fwd_fp8(
            _ptr(q), _ptr(q_scale), _ptr(kv), _ptr(kv_scale), _ptr(attn_sink),
            _ptr(topk_idxs), _ptr(out), B, M, N, Hq, Dqk, dv, K, float(sm_scale), wp, wn,
            _stream(q)))
    return out


def sparse_attn_bwd(q, kv, attn_sink, topk_idxs, o, dO, sm_scale=0.0, dq=None, dkv=None,
                    dsink=None):
    """Gradients (dq [B,M,Hq,Dqk], dkv [B,N,Dqk], dsink [Hq] or None), fp32,
    of dsa_sparse_attn_fwd with bf16 kv; o is the forward's output."""
    B, M, Hq, Dqk = _rank(q, "q", 4)
    N = _rank(kv, "kv", 3)[1]
    K = _rank(topk_idxs, "topk_idxs", 3)[2]
    Dv = _rank(dO, "dO", 4)[3]
    _tensor(q, "q", _BF16, (B, M, Hq, Dqk))
    _tensor(kv, "kv", _BF16, (B, N, Dqk))
    _tensor(attn_sink, "attn_sink", _F32, (Hq,))
    _tensor(topk_idxs, "topk_idxs", _I32, (B, M, K))
    _tensor(o, "o", _BF16, (B, M, Hq, Dv))
    _tensor(dO, "dO", _BF16, (B, M, Hq, Dv))
    _tensor(dq, "dq", _F32, (B, M, Hq, Dqk))
    _tensor(dkv, "dkv", _F32, (B, N, Dqk))
    _tensor(dsink, "dsink", _F32, (Hq,))
    _same_device(q, kv, attn_sink, topk_idxs, o, dO, dq, dkv, dsink)
    dev = q.device
    if dq is None:
        dq = torch.empty((B, M, Hq, Dqk), dtype=torch.float32, device=dev)
    if dkv is None:
        dkv = torch.empty((B, N, Dqk), dtype=torch.float32, device=dev)
    if attn_sink is not None and dsink is None:
        dsink = torch.empty((Hq,), dtype=torch.float32, device=dev)
    if attn_sink is None:
        dsink = None
    _check("dsa_sparse_attn_bwd", lib().dsa_sparse_attn_bwd(
        _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idxs), _ptr(o), _ptr(dO), _ptr(dq),
        _ptr(dkv), _ptr(dsink), B, M, N, Hq, Dqk, Dv, K, float(sm_scale), _stream(q)))
    return dq, dkv, dsink


def _prefill_args(index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q,
                  kv, attn_sink, sm_scale, dv, kv_scale, logits, topk_idxs, out):
    """Checked dsa_prefill_args and the output tensors (allocated if None)."""
    B, M, H, D = _rank(index_q, "index_q", 4)
    N = _rank(index_k, "index_k", 3)[1]
    Hq, Dqk = _rank(q, "q", 4)[2:]
    fp8 = kv_scale is not None
    dv = Dqk if dv is None else dv
    _tensor(index_q, "index_q", _FP8, (B, M, H, D))
    _tensor(index_k, "index_k", _FP8, (B, N, D))
    _tensor(index_q_scale, "index_q_scale", _F32, (B, M, H))
    _tensor(index_k_scale, "index_k_scale", _F32, (B, N))
    _tensor(index_weights, "index_weights", _F32, (B, M, H))
    _tensor(ks, "ks", _I32, (B, M))
    _tensor(ke, "ke", _I32, (B, M))
    _tensor(q, "q", _BF16, (B, M, Hq, Dqk))
    _tensor(kv, "kv", _FP8 if fp8 else _BF16, (B, N, Dqk))
    _tensor(kv_scale, "kv_scale", _F32, (B, N))
    _tensor(attn_sink, "attn_sink", _F32, (Hq,))
    _tensor(logits if logits is not False else None, "logits", _F32, (B, M, N))
    _tensor(topk_idxs, "topk_idxs", _I32, (B, M, K))
    _tensor(out, "out", _BF16, (B, M, Hq, dv))
    _same_device(q, index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, kv,
                 kv_scale, attn_sink, logits if logits is not False else None, topk_idxs, out)
    dev = q.device
    if logits is None:
        logits = torch.empty((B, M, N), dtype=torch.float32, device=dev)
    elif logits is False:  # slab mode: no [B, M, N] logits buffer
        logits = None
    if topk_idxs is None:
        topk_idxs = torch.empty((B, M, K), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, M, Hq, dv), dtype=torch.bfloat16, device=dev)
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
        logits=logits.data_ptr() if logits is not None else None,
        topk_idxs=topk_idxs.data_ptr(), workspace=None,
        workspace_bytes=0)
    return a, logits, topk_idxs, out


def prefill_workspace_size(args):
    """Bytes of scratch dsa_prefill needs for a PrefillArgs (0: none)."""
    n = ctypes.c_size_t(0)
    _check("dsa_prefill_workspace_size",
           lib().dsa_prefill_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def prefill(index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q, kv,
            attn_sink, sm_scale=0.0, dv=None, kv_scale=None, logits=None, topk_idxs=None,
            out=None, workspace="auto"):
    """The whole path on the current stream; returns (logits, topk_idxs, o).
    logits=False: no [B,M,N] logits buffer (indexer and top-k in workspace
    slabs); the returned logits is then None."""
    a, logits, topk_idxs, out = _prefill_args(
        index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q, kv,
        attn_sink, sm_scale, dv, kv_scale, logits, topk_idxs, out)
    with torch.cuda.device(q.device):
        need = prefill_workspace_size(a) if isinstance(workspace, str) else 0
        wp, wn, _keep = _workspace(workspace, need, q.device)
        a.workspace, a.workspace_bytes = (wp.value if wp is not None else None), wn
        _check("dsa_prefill", lib().dsa_prefill(ctypes.byref(a), _stream(q)))
    return logits, topk_idxs, out


def prefill_noalloc(index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q,
                    kv, attn_sink, sm_scale=0.0, dv=None, kv_scale=None, logits=None,
                    topk_idxs=None, out=None):
    """dsa_prefill_noalloc: the whole path with the library's static device
    scratch instead of a workspace (no device allocation by the library;
    outputs not passed in are still allocated here).  Calls on one device
    must not overlap."""
    a, logits, topk_idxs, out = _prefill_args(
        index_q, index_q_scale, index_k, index_k_scale, index_weights, ks, ke, K, q, kv,
        attn_sink, sm_scale, dv, kv_scale, logits, topk_idxs, out)
    with torch.cuda.device(q.device):
        _check("dsa_prefill_noalloc", lib().dsa_prefill_noalloc(ctypes.byref(a), _stream(q)))
    return logits, topk_idxs, out
