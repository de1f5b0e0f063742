"""Seeded synthetic inputs for the DSA hot path.

This module only draws and encodes input tensors; it holds none of the
method's arithmetic (no scores, no selection, no softmax).  Both the GPU tests
and the oracle are fed from here.

Recipe (numpy PCG64 streams; every tensor has its own id -- 0 decode
lengths, 1 indexer q, 2 indexer k, 3 indexer w, 4 attention q, 5 kv, 6 sink --
and is drawn in chunks of 2^22 values, chunk c from
Generator(PCG64(SeedSequence(seed, spawn_key=(id, c)))), so the values do not
depend on how many threads fill them):
  * indexer q and k: N(0,1) fp32, quantised to OCP e4m3fn per row with scale
    amax/448 (x/scale clamped to +-448, round-to-nearest-even by torch's
    float8_e4m3fn cast; an all-zero row gets scale 1);
  * indexer weights w: N(0, w_std) fp32 with w_std = H^-1/2;
  * attention q and kv: N(0,1) rounded to bf16 (RNE); for the fp8-KV workload
    kv is quantised per row like the indexer k and a per-row fp32 scale kept;
    for the full-FP8 attention workloads q is also quantised, per (token,
    head) row, with its fp32 scale kept;
  * attn_sink: N(0,1) fp32, one per attention head;
  * key windows: causal prefill ks = 0, ke = t+1; packed varlen ks = sequence
    start, ke = t+1; decode ks = 0, ke = L_b with L_b uniform in
    [4096, 65536], the query at the last position, keys >= L_b all zero.
"""
from dataclasses import dataclass, replace
import math

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

FP8_MAX = 448.0
_CHUNK = 1 << 22  # values per generation chunk
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    M: int          # query tokens per batch entry
    N: int          # keys per batch entry
    H: int          # indexer heads
    D: int          # indexer head dim
    K: int          # top-k
    Hq: int         # attention heads
    Dqk: int        # attention q/kv dim
    Dv: int         # attention output dim (first Dv dims of kv)
    kv_fp8: bool = False
    q_fp8: bool = False       # attention q in e4m3 (full-FP8 attention)
    windows: str = "causal"   # causal | packed | decode
    seg: int = 0              # packed: sequence length
    decode_min: int = 4096
    seed: int = 0

    @property
    def w_std(self):
        return 1.0 / math.sqrt(self.H)

    @property
    def sm_scale(self):
        return float(np.float32(1.0 / math.sqrt(self.Dqk)))

    def with_(self, **kw):
        return replace(self, **kw)


# The five workloads.  Sizes follow the DeepSeek-V3.2 shapes: indexer 64x128
# fp8, top-k 2048, 128 attention heads over 576-wide latent KV (512 + 64 rope).
WORKLOADS = {
    "tiny_causal_256": Workload("tiny_causal_256", B=1, M=256, N=256, H=4, D=64,
                                K=32, Hq=16, Dqk=64, Dv=64, seed=1),
    "prefill_4096": Workload("prefill_4096", B=1, M=4096, N=4096, H=64, D=128,
                             K=2048, Hq=128, Dqk=576, Dv=512, seed=2),
    "varlen_4x8192": Workload("varlen_4x8192", B=1, M=32768, N=32768, H=64,
                              D=128, K=2048, Hq=128, Dqk=576, Dv=512,
                              windows="packed", seg=8192, seed=3),
    "decode_b64": Workload("decode_b64", B=64, M=1, N=65536, H=64, D=128,
                           K=2048, Hq=128, Dqk=576, Dv=512, windows="decode",
                           seed=4),
    "prefill_8192_fp8kv": Workload("prefill_8192_fp8kv", B=1, M=8192, N=8192,
                                   H=32, D=128, K=2048, Hq=64, Dqk=576, Dv=512,
                                   kv_fp8=True, seed=5),
}


# Full-FP8 attention (e4m3 q and kv): the shapes of the 4096-token prefill
# (128 heads) and of the 8192-token fp8-KV prefill (64 heads).
FP8_ATTN_WORKLOADS = {
    "prefill_4096_fp8attn": WORKLOADS["prefill_4096"].with_(
        name="prefill_4096_fp8attn", kv_fp8=True, q_fp8=True),
    "prefill_8192_fp8attn": WORKLOADS["prefill_8192_fp8kv"].with_(
        name="prefill_8192_fp8attn", q_fp8=True),
}


def _gen(seed, tid, chunk):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(tid, chunk))))


def _normal(seed, tid, shape, std=1.0):
    """float32 N(0, std) of the given shape from tensor stream `tid`."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)

    def fill(c):
        s, e = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        _gen(seed, tid, c).standard_normal(e - s, dtype=np.float32, out=out[s:e])
        if std != 1.0:
            out[s:e] *= np.float32(std)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def quantize_e4m3fn_rows(x):
    """Per-row (last axis) e4m3fn quantisation: returns (codes as torch
    float8_e4m3fn tensor, fp32 scale per row)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (t / scale.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn), scale.to(torch.float32)


def to_bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def bounds(wl, rng=None, lengths=None):
    """ks, ke int32 [B, M] and (decode) the per-batch lengths."""
    B, M, N = wl.B, wl.M, wl.N
    t = np.arange(M, dtype=np.int64)
    if wl.windows == "causal":
        ks = np.zeros((B, M), np.int32)
        ke = np.broadcast_to((t + 1 + (N - M)).astype(np.int32), (B, M)).copy()
    elif wl.windows == "packed":
        ks = np.broadcast_to(((t // wl.seg) * wl.seg).astype(np.int32), (B, M)).copy()
        ke = np.broadcast_to((t + 1).astype(np.int32), (B, M)).copy()
    elif wl.windows == "decode":
        assert lengths is not None
        ks = np.zeros((B, M), np.int32)
        ke = np.broadcast_to(lengths.reshape(B, 1).astype(np.int32), (B, M)).copy()
    else:
        raise ValueError(wl.windows)
    return ks, ke


def make_inputs(wl, parts=("indexer", "attn"), seed=None):
    """Draw every input tensor of a workload.  Returns a dict of CPU tensors /
    numpy arrays:
      indexer: q8 [B,M,H,D] fp8, q_scale [B,M,H], k8 [B,N,D] fp8, k_scale [B,N],
               w [B,M,H]
      attn:    q [B,M,Hq,Dqk] bf16, or fp8 with qa_scale [B,M,Hq] (q_fp8);
               kv [B,N,Dqk] bf16 or fp8 (+ kv_scale [B,N]), sink [Hq] fp32
      always:  ks, ke [B,M] int32 (numpy), lengths (decode) or None"""
    import torch
    seed = wl.seed if seed is None else seed
    B, M, N = wl.B, wl.M, wl.N
    lengths = None
    if wl.windows == "decode":
        lengths = _gen(seed, 0, 0).integers(wl.decode_min, N, size=B,
                                            endpoint=True).astype(np.int64)
    ks, ke = bounds(wl, lengths=lengths)
    out = {"ks": ks, "ke": ke, "lengths": lengths}

    def key_mask(x):
        if lengths is not None:
            for b in range(B):
                x[b, lengths[b]:] = 0
        return x

    if "indexer" in parts:
        q = _normal(seed, 1, (B, M, wl.H, wl.D))
        out["q8"], out["q_scale"] = quantize_e4m3fn_rows(q)
        del q
        k = key_mask(_normal(seed, 2, (B, N, wl.D)))
        out["k8"], out["k_scale"] = quantize_e4m3fn_rows(k)
        del k
        out["w"] = torch.from_numpy(_normal(seed, 3, (B, M, wl.H), wl.w_std))
    if "attn" in parts:
        qa = _normal(seed, 4, (B, M, wl.Hq, wl.Dqk))
        if wl.q_fp8:
            out["q"], out["qa_scale"] = quantize_e4m3fn_rows(qa)
        else:
            out["q"] = to_bf16(qa)
            out["qa_scale"] = None
        del qa
        kv = key_mask(_normal(seed, 5, (B, N, wl.Dqk)))
        if wl.kv_fp8:
            out["kv"], out["kv_scale"] = quantize_e4m3fn_rows(kv)
        else:
            out["kv"] = to_bf16(kv)
            out["kv_scale"] = None
        del kv
        out["sink"] = torch.from_numpy(_normal(seed, 6, (wl.Hq,)))
    return out


def synthetic_logits(wl, seed=None, ties=False):
    """fp32 [B, M, N] stand-in scores for exercising top-k on its own:
    N(0,1) draws (tensor id 7); with ties=True they are rounded to multiples
    of 1/8 so that many keys share a value."""
    import torch
    seed = wl.seed if seed is None else seed
    x = _normal(seed, 7, (wl.B, wl.M, wl.N))
    if ties:
        x = np.round(x * 8.0) / 8.0
    return torch.from_numpy(x)


def synthetic_topk(wl, ks, ke, seed=None, pad_frac=0.0):
    """int32 [B, M, K] index lists shaped like a top-k result: a row whose
    window [s, e) holds at most K keys lists all of them, otherwise K distinct
    keys drawn uniformly from the window, ascending; -1 fills the rest.  With
    pad_frac > 0 that fraction of rows also gets random -1 holes."""
    import torch
    seed = wl.seed if seed is None else seed
    B, M, N, K = wl.B, wl.M, wl.N, wl.K
    out = np.full((B * M, K), -1, np.int32)
    s_all = np.clip(np.asarray(ks, np.int64).reshape(-1), 0, N)
    e_all = np.maximum(np.clip(np.asarray(ke, np.int64).reshape(-1), 0, N), s_all)

    def fill(r0):
        rng = _gen(seed, 8, r0)
        for r in range(r0, min(B * M, r0 + 256)):
            s, e = int(s_all[r]), int(e_all[r])
            if e - s <= K:
                out[r, :e - s] = np.arange(s, e, dtype=np.int32)
            else:
                sel = rng.choice(e - s, size=K, replace=False)
                out[r] = np.sort(sel).astype(np.int32) + s
            if pad_frac > 0 and rng.random() < pad_frac:
                holes = rng.random(K) < 0.3
                out[r, holes] = -1
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(0, B * M, 256)))
    return torch.from_numpy(out.reshape(B, M, K))
