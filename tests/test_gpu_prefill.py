"""GPU: the composed path (dsa_prefill) against the composed oracle.

On an exact-arithmetic workload (small-integer fp8 codes, integer weights,
power-of-two scales) every logit is exact in fp32 whatever the summation
order, so GPU and oracle logits are bit-identical, the top-k must match
exactly (with many ties), and the attention output is compared end to end.
At the full-size workloads every stage is checked on sampled rows against
the oracle applied to the GPU's own input to that stage."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import check_attn, compare_topk, dev, log, sample_rows

pytestmark = pytest.mark.gpu

# e4m3fn codes of small integers 0, +-1, +-2, +-3, +-4
_INT_CODES = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8], np.uint8)


def _exact_inputs(wl, seed=0):
    import torch as T
    rng = np.random.default_rng(seed)
    x = W.make_inputs(wl, parts=("attn",))
    x["q8"] = T.from_numpy(rng.choice(_INT_CODES, (wl.B, wl.M, wl.H, wl.D))).view(T.float8_e4m3fn)
    x["k8"] = T.from_numpy(rng.choice(_INT_CODES, (wl.B, wl.N, wl.D))).view(T.float8_e4m3fn)
    x["q_scale"] = T.from_numpy((2.0 ** rng.integers(-1, 2, (wl.B, wl.M, wl.H))).astype(np.float32))
    x["k_scale"] = T.from_numpy((2.0 ** rng.integers(-3, 1, (wl.B, wl.N))).astype(np.float32))
    x["w"] = T.from_numpy(rng.integers(-2, 3, (wl.B, wl.M, wl.H)).astype(np.float32))
    return x


def _prefill(x, wl):
    r = dsa.prefill(dev(x["q8"]), dev(x["q_scale"]), dev(x["k8"]), dev(x["k_scale"]),
                    dev(x["w"]), dev(x["ks"]), dev(x["ke"]), wl.K, dev(x["q"]), dev(x["kv"]),
                    dev(x["sink"]), sm_scale=wl.sm_scale, dv=wl.Dv, kv_scale=dev(x["kv_scale"]))
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("name,M,K", [("tiny_causal_256", 256, 32), ("prefill_4096", 600, 256),
                                      ("prefill_8192_fp8kv", 500, 128)])
def test_prefill_exact_arithmetic(name, M, K):
    wl = W.WORKLOADS[name].with_(M=M, N=M, K=K)
    log(f"prefill exact-arithmetic {name} M={M} K={K}")
    x = _exact_inputs(wl)
    logits, idx, o = _prefill(x, wl)
    R = wl.B * wl.M
    ref = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"], x["ks"],
                                x["ke"])
    g = logits.cpu().numpy().reshape(R, wl.N)
    win = ~np.isnan(ref)
    assert np.array_equal(g[win], ref[win]), "exact logits differ"
    ti = oracle.topk(ref, x["ks"], x["ke"], wl.B, wl.M, wl.N, wl.K)
    assert np.array_equal(idx.cpu().numpy().reshape(R, wl.K), ti), "top-k differs"
    ro = oracle.sparse_attn(x["q"], x["kv"], x["sink"], ti.reshape(wl.B, wl.M, wl.K),
                            wl.sm_scale, wl.Dv, kv_scale=x["kv_scale"])
    check_attn(o, ro, name)


def test_prefill_exact_arithmetic_decode():
    """Decode shapes through every path they take: one token per batch
    entry (the indexer's one-token layout), windows past 8192 keys with few
    rows (the top-k split into segments), few rows (attention split over
    workgroups with bf16 partials and a merge).  Exact logits, so the top-k
    must match exactly."""
    wl = W.WORKLOADS["decode_b64"].with_(B=6, N=20000, K=256, decode_min=300)
    log(f"prefill exact-arithmetic decode B={wl.B} N={wl.N} K={wl.K}")
    x = _exact_inputs(wl, seed=4)
    logits, idx, o = _prefill(x, wl)
    R = wl.B * wl.M
    ref = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"], x["ks"],
                                x["ke"])
    g = logits.cpu().numpy().reshape(R, wl.N)
    win = ~np.isnan(ref)
    assert np.array_equal(g[win], ref[win]), "exact logits differ"
    ti = oracle.topk(ref, x["ks"], x["ke"], wl.B, wl.M, wl.N, wl.K)
    assert np.array_equal(idx.cpu().numpy().reshape(R, wl.K), ti), "top-k differs"
    ro = oracle.sparse_attn(x["q"], x["kv"], x["sink"], ti.reshape(wl.B, wl.M, wl.K),
                            wl.sm_scale, wl.Dv, kv_scale=x["kv_scale"])
    check_attn(o, ro, "decode")


STAGEWISE = {  # workload: (sampled rows, rows that must be among them)
    "prefill_4096": (24, lambda wl: [0, 1, 2046, 2047, 2048, 2049, wl.M - 1]),
    # sequence starts and ends of the 4 packed sequences, and the rows where a
    # window passes K keys inside a sequence
    "varlen_4x8192": (20, lambda wl: [0, 8191, 8192, 16383, 16384, 24575, 24576, 32767,
                                      8192 + 2047, 8192 + 2048, 24576 + 2049]),
    "decode_b64": (12, lambda wl: [0, wl.B - 1]),
    "prefill_8192_fp8kv": (20, lambda wl: [0, 2047, 2048, 4096, wl.M - 1]),
}


@pytest.mark.parametrize("name", list(STAGEWISE))
def test_prefill_stagewise(name):
    """dsa_prefill at a full-size workload, checked stage by stage on sampled
    rows, each stage on the GPU's own input to it: logits against the oracle
    within 1e-4 * sum|terms|; top-k against the oracle's top-k of the GPU
    logits, bit-exact; o against the oracle's attention over the GPU's
    topk_idxs, max|d| <= 2e-2 and mean|d| <= 2e-3."""
    wl = W.WORKLOADS[name]
    n, must = STAGEWISE[name]
    log(f"prefill stagewise {name}")
    x = W.make_inputs(wl)
    logits, idx, o = _prefill(x, wl)
    R = wl.B * wl.M
    rows = sample_rows(R, n, seed=5, must=must(wl))
    rt = torch.from_numpy(rows).to(logits.device)
    lg_rows = logits.reshape(R, wl.N)[rt].cpu().numpy()
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       x["ks"], x["ke"], rows=rows, with_terms=True)
    win = ~np.isnan(ref)
    d = np.abs(lg_rows[win].astype(np.float64) - ref[win])
    assert np.all(d <= 1e-4 * terms[win]), f"logits: max|d| {d.max()}"
    # top-k of the GPU logits (outside each window the buffer is unspecified;
    # neither side reads it)
    idx_rows = idx.reshape(R, wl.K)[rt].cpu().numpy()
    ti = oracle.topk(lg_rows, x["ks"], x["ke"], wl.B, wl.M, wl.N, wl.K, rows=rows)
    compare_topk(idx_rows, ti, f"{name} top-k")
    # attention over the GPU's own indices
    ro = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx.cpu(), wl.sm_scale, wl.Dv,
                            kv_scale=x["kv_scale"], rows=rows)
    og = o.reshape(R, wl.Hq, wl.Dv)[rt]
    mx, mn = check_attn(og, ro, f"{name} attention")
    log(f"  logits max|d| {d.max():.3g}; top-k exact; attention max|d| {mx:.3g} mean {mn:.3g}")
