"""GPU: the composed path (dsa_prefill) against the composed oracle.

On an exact-arithmetic workload (small-integer fp8 codes, integer weights,
power-of-two scales) every logit is exact in fp32 whatever the summation
order, so GPU and oracle logits are bit-identical, the top-k must match
exactly (with many ties), and the attention output is compared end to end.
On the 4096-token workload the logits are checked on sampled rows and the
top-k output is checked for properties that hold at any size."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import check_attn, check_logits, dev, log, sample_rows

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


def _topk_properties(lg, ks, ke, idx, K):
    """Valid exact top-k of the given rows: ascending, in window, right count,
    every selected value >= every unselected one, ties to the lower index."""
    N = lg.shape[1]
    for r in range(lg.shape[0]):
        s = min(max(int(ks[r]), 0), N)
        e = min(max(int(ke[r]), s), N)
        sel = idx[r][idx[r] >= 0]
        assert sel.size == min(K, e - s)
        assert np.all(np.diff(sel) > 0) and (sel.size == 0 or (sel[0] >= s and sel[-1] < e))
        assert np.all(idx[r][sel.size:] == -1)
        if e - s > K:
            v = lg[r, s:e].astype(np.float64)
            v[np.isnan(v)] = -np.inf
            mask = np.zeros(e - s, bool)
            mask[sel - s] = True
            lo = v[mask].min()
            assert lo >= v[~mask].max()
            un_eq = np.nonzero(~mask & (v == lo))[0]
            se_eq = np.nonzero(mask & (v == lo))[0]
            if un_eq.size:
                assert se_eq.max() < un_eq.min()


def test_prefill_4096_stagewise():
    wl = W.WORKLOADS["prefill_4096"]
    log("prefill 4096 stagewise")
    x = W.make_inputs(wl)
    logits, idx, o = _prefill(x, wl)
    R = wl.B * wl.M
    rows = sample_rows(R, 24, seed=5, must=[0, 2047, 2048, R - 1])
    lg_rows = logits.reshape(R, wl.N)[torch.from_numpy(rows).to(logits.device)].cpu().numpy()
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       x["ks"], x["ke"], rows=rows, with_terms=True)
    win = ~np.isnan(ref)
    d = np.abs(lg_rows[win].astype(np.float64) - ref[win])
    assert np.all(d <= 1e-4 * terms[win]), d.max()
    idx_rows = idx.reshape(R, wl.K)[torch.from_numpy(rows).to(idx.device)].cpu().numpy()
    _topk_properties(lg_rows, x["ks"].reshape(-1)[rows], x["ke"].reshape(-1)[rows], idx_rows,
                     wl.K)
    og = o.float()
    assert torch.isfinite(og).all()
