"""GPU parity: dsa_indexer_logits against the oracle (|d| <= 1e-4 * sum|terms|
inside each window; nothing written outside it)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check_logits, indexer_gpu, log, sample_rows

pytestmark = pytest.mark.gpu


def _small(H, D, M=77, N=1100, B=2, seed=3):
    return W.Workload("small", B=B, M=M, N=N, H=H, D=D, K=32, Hq=16, Dqk=64, Dv=64, seed=seed)


@pytest.mark.parametrize("H,D", [(4, 64), (8, 128), (16, 128), (32, 128), (64, 128), (128, 128),
                                 (64, 64), (64, 256), (4, 256)])
def test_indexer_shapes_causal(H, D):
    wl = _small(H, D)
    log(f"indexer causal H={H} D={D} B={wl.B} M={wl.M} N={wl.N}")
    x = W.make_inputs(wl, parts=("indexer",))
    g = indexer_gpu(x, wl.N).cpu().numpy().reshape(-1, wl.N)
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       x["ks"], x["ke"], with_terms=True)
    check_logits(g, ref, terms, f"H{H}D{D}")


@pytest.mark.parametrize("H,D", [(64, 128), (4, 64), (32, 128)])
def test_indexer_random_windows(H, D):
    """ks < 0, ke > N, ks > ke, empty windows, windows past a chunk boundary."""
    wl = _small(H, D, M=150, N=2500, seed=9)
    log(f"indexer random windows H={H} D={D}")
    x = W.make_inputs(wl, parts=("indexer",))
    rng = np.random.default_rng(5)
    ks = rng.integers(-50, wl.N, (wl.B, wl.M)).astype(np.int32)
    ke = (ks + rng.integers(-20, 1500, (wl.B, wl.M))).astype(np.int32)
    ke[0, :5] = wl.N + 100
    ks[0, 5:10] = -7
    ke[1, :8] = ks[1, :8]          # empty
    ke[1, 8:12] = ks[1, 8:12] - 3  # inverted
    x["ks"], x["ke"] = ks, ke
    g = indexer_gpu(x, wl.N).cpu().numpy().reshape(-1, wl.N)
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       ks, ke, with_terms=True)
    check_logits(g, ref, terms, "random windows")


def test_indexer_no_q_scale_and_one_token():
    wl = _small(64, 128, M=1, N=700, B=3)
    x = W.make_inputs(wl, parts=("indexer",))
    x["w"] = (x["w"] * x["q_scale"]).contiguous()
    x["q_scale"] = None
    g = indexer_gpu(x, wl.N).cpu().numpy().reshape(-1, wl.N)
    ref, terms = oracle.indexer_logits(x["q8"], None, x["k8"], x["k_scale"], x["w"], x["ks"],
                                       x["ke"], with_terms=True)
    check_logits(g, ref, terms, "no q_scale")


@pytest.mark.parametrize("H,D,M", [(16, 128, 1), (32, 64, 1), (64, 128, 1), (64, 256, 1),
                                   (128, 128, 1), (64, 128, 2), (4, 64, 16)])
def test_indexer_decode_layouts(H, D, M):
    """Key-parallel layouts: one token per batch entry (H / 16 row tiles per
    wave) and a few tokens sharing a wave's 128 rows; windows of any length
    in several key chunks, empty and past-the-end ones included."""
    wl = _small(H, D, M=M, N=5000, B=5, seed=H + D + M)
    log(f"indexer decode layout H={H} D={D} M={M}")
    x = W.make_inputs(wl, parts=("indexer",))
    rng = np.random.default_rng(H * 7 + M)
    ks = rng.integers(-20, 200, (wl.B, wl.M)).astype(np.int32)
    ke = rng.integers(0, wl.N + 50, (wl.B, wl.M)).astype(np.int32)
    ks[0, 0], ke[0, 0] = 0, wl.N
    ks[1, 0], ke[1, 0] = 300, 300  # empty
    x["ks"], x["ke"] = ks, ke
    g = indexer_gpu(x, wl.N).cpu().numpy().reshape(-1, wl.N)
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       ks, ke, with_terms=True)
    check_logits(g, ref, terms, f"decode H{H}D{D}M{M}")


@pytest.mark.parametrize("B,N,empty", [(300, 3000, 0.5), (1100, 300, 0.2)])
def test_indexer_decode_balance(B, N, empty):
    """One token per batch entry.  Up to 1024 entries: the windows laid end
    to end are cut into equal ranges, one per workgroup, which straddle
    entries (about half of them empty here, lengths 1 to N).  Beyond 1024
    entries: one item per (entry, key chunk)."""
    wl = _small(64, 128, M=1, N=N, B=B, seed=B)
    log(f"indexer decode balance B={B} N={N}")
    x = W.make_inputs(wl, parts=("indexer",))
    rng = np.random.default_rng(B)
    ks = rng.integers(0, N, (B, 1)).astype(np.int32)
    ke = (ks + rng.integers(1, N + 1, (B, 1))).astype(np.int32)  # past the end: clamped
    ke[rng.random((B, 1)) < empty] = 0                            # empty
    ks[0, 0], ke[0, 0] = 0, N
    ks[B - 1, 0], ke[B - 1, 0] = N - 1, N                           # one key
    x["ks"], x["ke"] = ks, ke
    g = indexer_gpu(x, wl.N).cpu().numpy().reshape(-1, wl.N)
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       ks, ke, with_terms=True)
    check_logits(g, ref, terms, f"decode balance B{B}")


WORKLOAD_ROWS = {"tiny_causal_256": None, "prefill_4096": 40, "varlen_4x8192": 24,
                 "decode_b64": 12, "prefill_8192_fp8kv": 24}


@pytest.mark.parametrize("name", list(WORKLOAD_ROWS))
def test_indexer_workloads(name):
    wl = W.WORKLOADS[name]
    log(f"indexer workload {name}")
    x = W.make_inputs(wl, parts=("indexer",))
    g = indexer_gpu(x, wl.N)
    n = WORKLOAD_ROWS[name]
    R = wl.B * wl.M
    if n is None:
        rows = None
        gr = g.cpu().numpy().reshape(R, wl.N)
    else:
        must = [0, R - 1, wl.M // 2, wl.M // 2 - 1] + ([wl.seg - 1, wl.seg] if wl.seg else [])
        rows = sample_rows(R, n, seed=1, must=must)
        gr = g.reshape(R, wl.N)[rows].cpu().numpy()
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       x["ks"], x["ke"], rows=rows, with_terms=True)
    err = check_logits(gr, ref, terms, name)
    log(f"  max|d| {err:.3g}")
