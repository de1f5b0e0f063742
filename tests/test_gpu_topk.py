"""GPU parity: dsa_topk bit-exact against the oracle on the same logits."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import compare_topk, dev, log, sample_rows

pytestmark = pytest.mark.gpu


def _run(lg, ks, ke, K, workspace="auto"):
    out = dsa.topk(dev(lg), dev(ks), dev(ke), K, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _compare(lg, ks, ke, K, rows=None, what="", workspace="auto"):
    lg = np.ascontiguousarray(lg, np.float32)
    B, M, N = lg.shape
    g = _run(lg, ks, ke, K, workspace).reshape(B * M, K)
    flat = lg.reshape(B * M, N)
    if rows is None:
        ref = oracle.topk(flat, ks, ke, B, M, N, K)
        got = g
    else:
        ref = oracle.topk(flat[rows], ks, ke, B, M, N, K, rows=rows)
        got = g[rows]
    compare_topk(got, ref, what)


def _dist(kind, shape, rng):
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "ties":
        return rng.integers(-4, 5, shape).astype(np.float32)
    if kind == "special":
        x = rng.standard_normal(shape).astype(np.float32)
        m = rng.random(shape)
        x[m < 0.1] = 0.0
        x[(m >= 0.1) & (m < 0.2)] = -0.0
        x[(m >= 0.2) & (m < 0.23)] = np.nan
        x[(m >= 0.23) & (m < 0.26)] = -np.inf
        x[(m >= 0.26) & (m < 0.28)] = np.inf
        x[(m >= 0.28) & (m < 0.3)] = 1e-42  # denormal
        return x
    if kind == "narrow":  # one binade: the first radix digit sees a single bin
        return (1.0 + rng.random(shape)).astype(np.float32)
    if kind in ("sorted", "rsorted"):  # the largest keys at one end of the row
        x = np.sort(rng.standard_normal(shape).astype(np.float32), axis=-1)
        return np.ascontiguousarray(x[..., ::-1]) if kind == "rsorted" else x
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "narrow"])
@pytest.mark.parametrize("K", [1, 16, 100, 2048])
def test_topk_small(kind, K):
    rng = np.random.default_rng(K * 7 + len(kind))
    B, M, N = 2, 40, 5000
    lg = _dist(kind, (B, M, N), rng)
    ks = rng.integers(-10, N, (B, M)).astype(np.int32)
    ke = (ks + rng.integers(-5, 4500, (B, M))).astype(np.int32)
    # pin the length edge cases: len = K-1, K, K+1, whole row
    for i, ln in enumerate((K - 1, K, K + 1, N)):
        ks[0, i] = 0
        ke[0, i] = min(ln, N)
    log(f"topk small {kind} K={K}")
    _compare(lg, ks, ke, K, what=f"{kind}/K{K}")


@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "streaming"])
def test_topk_long_rows(workspace):
    """Rows longer than the register-resident limit (8192 keys), few rows,
    N > 65536: with a workspace the rows are split into segments sharing
    digit histograms; without one each long row takes one streaming
    workgroup."""
    rng = np.random.default_rng(11)
    B, M, N, K = 2, 3, 70000, 2048
    lg = _dist("special", (B, M, N), rng)
    ks = np.array([[0, 100, 60000], [0, 5, 0]], np.int32)
    ke = np.array([[70000, 8300, 70000], [65536, 8197, 2048]], np.int32)
    log(f"topk long rows workspace={workspace}")
    _compare(lg, ks, ke, K, what="long rows", workspace=workspace)
    lg2 = _dist("ties", (B, M, N), rng)
    _compare(lg2, ks, ke, 4096, what="long rows K=4096 ties", workspace=workspace)


def test_topk_deterministic():
    rng = np.random.default_rng(2)
    lg = _dist("ties", (1, 64, 9000), rng)
    ks = np.zeros((1, 64), np.int32)
    ke = np.full((1, 64), 9000, np.int32)
    a = _run(lg, ks, ke, 2048)
    b = _run(lg, ks, ke, 2048)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,nrows", [("tiny_causal_256", None), ("prefill_4096", None),
                                        ("varlen_4x8192", 1500), ("decode_b64", None),
                                        ("prefill_8192_fp8kv", 1500)])
def test_topk_workloads(name, nrows):
    wl = W.WORKLOADS[name]
    log(f"topk workload {name}")
    lengths = None
    if wl.windows == "decode":
        lengths = W._gen(wl.seed, 0, 0).integers(wl.decode_min, wl.N, size=wl.B,
                                                 endpoint=True).astype(np.int64)
    ks, ke = W.bounds(wl, lengths=lengths)
    lg = W.synthetic_logits(wl).numpy()
    R = wl.B * wl.M
    rows = None if nrows is None else sample_rows(R, nrows, seed=3,
                                                  must=[0, R - 1, wl.K, wl.K - 1, wl.K + 1])
    _compare(lg, ks, ke, wl.K, rows=rows, what=name)
    lg_t = W.synthetic_logits(wl, ties=True).numpy()
    _compare(lg_t, ks, ke, wl.K, rows=rows, what=name + "/ties")


@pytest.mark.parametrize("N", [40000, 65536, 70000], ids=["wide", "wide_max", "split"])
@pytest.mark.parametrize("kind", ["special", "ties", "narrow", "normal", "sorted", "rsorted"])
@pytest.mark.parametrize("K", [100, 2048, 4096])
def test_topk_few_long_rows(kind, K, N):
    """Few rows with N > 8192.  N <= 65536: one 1024-thread workgroup per
    row with the row in registers (lengths straddle the 4096-key wave
    segments; "sorted" and "rsorted" put the largest keys all in the last or
    the first waves).  N > 65536: every row is cut into 4096-key segments,
    one workgroup each, that share the row's digit histograms (lengths
    straddle segment boundaries)."""
    rng = np.random.default_rng(K + len(kind) + N)
    B, M = 1, 10
    lg = _dist(kind, (B, M, N), rng)
    # ... plus an empty row and a row shorter than K (written as -1 padded)
    ks = np.array([[0, 0, 0, 0, 0, 100, 31000, 5, 7, 0]], np.int32)
    ke = np.array([[N, K + 1, 8192, 8193, 16384 + 7, 24000, N, 5 + K, 7, K - 1]], np.int32)
    wide = N <= 65536
    assert (dsa.topk_workspace_size(B, M, N, K) == 0) == wide
    log(f"topk few long rows {kind} K={K} N={N}")
    _compare(lg, ks, ke, K, what=f"few long rows {kind}/K{K}/N{N}")


@pytest.mark.parametrize("workspace", ["auto", None], ids=["two_level", "streaming"])
@pytest.mark.parametrize("K", [100, 2048])
def test_topk_two_level_many_rows(K, workspace):
    """At least 256 rows with N > 8192: rows of up to 8192 keys go to the
    register-resident kernel; longer ones are cut into 8192-key segments
    whose top-K candidates are then reduced."""
    rng = np.random.default_rng(31 + K)
    B, M, N = 1, 300, 20000
    lg = _dist("ties" if K == 100 else "special", (B, M, N), rng)
    ks = rng.integers(0, 3000, (B, M)).astype(np.int32)
    ke = (ks + rng.integers(0, N - 3000, (B, M))).astype(np.int32)
    ks[0, :6] = [0, 0, 0, 5, 0, 19000]
    ke[0, :6] = [N, 8192, 8193, 16390, K, N]
    log(f"topk two-level many rows K={K} workspace={workspace}")
    _compare(lg, ks, ke, K, what=f"two-level many rows K{K}", workspace=workspace)


def test_topk_many_long_rows_streaming():
    """N > 8192 with more rows than the two-level candidate buffer allows
    (rows * ceil(N / 8192) * K * 4 bytes > 256 MiB): rows of up to 8192 keys
    go to the register-resident kernel, longer ones to one streaming
    workgroup each.  Sampled rows include every long row."""
    B, M, N, K = 1, 17000, 16384, 2048
    rng = np.random.default_rng(23)
    ks = rng.integers(0, 4000, (B, M)).astype(np.int32)
    ke = (ks + rng.integers(0, 8193, (B, M))).astype(np.int32)
    long_rows = np.array([3, 777, 8000, 16999])
    ks[0, long_rows] = [0, 5, 100, 0]
    ke[0, long_rows] = [N, 16000, 8293, 8193]
    log("topk many long rows (streaming)")
    gen = torch.Generator().manual_seed(5)
    lg = torch.randn((B, M, N), generator=gen, dtype=torch.float32)
    lg[0, :100] = torch.round(lg[0, :100] * 2) / 2  # some tie-heavy rows
    out = dsa.topk(lg.to("cuda"), dev(ks), dev(ke), K)
    torch.cuda.synchronize()
    g = out.cpu().numpy().reshape(M, K)
    rows = np.unique(np.concatenate([sample_rows(M, 60, seed=4, must=[0, 1, 50, M - 1]),
                                     long_rows]))
    flat = lg.numpy().reshape(M, N)
    ref = oracle.topk(flat[rows], ks, ke, B, M, N, K, rows=rows)
    compare_topk(g[rows], ref, "many long rows")
