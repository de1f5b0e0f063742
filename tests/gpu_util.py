"""Helpers shared by the GPU parity tests (device upload, comparisons)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(DEV)


def indexer_gpu(x, N, logits_fill=float("nan")):
    """Run dsa_indexer_logits on the inputs dict; returns host logits."""
    import fp8_indexer_amd as dsa
    B, M = x["q8"].shape[:2]
    out = torch.full((B, M, N), logits_fill, dtype=torch.float32, device=DEV)
    dsa.indexer_logits(dev(x["q8"]), dev(x.get("q_scale")), dev(x["k8"]), dev(x["k_scale"]),
                       dev(x["w"]), dev(x["ks"]), dev(x["ke"]), logits=out)
    torch.cuda.synchronize()
    return out


def check_logits(gpu_rows, ref, terms, what=""):
    """gpu_rows, ref: [n, N] (ref NaN outside windows).  Inside: |d| <=
    1e-4 * sum|terms| (an unwritten logit, still NaN, fails); outside: the
    GPU buffer must be untouched (NaN)."""
    g = np.asarray(gpu_rows, np.float64)
    win = ~np.isnan(ref)
    assert np.all(np.isnan(g[~win])), f"{what}: logits written outside the window"
    assert not np.isnan(g[win]).any(), f"{what}: {np.isnan(g[win]).sum()} window logits unwritten"
    d = np.abs(g[win] - ref[win])
    tol = 1e-4 * terms[win]
    bad = d > tol
    assert not bad.any(), (f"{what}: {bad.sum()} logits out of tolerance, "
                           f"worst {d[bad].max()} vs tol {tol[bad].min()}")
    return float(d.max()) if d.size else 0.0


def compare_topk(got, ref, what=""):
    """Top-k rows must be bit-identical: got, ref [n, K] int32."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    bad = np.nonzero(~np.all(got == ref, axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first row {bad[0]}"


def check_attn(o_gpu, o_ref, what=""):
    g = o_gpu.float().cpu().numpy().astype(np.float64).reshape(o_ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    d = np.abs(g - o_ref)
    assert d.max() <= 2e-2, f"{what}: max|d| {d.max()}"
    assert d.mean() <= 2e-3, f"{what}: mean|d| {d.mean()}"
    return float(d.max()), float(d.mean())


def sample_rows(n_rows, k, seed=0, must=()):
    rng = np.random.default_rng(seed)
    extra = rng.choice(n_rows, size=min(k, n_rows), replace=False)
    rows = sorted(set(int(r) for r in must if 0 <= r < n_rows) | set(int(r) for r in extra))
    return np.asarray(rows, np.int64)
