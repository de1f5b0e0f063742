"""GPU: indexer + top-k without the [B, M, N] logits buffer
(dsa_indexer_topk, and dsa_prefill with logits = NULL).  Its top-k must be
bit-identical to dsa_topk applied to dsa_indexer_logits' output for the same
arguments (every row), and equal to the oracle's top-k of those logits on
sampled rows; slab sizes that split batch entries, group them, and leave
short tails are covered."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import compare_topk, dev, log, sample_rows

pytestmark = pytest.mark.gpu


def _unfused(g, K):
    lg = dsa.indexer_logits(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"],
                            g["ke"])
    return lg, dsa.topk(lg, g["ks"], g["ke"], K)


def _upload(x):
    return {k: dev(v) for k, v in x.items() if k != "lengths"}


@pytest.mark.parametrize("name", ["prefill_4096", "varlen_4x8192", "prefill_8192_fp8kv",
                                  "decode_b64"])
def test_indexer_topk_matches_unfused(name):
    wl = W.WORKLOADS[name]
    log(f"fused indexer+top-k {name}")
    x = W.make_inputs(wl, parts=("indexer",))
    g = _upload(x)
    lg, ref = _unfused(g, wl.K)
    fused = dsa.indexer_topk(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"],
                             g["ke"], wl.K)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref), f"{name}: fused top-k differs from dsa_topk(logits)"
    R = wl.B * wl.M
    rows = sample_rows(R, 12, seed=7, must=[0, R - 1])
    lg_rows = lg.reshape(R, wl.N)[torch.from_numpy(rows).to(lg.device)].cpu().numpy()
    ti = oracle.topk(lg_rows, x["ks"], x["ke"], wl.B, wl.M, wl.N, wl.K, rows=rows)
    compare_topk(fused.reshape(R, wl.K).cpu().numpy()[rows], ti, f"{name} vs oracle")
    full = wl.B * wl.M * wl.N * 4
    ws = dsa.indexer_topk_workspace_size(wl.B, wl.M, wl.N, wl.H, wl.D, wl.K)
    log(f"  workspace {ws / 2**20:.1f} MiB vs logits buffer {full / 2**20:.1f} MiB")


@pytest.mark.parametrize("B,M,N,H,D,K,slab", [
    (1, 256, 256, 4, 64, 32, 50),     # token runs of 50; a short tail joins the last run
    (1, 300, 900, 64, 128, 100, 97),  # runs of 97, tail of 9 rows (>= 3) kept
    (1, 130, 500, 64, 128, 64, 128),  # tail of 2 rows (< 3) joins: one run of 130
    (5, 40, 700, 32, 128, 64, 100),   # two batch entries per slab
    (7, 1, 20000, 64, 128, 256, 3),   # decode shapes: 3 entries per slab, split top-k
])
def test_indexer_topk_slabs(B, M, N, H, D, K, slab):
    wl = W.Workload("slab", B=B, M=M, N=N, H=H, D=D, K=K, Hq=16, Dqk=64, Dv=64, seed=B + M,
                    windows="decode" if M == 1 else "causal", decode_min=K // 2)
    log(f"fused slabs B={B} M={M} N={N} H={H} K={K} slab={slab}")
    x = W.make_inputs(wl, parts=("indexer",))
    if M > 1:  # ragged windows: some empty, some past N
        rng = np.random.default_rng(M)
        ks = rng.integers(-5, N // 2, (B, M)).astype(np.int32)
        ke = (ks + rng.integers(-3, N, (B, M))).astype(np.int32)
        x["ks"], x["ke"] = ks, ke
    g = _upload(x)
    _, ref = _unfused(g, K)
    fused = dsa.indexer_topk(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"],
                             g["ke"], K, slab_rows=slab)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref)


@pytest.mark.parametrize("name,M", [("prefill_4096", 700), ("prefill_8192_fp8kv", 600)])
def test_prefill_without_logits_buffer(name, M):
    """dsa_prefill with logits = NULL: same top-k and attention output as with
    the buffer."""
    wl = W.WORKLOADS[name].with_(M=M, N=M)
    log(f"prefill without logits buffer {name} M={M}")
    x = W.make_inputs(wl)
    g = _upload(x)
    args = (g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"], wl.K,
            g["q"], g["kv"], g["sink"])
    kw = dict(sm_scale=wl.sm_scale, dv=wl.Dv, kv_scale=g.get("kv_scale"))
    _, i0, o0 = dsa.prefill(*args, **kw)
    lg1, i1, o1 = dsa.prefill(*args, logits=False, **kw)
    torch.cuda.synchronize()
    assert lg1 is None
    assert torch.equal(i0, i1)
    assert torch.equal(o0, o1)
