"""GPU parity: dsa_sparse_attn_bwd against the fp64 oracle.

Bar (derived): every GPU gradient element within 2^-7 of the sum of the
absolute values of its terms (oracle |term| sums, with ds_j = p_j (dp_j -
Delta) expanded into p_j dp_j and the products p_j dO[c] o[c] of Delta).
The GPU rounds P and dS to bf16 before the MFMA products (2^-9 relative per
term) and forms Delta from the bf16 forward output o (2^-9 relative per
product); everything else is fp32 (~1e-6), so the worst case is ~2^-8 of the
term sum and the bar leaves a factor 2."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import dev, log, sample_rows

pytestmark = pytest.mark.gpu
BAR = 2.0 ** -7


def check_grad(g, ref, terms, what):
    g = np.asarray(g, np.float64).reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    d = np.abs(g - ref)
    tol = BAR * terms + 1e-7
    bad = d > tol
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, worst "
                           f"{d[bad].max():.3g} vs tol {tol[bad].min():.3g}")
    return float(d.max())


def _indices(rng, B, M, N, K, kind):
    idx = np.stack([rng.choice(N, size=K, replace=False) for _ in range(B * M)])
    idx = idx.astype(np.int32).reshape(B, M, K)
    if kind == "ragged":
        for r in range(B * M):
            n = int(rng.integers(0, K + 1))
            idx.reshape(B * M, K)[r, n:] = -1
    elif kind == "messy":  # duplicates, out of range, -1 holes, an empty row
        m = rng.random(idx.shape)
        idx[m < 0.05] = N + 3
        idx[(m >= 0.05) & (m < 0.1)] = -1
        idx[..., 1] = idx[..., 0]
        idx[0, 0] = -1
    return idx


def _run(x, idx, dO, wl):
    o = dsa.sparse_attn_fwd(dev(x["q"]), dev(x["kv"]), dev(x["sink"]), dev(idx), wl.sm_scale,
                            wl.Dv)
    g = dsa.sparse_attn_bwd(dev(x["q"]), dev(x["kv"]), dev(x["sink"]), dev(idx), o, dev(dO),
                            wl.sm_scale)
    torch.cuda.synchronize()
    return g


CASES = [  # Hq, Dqk, Dv, K, sink
    (16, 64, 64, 32, True),
    (16, 64, 64, 50, False),
    (32, 64, 64, 100, True),
    (128, 64, 64, 64, True),
    (16, 576, 512, 64, True),
    (64, 576, 512, 96, False),
    (128, 576, 512, 2048, True),
    (128, 576, 512, 77, True),
]


@pytest.mark.parametrize("Hq,Dqk,Dv,K,sink", CASES)
@pytest.mark.parametrize("kind", ["full", "ragged", "messy"])
def test_attn_bwd_small(Hq, Dqk, Dv, K, sink, kind):
    B, M, N = 2, 3, 3000
    wl = W.Workload("bw", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=Dqk, Dv=Dv, seed=Hq + K)
    log(f"attn bwd Hq={Hq} Dqk={Dqk} Dv={Dv} K={K} sink={sink} {kind}")
    x = W.make_inputs(wl, parts=("attn",))
    if not sink:
        x["sink"] = None
    rng = np.random.default_rng(K + Hq)
    idx = _indices(rng, B, M, N, K, kind)
    dO = torch.from_numpy(rng.standard_normal((B, M, Hq, Dv)).astype(np.float32)).to(
        torch.bfloat16)
    dq, dkv, dsink = _run(x, idx, dO, wl)
    rq, rkv, rs, tq, tkv, ts = oracle.sparse_attn_bwd(x["q"], x["kv"], x["sink"], idx, dO,
                                                      wl.sm_scale, Dv, with_terms=True)
    check_grad(dq.cpu().numpy(), rq, tq, "dq")
    check_grad(dkv.cpu().numpy(), rkv, tkv, "dkv")
    if sink:
        check_grad(dsink.cpu().numpy(), rs, ts, "dsink")
    else:
        assert dsink is None
    if kind == "messy":  # the row without a valid index has no gradient
        assert torch.all(dq[0, 0] == 0)


@pytest.mark.parametrize("Hq,Dqk,Dv", [(48, 64, 64), (80, 576, 512)])
def test_attn_bwd_odd_head_groups(Hq, Dqk, Dv):
    """Head counts that are a multiple of 16 but not of 32 (the gradient
    runs in 16-head workgroups, several per token).  The forward has no
    kernel for them, so o is the oracle's forward output rounded to bf16,
    which stands for any forward within bf16 rounding."""
    B, M, N, K = 2, 3, 3000, 40
    wl = W.Workload("bw", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=Dqk, Dv=Dv, seed=Hq)
    log(f"attn bwd Hq={Hq} Dqk={Dqk} Dv={Dv} K={K}, o from the oracle")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(Hq)
    idx = _indices(rng, B, M, N, K, "ragged")
    dO = torch.from_numpy(rng.standard_normal((B, M, Hq, Dv)).astype(np.float32)).to(
        torch.bfloat16)
    o = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, Dv)
    o = torch.from_numpy(np.asarray(o, np.float32).reshape(B, M, Hq, Dv)).to(torch.bfloat16)
    dq, dkv, dsink = dsa.sparse_attn_bwd(dev(x["q"]), dev(x["kv"]), dev(x["sink"]), dev(idx),
                                         dev(o), dev(dO), wl.sm_scale)
    torch.cuda.synchronize()
    rq, rkv, rs, tq, tkv, ts = oracle.sparse_attn_bwd(x["q"], x["kv"], x["sink"], idx, dO,
                                                      wl.sm_scale, Dv, with_terms=True)
    check_grad(dq.cpu().numpy(), rq, tq, "dq")
    check_grad(dkv.cpu().numpy(), rkv, tkv, "dkv")
    check_grad(dsink.cpu().numpy(), rs, ts, "dsink")


@pytest.mark.parametrize("Hq,Dqk,Dv", [(32, 64, 64), (32, 576, 512)])
def test_attn_bwd_max_k(Hq, Dqk, Dv):
    """K = 4096, the largest supported top-k: 256 index tiles per token (one
    per thread when the list of non-empty tiles is built), every index slot
    of the token in LDS; ragged rows with -1 tails and one row of -1 only."""
    B, M, N, K = 1, 3, 5000, 4096
    wl = W.Workload("bw", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=Dqk, Dv=Dv, seed=7)
    log(f"attn bwd Hq={Hq} Dqk={Dqk} Dv={Dv} K={K}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(11)
    idx = _indices(rng, B, M, N, K, "full")
    idx[0, 1, 3000:] = -1
    idx[0, 2, :] = -1
    dO = torch.from_numpy(rng.standard_normal((B, M, Hq, Dv)).astype(np.float32)).to(
        torch.bfloat16)
    dq, dkv, dsink = _run(x, idx, dO, wl)
    rq, rkv, rs, tq, tkv, ts = oracle.sparse_attn_bwd(x["q"], x["kv"], x["sink"], idx, dO,
                                                      wl.sm_scale, Dv, with_terms=True)
    check_grad(dq.cpu().numpy(), rq, tq, "dq")
    check_grad(dkv.cpu().numpy(), rkv, tkv, "dkv")
    check_grad(dsink.cpu().numpy(), rs, ts, "dsink")
    assert torch.all(dq[0, 2] == 0)


def test_attn_bwd_workload_sampled_rows():
    """The 4096-token workload's shapes (128 heads, 576/512, K = 2048) on
    top-k-shaped index lists, dO nonzero on sampled rows only: the other
    rows contribute nothing, so the full dkv and dsink are the oracle's over
    the sampled rows; dq is compared on those rows and must be 0 elsewhere."""
    wl = W.WORKLOADS["prefill_4096"]
    log("attn bwd 4096-token workload, sampled rows")
    x = W.make_inputs(wl, parts=("attn",))
    idx = W.synthetic_topk(wl, x["ks"], x["ke"])
    R = wl.B * wl.M
    rows = sample_rows(R, 6, seed=9, must=[0, wl.K - 1, wl.K, R - 1])
    rng = np.random.default_rng(3)
    dOf = np.zeros((wl.B, wl.M, wl.Hq, wl.Dv), np.float32)
    dOf.reshape(R, wl.Hq, wl.Dv)[rows] = rng.standard_normal((len(rows), wl.Hq, wl.Dv))
    dO = torch.from_numpy(dOf).to(torch.bfloat16)
    dq, dkv, dsink = _run(x, idx, dO, wl)
    rq, rkv, rs, tq, tkv, ts = oracle.sparse_attn_bwd(x["q"], x["kv"], x["sink"], idx, dO,
                                                      wl.sm_scale, wl.Dv, rows=rows,
                                                      with_terms=True)
    dqh = dq.reshape(R, wl.Hq, wl.Dqk)
    m = check_grad(dqh[torch.from_numpy(rows).to(dq.device)].cpu().numpy(), rq, tq, "dq")
    others = torch.ones(R, dtype=torch.bool, device=dq.device)
    others[torch.from_numpy(rows).to(dq.device)] = False
    assert torch.all(dqh[others] == 0)
    mk = check_grad(dkv.cpu().numpy(), rkv, tkv, "dkv")
    ms = check_grad(dsink.cpu().numpy(), rs, ts, "dsink")
    log(f"  max|d| dq {m:.3g} dkv {mk:.3g} dsink {ms:.3g}")
