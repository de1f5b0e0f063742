"""GPU parity: dsa_sparse_attn_fwd against the fp64 oracle
(max|d| <= 2e-2, mean|d| <= 2e-3 on the bf16 output)."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import check_attn, dev, log, sample_rows

pytestmark = pytest.mark.gpu


def _run(x, idx, wl, workspace="auto"):
    o = dsa.sparse_attn_fwd(dev(x["q"]), dev(x["kv"]), dev(x["sink"]), dev(idx), wl.sm_scale,
                            wl.Dv, kv_scale=dev(x["kv_scale"]), workspace=workspace)
    torch.cuda.synchronize()
    return o


def _indices(rng, B, M, N, K, kind):
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            if kind == "full":
                n = K
            else:
                n = int(rng.integers(0, K + 1))
            sel = rng.choice(N, size=min(n, N), replace=False).astype(np.int32)
            idx[b, t, :sel.size] = sel
    if kind == "messy":  # out-of-range values, duplicates, holes, shuffled
        m = rng.random(idx.shape)
        idx[m < 0.05] = N + 7
        idx[(m >= 0.05) & (m < 0.08)] = -5
        idx[(m >= 0.08) & (m < 0.12)] = rng.integers(0, N)
        idx[..., : K // 2] = idx[..., : K // 2][..., ::-1]
    return idx


CASES = [  # Hq, Dqk, Dv, K, fp8, sink
    (16, 64, 64, 32, False, True),
    (16, 64, 64, 50, False, False),
    (32, 64, 64, 100, False, True),
    (128, 64, 64, 64, False, True),
    (16, 576, 512, 64, False, True),
    (64, 576, 512, 96, False, False),
    (128, 576, 512, 2048, False, True),
    (128, 576, 512, 77, False, True),
    (64, 576, 512, 2048, True, True),
    (16, 576, 512, 40, True, False),
    (128, 576, 512, 64, True, True),
]


@pytest.mark.parametrize("Hq,Dqk,Dv,K,fp8,sink", CASES)
@pytest.mark.parametrize("kind", ["full", "ragged", "messy"])
def test_attn_small(Hq, Dqk, Dv, K, fp8, sink, kind):
    B, M, N = 2, 3, 3000
    wl = W.Workload("a", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=Dqk, Dv=Dv, kv_fp8=fp8,
                    seed=Hq + K)
    log(f"attn small Hq={Hq} Dqk={Dqk} Dv={Dv} K={K} fp8={fp8} sink={sink} {kind}")
    x = W.make_inputs(wl, parts=("attn",))
    if not sink:
        x["sink"] = None
    rng = np.random.default_rng(K)
    idx = _indices(rng, B, M, N, K, kind)
    o = _run(x, idx, wl)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, Dv,
                             kv_scale=x["kv_scale"])
    check_attn(o, ref, f"Hq{Hq}/{Dqk}/{K}/{kind}")


@pytest.mark.parametrize("sink", [True, False])
@pytest.mark.parametrize("kind", ["full", "ragged", "messy"])
@pytest.mark.parametrize("K", [1, 31, 32, 33, 77, 300, 2048, 3000])
def test_attn_unsplit_128_heads(K, kind, sink):
    """128 heads, bf16, no workspace: the unsplit instance (two waves per
    SIMD for K <= 2048; K = 3000 takes the one-wave-per-SIMD kernel), at
    tile-boundary lengths, with empty, ragged and messy index lists."""
    B, M, N = 2, 3, 3000
    wl = W.Workload("u", B=B, M=M, N=N, H=4, D=64, K=K, Hq=128, Dqk=576, Dv=512, seed=K + 5)
    log(f"attn unsplit 128 heads K={K} {kind} sink={sink}")
    x = W.make_inputs(wl, parts=("attn",))
    if not sink:
        x["sink"] = None
    idx = _indices(np.random.default_rng(K + 1), B, M, N, K, kind)
    o = _run(x, idx, wl, workspace=None)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv)
    check_attn(o, ref, f"unsplit K{K}/{kind}")


@pytest.mark.parametrize("fp8", [False, True])
def test_attn_all_invalid_rows_are_zero(fp8):
    B, M, N, K = 1, 4, 500, 64
    wl = W.Workload("z", B=B, M=M, N=N, H=4, D=64, K=K, Hq=64, Dqk=576, Dv=512, kv_fp8=fp8, seed=4)
    x = W.make_inputs(wl, parts=("attn",))
    idx = np.full((B, M, K), -1, np.int32)
    idx[0, 1, :] = N + 3        # all out of range
    idx[0, 2, 10] = 17          # one valid index
    o = _run(x, idx, wl).float().cpu().numpy()
    assert np.all(o[0, 0] == 0) and np.all(o[0, 1] == 0) and np.all(o[0, 3] == 0)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(torch.from_numpy(o), ref, "one valid")
    x["sink"] = None
    o2 = _run(x, idx, wl).float().cpu().numpy()
    assert np.all(o2[0, 0] == 0)


WORKLOAD_ROWS = {"tiny_causal_256": None, "prefill_4096": 24, "varlen_4x8192": 12,
                 "decode_b64": 12, "prefill_8192_fp8kv": 16}


@pytest.mark.parametrize("name", list(WORKLOAD_ROWS))
def test_attn_workloads(name):
    wl = W.WORKLOADS[name]
    log(f"attn workload {name}")
    x = W.make_inputs(wl, parts=("attn",))
    idx = W.synthetic_topk(wl, x["ks"], x["ke"])
    o = _run(x, idx, wl)
    R = wl.B * wl.M
    n = WORKLOAD_ROWS[name]
    rows = None if n is None else sample_rows(R, n, seed=2, must=[0, R - 1, wl.K - 1, wl.K])
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"], rows=rows)
    og = o.reshape(R, wl.Hq, wl.Dv)
    if rows is not None:
        og = og[torch.from_numpy(rows).to(og.device)]
    mx, mn = check_attn(og, ref, name)
    log(f"  max|d| {mx:.3g} mean|d| {mn:.3g}")


@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "unsplit"])
@pytest.mark.parametrize("Hq", [128, 64])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("where", ["middle", "last", "first", "moderate", "second_half"])
def test_attn_reference_restart(fp8, where, Hq, workspace):
    """A score far above every score of the first tile (the kernel's fixed
    softmax reference: 72 natural units, p ~ 2^104) forces the max-only
    pre-pass and the second pass.  "moderate": ~21 natural units above (p ~
    2^30), which the fixed reference carries exactly without a restart.
    "second_half": the big score in rows 16-31 of the first tile (the second
    16-row MFMA tile of the first gathered tile).  Two query rows: with a
    workspace they run the split instance (each row's indices over several
    workgroups), without one the unsplit instance that every prefill row
    runs."""
    B, M, N, K = 1, 2, 600, 256
    wl = W.Workload("r", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512, kv_fp8=fp8,
                    seed=6)
    x = W.make_inputs(wl, parts=("attn",))
    big = {"middle": 300, "last": 599, "first": 3, "moderate": 300, "second_half": 301}[where]
    qv = torch.ones((B, M, wl.Hq, wl.Dqk), dtype=torch.float32) * 0.5
    qv[..., ::2] = 1.0
    x["q"] = qv.to(torch.bfloat16)
    kvf = torch.from_numpy(np.random.default_rng(1).standard_normal((B, N, wl.Dqk))
                           .astype(np.float32))
    if where == "moderate":
        kvf[0, big] = 1.25     # q.k/24 = 22.5; o ~ 1.25, exact in bf16
    else:
        kvf[0, big] = 4.0      # q.k/24 = 72 (natural units) above the others
        kvf[0, big, :8] = -3.0
    if fp8:
        x["kv"], x["kv_scale"] = W.quantize_e4m3fn_rows(kvf.numpy())
    else:
        x["kv"] = kvf.to(torch.bfloat16)
    idx = np.tile(np.arange(0, 2 * K, 2, dtype=np.int32), (B, M, 1))  # rows 0,2,..,510
    idx[0, 0, K // 2] = big
    idx[0, 1, {"first": 0, "second_half": 20}.get(where, K - 1)] = big
    log(f"attn restart {where} fp8={fp8} Hq={Hq} workspace={workspace}")
    o = _run(x, idx, wl, workspace)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(o, ref, f"restart/{where}")


@pytest.mark.parametrize("Hq", [128, 64])
@pytest.mark.parametrize("fp8", [False, True])
def test_attn_split_rows_edge_cases(fp8, Hq):
    """Few rows with K = 2048: each row's indices are split over several
    workgroups and merged.  Row 0 has no valid index (zero output), row 1
    only valid indices in the last split, row 2 a full set."""
    B, M, N, K = 1, 3, 5000, 2048
    wl = W.Workload("s", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512, kv_fp8=fp8,
                    seed=9)
    log(f"attn split edge fp8={fp8} Hq={Hq}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(5)
    idx = np.full((B, M, K), -1, np.int32)
    idx[0, 1, K - 100:] = rng.choice(N, size=100, replace=False)
    idx[0, 2, :] = rng.choice(N, size=K, replace=False)
    o = _run(x, idx, wl)
    assert torch.all(o[0, 0].float() == 0)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(o, ref, "split edge")


@pytest.mark.parametrize("Hq,fp8", [(128, False), (64, True)])
def test_attn_split_rows_multiple_of_8(Hq, fp8):
    """16 rows (a multiple of the 8 XCDs, so the splits of each row are
    placed together), each split over several workgroups: every row of o
    against the oracle, rows of different lengths, one row without a valid
    index."""
    B, M, N, K = 2, 8, 4000, 1024
    wl = W.Workload("s8", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512, kv_fp8=fp8,
                    seed=21)
    log(f"attn split 16 rows fp8={fp8} Hq={Hq}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(21)
    idx = np.full((B, M, K), -1, np.int32)
    for r in range(B * M):
        n = 0 if r == 5 else int(rng.integers(1, K + 1))
        idx.reshape(B * M, K)[r, :n] = rng.choice(N, size=n, replace=False)
    o = _run(x, idx, wl)
    assert torch.all(o.reshape(B * M, Hq, wl.Dv)[5].float() == 0)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(o, ref, "split 16 rows")


@pytest.mark.parametrize("Hq,fp8", [(128, False), (64, True)])
def test_attn_restart_many_rows(Hq, fp8):
    """160 query rows (more than half the compute units: the unsplit
    instance whatever the workspace) at the prefill head counts; every 7th
    row holds one score ~72 natural units above its first tile's maximum
    (a restart of that row's workgroup), at a varying position, the other
    rows none."""
    B, M, N, K = 1, 160, 3000, 512
    wl = W.Workload("rm", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512, kv_fp8=fp8,
                    seed=12)
    log(f"attn restart many rows Hq={Hq} fp8={fp8}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(3)
    qv = torch.ones((B, M, Hq, wl.Dqk), dtype=torch.float32) * 0.5
    qv[..., ::2] = 1.0
    x["q"] = qv.to(torch.bfloat16)
    kvf = torch.from_numpy(rng.standard_normal((B, N, wl.Dqk)).astype(np.float32))
    big = 2999
    kvf[0, big] = 4.0
    kvf[0, big, :8] = -3.0
    if fp8:
        x["kv"], x["kv_scale"] = W.quantize_e4m3fn_rows(kvf.numpy())
    else:
        x["kv"] = kvf.to(torch.bfloat16)
    idx = np.stack([rng.choice(N - 1, size=K, replace=False) for _ in range(M)]).astype(np.int32)
    idx = idx.reshape(B, M, K)
    for t in range(0, M, 7):
        idx[0, t, (37 * t) % K] = big
    assert dsa.sparse_attn_workspace_size(B, M, Hq, 576, 512, K) == 0  # unsplit
    o = _run(x, idx, wl)
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(o, ref, "restart many rows")


@pytest.mark.parametrize("Hq,fp8", [(128, False), (64, True)])
def test_attn_split_and_unsplit_agree(Hq, fp8):
    """Decode-shaped rows (batch 8, K = 2048): the split instance (with a
    workspace) and the unsplit one (without) both match the oracle."""
    B, M, N, K = 8, 1, 6000, 2048
    wl = W.Workload("su", B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512, kv_fp8=fp8,
                    seed=13)
    log(f"attn split/unsplit Hq={Hq} fp8={fp8}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(8)
    idx = np.stack([rng.choice(N, size=K, replace=False) for _ in range(B * M)]).astype(np.int32)
    idx = idx.reshape(B, M, K)
    idx[1, 0, 100:] = -1
    assert dsa.sparse_attn_workspace_size(B, M, Hq, 576, 512, K) > 0
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                             kv_scale=x["kv_scale"])
    check_attn(_run(x, idx, wl, "auto"), ref, "split")
    check_attn(_run(x, idx, wl, None), ref, "unsplit")
