"""GPU parity: dsa_sparse_attn_fwd_fp8 (full-FP8 attention: e4m3 q and KV,
bf16 output) against the fp64 oracle on the same e4m3 inputs.

Bar (derived from the arithmetic; the probabilities enter PV as e4m3, which
the bf16 path's 2e-2 / 2e-3 bar does not allow for when a few terms dominate
an output):
  * per element |d| <= 2^-4 * T + 2^-8 * |o| + 4e-3, where T = sum_j p_j
    |v_jc| (the oracle's term sums): each scaled probability is rounded to
    e4m3 (relative error at most 2^-4 in the format's normal range), o to bf16
    (2^-9 relative), and the floor covers probabilities in the e4m3 subnormal
    range (rounded to a multiple of 2^-9 of the scaled range);
  * where many independent terms make up each output (random indices without
    heavy duplication, K >= 300), the least-squares slope of the GPU output
    on the oracle's is 1 within 4e-3: the roundings are to nearest even and
    unbiased, so a systematic scale error shows here long before it reaches
    the per-element bound."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import oracle
import workloads as W
from gpu_util import dev, log, sample_rows
from test_gpu_attn import _indices

pytestmark = pytest.mark.gpu


def _run(x, idx, wl, workspace="auto", q_scale="keep"):
    qs = x["qa_scale"] if q_scale == "keep" else q_scale
    o = dsa.sparse_attn_fwd_fp8(dev(x["q"]), dev(qs), dev(x["kv"]), dev(x["kv_scale"]),
                                dev(x["sink"]), dev(idx), wl.sm_scale, wl.Dv,
                                workspace=workspace)
    torch.cuda.synchronize()
    return o


def _ref(x, idx, wl, rows=None, q_scale="keep"):
    qs = x["qa_scale"] if q_scale == "keep" else q_scale
    return oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv,
                              kv_scale=x["kv_scale"], rows=rows, q_scale=qs, q_fp8=True,
                              with_terms=True)


def check_fp8(o_gpu, ref, what="", slope_tol=None):
    o_ref, terms = ref
    g = o_gpu.float().cpu().numpy().astype(np.float64).reshape(o_ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    d = np.abs(g - o_ref)
    bound = 2.0 ** -4 * terms + 2.0 ** -8 * np.abs(o_ref) + 4e-3
    den = float((o_ref * o_ref).sum())
    slope = float((g * o_ref).sum()) / den if den > 0 else 1.0
    log(f"  {what}: max|d| {d.max():.4g} mean|d| {d.mean():.4g} mean T {terms.mean():.4g} "
        f"max d/bound {(d / bound).max():.3f} slope {slope:.5f}")
    bad = d > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the e4m3 bound, worst "
                           f"{(d - bound).max()}")
    if slope_tol is not None:
        assert abs(slope - 1.0) <= slope_tol, f"{what}: slope {slope}"
    return float(d.max()), float(d.mean())


def _wl(name, B, M, N, K, Hq, seed):
    return W.Workload(name, B=B, M=M, N=N, H=4, D=64, K=K, Hq=Hq, Dqk=576, Dv=512,
                      kv_fp8=True, q_fp8=True, seed=seed)


CASES = [  # Hq, K, sink
    (128, 64, True),
    (128, 77, False),
    (128, 300, True),
    (128, 2048, True),
    (64, 64, True),
    (64, 130, True),
    (64, 2048, False),
]


@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "unsplit"])
@pytest.mark.parametrize("Hq,K,sink", CASES)
@pytest.mark.parametrize("kind", ["full", "ragged", "messy"])
def test_fp8_attn_small(Hq, K, sink, kind, workspace):
    """Two batch entries of 3 query rows over 3000 keys: with a workspace
    the rows with K >= 512 run split (each row's indices over several
    workgroups and a merge), without one unsplit."""
    B, M, N = 2, 3, 3000
    wl = _wl("f", B, M, N, K, Hq, seed=Hq + K)
    log(f"fp8 attn small Hq={Hq} K={K} sink={sink} {kind} workspace={workspace}")
    x = W.make_inputs(wl, parts=("attn",))
    if not sink:
        x["sink"] = None
    idx = _indices(np.random.default_rng(K), B, M, N, K, kind)
    many = K >= 300 and kind != "messy"
    check_fp8(_run(x, idx, wl, workspace), _ref(x, idx, wl), f"Hq{Hq}/K{K}/{kind}",
              slope_tol=4e-3 if many else None)


def test_fp8_attn_without_q_scale():
    B, M, N, K = 1, 4, 900, 256
    wl = _wl("n", B, M, N, K, 128, seed=3)
    log("fp8 attn without q_scale")
    x = W.make_inputs(wl, parts=("attn",))
    idx = _indices(np.random.default_rng(1), B, M, N, K, "ragged")
    check_fp8(_run(x, idx, wl, q_scale=None), _ref(x, idx, wl, q_scale=None), "no q_scale")


@pytest.mark.parametrize("Hq", [128, 64])
def test_fp8_attn_all_invalid_rows_are_zero(Hq):
    B, M, N, K = 1, 4, 500, 64
    wl = _wl("z", B, M, N, K, Hq, seed=4)
    log(f"fp8 attn all-invalid rows Hq={Hq}")
    x = W.make_inputs(wl, parts=("attn",))
    idx = np.full((B, M, K), -1, np.int32)
    idx[0, 1, :] = N + 3        # all out of range
    idx[0, 2, 10] = 17          # one valid index
    o = _run(x, idx, wl)
    of = o.float().cpu().numpy()
    assert np.all(of[0, 0] == 0) and np.all(of[0, 1] == 0) and np.all(of[0, 3] == 0)
    check_fp8(o, _ref(x, idx, wl), "one valid")
    x["sink"] = None
    assert torch.all(_run(x, idx, wl)[0, 0].float() == 0)


def _spiky(wl, big, N, B=1, seed=1):
    """q codes of a fixed positive pattern and N(0,1) KV rows, except row
    `big`, whose score is ~72 natural units above the others."""
    x = W.make_inputs(wl, parts=("attn",))
    qv = np.full((B, wl.M, wl.Hq, wl.Dqk), 0.5, np.float32)
    qv[..., ::2] = 1.0
    x["q"], x["qa_scale"] = W.quantize_e4m3fn_rows(qv)
    kvf = np.random.default_rng(seed).standard_normal((B, N, wl.Dqk)).astype(np.float32)
    kvf[0, big] = 4.0
    kvf[0, big, :8] = -3.0
    x["kv"], x["kv_scale"] = W.quantize_e4m3fn_rows(kvf)
    return x


@pytest.mark.parametrize("workspace", ["auto", None], ids=["split", "unsplit"])
@pytest.mark.parametrize("Hq", [128, 64])
@pytest.mark.parametrize("where", ["first", "second_half", "middle", "last"])
def test_fp8_attn_reference_restart(where, Hq, workspace):
    """A score far above every score of the first tile (the kernel's fixed
    reference; P would pass the e4m3 maximum) forces the max-only pre-pass
    and the exact-max pass.  "second_half": in rows 32-63 of the first
    64-row tile (the other row half, with 64 heads another wave's)."""
    B, M, N, K = 1, 2, 1200, 512
    wl = _wl("r", B, M, N, K, Hq, seed=6)
    big = {"first": 3, "second_half": 1101, "middle": 600, "last": 1199}[where]
    x = _spiky(wl, big, N)
    idx = np.tile(np.arange(0, 2 * K, 2, dtype=np.int32), (B, M, 1))  # rows 0, 2, .., 1022
    idx[0, 0, K // 2] = big
    idx[0, 1, {"first": 0, "second_half": 40}.get(where, K - 1)] = big
    log(f"fp8 attn restart {where} Hq={Hq} workspace={workspace}")
    check_fp8(_run(x, idx, wl, workspace), _ref(x, idx, wl), f"restart/{where}")


@pytest.mark.parametrize("Hq", [128, 64])
def test_fp8_attn_restart_many_rows(Hq):
    """160 query rows (the unsplit instance); every 7th holds one score far
    above its first tile's maximum, at a varying position."""
    B, M, N, K = 1, 160, 3000, 512
    wl = _wl("rm", B, M, N, K, Hq, seed=12)
    log(f"fp8 attn restart many rows Hq={Hq}")
    big = 2999
    x = _spiky(wl, big, N, seed=3)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(N - 1, size=K, replace=False) for _ in range(M)]).astype(np.int32)
    idx = idx.reshape(B, M, K)
    for t in range(0, M, 7):
        idx[0, t, (37 * t) % K] = big
    assert dsa.sparse_attn_fp8_workspace_size(B, M, Hq, 576, 512, K) == 0
    check_fp8(_run(x, idx, wl), _ref(x, idx, wl), "restart many rows")


@pytest.mark.parametrize("Hq", [128, 64])
def test_fp8_attn_split_and_unsplit_agree(Hq):
    """Decode-shaped rows (batch 8, K = 2048): split (with a workspace) and
    unsplit (without) both match the oracle; one row has 100 valid
    indices, another only valid indices in its last split."""
    B, M, N, K = 8, 1, 6000, 2048
    wl = _wl("su", B, M, N, K, Hq, seed=13)
    log(f"fp8 attn split/unsplit Hq={Hq}")
    x = W.make_inputs(wl, parts=("attn",))
    rng = np.random.default_rng(8)
    idx = np.stack([rng.choice(N, size=K, replace=False) for _ in range(B * M)]).astype(np.int32)
    idx = idx.reshape(B, M, K)
    idx[1, 0, 100:] = -1
    idx[2, 0, :K - 70] = -1
    idx[3, 0, :] = -1
    assert dsa.sparse_attn_fp8_workspace_size(B, M, Hq, 576, 512, K) > 0
    ref = _ref(x, idx, wl)
    o1 = _run(x, idx, wl, "auto")
    o2 = _run(x, idx, wl, None)
    assert torch.all(o1[3].float() == 0) and torch.all(o2[3].float() == 0)
    check_fp8(o1, ref, "split", slope_tol=4e-3)
    check_fp8(o2, ref, "unsplit", slope_tol=4e-3)


@pytest.mark.parametrize("name", list(W.FP8_ATTN_WORKLOADS))
def test_fp8_attn_workloads(name):
    """The full-size full-FP8 workloads (causal top-k indices), sampled rows."""
    wl = W.FP8_ATTN_WORKLOADS[name]
    log(f"fp8 attn workload {name}")
    x = W.make_inputs(wl, parts=("attn",))
    idx = W.synthetic_topk(wl, x["ks"], x["ke"])
    o = _run(x, idx, wl)
    R = wl.B * wl.M
    rows = sample_rows(R, 16, seed=2, must=[0, R - 1, wl.K - 1, wl.K])
    ref = _ref(x, idx, wl, rows=rows)
    og = o.reshape(R, wl.Hq, wl.Dv)[torch.from_numpy(rows).to(o.device)]
    mx, mn = check_fp8(og, ref, name, slope_tol=4e-3)
    log(f"  max|d| {mx:.3g} mean|d| {mn:.3g}")
