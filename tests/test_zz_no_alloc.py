"""GPU: dsa_prefill_noalloc (static device scratch, no allocation by the
library) against dsa_prefill with a caller workspace, through the C ABI, on
decode-shaped inputs whose top-k and attention both take their scratch
paths (rows split into segments sharing digit histograms; attention rows
split over workgroups with a merge).  Two calls in a row, the second with a
smaller input, so the second runs on scratch holding the first call's
contents.  Same kernels and the same split decisions: the logits inside each
window, the top-k indices and the attention output must be identical."""
import numpy as np
import pytest
import torch

import fp8_indexer_amd as dsa
import workloads as W
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

CALLS = [  # (B, N, K, seed): the second smaller than the first
    (8, 20000, 512, 1),
    (3, 12000, 256, 2),
]


def _inputs(B, N, K, seed):
    wl = W.WORKLOADS["decode_b64"].with_(B=B, N=N, K=K, decode_min=K + 100, seed=seed)
    return wl, W.make_inputs(wl)


def _run(fn, wl, x, **kw):
    g = {k: dev(v) for k, v in x.items() if k != "lengths"}
    logits = torch.full((wl.B, wl.M, wl.N), float("nan"), dtype=torch.float32, device="cuda")
    r = fn(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"], wl.K, g["q"],
           g["kv"], g["sink"], sm_scale=wl.sm_scale, dv=wl.Dv, kv_scale=g["kv_scale"],
           logits=logits, **kw)
    torch.cuda.synchronize()
    return [t.cpu() for t in r]


def test_noalloc_matches_prefill_twice():
    for B, N, K, seed in CALLS:
        wl, x = _inputs(B, N, K, seed)
        a = dsa._prefill_args(*(dev(x[k]) for k in ("q8", "q_scale", "k8", "k_scale", "w", "ks",
                                                    "ke")), K, dev(x["q"]), dev(x["kv"]),
                              dev(x["sink"]), wl.sm_scale, wl.Dv, None, None, None, None)[0]
        need = dsa.prefill_workspace_size(a)
        log(f"noalloc B={B} N={N} K={K}: scratch {need} bytes")
        assert 0 < need <= dsa.NOALLOC_SCRATCH_BYTES
        lg0, ix0, o0 = _run(dsa.prefill, wl, x, workspace="auto")
        lg1, ix1, o1 = _run(dsa.prefill_noalloc, wl, x)
        win = ~torch.isnan(lg0)
        assert torch.equal(win, ~torch.isnan(lg1)), "logits written outside a window"
        assert torch.equal(lg0[win], lg1[win]), "logits differ"
        assert torch.equal(ix0, ix1), "top-k differs"
        assert torch.equal(o0, o1), "attention output differs"
