"""Checker-mutation tests of the GPU parity comparators, on the CPU: the
oracle's own results, with one plausible GPU mistake planted, must fail the
comparison each GPU test applies (a swapped or wrong top-k index, a logit
moved by twice its tolerance or written outside its window, an attention
output element moved by 0.03 or a small bias over the whole output), while
the unmodified results pass."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import check_attn, check_logits, compare_topk


def _expect_fail(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_compare_topk_catches_index_mistakes():
    rng = np.random.default_rng(0)
    B, M, N, K = 1, 20, 300, 16
    lg = rng.integers(-3, 4, (B * M, N)).astype(np.float32)  # many ties
    ks = np.zeros((B, M), np.int32)
    ke = np.full((B, M), N, np.int32)
    ref = oracle.topk(lg, ks, ke, B, M, N, K)
    compare_topk(ref.copy(), ref)
    got = ref.copy()
    got[3, [2, 7]] = got[3, [7, 2]]          # two slots swapped (order broken)
    _expect_fail(compare_topk, got, ref)
    got = ref.copy()
    sel = set(got[5].tolist())
    other = next(i for i in range(N) if i not in sel)
    got[5, 4] = other                        # one index replaced by an unselected key
    _expect_fail(compare_topk, got, ref)
    got = ref.copy()
    got[0, -1] = -1                          # a selected key dropped
    _expect_fail(compare_topk, got, ref)
    # a tie resolved to the higher index
    row = 9
    v = lg[row]
    tau = np.sort(v)[::-1][K - 1]
    sel_eq = [i for i in ref[row] if v[i] == tau]
    uns_eq = [i for i in range(N) if v[i] == tau and i not in set(ref[row].tolist())]
    if sel_eq and uns_eq:
        got = ref.copy()
        got[row] = np.sort(np.where(got[row] == max(sel_eq), uns_eq[0], got[row]))
        _expect_fail(compare_topk, got, ref)


def test_check_logits_catches_value_and_window_mistakes():
    wl = W.WORKLOADS["tiny_causal_256"].with_(M=40, N=40)
    x = W.make_inputs(wl, parts=("indexer",))
    ref, terms = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                       x["ks"], x["ke"], with_terms=True)
    gpu = ref.astype(np.float64).copy()      # NaN outside windows = untouched
    check_logits(gpu, ref, terms)
    win = np.argwhere(~np.isnan(ref) & (terms > 0))
    r, c = win[len(win) // 2]
    g = gpu.copy()
    g[r, c] += 2e-4 * terms[r, c]            # twice the tolerance
    _expect_fail(check_logits, g, ref, terms)
    g = gpu.copy()
    g[r, c] -= 2e-4 * terms[r, c]
    _expect_fail(check_logits, g, ref, terms)
    g = gpu.copy()
    g[0, 5] = 0.0                            # row 0's window is [0, 1): written outside it
    _expect_fail(check_logits, g, ref, terms)
    g = gpu.copy()
    g[r, c] = np.nan                         # a window logit left unwritten
    _expect_fail(check_logits, g, ref, terms)


def test_check_attn_catches_output_mistakes():
    wl = W.WORKLOADS["tiny_causal_256"].with_(M=12, N=12, K=8)
    x = W.make_inputs(wl, parts=("attn",))
    idx = W.synthetic_topk(wl, x["ks"], x["ke"])
    ref = oracle.sparse_attn(x["q"], x["kv"], x["sink"], idx, wl.sm_scale, wl.Dv)
    check_attn(torch.from_numpy(ref.copy()), ref)
    g = ref.copy()
    g[3, 2, 7] += 0.03                       # one element moved by 0.03
    _expect_fail(check_attn, torch.from_numpy(g), ref)
    g = ref + 0.0025                         # a small bias everywhere (mean bound)
    _expect_fail(check_attn, torch.from_numpy(g), ref)
    g = ref.copy()
    g[0, 0, 0] = np.nan
    _expect_fail(check_attn, torch.from_numpy(g), ref)
