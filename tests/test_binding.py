"""CPU checks of the Python binding's argument validation: every shape, dtype
and device mismatch raises before the C call, which sees pointers only and
could otherwise read or write out of bounds.  No GPU needed: shapes are
checked before devices, so CPU tensors of the right shapes reach the device
check (TypeError) and mismatched ones stop at the shape check (ValueError)."""
import pytest
import torch

import fp8_indexer_amd as dsa

B, M, N, H, D, K, HQ, DQK, DV = 2, 5, 40, 4, 64, 8, 16, 64, 64


def _indexer():
    return dict(q=torch.zeros((B, M, H, D), dtype=torch.uint8),
                q_scale=torch.ones((B, M, H)), k=torch.zeros((B, N, D), dtype=torch.uint8),
                k_scale=torch.ones((B, N)), weights=torch.ones((B, M, H)),
                ks=torch.zeros((B, M), dtype=torch.int32), ke=torch.ones((B, M), dtype=torch.int32))


def _attn():
    return dict(q=torch.zeros((B, M, HQ, DQK), dtype=torch.bfloat16),
                kv=torch.zeros((B, N, DQK), dtype=torch.bfloat16),
                attn_sink=torch.zeros((HQ,)),
                topk_idxs=torch.zeros((B, M, K), dtype=torch.int32))


def test_indexer_shapes_checked():
    a = _indexer()
    with pytest.raises(TypeError, match="CUDA"):
        dsa.indexer_logits(**a)
    bad = {"q_scale": (B, M, H + 1), "k": (B, N, D + 1), "k_scale": (B, N + 1),
           "weights": (B, M - 1, H), "ks": (B, M + 1), "ke": (B + 1, M)}
    for name, shape in bad.items():
        x = dict(a)
        x[name] = torch.zeros(shape, dtype=a[name].dtype)
        with pytest.raises(ValueError, match=name):
            dsa.indexer_logits(**x)
    with pytest.raises(ValueError, match="logits"):
        dsa.indexer_logits(**a, logits=torch.zeros((B, M, N - 1)))
    x = dict(a)
    x["weights"] = torch.ones((B, M, H), dtype=torch.float64)
    with pytest.raises(TypeError, match="weights"):
        dsa.indexer_logits(**x)
    x = dict(a)
    x["q"] = torch.zeros((B, M, D, H), dtype=torch.uint8).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        dsa.indexer_logits(**x)


def test_topk_shapes_checked():
    lg = torch.zeros((B, M, N))
    ks = torch.zeros((B, M), dtype=torch.int32)
    ke = torch.ones((B, M), dtype=torch.int32)
    with pytest.raises(TypeError, match="CUDA"):
        dsa.topk(lg, ks, ke, K)
    with pytest.raises(ValueError, match="ks"):
        dsa.topk(lg, torch.zeros((B, M + 1), dtype=torch.int32), ke, K)
    with pytest.raises(ValueError, match="out"):
        dsa.topk(lg, ks, ke, K, out=torch.zeros((B, M, K + 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="logits"):
        dsa.topk(torch.zeros((B * M, N)), ks, ke, K)


def test_attention_shapes_checked():
    a = _attn()
    with pytest.raises(TypeError, match="CUDA"):
        dsa.sparse_attn_fwd(**a, dv=DV)
    bad = {"kv": (B, N, DQK + 8), "attn_sink": (HQ + 1,), "topk_idxs": (B, M + 1, K)}
    for name, shape in bad.items():
        x = dict(a)
        x[name] = torch.zeros(shape, dtype=a[name].dtype)
        with pytest.raises(ValueError, match=name):
            dsa.sparse_attn_fwd(**x, dv=DV)
    with pytest.raises(ValueError, match="out"):
        dsa.sparse_attn_fwd(**a, dv=DV, out=torch.zeros((B, M, HQ, DV - 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="kv_scale"):
        x = dict(a)
        x["kv"] = torch.zeros((B, N, DQK), dtype=torch.uint8)
        dsa.sparse_attn_fwd(**x, dv=DV, kv_scale=torch.ones((B, N + 1)))
    with pytest.raises(TypeError, match="kv"):  # fp8 kv without its scale
        x = dict(a)
        x["kv"] = torch.zeros((B, N, DQK), dtype=torch.uint8)
        dsa.sparse_attn_fwd(**x, dv=DV)


def test_prefill_shapes_checked():
    i, a = _indexer(), _attn()
    args = (i["q"], i["q_scale"], i["k"], i["k_scale"], i["weights"], i["ks"], i["ke"], K, a["q"],
            a["kv"], a["attn_sink"])
    with pytest.raises(TypeError, match="CUDA"):
        dsa.prefill(*args, dv=DV)
    with pytest.raises(ValueError, match="topk_idxs"):
        dsa.prefill(*args, dv=DV, topk_idxs=torch.zeros((B, M, K - 1), dtype=torch.int32))
    bad_q = torch.zeros((B, M + 1, HQ, DQK), dtype=torch.bfloat16)  # attention rows != indexer rows
    with pytest.raises(ValueError, match="q"):
        dsa.prefill(*args[:8], bad_q, *args[9:], dv=DV)
    bad_kv = torch.zeros((B, N + 3, DQK), dtype=torch.bfloat16)  # kv keys != indexer keys
    with pytest.raises(ValueError, match="kv"):
        dsa.prefill(*args[:9], bad_kv, args[10], dv=DV)
