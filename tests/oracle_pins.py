"""Pins of the CPU oracle to things other than itself.

Each check_* function raises AssertionError when the oracle disagrees with an
independent fact: the format definitions as implemented by torch, hand-worked
fixtures (tests/golden/), exact rational arithmetic, a full sort, the dense
textbook softmax, closed forms and invariants.  The same checks run against
deliberately broken copies of the oracle in test_oracle_mutants.py, which
proves that each plausible mistake is caught by at least one of them.
"""
import contextlib
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@contextlib.contextmanager
def oracle_lib(path):
    """Temporarily route the oracle wrappers to another build of the library."""
    saved = oracle._lib
    oracle._lib = oracle.lib(path)
    try:
        yield
    finally:
        oracle._lib = saved


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _code(c):
    return int(c, 16) if isinstance(c, str) else int(c)


def _val(v):
    if isinstance(v, str):
        return float(v)  # "nan", "-inf", "-0.0"
    return float(v)


def _torch_e4m3(codes):
    t = torch.as_tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def _torch_bf16(bits):
    t = torch.as_tensor(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).numpy().astype(np.float64)


def _rand_e4m3(rng, shape, allow_sub=True):
    """Random finite e4m3fn codes (every finite code, incl. subnormals)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E  # replace NaN codes
    if not allow_sub:
        c[(c & 0x78) == 0] |= 0x08
    return c


# ---------------------------------------------------------------- formats --

def check_e4m3_decode():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3(codes)
    got = np.array([oracle.e4m3fn_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN codes differ"
    assert np.array_equal(got[~nan], ref[~nan]), "e4m3fn decode differs from torch"
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert oracle.e4m3fn_value(0x7E) == 448.0
    assert oracle.e4m3fn_value(0x01) == 2.0 ** -9
    assert oracle.e4m3fn_value(0x08) == 2.0 ** -6
    assert oracle.e4m3fn_value(0x80) == 0.0 and math.copysign(1, oracle.e4m3fn_value(0x80)) < 0


def check_bf16_decode():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _torch_bf16(bits)
    got = np.array([oracle.bf16_value(int(b)) for b in bits[::97]])
    r = ref[::97]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan]), "bf16 decode differs from torch"


# ---------------------------------------------------------------- indexer --

def check_indexer_hand():
    for case in _load("indexer_hand.json")["cases"]:
        B, M, N, H, D = (case[x] for x in "BMNHD")
        q = np.vectorize(_code)(np.array(case["q_codes"], dtype=object)).astype(np.uint8)
        k = np.vectorize(_code)(np.array(case["k_codes"], dtype=object)).astype(np.uint8)
        got = oracle.indexer_logits(q.reshape(B, M, H, D), np.float32(case["q_scale"]),
                                    k.reshape(B, N, D), np.float32(case["k_scale"]),
                                    np.float32(case["w"]), np.int32(case["ks"]),
                                    np.int32(case["ke"]))
        exp = np.array([[np.nan if v is None else v for v in row]
                        for bb in case["logits"] for row in bb], np.float64)
        assert got.shape == exp.shape
        for a, b in zip(got.ravel(), exp.ravel()):
            if math.isnan(b):
                assert math.isnan(a), case["name"]
            else:
                assert a == b, (case["name"], a, b)


def _exact_logit(qv, qs, kv, ks_, w, t_row, key, H, D):
    """Exact rational score for one (row, key) from torch-decoded values."""
    acc = Fraction(0)
    for h in range(H):
        dot = sum(Fraction(float(qv[t_row, h, d])) * Fraction(float(kv[key, d]))
                  for d in range(D))
        if dot > 0:
            acc += dot * Fraction(float(w[t_row, h])) * Fraction(float(qs[t_row, h]))
    return acc * Fraction(float(ks_[key]))


def check_indexer_exact(seed=7):
    rng = np.random.default_rng(seed)
    B, M, N, H, D = 2, 4, 6, 3, 5
    q = _rand_e4m3(rng, (B, M, H, D))
    k = _rand_e4m3(rng, (B, N, D))
    qs = rng.uniform(0.25, 2.0, (B, M, H)).astype(np.float32)
    ksc = rng.uniform(0.25, 2.0, (B, N)).astype(np.float32)
    w = rng.standard_normal((B, M, H)).astype(np.float32)
    ks = rng.integers(-2, N, (B, M)).astype(np.int32)
    ke = rng.integers(0, N + 3, (B, M)).astype(np.int32)
    got = oracle.indexer_logits(q, qs, k, ksc, w, ks, ke)
    qv = _torch_e4m3(q.ravel()).reshape(q.shape)
    kv = _torch_e4m3(k.ravel()).reshape(k.shape)
    for b in range(B):
        for t in range(M):
            r = b * M + t
            s = min(max(int(ks[b, t]), 0), N)
            e = min(max(int(ke[b, t]), s), N)
            for key in range(N):
                g = got[r, key]
                if not (s <= key < e):
                    assert math.isnan(g), ("outside window must be NaN", b, t, key)
                    continue
                ex = _exact_logit(qv[b], qs[b], kv[b], ksc[b], w[b], t, key, H, D)
                ref = np.float32(float(ex))
                # correctly rounded exact value, or its neighbour (double rounding)
                assert abs(float(g) - float(ref)) <= float(np.spacing(np.abs(ref))) + 1e-45, \
                    (b, t, key, g, float(ex))


def _rand_indexer(rng, B=1, M=5, N=9, H=4, D=16):
    q = _rand_e4m3(rng, (B, M, H, D))
    k = _rand_e4m3(rng, (B, N, D))
    qs = np.float32(2.0) ** rng.integers(-3, 3, (B, M, H)).astype(np.float32)
    ksc = rng.uniform(0.5, 2.0, (B, N)).astype(np.float32)
    w = rng.standard_normal((B, M, H)).astype(np.float32)
    ks = np.zeros((B, M), np.int32)
    ke = np.full((B, M), N, np.int32)
    return q, qs, k, ksc, w, ks, ke


def check_indexer_invariants(seed=11):
    rng = np.random.default_rng(seed)
    q, qs, k, ksc, w, ks, ke = _rand_indexer(rng)
    base = oracle.indexer_logits(q, qs, k, ksc, w, ks, ke)
    # negating the head weights negates every logit exactly
    neg = oracle.indexer_logits(q, qs, k, ksc, -w, ks, ke)
    assert np.array_equal(neg, -base), "w -> -w must negate logits"
    # a power-of-two q_scale folded into w gives identical logits
    fold = oracle.indexer_logits(q, None, k, ksc, (w * qs).astype(np.float32), ks, ke)
    assert np.array_equal(fold, base), "q_scale folding"
    # permuting keys permutes the logits
    perm = rng.permutation(k.shape[1])
    pk = oracle.indexer_logits(q, qs, k[:, perm], ksc[:, perm], w, ks, ke)
    assert np.array_equal(pk, base[:, perm]), "key permutation equivariance"
    # linear in k_scale
    dbl = oracle.indexer_logits(q, qs, k, ksc * 2, w, ks, ke)
    assert np.array_equal(dbl, base * 2), "linear in k_scale"
    # relu: a head whose every dot is negative contributes nothing
    q2 = q.copy()
    q2[..., 0, :] = k[0, 0, :] ^ 0x80  # head 0 = -key0 -> dot with key 0 < 0
    a = oracle.indexer_logits(q2, qs, k, ksc, w, ks, ke)
    w2 = w.copy()
    w2[..., 0] = 0
    b_ = oracle.indexer_logits(q2, qs, k, ksc, w2, ks, ke)
    nz = np.any(k[0, 0] & 0x7F)
    if nz:
        assert np.array_equal(a[:, 0], b_[:, 0]), "relu must drop negative dots"
    # row subset equals the same rows of the full computation
    rows = np.array([3, 0], np.int64)
    sub = oracle.indexer_logits(q, qs, k, ksc, w, ks, ke, rows=rows)
    assert np.array_equal(sub, base[rows])


def check_indexer_terms(seed=5):
    rng = np.random.default_rng(seed)
    q, qs, k, ksc, w, ks, ke = _rand_indexer(rng, M=3, N=4, H=2, D=3)
    lg, terms = oracle.indexer_logits(q, qs, k, ksc, w, ks, ke, with_terms=True)
    qv = _torch_e4m3(q.ravel()).reshape(q.shape)
    kv = _torch_e4m3(k.ravel()).reshape(k.shape)
    for t in range(3):
        for key in range(4):
            tt = sum(abs(float(w[0, t, h]) * float(qs[0, t, h])) *
                     sum(abs(qv[0, t, h, d] * kv[0, key, d]) for d in range(3))
                     for h in range(2)) * abs(float(ksc[0, key]))
            assert math.isclose(terms[t, key], tt, rel_tol=1e-12)
            assert abs(lg[t, key]) <= terms[t, key] * (1 + 1e-6)


# ------------------------------------------------------------------- top-k --

def _topk_ref(row, s, e, K):
    """Full stable sort by (value desc, index asc); independent of the oracle."""
    vals = []
    for i in range(s, e):
        v = float(row[i])
        if math.isnan(v):
            v = -math.inf
        vals.append((v, i))
    if e - s <= K:
        sel = list(range(s, e))
    else:
        sel = [i for _, i in sorted(vals, key=lambda p: (-p[0], p[1]))[:K]]
    sel = sorted(sel)
    return sel + [-1] * (K - len(sel))


def check_topk_hand():
    for case in _load("topk_hand.json")["cases"]:
        row = np.array([_val(v) for v in case["row"]], np.float32)
        N = row.size
        got = oracle.topk(row.reshape(1, N), np.int32([case["ks"]]), np.int32([case["ke"]]),
                          1, 1, N, case["K"])
        assert got[0].tolist() == case["expect"], (case, got[0].tolist())


def check_topk_bruteforce(seed=3):
    rng = np.random.default_rng(seed)
    for trial in range(60):
        N = int(rng.integers(1, 40))
        M = int(rng.integers(1, 5))
        K = int(rng.integers(1, 12))
        kind = trial % 4
        if kind == 0:    # tie-heavy small integers
            lg = rng.integers(-3, 4, (M, N)).astype(np.float32)
        elif kind == 1:  # many signed zeros and infinities
            lg = rng.choice(np.float32([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan]),
                            (M, N)).astype(np.float32)
        elif kind == 2:
            lg = rng.standard_normal((M, N)).astype(np.float32)
        else:            # tiny magnitudes and denormals
            lg = (rng.standard_normal((M, N)) * 1e-40).astype(np.float32)
        ks = rng.integers(-3, N + 2, M).astype(np.int32)
        ke = rng.integers(-1, N + 4, M).astype(np.int32)
        got = oracle.topk(lg, ks, ke, 1, M, N, K)
        for t in range(M):
            s = min(max(int(ks[t]), 0), N)
            e = min(max(int(ke[t]), s), N)
            assert got[t].tolist() == _topk_ref(lg[t], s, e, K), (trial, t)


def check_topk_invariants(seed=4):
    rng = np.random.default_rng(seed)
    N, M, K = 300, 6, 37
    lg = rng.integers(-20, 20, (M, N)).astype(np.float32)
    ks = np.int32([0, 5, 100, 0, 250, 290])
    ke = np.int32([300, 41, 137, 37, 300, 300])
    got = oracle.topk(lg, ks, ke, 1, M, N, K)
    for t in range(M):
        s, e = int(ks[t]), int(ke[t])
        sel = [i for i in got[t] if i >= 0]
        assert len(sel) == min(K, e - s)
        assert sel == sorted(sel) and len(set(sel)) == len(sel)
        assert all(s <= i < e for i in sel)
        uns = [i for i in range(s, e) if i not in set(sel)]
        if uns:
            mn = min(lg[t, i] for i in sel)
            mx = max(lg[t, i] for i in uns)
            assert mn >= mx
            # at the threshold value, selected indices precede unselected ones
            thr_sel = [i for i in sel if lg[t, i] == mn]
            thr_uns = [i for i in uns if lg[t, i] == mn]
            if thr_uns:
                assert max(thr_sel) < min(thr_uns)
    # all-equal row: first K of the window
    eq = np.ones((1, 50), np.float32)
    assert oracle.topk(eq, np.int32([7]), np.int32([50]), 1, 1, 50, 5)[0].tolist() == \
        [7, 8, 9, 10, 11]


# -------------------------------------------------------------- attention --

def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def _attn_dense(qv, kvv, sink, idx, sm_scale, dv, vals=None):
    """Textbook softmax over ALL N keys plus one sink column with a zero value
    row; keys not in idx are masked with weight 0 (idx without duplicates).
    vals: the value rows (default: the first dv columns of kvv)."""
    B, M, Hq, Dqk = qv.shape
    N = kvv.shape[1]
    out = np.zeros((B * M, Hq, dv))
    for b in range(B):
        for t in range(M):
            mask = np.zeros(N, bool)
            for j in idx[b, t]:
                if 0 <= j < N:
                    mask[j] = True
            if not mask.any():
                continue
            for h in range(Hq):
                s = sm_scale * (kvv[b] @ qv[b, t, h])            # [N]
                cols = np.concatenate([s, [sink[h] if sink is not None else -np.inf]])
                wts = np.concatenate([mask.astype(np.float64), [1.0]])
                mx = cols[wts > 0].max()
                ex = wts * np.exp(cols - mx)
                p = ex / ex.sum()
                vb = (kvv if vals is None else vals)[b][:, :dv]
                vrows = np.concatenate([vb, np.zeros((1, dv))])  # sink value row 0
                out[b * M + t, h] = p @ vrows
    return out


def _rand_attn(rng, B=2, M=3, N=11, Hq=4, Dqk=8, K=6, dup=False):
    qv = rng.standard_normal((B, M, Hq, Dqk)).astype(np.float32)
    kvv = rng.standard_normal((B, N, Dqk)).astype(np.float32)
    qb, kvb = _bf16_bits(qv), _bf16_bits(kvv)
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            n = int(rng.integers(0, K + 1))
            if dup:
                idx[b, t, :n] = rng.integers(0, N, n)
            else:
                idx[b, t, :n] = rng.choice(N, size=min(n, N), replace=False)
            rng.shuffle(idx[b, t])
    sink = rng.standard_normal(Hq).astype(np.float32)
    return qb, kvb, idx, sink


def check_attn_hand():
    for case in _load("attn_hand.json")["cases"]:
        q = np.float32(case["q"]).reshape(1, 1, 1, -1)
        kv = np.float32(case["kv"]).reshape(1, len(case["kv"]), -1)
        idx = np.int32(case["idx"]).reshape(1, 1, -1)
        sink = None if case["sink"] is None else np.float32([case["sink"]])
        got = oracle.sparse_attn(_bf16_bits(q), _bf16_bits(kv), sink, idx,
                                 case["sm_scale"], case["Dv"])
        assert np.allclose(got.ravel(), case["o"], rtol=1e-14, atol=1e-14), \
            (case["name"], got.ravel())


def check_attn_dense(seed=21):
    rng = np.random.default_rng(seed)
    qb, kvb, idx, sink = _rand_attn(rng)
    qv = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
    kvv = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
    for dv in (8, 5):
        for sk in (sink, None):
            got = oracle.sparse_attn(qb, kvb, sk, idx, 0.35, dv)
            ref = _attn_dense(qv, kvv, sk, idx, 0.35, dv)
            assert np.allclose(got, ref, rtol=1e-11, atol=1e-13), np.abs(got - ref).max()


def check_attn_closed_forms(seed=22):
    rng = np.random.default_rng(seed)
    qb, kvb, idx, sink = _rand_attn(rng, B=1, M=1, N=5, Hq=3, Dqk=6, K=4)
    qv = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
    kvv = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
    # one valid index: o = v * logistic(s - sink)
    one = np.int32([[[-1, 3, -1, -1]]])
    got = oracle.sparse_attn(qb, kvb, sink, one, 0.5, 6)
    for h in range(3):
        s = 0.5 * float(qv[0, 0, h] @ kvv[0, 3])
        sig = 1.0 / (1.0 + math.exp(-(s - float(sink[h]))))
        assert np.allclose(got[0, h], kvv[0, 3] * sig, rtol=1e-12, atol=1e-14)
    # no sink at all: one index gives exactly its row
    got = oracle.sparse_attn(qb, kvb, None, one, 0.5, 6)
    assert np.allclose(got[0], np.broadcast_to(kvv[0, 3], (3, 6)), rtol=1e-14)
    # sink = -inf equals no sink
    full = np.int32([[[0, 1, 2, 4]]])
    a = oracle.sparse_attn(qb, kvb, np.full(3, -np.inf, np.float32), full, 0.5, 6)
    b = oracle.sparse_attn(qb, kvb, None, full, 0.5, 6)
    assert np.array_equal(a, b)
    # all -1 gives zero, with or without a sink
    none = np.full((1, 1, 4), -1, np.int32)
    assert not oracle.sparse_attn(qb, kvb, sink, none, 0.5, 6).any()
    assert not oracle.sparse_attn(qb, kvb, None, none, 0.5, 6).any()
    # a duplicated index counts twice: same as one copy with score + ln 2
    dup = np.int32([[[2, 2, -1, -1]]])
    got = oracle.sparse_attn(qb, kvb, sink, dup, 0.5, 6)
    for h in range(3):
        s = 0.5 * float(qv[0, 0, h] @ kvv[0, 2]) + math.log(2.0)
        sig = 1.0 / (1.0 + math.exp(-(s - float(sink[h]))))
        assert np.allclose(got[0, h], kvv[0, 2] * sig, rtol=1e-12, atol=1e-14)


def check_attn_invariants(seed=23):
    rng = np.random.default_rng(seed)
    qb, kvb, idx, sink = _rand_attn(rng, dup=True)
    base = oracle.sparse_attn(qb, kvb, sink, idx, 0.3, 8)
    perm = rng.permutation(idx.shape[-1])
    assert np.allclose(oracle.sparse_attn(qb, kvb, sink, idx[..., perm], 0.3, 8), base,
                       rtol=1e-13, atol=1e-15)
    pad = np.concatenate([idx, np.full(idx.shape[:-1] + (5,), -1, np.int32)], -1)
    assert np.allclose(oracle.sparse_attn(qb, kvb, sink, pad, 0.3, 8), base,
                       rtol=1e-13, atol=1e-15)
    bad = idx.copy()
    bad[bad < 0] = np.int32(kvb.shape[1] + 100)  # out of range -> skipped like -1
    assert np.array_equal(oracle.sparse_attn(qb, kvb, sink, bad, 0.3, 8), base)
    rows = np.int64([4, 1])
    assert np.array_equal(oracle.sparse_attn(qb, kvb, sink, idx, 0.3, 8, rows=rows),
                          base[rows])


def check_attn_fp8_kv(seed=24):
    """fp8 KV: the value is decode(code) * row scale, as the dense formula
    computed from torch-decoded codes."""
    rng = np.random.default_rng(seed)
    B, M, N, Hq, Dqk, K = 1, 2, 7, 2, 8, 5
    qv = rng.standard_normal((B, M, Hq, Dqk)).astype(np.float32)
    qb = _bf16_bits(qv)
    kv8 = _rand_e4m3(rng, (B, N, Dqk))
    scale = rng.uniform(0.01, 0.1, (B, N)).astype(np.float32)
    idx = np.int32(rng.choice(N, size=(B, M, K)))
    idx[0, 1, :] = rng.permutation(N)[:K]
    idx[0, 0, :] = rng.permutation(N)[:K]
    sink = rng.standard_normal(Hq).astype(np.float32)
    got = oracle.sparse_attn(qb, kv8, sink, idx, 0.4, 6, kv_scale=scale)
    kvv = _torch_e4m3(kv8.ravel()).reshape(kv8.shape) * scale[..., None].astype(np.float64)
    qd = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
    ref = _attn_dense(qd, kvv, sink, idx, 0.4, 6)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)


def check_attn_fp8_q(seed=25):
    """fp8 query (the full-FP8 attention's input): the query value is
    decode(code) * q_scale[b,t,h].  With power-of-two scales those values are
    exact in bf16, so the result must equal the bf16-query path fed with
    them; with any scale it must equal the dense formula on torch-decoded
    values; a scale common to every (t, h) is the same as folding it into
    sm_scale."""
    rng = np.random.default_rng(seed)
    B, M, N, Hq, Dqk, K = 1, 3, 9, 3, 8, 5
    q8 = _rand_e4m3(rng, (B, M, Hq, Dqk))
    qs = np.float32(2.0) ** rng.integers(-3, 4, (B, M, Hq)).astype(np.float32)
    kvv = rng.standard_normal((B, N, Dqk)).astype(np.float32)
    kvb = _bf16_bits(kvv)
    idx = np.int32(np.stack([rng.permutation(N)[:K] for _ in range(B * M)]).reshape(B, M, K))
    idx[0, 1, 2:] = -1
    idx[0, 2, :] = -1
    sink = rng.standard_normal(Hq).astype(np.float32)
    got = oracle.sparse_attn(q8, kvb, sink, idx, 0.4, 6, q_scale=qs)
    qd = _torch_e4m3(q8.ravel()).reshape(q8.shape) * qs[..., None].astype(np.float64)
    same = oracle.sparse_attn(_bf16_bits(qd.astype(np.float32)), kvb, sink, idx, 0.4, 6)
    assert np.allclose(got, same, rtol=1e-14, atol=1e-16)
    kd = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
    ref = _attn_dense(qd, kd, sink, idx, 0.4, 6)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)
    assert not got[2].any()
    # no scale = scale 1; a common non-power-of-two scale folds into sm_scale
    one = oracle.sparse_attn(q8, kvb, sink, idx, 0.4, 6)
    assert np.array_equal(one, oracle.sparse_attn(q8, kvb, sink, idx, 0.4, 6,
                                                  q_scale=np.ones((B, M, Hq), np.float32)))
    a = np.float32(0.37)
    sc = oracle.sparse_attn(q8, kvb, sink, idx, 0.4, 6, q_scale=np.full((B, M, Hq), a))
    assert np.allclose(sc, oracle.sparse_attn(q8, kvb, sink, idx, 0.4 * float(a), 6),
                       rtol=1e-12, atol=1e-15)
    # fp8 query and fp8 KV together
    kv8 = _rand_e4m3(rng, (B, N, Dqk))
    ks = rng.uniform(0.01, 0.1, (B, N)).astype(np.float32)
    got = oracle.sparse_attn(q8, kv8, sink, idx, 0.4, 6, kv_scale=ks, q_scale=qs)
    kvd = _torch_e4m3(kv8.ravel()).reshape(kv8.shape) * ks[..., None].astype(np.float64)
    ref = _attn_dense(qd, kvd, sink, idx, 0.4, 6)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)


def check_attn_terms(seed=26):
    """The per-element term sums sum_j p_j |v_jc| that bound the GPU path's
    rounding: the dense formula on |v|, equal to o when every value is >= 0,
    never below |o|, zero for rows without a valid index."""
    rng = np.random.default_rng(seed)
    qb, kvb, idx, sink = _rand_attn(rng, dup=True)
    o, t = oracle.sparse_attn(qb, kvb, sink, idx, 0.3, 8, with_terms=True)
    assert np.array_equal(o, oracle.sparse_attn(qb, kvb, sink, idx, 0.3, 8))
    assert (t >= np.abs(o) * (1 - 1e-12)).all()
    qd = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
    kd = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
    nodup = _rand_attn(np.random.default_rng(seed + 1))[2]
    _, t2 = oracle.sparse_attn(qb, kvb, sink, nodup, 0.3, 7, with_terms=True)
    assert np.allclose(t2, _attn_dense(qd, kd, sink, nodup, 0.3, 7, vals=np.abs(kd)),
                       rtol=1e-11, atol=1e-13)
    kpos = _bf16_bits(np.abs(kd).astype(np.float32))
    o3, t3 = oracle.sparse_attn(qb, kpos, sink, idx, 0.3, 8, with_terms=True)
    assert np.allclose(o3, t3, rtol=1e-13, atol=1e-15)
    empty = ~(idx >= 0).any(-1).reshape(-1)
    assert empty.any() and not t[empty].any()


# ------------------------------------------------ row subsets (rows=...) --

def check_rows_subsets(seed=31):
    """The `rows=` path of each stage (the GPU tests compare sampled rows of
    full-size workloads through it): every listed row, in the listed order,
    must equal the independent reference for that row -- the brute-force sort
    for top-k, exact rational scores for the indexer, the dense softmax for
    attention -- with rows whose windows and index lists all differ, so a
    wrong row mapping cannot pass."""
    rng = np.random.default_rng(seed)
    # top-k: distinct windows per row, rows listed out of order
    M, N, K = 9, 60, 7
    lg = rng.integers(-4, 5, (M, N)).astype(np.float32)
    ks = np.int32([0, 3, 10, 20, 1, 33, 40, 0, 50])
    ke = np.int32([60, 30, 18, 59, 9, 60, 47, 5, 58])
    rows = np.int64([7, 2, 5, 0, 8])
    got = oracle.topk(lg[rows], ks, ke, 1, M, N, K, rows=rows)
    for i, r in enumerate(rows):
        s, e = int(ks[r]), int(ke[r])
        assert got[i].tolist() == _topk_ref(lg[r], s, e, K), ("topk rows", r)
    # indexer: B = 2 so that rows of the second batch entry use its own keys
    B, M2, N2, H, D = 2, 3, 7, 2, 4
    q, qs, k, ksc, w, _, _ = _rand_indexer(rng, B=B, M=M2, N=N2, H=H, D=D)
    ks2 = np.int32([[0, 2, 1], [3, 0, 5]])
    ke2 = np.int32([[7, 5, 3], [7, 4, 7]])
    rows2 = np.int64([4, 1, 5])
    lg2 = oracle.indexer_logits(q, qs, k, ksc, w, ks2, ke2, rows=rows2)
    qv = _torch_e4m3(q.ravel()).reshape(q.shape)
    kv = _torch_e4m3(k.ravel()).reshape(k.shape)
    for i, r in enumerate(rows2):
        b, t = divmod(int(r), M2)
        for key in range(N2):
            inside = ks2[b, t] <= key < ke2[b, t]
            assert np.isnan(lg2[i, key]) == (not inside), ("indexer window", r, key)
            if inside:
                acc = Fraction(0)
                for h in range(H):
                    dot = sum(Fraction(qv[b, t, h, d]) * Fraction(kv[b, key, d])
                              for d in range(D))
                    if dot > 0:
                        acc += dot * Fraction(float(w[b, t, h])) * Fraction(float(qs[b, t, h]))
                want = np.float32(float(acc * Fraction(float(ksc[b, key]))))
                assert lg2[i, key] == want, ("indexer rows", r, key)
    # attention: every row its own index list
    qb, kvb, idx, sink = _rand_attn(rng, B=2, M=3, N=11, Hq=4, Dqk=8, K=6)
    rows3 = np.int64([5, 0, 3])
    got3 = oracle.sparse_attn(qb, kvb, sink, idx, 0.3, 8, rows=rows3)
    qv3 = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
    kvv3 = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
    dense = _attn_dense(qv3, kvv3, sink, idx, 0.3, 8)
    assert np.allclose(got3, dense[rows3], rtol=1e-12, atol=1e-12), "attention rows"


# -------------------------------------------------------------- backward --

def _attn_multiset(qv, kvv, sink, idx, sm_scale, dv):
    """Forward of the sparse attention in numpy fp64, looping over index
    occurrences (a duplicated index counts each time), for finite differences
    of the backward; independent of the oracle's C code."""
    B, M, Hq, Dqk = qv.shape
    N = kvv.shape[1]
    out = np.zeros((B * M, Hq, dv))
    for b in range(B):
        for t in range(M):
            J = [int(j) for j in idx[b, t] if 0 <= j < N]
            if not J:
                continue
            for h in range(Hq):
                s = np.array([sm_scale * float(qv[b, t, h] @ kvv[b, j]) for j in J])
                mx = max(s.max(), sink[h] if sink is not None else -np.inf)
                e = np.exp(s - mx)
                den = e.sum() + (np.exp(sink[h] - mx) if sink is not None else 0.0)
                out[b * M + t, h] = sum(e[k] * kvv[b, J[k], :dv] for k in range(len(J))) / den
    return out


def check_attn_bwd_finite_differences(seed=41):
    """Oracle gradients of L = sum(dO * o) against central differences of the
    numpy forward, for every element of q, kv and the sink, with duplicated
    and -1 indices, with and without a sink."""
    rng = np.random.default_rng(seed)
    B, M, N, Hq, Dqk, Dv, K = 1, 3, 6, 2, 5, 4, 5
    for with_sink in (True, False):
        qb = _bf16_bits(rng.standard_normal((B, M, Hq, Dqk)))
        kvb = _bf16_bits(rng.standard_normal((B, N, Dqk)))
        gb = _bf16_bits(rng.standard_normal((B, M, Hq, Dv)))
        sink = rng.standard_normal(Hq).astype(np.float32) if with_sink else None
        idx = np.array([[[0, 3, 3, -1, 5], [2, -1, -1, 4, 1], [-1, -1, -1, -1, -1]]], np.int32)
        qv = _torch_bf16(qb.view(np.uint16).ravel()).reshape(qb.shape)
        kvv = _torch_bf16(kvb.view(np.uint16).ravel()).reshape(kvb.shape)
        gv = _torch_bf16(gb.view(np.uint16).ravel()).reshape(gb.shape)
        sc = 0.4
        dq, dkv, dsink = oracle.sparse_attn_bwd(qb, kvb, sink, idx, gb, sc, Dv)
        sk64 = None if sink is None else sink.astype(np.float64)

        def loss(qx, kx, sx):
            return float((_attn_multiset(qx, kx, sx, idx, sc, Dv) *
                          gv.reshape(B * M, Hq, Dv)).sum())

        eps = 1e-6
        for arr, grad, name in ((qv, dq.reshape(qv.shape), "q"), (kvv, dkv, "kv")):
            for pos in np.ndindex(arr.shape):
                a1, a2 = arr.copy(), arr.copy()
                a1[pos] += eps
                a2[pos] -= eps
                args1 = (a1, kvv, sk64) if name == "q" else (qv, a1, sk64)
                args2 = (a2, kvv, sk64) if name == "q" else (qv, a2, sk64)
                fd = (loss(*args1) - loss(*args2)) / (2 * eps)
                assert abs(fd - grad[pos]) <= 1e-6 * (1 + abs(fd)), (name, pos, fd, grad[pos])
        if sink is not None:
            for h in range(Hq):
                s1, s2 = sk64.copy(), sk64.copy()
                s1[h] += eps
                s2[h] -= eps
                fd = (loss(qv, kvv, s1) - loss(qv, kvv, s2)) / (2 * eps)
                assert abs(fd - dsink[h]) <= 1e-6 * (1 + abs(fd)), ("sink", h, fd, dsink[h])
        else:
            assert dsink is None


def check_attn_bwd_closed_forms(seed=42):
    """One valid index and no sink: p = 1, so dS = 0 (dq = 0) and the row's
    dkv is dO on the first Dv columns, 0 beyond; a row without a valid index
    contributes nothing; -1 padding changes nothing; rows= lists the
    contributions of the listed rows only."""
    rng = np.random.default_rng(seed)
    B, M, N, Hq, Dqk, Dv, K = 1, 2, 5, 3, 6, 4, 4
    qb = _bf16_bits(rng.standard_normal((B, M, Hq, Dqk)))
    kvb = _bf16_bits(rng.standard_normal((B, N, Dqk)))
    gb = _bf16_bits(rng.standard_normal((B, M, Hq, Dv)))
    gv = _torch_bf16(gb.view(np.uint16).ravel()).reshape(gb.shape)
    idx = np.array([[[2, -1, -1, -1], [-1, -1, -1, -1]]], np.int32)
    dq, dkv, _ = oracle.sparse_attn_bwd(qb, kvb, None, idx, gb, 0.5, Dv)
    assert np.all(dq == 0.0)
    want = np.zeros((B, N, Dqk))
    want[0, 2, :Dv] = gv[0, 0].sum(axis=0)  # every head's dO lands on row 2
    assert np.allclose(dkv, want, rtol=0, atol=1e-15), np.abs(dkv - want).max()
    # padding with -1 and a second copy of the idx layout give the same result
    idx2 = np.array([[[-1, 4, 1, -1], [3, 0, -1, -1]]], np.int32)
    sink = rng.standard_normal(Hq).astype(np.float32)
    a = oracle.sparse_attn_bwd(qb, kvb, sink, idx2, gb, 0.5, Dv)
    idx3 = np.concatenate([idx2, np.full((B, M, 3), -1, np.int32)], axis=2)
    b_ = oracle.sparse_attn_bwd(qb, kvb, sink, idx3, gb, 0.5, Dv)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y)
    # the |term| sums bound the gradients (triangle inequality) and vanish
    # with them
    _, _, _, tq, tk, ts = oracle.sparse_attn_bwd(qb, kvb, sink, idx2, gb, 0.5, Dv,
                                                 with_terms=True)
    assert np.all(tq >= np.abs(a[0]) * (1 - 1e-12)) and np.all(tk >= np.abs(a[1]) * (1 - 1e-12))
    assert np.all(ts >= np.abs(a[2]) * (1 - 1e-12)) and ts.max() > 0
    assert tq.max() > 0 and tk.max() > 0
    assert np.all(tk[0, 2] == 0.0)  # row 2 is gathered by no token
    # rows=[1] equals the full call with row 0's dO set to zero
    r1 = oracle.sparse_attn_bwd(qb, kvb, sink, idx2, gb, 0.5, Dv, rows=[1])
    g0 = gb.copy()
    g0[0, 0] = 0
    full0 = oracle.sparse_attn_bwd(qb, kvb, sink, idx2, g0, 0.5, Dv)
    assert np.allclose(r1[0], full0[0][1:], rtol=1e-13, atol=1e-15)
    assert np.allclose(r1[1], full0[1], rtol=1e-13, atol=1e-15)
    assert np.allclose(r1[2], full0[2], rtol=1e-13, atol=1e-15)


ALL_CHECKS = [
    check_e4m3_decode, check_bf16_decode,
    check_indexer_hand, check_indexer_exact, check_indexer_invariants, check_indexer_terms,
    check_topk_hand, check_topk_bruteforce, check_topk_invariants,
    check_attn_hand, check_attn_dense, check_attn_closed_forms, check_attn_invariants,
    check_attn_fp8_kv, check_attn_fp8_q, check_attn_terms, check_rows_subsets,
    check_attn_bwd_finite_differences, check_attn_bwd_closed_forms,
]
