"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, the ctypes struct matches the C layout, and invalid arguments are
rejected on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_indexer_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return dsa.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_stages():
    fns = header_functions()
    for f in dsa.EXPORTS:
        assert f in fns


def test_library_exports_every_declared_symbol():
    L = _lib()
    for f in header_functions():
        assert hasattr(L, f), f"libdsa.so does not export {f}"
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True,
                         text=True).stdout
    for f in header_functions():
        assert re.search(rf"\bT {f}\b", out), f


def test_version_and_status_strings():
    L = _lib()
    assert dsa.version() == 200
    for s in range(5):
        assert L.dsa_status_string(s)
    assert b"unknown" in L.dsa_status_string(99)


def test_prefill_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in dsa.PrefillArgs._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "dsa.h"\nint main(void){\n'
                    + 'printf("%zu\\n", sizeof(dsa_prefill_args));\n'
                    + "".join(f'printf("%zu\\n", offsetof(dsa_prefill_args, {f}));\n'
                              for f in fields) + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(dsa.PrefillArgs)
    for f, off in zip(fields, vals[1:]):
        assert getattr(dsa.PrefillArgs, f).offset == off, f


INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 4
P = ctypes.c_void_p
A16 = ctypes.c_void_p(0x10000)   # aligned fake pointers: never dereferenced,
A4 = ctypes.c_void_p(0x20004)    # validation fails before any HIP call


def test_indexer_rejects_bad_arguments():
    L = _lib()
    f = L.dsa_indexer_logits
    ok = dict(q=A16, qs=None, k=A16, ksc=A16, w=A16, ks=A16, ke=A16, out=A16, B=1, M=4, N=4,
              H=64, D=128)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["q"], a["qs"], a["k"], a["ksc"], a["w"], a["ks"], a["ke"], a["out"], a["B"],
                 a["M"], a["N"], a["H"], a["D"], None)

    assert call(q=None) == INVALID
    assert call(k=None) == INVALID
    assert call(out=None) == INVALID
    assert call(B=0) == INVALID
    assert call(M=-1) == INVALID
    assert call(N=0) == INVALID
    assert call(q=ctypes.c_void_p(0x10008)) == INVALID      # q not 16-byte aligned
    assert call(ks=ctypes.c_void_p(0x10002)) == INVALID     # bounds not 4-byte aligned
    assert call(N=1 << 31) == INVALID
    assert call(H=5) == UNSUPPORTED
    assert call(D=96) == UNSUPPORTED


def test_topk_rejects_bad_arguments():
    L = _lib()
    f = L.dsa_topk

    def call(*a, ws=None, wsb=0):
        return f(*a, ws, wsb, None)

    assert call(None, A16, A16, A16, 1, 4, 8, 2) == INVALID
    assert call(A16, A16, A16, A16, 1, 4, 8, 0) == INVALID
    assert call(A16, A16, A16, A16, 0, 4, 8, 2) == INVALID
    assert call(A16, A16, A16, A16, 1, 4, 8, 4097) == UNSUPPORTED
    assert call(A16, A16, ctypes.c_void_p(0x10001), A16, 1, 4, 8, 2) == INVALID
    # decode-shaped rows beyond 65536 keys need scratch: a workspace one byte
    # short is refused
    need = dsa.topk_workspace_size(64, 1, 131072, 2048)
    assert need > 0
    assert call(A16, A16, A16, A16, 64, 1, 131072, 2048, ws=A16, wsb=need - 1) == WORKSPACE
    assert call(A16, A16, A16, A16, 64, 1, 131072, 2048, ws=ctypes.c_void_p(0x10008),
                wsb=need) == INVALID  # workspace not 16-byte aligned


def test_attention_rejects_bad_arguments():
    L = _lib()
    f = L.dsa_sparse_attn_fwd

    def call(kv_dtype=0, kv_scale=None, Hq=128, Dqk=576, Dv=512, K=2048, q=A16, o=A16, ws=None,
             wsb=0, M=4):
        return f(q, A16, kv_dtype, kv_scale, None, A16, o, 1, M, 8, Hq, Dqk, Dv, K, 0.0, ws, wsb,
                 None)

    assert call(q=None) == INVALID
    assert call(kv_dtype=1) == INVALID                # fp8 kv needs kv_scale
    assert call(kv_dtype=0, kv_scale=A16) == INVALID  # bf16 kv must not have one
    assert call(kv_dtype=7) == INVALID
    assert call(Dv=600) == INVALID                    # Dv > Dqk
    assert call(K=0) == INVALID
    assert call(o=ctypes.c_void_p(0x10004)) == INVALID
    assert call(Hq=24) == UNSUPPORTED
    assert call(Dqk=128, Dv=128) == UNSUPPORTED
    assert call(K=5000) == UNSUPPORTED
    assert call(kv_dtype=1, kv_scale=A16, Dqk=64, Dv=64, Hq=16) == UNSUPPORTED
    need = dsa.sparse_attn_workspace_size(1, 4, 128, 576, 512, 2048)
    if need > 0:
        assert call(ws=A16, wsb=need - 1) == WORKSPACE


def test_fp8_attention_rejects_bad_arguments():
    L = _lib()
    f = L.dsa_sparse_attn_fwd_fp8

    def call(q=A16, qs=None, kvs=A16, Hq=128, Dqk=576, Dv=512, K=2048, o=A16, ws=None, wsb=0,
             M=4):
        return f(q, qs, A16, kvs, None, A16, o, 1, M, 8, Hq, Dqk, Dv, K, 0.0, ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(kvs=None) == INVALID                  # the KV scales are required
    assert call(qs=ctypes.c_void_p(0x10002)) == INVALID
    assert call(K=0) == INVALID
    assert call(Dv=600) == INVALID
    assert call(o=ctypes.c_void_p(0x10004)) == INVALID
    assert call(Hq=32) == UNSUPPORTED
    assert call(Hq=16) == UNSUPPORTED
    assert call(Dqk=64, Dv=64) == UNSUPPORTED
    assert call(K=5000) == UNSUPPORTED
    need = dsa.sparse_attn_fp8_workspace_size(64, 1, 128, 576, 512, 2048)
    assert need > 0
    assert f(A16, None, A16, A16, None, A16, A16, 64, 1, 8, 128, 576, 512, 2048, 0.0, A16,
             need - 1, None) == WORKSPACE
    # 64-row tiles: at least 4 per split
    S = need // (64 * 128 * (2 * 512 + 8))
    assert need % (64 * 128 * (2 * 512 + 8)) == 0 and 2 <= S <= 2048 // 256
    assert dsa.sparse_attn_fp8_workspace_size(1, 4096, 128, 576, 512, 2048) == 0


def test_workspace_size_queries():
    """Sizes follow the documented formulas: none for short rows and many
    query rows, per-row digit histograms for few long rows, candidates for
    many long rows, and bf16 partials plus (m, l) for split attention rows;
    invalid shapes are rejected like the calls themselves."""
    assert dsa.topk_workspace_size(1, 4096, 4096, 2048) == 0
    assert dsa.topk_workspace_size(1, 4096, 8192, 2048) == 0
    # few rows of up to 65536 keys: one workgroup per row, no scratch
    assert dsa.topk_workspace_size(64, 1, 65536, 2048) == 0
    # 64 rows, N = 131072: 32 segments of 4096 keys per row
    assert dsa.topk_workspace_size(64, 1, 131072, 2048) == 64 * (6144 + 32 * 1028) * 4
    # 300 rows of 20000 keys: 3 segments of 8192 keys, K candidates each
    assert dsa.topk_workspace_size(1, 300, 20000, 100) == 300 * 3 * 100 * 4
    # candidates beyond 256 MiB: none (streaming)
    assert dsa.topk_workspace_size(1, 32768, 32768, 2048) == 0
    # attention: many rows run unsplit; B*M <= CUs/2 rows are split
    assert dsa.sparse_attn_workspace_size(1, 4096, 128, 576, 512, 2048) == 0
    n = dsa.sparse_attn_workspace_size(64, 1, 128, 576, 512, 2048)
    assert n > 0 and n % (64 * 128 * (2 * 512 + 8)) == 0
    S = n // (64 * 128 * (2 * 512 + 8))
    assert 2 <= S <= 2048 // 128
    with pytest.raises(dsa.DSAError):
        dsa.topk_workspace_size(1, 4, 8, 0)
    with pytest.raises(dsa.DSAError):
        dsa.sparse_attn_workspace_size(1, 4, 24, 576, 512, 2048)


def test_prefill_rejects_null_and_inconsistent():
    L = _lib()
    assert L.dsa_prefill(None, None) == INVALID
    a = dsa.PrefillArgs()  # all zero
    assert L.dsa_prefill(ctypes.byref(a), None) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dsa, "_lib", None)
    monkeypatch.setattr(dsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        dsa.lib()


def test_prefill_noalloc_rejects_before_launch():
    """The static-scratch entry point refuses a workspace argument and a
    shape whose scratch need exceeds its static array, before any HIP call."""
    L = _lib()
    a = dsa.PrefillArgs(batch=100, seq_q=1, seq_kv=1 << 24, index_q=0x10000,
                        index_k=0x10000, index_k_scale=0x10000, index_weights=0x10000,
                        ks=0x10000, ke=0x10000, index_heads=64, index_dim=128, topk=2048,
                        q=0x10000, kv=0x10000, kv_dtype=0, o=0x10000, heads=128, dqk=576,
                        dv=512, logits=0x10000, topk_idxs=0x10000)
    assert dsa.prefill_workspace_size(a) > dsa.NOALLOC_SCRATCH_BYTES
    assert L.dsa_prefill_noalloc(ctypes.byref(a), None) == WORKSPACE
    a.workspace, a.workspace_bytes = 0x10000, 1 << 30
    assert L.dsa_prefill_noalloc(ctypes.byref(a), None) == INVALID
    assert L.dsa_prefill_noalloc(None, None) == INVALID
