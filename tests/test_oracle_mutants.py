"""Checker-mutation tests: plant a plausible mistake in a copy of the oracle
(on the CPU), rebuild it, and require that the pins catch it.  This shows that
the pins in oracle_pins.py can fail, and that each kind of mistake -- a
dropped term, a wrong sign, an off-by-one index, a wrong operand slice, a
wrong tie rule -- is covered."""
import multiprocessing as mp
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402
from oracle import build as obuild  # noqa: E402

SRC = open(obuild.SRC).read()

# (id, original text, mutated text)
MUTANTS = [
    ("e4m3_bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3_int_subnormal", "(e == 0) ? (int64_t)m :", "(e == 0) ? (int64_t)(m + 1) :"),
    ("relu_dropped", "if (x > 0.0) acc += x * wq;", "acc += x * wq;"),
    ("qscale_ignored", "(q_scale ? (double)q_scale[r * H + h] : 1.0)", "1.0"),
    ("kscale_ignored", "out[key] = (float)(acc * ksc);", "out[key] = (float)(acc);"),
    ("window_off_by_one", "for (int64_t key = s; key < e; ++key) {\n      const uint8_t* kr",
     "for (int64_t key = s + 1; key < e; ++key) {\n      const uint8_t* kr"),
    ("k_transposed_index", "const uint8_t* kr = k + (b * N + key) * D;",
     "const uint8_t* kr = k + (b * N + (N - 1 - key)) * D;"),
    ("clamp_ke_missing", "  if (b > N) b = N;\n", "\n"),
    ("tie_to_higher", "return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    ("topk_not_sorted", "qsort(o, (size_t)K, sizeof(int32_t), cmp_int_asc);", ";"),
    ("topk_short_row_offset", "o[j] = (int32_t)(s + j);", "o[j] = (int32_t)j;"),
    ("sink_dropped", "if (sink) den += exp(sk - mx);", ";"),
    ("sink_scaled", "double sk = sink ? (double)sink[h] : -INFINITY;\n        if (sk > mx) mx = sk;\n        double den = 0.0;",
     "double sk = sink ? sm_scale * (double)sink[h] : -INFINITY;\n        if (sk > mx) mx = sk;\n        double den = 0.0;"),
    ("v_wrong_slice", "oh[c] += p * vr[c];", "oh[c] += p * vr[c + (Dqk - Dv)];"),
    ("scale_ignored", "sc[j] = sm_scale * acc;\n          if (sc[j] > mx)", "sc[j] = acc;\n          if (sc[j] > mx)"),
    ("minus_one_not_masked", "if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];\n      /* decode",
     "if (idx[j] < N) J[nj++] = idx[j] < 0 ? 0 : idx[j];\n      /* decode"),
    ("bwd_minus_one_not_masked", "if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];\n      for (int32_t h",
     "if (idx[j] < N) J[nj++] = idx[j] < 0 ? 0 : idx[j];\n      for (int32_t h"),
    ("fp8_kv_scale_ignored", "(double)kv_scale[b * N + J[j]];", "1.0;"),
    # row-subset paths: the listed row's own window / query / index list
    ("topk_rows_window", "window(ks, ke, r, N, &s, &e);\n      int32_t* o = out + i * K;",
     "window(ks, ke, i, N, &s, &e);\n      int32_t* o = out + i * K;"),
    ("indexer_rows_query", "const uint8_t* qr = q + (r * H + h) * D;",
     "const uint8_t* qr = q + (i * H + h) * D;"),
    ("attn_rows_indices", "const int32_t* idx = topk_idxs + r * K;\n      int32_t nj = 0;\n      for (int32_t j = 0; j < K; ++j)\n        if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];\n      /* decode",
     "const int32_t* idx = topk_idxs + i * K;\n      int32_t nj = 0;\n      for (int32_t j = 0; j < K; ++j)\n        if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];\n      /* decode"),
    # fp8 query and the term sums
    ("q8_scale_ignored", "const double qsc = q_scale ? (double)q_scale[r * Hq + h] : 1.0;",
     "const double qsc = 1.0;"),
    ("q8_scale_wrong_head", "(double)q_scale[r * Hq + h] : 1.0;", "(double)q_scale[r * Hq] : 1.0;"),
    ("terms_signed", "th[c] += p * fabs(vr[c]);", "th[c] += p * vr[c];"),
    ("terms_unnormalised", "for (int32_t c = 0; c < Dv; ++c) th[c] /= den;", ";"),
    # backward
    ("bwd_delta_dropped", "double ds = p * (dp[j] - delta);", "double ds = p * dp[j];"),
    ("bwd_dq_unscaled", "g[d] += sm_scale * ds * kvd;", "g[d] += ds * kvd;"),
    ("bwd_dv_dropped", "(d < Dv ? p * gv[d] : 0.0);\n#pragma omp atomic\n            gk[d] += add;",
     "0.0;\n#pragma omp atomic\n            gk[d] += add;"),
    ("bwd_dk_wrong_q", "double add = sm_scale * ds * qv[d]", "double add = sm_scale * ds * kvd"),
    ("bwd_dsink_sign", "dsink[h] += -ps * delta;", "dsink[h] += ps * delta;"),
    ("bwd_sink_in_max_only", "double den = sink ? exp(sk - mx) : 0.0;", "double den = 0.0;"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant_dir, name, orig, mut):
    assert SRC.count(orig) == 1, f"mutation anchor for {name} not unique/found"
    src = mutant_dir / f"{name}.c"
    src.write_text(SRC.replace(orig, mut).replace(
        '#include "dsa_oracle.h"', f'#include "{os.path.join(os.path.dirname(obuild.SRC), "dsa_oracle.h")}"'))
    lib = str(mutant_dir / f"lib{name}.so")
    obuild.build(out=lib, src=str(src), extra_flags=("-w",))
    # A mutant may write out of bounds: run it in a child process so it cannot
    # corrupt this process.  A crash also counts as caught.  The child is
    # spawned, not forked: a fork after this process has run OpenMP regions
    # (any earlier oracle call) would leave the child's thread pool unusable.
    ctx = mp.get_context("spawn")
    rd, wr = ctx.Pipe(duplex=False)
    proc = ctx.Process(target=_run_checks, args=(lib, wr))
    proc.start()
    wr.close()
    try:
        caught = rd.recv()
    except EOFError:
        caught = ["<crashed>"]
    proc.join()
    assert caught, f"no pin catches mutant {name}"


def _run_checks(lib, conn):
    import faulthandler
    faulthandler.disable()  # a crashing mutant is expected; keep the log quiet
    caught = []
    with P.oracle_lib(lib):
        for chk in P.ALL_CHECKS:
            try:
                chk()
            except AssertionError:
                caught.append(chk.__name__)
    conn.send(caught)
    conn.close()
    os._exit(0)
