/*
 * dsa_oracle.c -- plain CPU reference for the DSA hot path (test
 * infrastructure only; see dsa_oracle.h).  Built with gcc -O2 -fopenmp and
 * without fast-math.  Nothing here is shared with the GPU library.
 *
 * Sources, by function:
 *   indexer  -- Modular "sparse_index_fp8_sm100_prefill" page, the score
 *               formula; TileLang "deepseek_v32" examples page, section
 *               "Lightning Indexer" (relu, weights, k-scale, head sum, and the
 *               per-token key bounds CuSeqLenKS / CuSeqLenKE clamped to the
 *               key count).
 *   top-k    -- TileLang "deepseek_v32" page, section "Top-k Selector" (exact
 *               top-k over [start, end) of each row); ties to the lower index
 *               and ascending output are this library's stated contract.
 *   attention-- DeepSeek V4.1 atlas page, sparse_attn_kernel and sparse_attn
 *               (gather by index, -1 masked, softmax with a per-head sink in
 *               the denominator only, all-invalid rows give zero).
 *   backward -- TileLang "deepseek_v32" page, section "Sparse MLA Backward"
 *               (Delta = rowsum(dO * O), dS = P * (dP - Delta), dQ and the
 *               scattered dKV), applied to the forward above.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

double dsa_oracle_e4m3fn_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN; /* the only NaN pattern, either sign */
  if (e == 0)
    mag = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* e4m3fn code as an exact integer multiple of 2^-9: value = int * 2^-9.
 * Finite codes only.  Largest magnitude: 448 * 2^9 = 229376 < 2^18. */
static int64_t e4m3fn_times_512(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  int64_t mag = (e == 0) ? (int64_t)m : ((int64_t)(8 + m) << (e - 1));
  return sign ? -mag : mag;
}

double dsa_oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int dsa_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 0;
#endif
}

/* Per-token key window: s = clamp(ks, 0, N), e = clamp(ke, s, N). */
static void window(const int32_t* ks, const int32_t* ke, int64_t r, int64_t N,
                   int64_t* s, int64_t* e) {
  int64_t a = ks[r], b = ke[r];
  if (a < 0) a = 0;
  if (a > N) a = N;
  if (b < a) b = a;
  if (b > N) b = N;
  *s = a;
  *e = b;
}

static int64_t row_id(const int64_t* rows, int64_t i) {
  return rows ? rows[i] : i;
}

/* ------------------------------------------------------------------------ */
/* Indexer logits                                                            */
/* ------------------------------------------------------------------------ */

int dsa_oracle_indexer_logits(const uint8_t* q, const float* q_scale,
                              const uint8_t* k, const float* k_scale,
                              const float* w, const int32_t* ks,
                              const int32_t* ke, int64_t B, int64_t M,
                              int64_t N, int32_t H, int32_t D,
                              const int64_t* rows, int64_t n_rows,
                              float* logits, double* terms) {
  if (!q || !k || !k_scale || !w || !ks || !ke || !logits) return -1;
  if (B <= 0 || M <= 0 || N <= 0 || H <= 0 || D <= 0 || D > 1024) return -1;
  if (!rows) n_rows = B * M;
  for (int64_t i = 0; i < n_rows; ++i)
    if (row_id(rows, i) < 0 || row_id(rows, i) >= B * M) return -1;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = row_id(rows, i);
    int64_t b = r / M;
    int64_t s, e;
    window(ks, ke, r, N, &s, &e);
    float* out = logits + i * N;
    double* tout = terms ? terms + i * N : NULL;
    for (int64_t key = 0; key < N; ++key) {
      out[key] = NAN;
      if (tout) tout[key] = NAN;
    }
    for (int64_t key = s; key < e; ++key) {
      const uint8_t* kr = k + (b * N + key) * D;
      double acc = 0.0, tacc = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        const uint8_t* qr = q + (r * H + h) * D;
        int64_t dot = 0, adot = 0; /* exact: |dot| < 2^43 */
        for (int32_t d = 0; d < D; ++d) {
          int64_t p = e4m3fn_times_512(qr[d]) * e4m3fn_times_512(kr[d]);
          dot += p;
          adot += p < 0 ? -p : p;
        }
        double x = ldexp((double)dot, -18); /* exact q.k */
        double wq = (double)w[r * H + h] *
                    (q_scale ? (double)q_scale[r * H + h] : 1.0);
        if (x > 0.0) acc += x * wq; /* relu(q.k) * w * q_scale */
        tacc += ldexp((double)adot, -18) * fabs(wq);
      }
      double ksc = (double)k_scale[b * N + key];
      out[key] = (float)(acc * ksc);
      if (tout) tout[key] = tacc * fabs(ksc);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Top-k                                                                     */
/* ------------------------------------------------------------------------ */

typedef struct {
  float v;
  int32_t i;
} vi_pair;

/* -0 compares equal to +0 already; NaN is ranked as -inf. */
static float canon(float x) { return isnan(x) ? -INFINITY : (x == 0.0f ? 0.0f : x); }

/* (value descending, index ascending) */
static int cmp_desc(const void* pa, const void* pb) {
  const vi_pair* a = (const vi_pair*)pa;
  const vi_pair* b = (const vi_pair*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

static int cmp_int_asc(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int dsa_oracle_topk(const float* logits, const int32_t* ks, const int32_t* ke,
                    int64_t B, int64_t M, int64_t N, int32_t K,
                    const int64_t* rows, int64_t n_rows, int32_t* out) {
  if (!logits || !ks || !ke || !out) return -1;
  if (B <= 0 || M <= 0 || N <= 0 || K <= 0 || N > 0x7fffffff) return -1;
  if (!rows) n_rows = B * M;
  for (int64_t i = 0; i < n_rows; ++i)
    if (row_id(rows, i) < 0 || row_id(rows, i) >= B * M) return -1;
  int failed = 0;

#pragma omp parallel
  {
    vi_pair* buf = (vi_pair*)malloc(sizeof(vi_pair) * (size_t)N);
    if (!buf) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
      if (!buf) continue;
      int64_t r = row_id(rows, i);
      int64_t s, e;
      window(ks, ke, r, N, &s, &e);
      int32_t* o = out + i * K;
      int64_t len = e - s;
      for (int32_t j = 0; j < K; ++j) o[j] = -1;
      if (len <= K) {
        for (int64_t j = 0; j < len; ++j) o[j] = (int32_t)(s + j);
        continue;
      }
      const float* row = logits + i * N;
      for (int64_t j = 0; j < len; ++j) {
        buf[j].v = canon(row[s + j]);
        buf[j].i = (int32_t)(s + j);
      }
      qsort(buf, (size_t)len, sizeof(vi_pair), cmp_desc);
      for (int32_t j = 0; j < K; ++j) o[j] = buf[j].i;
      qsort(o, (size_t)K, sizeof(int32_t), cmp_int_asc);
    }
    free(buf);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention with sink                                                */
/* ------------------------------------------------------------------------ */

int dsa_oracle_sparse_attn_ex(const void* q, int32_t q_fp8, const float* q_scale,
                              const void* kv, int32_t kv_fp8,
                              const float* kv_scale, const float* sink,
                              const int32_t* topk_idxs, int64_t B, int64_t M,
                              int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                              int32_t K, double sm_scale, const int64_t* rows,
                              int64_t n_rows, double* o, double* terms) {
  if (!q || !kv || !topk_idxs || !o) return -1;
  if (!q_fp8 && q_scale) return -1;
  if (kv_fp8 && !kv_scale) return -1;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Dqk <= 0 || Dv <= 0 ||
      Dv > Dqk || K <= 0)
    return -1;
  if (!rows) n_rows = B * M;
  for (int64_t i = 0; i < n_rows; ++i)
    if (row_id(rows, i) < 0 || row_id(rows, i) >= B * M) return -1;
  int failed = 0;

#pragma omp parallel
  {
    /* per thread: decoded rows of the gathered set and their scores */
    double* rowv = (double*)malloc(sizeof(double) * (size_t)K * (size_t)Dqk);
    double* sc = (double*)malloc(sizeof(double) * (size_t)K);
    double* qv = (double*)malloc(sizeof(double) * (size_t)Dqk);
    int32_t* J = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    if (!rowv || !sc || !qv || !J) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      if (!rowv || !sc || !qv || !J) continue;
      int64_t r = row_id(rows, i);
      int64_t b = r / M;
      const int32_t* idx = topk_idxs + r * K;
      int32_t nj = 0;
      for (int32_t j = 0; j < K; ++j)
        if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];
      /* decode the gathered KV rows once per (b, t) */
      for (int32_t j = 0; j < nj; ++j) {
        int64_t base = (b * N + J[j]) * (int64_t)Dqk;
        for (int32_t d = 0; d < Dqk; ++d) {
          double v;
          if (kv_fp8)
            v = dsa_oracle_e4m3fn_value(((const uint8_t*)kv)[base + d]) *
                (double)kv_scale[b * N + J[j]];
          else
            v = dsa_oracle_bf16_value(((const uint16_t*)kv)[base + d]);
          rowv[(int64_t)j * Dqk + d] = v;
        }
      }
      for (int32_t h = 0; h < Hq; ++h) {
        double* oh = o + (i * Hq + h) * (int64_t)Dv;
        double* th = terms ? terms + (i * Hq + h) * (int64_t)Dv : NULL;
        for (int32_t c = 0; c < Dv; ++c) oh[c] = 0.0;
        if (th)
          for (int32_t c = 0; c < Dv; ++c) th[c] = 0.0;
        if (nj == 0) continue; /* all-invalid row: zero output */
        const int64_t qoff = (r * Hq + h) * (int64_t)Dqk;
        if (q_fp8) {
          /* fp8 query: decoded code times the (token, head) scale */
          const double qsc = q_scale ? (double)q_scale[r * Hq + h] : 1.0;
          for (int32_t d = 0; d < Dqk; ++d)
            qv[d] = dsa_oracle_e4m3fn_value(((const uint8_t*)q)[qoff + d]) * qsc;
        } else {
          for (int32_t d = 0; d < Dqk; ++d)
            qv[d] = dsa_oracle_bf16_value(((const uint16_t*)q)[qoff + d]);
        }
        double mx = -INFINITY;
        for (int32_t j = 0; j < nj; ++j) {
          double acc = 0.0;
          const double* kr = rowv + (int64_t)j * Dqk;
          for (int32_t d = 0; d < Dqk; ++d) acc += qv[d] * kr[d];
          sc[j] = sm_scale * acc;
          if (sc[j] > mx) mx = sc[j];
        }
        double sk = sink ? (double)sink[h] : -INFINITY;
        if (sk > mx) mx = sk;
        double den = 0.0;
        for (int32_t j = 0; j < nj; ++j) {
          double p = exp(sc[j] - mx);
          den += p;
          const double* vr = rowv + (int64_t)j * Dqk;
          for (int32_t c = 0; c < Dv; ++c) oh[c] += p * vr[c];
          if (th)
            for (int32_t c = 0; c < Dv; ++c) th[c] += p * fabs(vr[c]);
        }
        if (sink) den += exp(sk - mx);
        for (int32_t c = 0; c < Dv; ++c) oh[c] /= den;
        if (th)
          for (int32_t c = 0; c < Dv; ++c) th[c] /= den;
      }
    }
    free(rowv);
    free(sc);
    free(qv);
    free(J);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention backward                                                 */
int dsa_oracle_sparse_attn(const uint16_t* q, const void* kv, int32_t kv_fp8,
                           const float* kv_scale, const float* sink,
                           const int32_t* topk_idxs, int64_t B, int64_t M,
                           int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                           int32_t K, double sm_scale, const int64_t* rows,
                           int64_t n_rows, double* o) {
  return dsa_oracle_sparse_attn_ex(q, 0, NULL, kv, kv_fp8, kv_scale, sink, topk_idxs, B, M,
                                   N, Hq, Dqk, Dv, K, sm_scale, rows, n_rows, o, NULL);
}

/* ------------------------------------------------------------------------ */

int dsa_oracle_sparse_attn_bwd(const uint16_t* q, const uint16_t* kv,
                               const float* sink, const int32_t* topk_idxs,
                               const uint16_t* dO, int64_t B, int64_t M,
                               int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                               int32_t K, double sm_scale, const int64_t* rows,
                               int64_t n_rows, double* dq, double* dkv,
                               double* dsink, double* tdq, double* tdkv,
                               double* tdsink) {
  if (!q || !kv || !topk_idxs || !dO || !dq || !dkv) return -1;
  if (sink && !dsink) return -1;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Dqk <= 0 || Dv <= 0 ||
      Dv > Dqk || K <= 0)
    return -1;
  if (!rows) n_rows = B * M;
  for (int64_t i = 0; i < n_rows; ++i)
    if (row_id(rows, i) < 0 || row_id(rows, i) >= B * M) return -1;
  for (int64_t x = 0; x < B * N * Dqk; ++x) {
    dkv[x] = 0.0;
    if (tdkv) tdkv[x] = 0.0;
  }
  if (dsink)
    for (int32_t h = 0; h < Hq; ++h) dsink[h] = 0.0;
  if (tdsink)
    for (int32_t h = 0; h < Hq; ++h) tdsink[h] = 0.0;
  int failed = 0;

#pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)K);
    double* dp = (double*)malloc(sizeof(double) * (size_t)K);
    double* qv = (double*)malloc(sizeof(double) * (size_t)Dqk);
    double* gv = (double*)malloc(sizeof(double) * (size_t)Dv);
    int32_t* J = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    if (!sc || !dp || !qv || !gv || !J) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      if (!sc || !dp || !qv || !gv || !J) continue;
      int64_t r = row_id(rows, i);
      int64_t b = r / M;
      const int32_t* idx = topk_idxs + r * K;
      int32_t nj = 0;
      for (int32_t j = 0; j < K; ++j)
        if (idx[j] >= 0 && idx[j] < N) J[nj++] = idx[j];
      for (int32_t h = 0; h < Hq; ++h) {
        double* g = dq + (i * Hq + h) * (int64_t)Dqk;
        double* tg = tdq ? tdq + (i * Hq + h) * (int64_t)Dqk : NULL;
        for (int32_t d = 0; d < Dqk; ++d) {
          g[d] = 0.0;
          if (tg) tg[d] = 0.0;
        }
        if (nj == 0) continue; /* o = 0 whatever q, kv and the sink */
        const uint16_t* qh = q + (r * Hq + h) * (int64_t)Dqk;
        const uint16_t* gh = dO + (r * Hq + h) * (int64_t)Dv;
        for (int32_t d = 0; d < Dqk; ++d) qv[d] = dsa_oracle_bf16_value(qh[d]);
        for (int32_t c = 0; c < Dv; ++c) gv[c] = dsa_oracle_bf16_value(gh[c]);
        /* forward statistics */
        double mx = -INFINITY;
        for (int32_t j = 0; j < nj; ++j) {
          const uint16_t* kr = kv + (b * N + J[j]) * (int64_t)Dqk;
          double acc = 0.0, dacc = 0.0;
          for (int32_t d = 0; d < Dqk; ++d) acc += qv[d] * dsa_oracle_bf16_value(kr[d]);
          for (int32_t c = 0; c < Dv; ++c) dacc += gv[c] * dsa_oracle_bf16_value(kr[c]);
          sc[j] = sm_scale * acc;
          dp[j] = dacc;
          if (sc[j] > mx) mx = sc[j];
        }
        double sk = sink ? (double)sink[h] : -INFINITY;
        if (sk > mx) mx = sk;
        double den = sink ? exp(sk - mx) : 0.0;
        for (int32_t j = 0; j < nj; ++j) den += exp(sc[j] - mx);
        /* Delta = sum_j p_j dp_j */
        double delta = 0.0;
        for (int32_t j = 0; j < nj; ++j) delta += exp(sc[j] - mx) / den * dp[j];
        /* for the |term| sums: sum_c |dO[c]| |o[c]|, the terms of Delta
         * written as dO . o */
        double dabs = 0.0;
        if (tg || tdkv || tdsink) {
          for (int32_t c = 0; c < Dv; ++c) {
            double oc = 0.0;
            for (int32_t j = 0; j < nj; ++j)
              oc += exp(sc[j] - mx) / den *
                    dsa_oracle_bf16_value(kv[(b * N + J[j]) * (int64_t)Dqk + c]);
            dabs += fabs(gv[c]) * fabs(oc);
          }
        }
        if (sink) {
          double ps = exp(sk - mx) / den;
#pragma omp atomic
          dsink[h] += -ps * delta;
          if (tdsink) {
#pragma omp atomic
            tdsink[h] += ps * dabs;
          }
        }
        for (int32_t j = 0; j < nj; ++j) {
          double p = exp(sc[j] - mx) / den;
          double ds = p * (dp[j] - delta);
          double dsabs = p * (fabs(dp[j]) + dabs); /* |terms| of ds */
          const uint16_t* kr = kv + (b * N + J[j]) * (int64_t)Dqk;
          double* gk = dkv + (b * N + J[j]) * (int64_t)Dqk;
          double* tk = tdkv ? tdkv + (b * N + J[j]) * (int64_t)Dqk : NULL;
          for (int32_t d = 0; d < Dqk; ++d) {
            double kvd = dsa_oracle_bf16_value(kr[d]);
            g[d] += sm_scale * ds * kvd;
            if (tg) tg[d] += sm_scale * dsabs * fabs(kvd);
            double add = sm_scale * ds * qv[d] + (d < Dv ? p * gv[d] : 0.0);
#pragma omp atomic
            gk[d] += add;
            if (tk) {
              double tadd = sm_scale * dsabs * fabs(qv[d]) + (d < Dv ? p * fabs(gv[d]) : 0.0);
#pragma omp atomic
              tk[d] += tadd;
            }
          }
        }
      }
    }
    free(sc);
    free(dp);
    free(qv);
    free(gv);
    free(J);
  }
  return failed ? -1 : 0;
}
