/*
 * dsa_oracle.h -- plain, slow, CPU reference for the DeepSeek-style sparse
 * attention (DSA) hot path: indexer logits, exact per-row top-k, and gathered
 * sparse attention with an attention sink.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU path.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the GPU library.
 *
 * Every function computes the plain definition of its result in fp64 (the
 * pages' fast methods -- radix select, online softmax, MFMA tiling -- reach the
 * same result and are deliberately NOT reproduced here).
 *
 * Row subsets: every entry point takes an optional list `rows` of flattened
 * (batch, token) row ids r = b*M + t (NULL = all B*M rows in order) and writes
 * its output compactly, one output row per listed row.
 *
 * Return value: 0 on success, -1 on an invalid argument (nothing written).
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Value of an OCP FP8 e4m3fn code, from the format definition (sign, 4-bit
 * exponent with bias 7, 3-bit mantissa, exponent 0 subnormal, S.1111.111 NaN,
 * no infinities, largest finite 448).  Returns NaN for the two NaN codes. */
double dsa_oracle_e4m3fn_value(uint8_t code);

/* Value of a bfloat16 bit pattern (the upper half of an IEEE binary32). */
double dsa_oracle_bf16_value(uint16_t bits);

/* Indexer logits (Modular sparse_index_fp8_sm100_prefill page, score formula;
 * TileLang deepseek_v32 page, "Lightning Indexer"):
 *   logit[b,t,key] = k_scale[b,key] * sum_h relu(q[b,t,h,:] . k[b,key,:])
 *                                         * w[b,t,h] * q_scale[b,t,h]
 * for key in [s, e), s = clamp(ks,0,N), e = clamp(ke,s,N).
 *   q  [B,M,H,D] e4m3fn codes     q_scale [B,M,H] fp32 or NULL (= 1)
 *   k  [B,N,D]   e4m3fn codes     k_scale [B,N] fp32
 *   w  [B,M,H]   fp32             ks, ke  [B,M] int32
 * logits: [n_rows, N] fp32; keys outside [s, e) are set to NaN.
 * terms (optional, [n_rows, N] fp64): k_scale * sum_h |w*q_scale| *
 *   sum_d |q*k| -- the sum of absolute values of every term, for tolerances.
 * The FP8 codes must be finite (not 0x7F / 0xFF).                         */
int dsa_oracle_indexer_logits(const uint8_t* q, const float* q_scale,
                              const uint8_t* k, const float* k_scale,
                              const float* w, const int32_t* ks,
                              const int32_t* ke, int64_t B, int64_t M,
                              int64_t N, int32_t H, int32_t D,
                              const int64_t* rows, int64_t n_rows,
                              float* logits, double* terms);

/* Exact top-k per row (TileLang deepseek_v32 page, "Top-k Selector"):
 * the K keys of [s, e) that come first in the order (value descending,
 * index ascending), -0 equal to +0 and NaN ranked as -inf, written in
 * ascending index order; a row with len = e - s <= K yields s..e-1.  Unused
 * slots hold -1.
 *   logits: [n_rows, N] fp32, one row per listed row (compact)
 *   out:    [n_rows, K] int32                                             */
int dsa_oracle_topk(const float* logits, const int32_t* ks, const int32_t* ke,
                    int64_t B, int64_t M, int64_t N, int32_t K,
                    const int64_t* rows, int64_t n_rows, int32_t* out);

/* Sparse attention forward with a sink (DeepSeek V4.1 atlas page,
 * sparse_attn_kernel).  For each (b,t,h), with J the multiset of indices j in
 * topk_idxs[b,t,:] with 0 <= j < N (-1 and other values are skipped):
 *   s_j  = sm_scale * sum_{d<Dqk} q[b,t,h,d] * kv[b,j,d]
 *   Mx   = max(max_j s_j, sink_h)     (sink term omitted when sink == NULL)
 *   den  = sum_j exp(s_j - Mx) + exp(sink_h - Mx)
 *   o[c] = sum_j exp(s_j - Mx) * kv[b,j,c] / den,   c < Dv
 * and o = 0 when J is empty.
 *   q   [B,M,Hq,Dqk] bf16 bits
 *   kv  [B,N,Dqk]    bf16 bits (kv_fp8 = 0) or e4m3fn codes (kv_fp8 = 1); with
 *                    fp8 the value is code_value * kv_scale[b,j]
 *   sink [Hq] fp32 or NULL; topk_idxs [B,M,K] int32
 * o: [n_rows, Hq, Dv] fp64.                                                */
int dsa_oracle_sparse_attn(const uint16_t* q, const void* kv, int32_t kv_fp8,
                           const float* kv_scale, const float* sink,
                           const int32_t* topk_idxs, int64_t B, int64_t M,
                           int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                           int32_t K, double sm_scale, const int64_t* rows,
                           int64_t n_rows, double* o);

/* The same attention with the query optionally in fp8 (full-FP8 attention:
 * TileLang "deepseek_v32" page, section "Sparse MLA Forward (FP8)", an e4m3
 * query and KV cache with a bf16 output).  q_fp8 = 0: q holds bf16 bits and
 * q_scale must be NULL; q_fp8 = 1: q holds e4m3fn codes and the query value
 * is code_value * q_scale[b,t,h] (q_scale [B,M,Hq] fp32, NULL = 1).  The
 * result is the exact attention of those values: the fp8 rounding of the
 * probabilities that the GPU path applies is not modelled here (it is the
 * GPU path's rounding, bounded through `terms`).
 * terms (NULL or [n_rows, Hq, Dv] fp64): terms[c] = sum_j exp(s_j - Mx) *
 * |kv_value[b,j,c]| / den, the magnitude of what each output element sums
 * (equal to o[c] when every value is >= 0).                                 */
int dsa_oracle_sparse_attn_ex(const void* q, int32_t q_fp8, const float* q_scale,
                              const void* kv, int32_t kv_fp8,
                              const float* kv_scale, const float* sink,
                              const int32_t* topk_idxs, int64_t B, int64_t M,
                              int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                              int32_t K, double sm_scale, const int64_t* rows,
                              int64_t n_rows, double* o, double* terms);

/* Gradients of that sparse attention (TileLang deepseek_v32 page, "Sparse
 * MLA Backward": dP from dO and V, Delta = rowsum(dO * O), dS = P * (dP -
 * Delta), dQ from dS and K, dKV scattered back to the gathered rows).  For
 * each listed (b,t) and head h, with p_j = exp(s_j - Mx) / den and p_sink =
 * exp(sink_h - Mx) / den as in the forward:
 *   dp_j      = sum_{c<Dv} dO[b,t,h,c] * kv[b,j,c]
 *   Delta     = sum_j p_j * dp_j              (= sum_c dO[c] * o[c])
 *   ds_j      = p_j * (dp_j - Delta)
 *   dq[d]     = sm_scale * sum_j ds_j * kv[b,j,d]               d < Dqk
 *   dkv[b,j,d] += sm_scale * ds_j * q[d] + (d < Dv ? p_j * dO[d] : 0)
 *   dsink[h]  += -p_sink * Delta
 * Each occurrence of a duplicated index contributes; rows without a valid
 * index contribute nothing.  q, kv, dO are bf16 bits.
 *   dq    [n_rows, Hq, Dqk] fp64 (listed rows)
 *   dkv   [B, N, Dqk] fp64: the listed rows' contributions (overwritten)
 *   dsink [Hq] fp64 (listed rows), or NULL when sink is NULL
 *   tdq, tdkv: NULL, or the same shapes holding the sums of the absolute
 *   values of the terms above, with ds_j expanded into its terms p_j dp_j
 *   and p_j dO[c] o[c] (c < Dv): with A_j = p_j (|dp_j| + sum_c |dO[c]|
 *   |o[c]|), sm_scale A_j |kv_j[d]|, and sm_scale A_j |q[d]| + p_j |dO[d]|;
 *   tdsink: NULL, or [Hq] with sum p_sink sum_c |dO[c]| |o[c]|; for
 *   tolerances.                                                            */
int dsa_oracle_sparse_attn_bwd(const uint16_t* q, const uint16_t* kv,
                               const float* sink, const int32_t* topk_idxs,
                               const uint16_t* dO, int64_t B, int64_t M,
                               int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv,
                               int32_t K, double sm_scale, const int64_t* rows,
                               int64_t n_rows, double* dq, double* dkv,
                               double* dsink, double* tdq, double* tdkv,
                               double* tdsink);

/* Number of OpenMP threads the oracle runs with (0 if built without). */
int dsa_oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
