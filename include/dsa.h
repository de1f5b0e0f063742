/*
 * dsa.h -- C ABI of libdsa: the DeepSeek-style sparse-attention (DSA) hot
 * path on AMD Instinct MI355X (gfx950).
 *
 *   1. dsa_indexer_logits  -- FP8 lightning-indexer scores
 *   2. dsa_topk            -- exact per-row top-k over those scores
 *   3. dsa_sparse_attn_fwd -- gathered sparse attention forward with a sink
 *   4. dsa_prefill         -- 1 -> 2 -> 3 on one stream
 * and dsa_indexer_topk (1 + 2 without the logits buffer),
 * dsa_sparse_attn_fwd_fp8 (3 with an fp8 query and KV cache: full-FP8
 * attention) and dsa_sparse_attn_bwd (the gradients of 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Tensor arguments are DEVICE pointers to dense row-major arrays (the last
 *    dimension is contiguous).  Pointers must be 16-byte aligned, except the
 *    per-row scale, weight, bound and sink arrays, which need 4-byte alignment.
 *  * Every call only ENQUEUES work on `stream` (a hipStream_t, NULL = the
 *    default stream) and returns; there is no host synchronisation unless the
 *    environment variable DSA_SYNC_CHECK=1 is set, in which case the call
 *    waits for its kernels and reports their errors.
 *  * Ownership: the caller allocates and owns every buffer, including the
 *    intermediates of dsa_prefill and any device scratch ("workspace").  The
 *    library allocates no device memory, keeps no pointer after a call
 *    returns and holds no mutable global state other than a mutex-guarded
 *    cache of each device's compute-unit count; calls are thread-safe.
 *    Calls that can use scratch (dsa_topk, dsa_sparse_attn_fwd[_fp8], dsa_prefill)
 *    take a `workspace` pointer and its size in bytes; the matching
 *    *_workspace_size call gives the bytes the fastest path needs for a
 *    shape on the current device.  A NULL workspace (or a size of 0 bytes
 *    needed) selects paths that need none, with the same results; a
 *    non-NULL workspace smaller than the size query's answer gives
 *    DSA_ERR_WORKSPACE.  The workspace must be 16-byte aligned.
 *    The workspace is read and written by the enqueued kernels only, in
 *    stream order: it must stay allocated until the stream has passed the
 *    call, and two calls in flight at once need two workspaces.
 *  * Errors: arguments are checked on the host before anything is enqueued.
 *    NULL pointers, non-positive sizes, misalignment or inconsistent sizes
 *    give DSA_ERR_INVALID_VALUE; a valid shape with no compiled kernel gives
 *    DSA_ERR_NOT_SUPPORTED; a too small workspace DSA_ERR_WORKSPACE.  In
 *    these cases nothing is launched and no output is written.  A failed
 *    launch gives DSA_ERR_LAUNCH.  The *_workspace_size calls validate
 *    their sizes the same way and write *bytes only on DSA_OK.
 *  * Device-side data contracts are clamped or masked, never trapped: bounds
 *    are clamped, out-of-range indices are treated as -1.
 *  * FP8 means OCP float8 e4m3fn (1 sign, 4 exponent bits with bias 7, 3
 *    mantissa bits, largest finite 448, 0x7F/0xFF NaN).  NaN codes are not
 *    valid inputs; results that depend on them are unspecified.
 *  * bf16 is the upper half of an IEEE binary32.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_VERSION 200 /* 2.0.0: caller-owned workspace arguments */

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_VALUE = 1,
  DSA_ERR_NOT_SUPPORTED = 2,
  DSA_ERR_LAUNCH = 3,
  DSA_ERR_WORKSPACE = 4, /* workspace given but smaller than the call needs */
  DSA_STATUS_INT_ = 0x7fffffff /* not a status: makes every int value
                                  representable (dsa_status_string accepts
                                  any value) */
} dsa_status;

typedef enum dsa_kv_dtype {
  DSA_KV_BF16 = 0,       /* kv holds bf16 values                             */
  DSA_KV_FP8_E4M3FN = 1, /* kv holds e4m3fn codes; value = code * kv_scale   */
  DSA_KV_DTYPE_INT_ = 0x7fffffff /* not a dtype: makes every int value
                                    representable, so that an invalid value
                                    can be passed and rejected */
} dsa_kv_dtype;

/*
 * dsa_indexer_logits -- lightning-indexer scores.
 *
 * Defined by the Modular "sparse_index_fp8_sm100_prefill" page (score
 * formula, with the per-(token, head) query scale in the weight position) and
 * the TileLang "deepseek_v32" examples page, section "Lightning Indexer"
 * (relu, head weights, key scale, sum over heads, per-token key bounds):
 *
 *   logits[b,t,key] = k_scale[b,key] *
 *        sum_h relu( sum_d q[b,t,h,d] * k[b,key,d] ) * weights[b,t,h] * q_scale[b,t,h]
 *
 * for every key in [s, e) with s = clamp(ks[b,t], 0, N), e = clamp(ke[b,t], s, N).
 *
 *   q        [B, M, H, D]  e4m3fn codes (1 byte each)
 *   q_scale  [B, M, H]     fp32, or NULL for 1 (may also be folded into
 *                          weights by the caller: relu(s*x) = s*relu(x), s > 0)
 *   k        [B, N, D]     e4m3fn codes
 *   k_scale  [B, N]        fp32
 *   weights  [B, M, H]     fp32
 *   ks, ke   [B, M]        int32 per-token key bounds
 *   logits   [B, M, N]     fp32 output.  Only keys inside each token's window
 *                          are written; entries outside it are left untouched
 *                          (unspecified to the caller).
 * Supported: H in {4, 8, 16, 32, 64, 128}, D in {64, 128, 256}; N < 2^31.
 * Products are exact and accumulate in fp32; the head sum is fp32.
 */
dsa_status dsa_indexer_logits(const void* q, const float* q_scale,
                              const void* k, const float* k_scale,
                              const float* weights, const int32_t* ks,
                              const int32_t* ke, float* logits, int64_t B,
                              int64_t M, int64_t N, int32_t H, int32_t D,
                              void* stream);

/*
 * dsa_topk -- exact top-k per row.
 *
 * Defined by the TileLang "deepseek_v32" examples page, section "Top-k
 * Selector" (exact selection over each row's [start, end) without a full
 * sort; indices are absolute key positions).  For row (b,t) with window
 * [s, e) clamped as in dsa_indexer_logits and len = e - s:
 *   * len <= K: the output is s, s+1, ..., e-1 followed by -1s (the logits
 *     are not read);
 *   * len  > K: the output is the K keys of [s, e) that come first in the
 *     order (value descending, index ascending) -- ties go to the lower index,
 *     -0 equals +0, NaN ranks as -inf -- in ascending index order.
 *
 *   logits     [B, M, N] fp32 (only each row's window is read)
 *   ks, ke     [B, M]    int32
 *   topk_idxs  [B, M, K] int32 output
 * Supported: 1 <= K <= 4096, N < 2^31.  Output is deterministic.
 * Workspace (dsa_topk_workspace_size; only N > 8192 needs any): with fewer
 * than 256 rows every row is cut into 4096-key segments that share per-row
 * digit histograms, B*M*(6144 + ceil(N/4096)*1028)*4 bytes; with more rows,
 * windows longer than 8192 keys go through a candidate buffer of
 * B*M*ceil(N/8192)*K*4 bytes when that is at most 256 MiB (0 bytes
 * otherwise).  Without a workspace, rows longer than 8192 keys take one
 * streaming workgroup each.
 */
dsa_status dsa_topk_workspace_size(int64_t B, int64_t M, int64_t N, int32_t K, size_t* bytes);

dsa_status dsa_topk(const float* logits, const int32_t* ks, const int32_t* ke,
                    int32_t* topk_idxs, int64_t B, int64_t M, int64_t N,
                    int32_t K, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * dsa_indexer_topk -- dsa_indexer_logits followed by dsa_topk without the
 * [B, M, N] logits buffer: the pages' planned fused score + top-k-select
 * step (Modular "sparse_index_fp8_sm100_prefill" page, the paragraph on the
 * next step: scoring and top-k selection together, with no materialised
 * [total_seq, max_num_keys] score buffer).  Rows are scored and selected in
 * slabs of about `slab_rows` rows (0 = 2048) whose logits live in the
 * workspace: peak scratch is one slab's logits (slab_rows * N * 4 bytes)
 * plus the top-k's scratch for a slab, instead of B * M * N * 4 bytes.
 * topk_idxs is exactly what dsa_topk returns on dsa_indexer_logits' output
 * for the same arguments (same arithmetic per logit; the selection is
 * exact).  Arguments as in dsa_indexer_logits and dsa_topk.  The
 * workspace is required (NULL or smaller than
 * dsa_indexer_topk_workspace_size gives DSA_ERR_WORKSPACE) and must be
 * 256-byte aligned.
 */
dsa_status dsa_indexer_topk_workspace_size(int64_t B, int64_t M, int64_t N, int32_t H,
                                           int32_t D, int32_t K, int64_t slab_rows,
                                           size_t* bytes);
dsa_status dsa_indexer_topk(const void* q, const float* q_scale, const void* k,
                            const float* k_scale, const float* weights,
                            const int32_t* ks, const int32_t* ke, int32_t* topk_idxs,
                            int64_t B, int64_t M, int64_t N, int32_t H, int32_t D,
                            int32_t K, int64_t slab_rows, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn_fwd -- gathered sparse attention forward with a sink.
 *
 * Defined by the DeepSeek V4.1 atlas page, sparse_attn_kernel and its wrapper
 * sparse_attn (gather the top-k KV rows by index, online softmax, per-head
 * attn_sink added to the denominator only, -1 indices masked, a row without
 * a valid index gives zero), with the value read from the first Dv columns
 * of the shared latent KV row.  For each (b, t, h), J = the indices j of
 * topk_idxs[b,t,:] with 0 <= j < N (others are skipped like -1):
 *   s_j  = sm_scale * sum_{d < Dqk} q[b,t,h,d] * kv[b,j,d]
 *   o[b,t,h,c] = sum_j exp(s_j) kv[b,j,c] / (sum_j exp(s_j) + exp(attn_sink[h]))
 * for c < Dv (the sink term is absent when attn_sink is NULL); o = 0 if J is
 * empty.  Softmax runs in base 2 with sm_scale*log2(e) folded in, in fp32;
 * QK^T and PV use bf16 MFMA with fp32 accumulation (P rounded to bf16).
 *
 *   q          [B, M, Hq, Dqk] bf16
 *   kv         [B, N, Dqk]     bf16, or e4m3fn codes (kv_dtype = FP8)
 *   kv_scale   [B, N] fp32 per-row scale for FP8 kv; must be NULL for bf16
 *   attn_sink  [Hq] fp32 or NULL
 *   topk_idxs  [B, M, K] int32
 *   o          [B, M, Hq, Dv] bf16 output
 *   sm_scale   softmax scale; <= 0 selects 1/sqrt(Dqk)
 * Supported: Hq in {16, 32, 64, 128}; (Dqk, Dv) in {(64, 64), (576, 512)}
 * (FP8 kv with (576, 512) only); 1 <= K <= 4096.
 * Workspace (dsa_sparse_attn_workspace_size): with few query rows (B*M at
 * most half the device's compute units, as in decode) each row's K indices
 * are split over S workgroups whose partial results a second kernel merges;
 * the partials take B*M*S*Hq*(2*Dv + 8) bytes (S <= K/128, chosen from the
 * device's compute-unit count).  Without a workspace the rows run unsplit,
 * with the same result up to rounding (the split stores its normalised
 * partials in bf16).
 */
dsa_status dsa_sparse_attn_workspace_size(int64_t B, int64_t M, int32_t Hq, int32_t Dqk,
                                          int32_t Dv, int32_t K, size_t* bytes);

dsa_status dsa_sparse_attn_fwd(const void* q, const void* kv,
                               dsa_kv_dtype kv_dtype, const float* kv_scale,
                               const float* attn_sink,
                               const int32_t* topk_idxs, void* o, int64_t B,
                               int64_t M, int64_t N, int32_t Hq, int32_t Dqk,
                               int32_t Dv, int32_t K, float sm_scale,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * dsa_sparse_attn_fwd_fp8 -- full-FP8 sparse attention forward: the
 * attention of dsa_sparse_attn_fwd with an e4m3 query and KV cache and a
 * bf16 output (TileLang "deepseek_v32" examples page, section "Sparse MLA
 * Forward (FP8)"), both products on fp8 MFMA.  The values are
 *   q[b,t,h,d] = e4m3(q codes) * q_scale[b,t,h]   (q_scale NULL: 1)
 *   kv[b,j,d]  = e4m3(kv codes) * kv_scale[b,j]
 * and o is defined by the formula of dsa_sparse_attn_fwd on those values
 * (sink, -1 / out-of-range indices and rows without a valid index alike).
 * Rounding: QK^T is exact products with fp32 accumulation; the softmax runs
 * in base 2 in fp32; each probability enters PV as an e4m3 number after
 * scaling by 2^c * kv_scale[b,j] / sigma (sigma = the largest kv_scale of
 * the row's indices, 2^c between 16 and 448 relative to the head's running
 * reference, following the FlashInfer MLA pull-request discussion's
 * scaling by the e4m3 maximum), so each term of o carries up to 2^-4
 * relative error (plus e4m3 underflow below 2^-9 of the scaled maximum); the
 * denominator sums unrounded fp32 probabilities; o is rounded to bf16.
 *
 *   q          [B, M, Hq, Dqk] e4m3fn codes
 *   q_scale    [B, M, Hq] fp32 or NULL
 *   kv         [B, N, Dqk]     e4m3fn codes
 *   kv_scale   [B, N] fp32 (required)
 *   attn_sink  [Hq] fp32 or NULL; topk_idxs [B, M, K] int32
 *   o          [B, M, Hq, Dv] bf16 output
 *   sm_scale   softmax scale; <= 0 selects 1/sqrt(Dqk)
 * Supported: Hq in {64, 128}; (Dqk, Dv) = (576, 512); 1 <= K <= 4096.
 * Workspace (dsa_sparse_attn_fp8_workspace_size): as dsa_sparse_attn_fwd,
 * splits of each row's indices over S workgroups when B*M is at most half
 * the device's compute units (S <= K/256); without a workspace the rows run
 * unsplit, with the same result up to rounding.
 */
dsa_status dsa_sparse_attn_fp8_workspace_size(int64_t B, int64_t M, int32_t Hq, int32_t Dqk,
                                              int32_t Dv, int32_t K, size_t* bytes);

dsa_status dsa_sparse_attn_fwd_fp8(const void* q, const float* q_scale, const void* kv,
                                   const float* kv_scale, const float* attn_sink,
                                   const int32_t* topk_idxs, void* o, int64_t B, int64_t M,
                                   int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K,
                                   float sm_scale, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * dsa_sparse_attn_bwd -- gradients of dsa_sparse_attn_fwd (bf16 kv).
 *
 * Defined by the TileLang "deepseek_v32" examples page, section "Sparse MLA
 * Backward" (dP from dO and V, Delta = rowsum(dO * O), dS = P * (dP -
 * Delta), dQ from dS and K, dKV scattered to the gathered rows with
 * atomics), applied to the forward above: for each (b, t, h), with p_j the
 * softmax weight of index j (sink in the denominator) and p_sink the sink's,
 *   dp_j  = sum_{c<Dv} dO[b,t,h,c] kv[b,j,c]
 *   Delta = sum_{c<Dv} dO[b,t,h,c] o[b,t,h,c]
 *   ds_j  = p_j (dp_j - Delta)
 *   dq[b,t,h,d]  = sm_scale sum_j ds_j kv[b,j,d]                   d < Dqk
 *   dkv[b,j,d]  += sm_scale ds_j q[b,t,h,d] + (d < Dv ? p_j dO[b,t,h,d] : 0)
 *   dsink[h]    += -p_sink Delta
 * summed over every (t, h) and every occurrence of j; invalid indices (-1 or
 * outside [0, N)) and rows without a valid index contribute nothing.
 *
 *   q [B,M,Hq,Dqk], kv [B,N,Dqk], o and dO [B,M,Hq,Dv]: bf16 (o is the
 *   forward's output for the same inputs); attn_sink [Hq] fp32 or NULL;
 *   topk_idxs [B,M,K] int32
 *   dq [B,M,Hq,Dqk], dkv [B,N,Dqk], dsink [Hq] (NULL iff attn_sink is NULL):
 *   fp32 outputs, overwritten (the call zero-fills them, then accumulates).
 * Supported: Hq a multiple of 16 up to 128; (Dqk, Dv) in {(64, 64), (576,
 * 512)}; 1 <= K <= 4096.  P and dS enter the MFMA products rounded to bf16,
 * everything else is fp32; dkv and dq are accumulated with fp32 atomics, so
 * their last bits depend on the order the hardware applies them in.
 */
dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, const float* attn_sink,
                               const int32_t* topk_idxs, const void* o, const void* dO,
                               float* dq, float* dkv, float* dsink, int64_t B, int64_t M,
                               int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K,
                               float sm_scale, void* stream);

/*
 * dsa_prefill -- the whole path on one stream: indexer scores into `logits`,
 * top-k into `topk_idxs`, sparse attention into `o`.  Every field has the
 * meaning, layout and constraints of the same argument above; `logits` and
 * `topk_idxs` are caller-owned intermediates that hold the stage results when
 * the stream reaches the end of the call.  The argument struct is read during
 * the call only.  The stages run one after the other on `stream`, so one
 * workspace serves both the top-k and the attention:
 * dsa_prefill_workspace_size gives the larger of their needs.
 * With logits == NULL the indexer and top-k run as dsa_indexer_topk (slabs
 * of 2048 rows, no [B, M, N] buffer; same topk_idxs); the workspace is then
 * required and its size includes a slab's logits.
 */
typedef struct dsa_prefill_args {
  /* sizes */
  int64_t batch;       /* B */
  int64_t seq_q;       /* M: query tokens per batch entry */
  int64_t seq_kv;      /* N: keys per batch entry */
  /* indexer */
  const void* index_q;        /* [B, M, H, D] e4m3fn */
  const float* index_q_scale; /* [B, M, H] or NULL */
  const void* index_k;        /* [B, N, D] e4m3fn */
  const float* index_k_scale; /* [B, N] */
  const float* index_weights; /* [B, M, H] */
  const int32_t* ks;          /* [B, M] */
  const int32_t* ke;          /* [B, M] */
  int32_t index_heads;        /* H */
  int32_t index_dim;          /* D */
  /* top-k */
  int32_t topk;               /* K */
  /* attention */
  const void* q;              /* [B, M, Hq, Dqk] bf16 */
  const void* kv;             /* [B, N, Dqk] */
  dsa_kv_dtype kv_dtype;
  const float* kv_scale;      /* [B, N] (FP8 kv) or NULL */
  const float* attn_sink;     /* [Hq] or NULL */
  void* o;                    /* [B, M, Hq, Dv] bf16 */
  int32_t heads;              /* Hq */
  int32_t dqk;                /* Dqk */
  int32_t dv;                 /* Dv */
  float sm_scale;             /* <= 0 -> 1/sqrt(Dqk) */
  /* caller-owned intermediates */
  float* logits;              /* [B, M, N], or NULL: scored in workspace slabs */
  int32_t* topk_idxs;         /* [B, M, K] */
  void* workspace;            /* device scratch or NULL */
  size_t workspace_bytes;
} dsa_prefill_args;

dsa_status dsa_prefill_workspace_size(const dsa_prefill_args* args, size_t* bytes);
dsa_status dsa_prefill(const dsa_prefill_args* args, void* stream);

/*
 * dsa_prefill_noalloc -- dsa_prefill for callers that cannot allocate device
 * memory at all: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  It computes exactly what dsa_prefill
 * computes with a workspace of dsa_prefill_workspace_size bytes, taking that
 * scratch from a static device array of DSA_NOALLOC_SCRATCH_BYTES inside the
 * library (one copy per device, held from the library's load until the
 * process ends) instead of a caller workspace.  `args->workspace` must be
 * NULL and `args->workspace_bytes` 0.
 *  * A shape whose scratch need exceeds DSA_NOALLOC_SCRATCH_BYTES is
 *    rejected with DSA_ERR_WORKSPACE before anything is enqueued (e.g. the
 *    top-k of fewer than 256 rows of more than ~3M keys).
 *  * The array is shared by every call on a device and keeps the last
 *    call's contents (the kernels clear what they need cleared themselves):
 *    calls that overlap on one device -- two streams, or two host threads --
 *    race on it and must be serialised by the caller.
 *  * The first call on a device looks up that device's copy of the array
 *    (no allocation); calls are otherwise like dsa_prefill.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
dsa_status dsa_prefill_noalloc(const dsa_prefill_args* args, void* stream);

/* Static description of a status code (never NULL). */
const char* dsa_status_string(dsa_status s);

/* DSA_VERSION of the built library. */
int dsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
