// api.hip -- the C ABI of libdsa (declared in include/dsa.h): host-side
// argument validation, kernel dispatch, launch error mapping.
#include <cstdlib>
#include <cstring>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

constexpr int64_t kMaxI32 = 0x7fffffffLL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool sync_check() {
  static const bool on = [] {
    const char* e = std::getenv("DSA_SYNC_CHECK");
    return e && std::strcmp(e, "0") != 0 && e[0] != '\0';
  }();
  return on;
}

dsa_status finish(hipError_t launched, hipStream_t stream) {
  if (launched != hipSuccess) return DSA_ERR_LAUNCH;
  if (sync_check()) {
    if (hipStreamSynchronize(stream) != hipSuccess) return DSA_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

dsa_status check_indexer(const void* q, const float* q_scale, const void* k, const float* k_scale,
                         const float* weights, const int32_t* ks, const int32_t* ke,
                         const float* logits, int64_t B, int64_t M, int64_t N, int32_t H,
                         int32_t D) {
  if (!q || !k || !k_scale || !weights || !ks || !ke || !logits) return DSA_ERR_INVALID_VALUE;
  if (B <= 0 || M <= 0 || N <= 0 || H <= 0 || D <= 0) return DSA_ERR_INVALID_VALUE;
  if (B * M > kMaxI32 || N > kMaxI32 || B > kMaxI32 / N) return DSA_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(k_scale, 4) || !aligned(weights, 4) ||
      !aligned(ks, 4) || !aligned(ke, 4) || !aligned(logits, 4) ||
      (q_scale && !aligned(q_scale, 4)))
    return DSA_ERR_INVALID_VALUE;
  if (!dsa::indexer_supported(H, D)) return DSA_ERR_NOT_SUPPORTED;
  return DSA_OK;
}

dsa_status check_topk(const float* logits, const int32_t* ks, const int32_t* ke,
                      const int32_t* out, int64_t B, int64_t M, int64_t N, int32_t K) {
  if (!logits || !ks || !ke || !out) return DSA_ERR_INVALID_VALUE;
  if (B <= 0 || M <= 0 || N <= 0 || K <= 0) return DSA_ERR_INVALID_VALUE;
  if (B * M > kMaxI32 || N > kMaxI32) return DSA_ERR_INVALID_VALUE;
  if (!aligned(logits, 4) || !aligned(ks, 4) || !aligned(ke, 4) || !aligned(out, 4))
    return DSA_ERR_INVALID_VALUE;
  if (K > 4096) return DSA_ERR_NOT_SUPPORTED;
  return DSA_OK;
}

dsa_status check_attn(const void* q, const void* kv, int kv_dtype, const float* kv_scale,
                      const float* sink, const int32_t* idx, const void* o, int64_t B, int64_t M,
                      int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K) {
  if (!q || !kv || !idx || !o) return DSA_ERR_INVALID_VALUE;
  if (kv_dtype != DSA_KV_BF16 && kv_dtype != DSA_KV_FP8_E4M3FN) return DSA_ERR_INVALID_VALUE;
  const bool fp8 = kv_dtype == DSA_KV_FP8_E4M3FN;
  if (fp8 != (kv_scale != nullptr)) return DSA_ERR_INVALID_VALUE;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Dqk <= 0 || Dv <= 0 || K <= 0 || Dv > Dqk)
    return DSA_ERR_INVALID_VALUE;
  if (B * M > kMaxI32 || N > kMaxI32 || B > kMaxI32 / N) return DSA_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(o, 16) || !aligned(idx, 4) ||
      (kv_scale && !aligned(kv_scale, 4)) || (sink && !aligned(sink, 4)))
    return DSA_ERR_INVALID_VALUE;
  if (K > 4096 || !dsa::attn_supported(Hq, Dqk, Dv, fp8)) return DSA_ERR_NOT_SUPPORTED;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_logits(const void* q, const float* q_scale, const void* k,
                              const float* k_scale, const float* weights, const int32_t* ks,
                              const int32_t* ke, float* logits, int64_t B, int64_t M, int64_t N,
                              int32_t H, int32_t D, void* stream) {
  const dsa_status st = check_indexer(q, q_scale, k, k_scale, weights, ks, ke, logits, B, M, N, H, D);
  if (st != DSA_OK) return st;
  dsa::IndexerArgs a{q, q_scale, k, k_scale, weights, ks, ke, logits, B, M, N, H, D};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_indexer(a, s), s);
}

dsa_status dsa_topk(const float* logits, const int32_t* ks, const int32_t* ke, int32_t* topk_idxs,
                    int64_t B, int64_t M, int64_t N, int32_t K, void* stream) {
  const dsa_status st = check_topk(logits, ks, ke, topk_idxs, B, M, N, K);
  if (st != DSA_OK) return st;
  dsa::TopkArgs a{logits, ks, ke, topk_idxs, B, M, N, K};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_topk(a, s), s);
}

dsa_status dsa_sparse_attn_fwd(const void* q, const void* kv, dsa_kv_dtype kv_dtype,
                               const float* kv_scale, const float* attn_sink,
                               const int32_t* topk_idxs, void* o, int64_t B, int64_t M, int64_t N,
                               int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K, float sm_scale,
                               void* stream) {
  const dsa_status st = check_attn(q, kv, (int)kv_dtype, kv_scale, attn_sink, topk_idxs, o, B, M,
                                   N, Hq, Dqk, Dv, K);
  if (st != DSA_OK) return st;
  dsa::AttnArgs a{q,  kv, kv_dtype == DSA_KV_FP8_E4M3FN, kv_scale, attn_sink, topk_idxs, o, B, M,
                  N,  Hq, Dqk, Dv, K, sm_scale};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_attn(a, s), s);
}

dsa_status dsa_prefill(const dsa_prefill_args* p, void* stream) {
  if (!p) return DSA_ERR_INVALID_VALUE;
  dsa_status st = check_indexer(p->index_q, p->index_q_scale, p->index_k, p->index_k_scale,
                                p->index_weights, p->ks, p->ke, p->logits, p->batch, p->seq_q,
                                p->seq_kv, p->index_heads, p->index_dim);
  if (st == DSA_OK)
    st = check_topk(p->logits, p->ks, p->ke, p->topk_idxs, p->batch, p->seq_q, p->seq_kv, p->topk);
  if (st == DSA_OK)
    st = check_attn(p->q, p->kv, (int)p->kv_dtype, p->kv_scale, p->attn_sink, p->topk_idxs, p->o,
                    p->batch, p->seq_q, p->seq_kv, p->heads, p->dqk, p->dv, p->topk);
  if (st != DSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  dsa::IndexerArgs ia{p->index_q, p->index_q_scale, p->index_k, p->index_k_scale,
                      p->index_weights, p->ks, p->ke, p->logits, p->batch, p->seq_q,
                      p->seq_kv, p->index_heads, p->index_dim};
  st = finish(dsa::launch_indexer(ia, s), s);
  if (st != DSA_OK) return st;
  dsa::TopkArgs ta{p->logits, p->ks, p->ke, p->topk_idxs, p->batch, p->seq_q, p->seq_kv, p->topk};
  st = finish(dsa::launch_topk(ta, s), s);
  if (st != DSA_OK) return st;
  dsa::AttnArgs aa{p->q,     p->kv,     p->kv_dtype == DSA_KV_FP8_E4M3FN,
                   p->kv_scale, p->attn_sink, p->topk_idxs,
                   p->o,     p->batch,  p->seq_q,
                   p->seq_kv, p->heads, p->dqk,
                   p->dv,    p->topk,   p->sm_scale};
  return finish(dsa::launch_attn(aa, s), s);
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_VALUE: return "DSA_ERR_INVALID_VALUE: invalid argument";
    case DSA_ERR_NOT_SUPPORTED: return "DSA_ERR_NOT_SUPPORTED: no kernel for this shape";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: kernel launch or execution failed";
  }
  return "unknown dsa_status";
}

int dsa_version(void) { return DSA_VERSION; }

}  // extern "C"
