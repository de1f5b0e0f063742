// api.hip -- the C ABI of libdsa (declared in include/dsa.h): host-side
// argument validation, kernel dispatch, launch error mapping.
#include <cstdlib>
#include <cstring>
#include <mutex>

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

dsa_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr) return DSA_OK;  // paths without scratch
  if (!aligned(ws, 16)) return DSA_ERR_INVALID_VALUE;
  return ws_bytes < need ? DSA_ERR_WORKSPACE : DSA_OK;
}

dsa::AttnArgs attn_args(const void* q, const void* kv, int kv_dtype, const float* kv_scale,
                        const float* sink, const int32_t* idx, void* o, int64_t B, int64_t M,
                        int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K,
                        float sm_scale) {
  return dsa::AttnArgs{q, kv, kv_dtype == DSA_KV_FP8_E4M3FN, kv_scale, sink, idx, o, B, M,
                       N, Hq, Dqk, Dv, K, sm_scale};
}

constexpr int kMaxDevices = 64;

}  // namespace

namespace dsa {

int device_cus() {
  static std::mutex mu;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  auto query = [dev] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    return v;
  };
  if (dev < 0 || dev >= kMaxDevices) return query();
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) cache[dev] = query();
  return cache[dev];
}

}  // namespace dsa

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

dsa_status dsa_topk_workspace_size(int64_t B, int64_t M, int64_t N, int32_t K, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_VALUE;
  const int32_t one = 0;
  const dsa_status st = check_topk(reinterpret_cast<const float*>(&one), &one, &one, &one, B, M,
                                   N, K);
  if (st != DSA_OK) return st;
  *bytes = dsa::topk_workspace_bytes(dsa::TopkArgs{nullptr, nullptr, nullptr, nullptr, B, M, N, K});
  return DSA_OK;
}

dsa_status dsa_topk(const float* logits, const int32_t* ks, const int32_t* ke, int32_t* topk_idxs,
                    int64_t B, int64_t M, int64_t N, int32_t K, void* workspace,
                    size_t workspace_bytes, void* stream) {
  dsa_status st = check_topk(logits, ks, ke, topk_idxs, B, M, N, K);
  if (st != DSA_OK) return st;
  dsa::TopkArgs a{logits, ks, ke, topk_idxs, B, M, N, K};
  st = check_workspace(workspace, workspace_bytes, dsa::topk_workspace_bytes(a));
  if (st != DSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_topk(a, dsa::Workspace{workspace, workspace_bytes}, s), s);
}

dsa_status dsa_sparse_attn_workspace_size(int64_t B, int64_t M, int32_t Hq, int32_t Dqk,
                                          int32_t Dv, int32_t K, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_VALUE;
  alignas(16) static const int64_t dummy[2] = {0, 0};  // stand-in pointers: never dereferenced
  const dsa_status st = check_attn(dummy, dummy, DSA_KV_BF16, nullptr, nullptr,
                                   reinterpret_cast<const int32_t*>(dummy), dummy, B, M, 1, Hq,
                                   Dqk, Dv, K);
  if (st != DSA_OK) return st;
  *bytes = dsa::attn_workspace_bytes(
      attn_args(nullptr, nullptr, DSA_KV_BF16, nullptr, nullptr, nullptr, nullptr, B, M, 1, Hq,
                Dqk, Dv, K, 0.f));
  return DSA_OK;
}

dsa_status dsa_sparse_attn_fwd(const void* q, const void* kv, dsa_kv_dtype kv_dtype,
                               const float* kv_scale, const float* attn_sink,
                               const int32_t* topk_idxs, void* o, int64_t B, int64_t M, int64_t N,
                               int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K, float sm_scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_attn(q, kv, (int)kv_dtype, kv_scale, attn_sink, topk_idxs, o, B, M, N,
                             Hq, Dqk, Dv, K);
  if (st != DSA_OK) return st;
  const dsa::AttnArgs a = attn_args(q, kv, (int)kv_dtype, kv_scale, attn_sink, topk_idxs, o, B,
                                    M, N, Hq, Dqk, Dv, K, sm_scale);
  st = check_workspace(workspace, workspace_bytes, dsa::attn_workspace_bytes(a));
  if (st != DSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_attn(a, dsa::Workspace{workspace, workspace_bytes}, s), s);
}

}  // extern "C"

namespace {

dsa_status check_attn_fp8(const void* q, const float* q_scale, const void* kv,
                          const float* kv_scale, const float* sink, const int32_t* idx,
                          const void* o, int64_t B, int64_t M, int64_t N, int32_t Hq,
                          int32_t Dqk, int32_t Dv, int32_t K) {
  if (!q || !kv || !kv_scale || !idx || !o) return DSA_ERR_INVALID_VALUE;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Dqk <= 0 || Dv <= 0 || K <= 0 || Dv > Dqk)
    return DSA_ERR_INVALID_VALUE;
  if (B * M > kMaxI32 || N > kMaxI32 || B > kMaxI32 / N) return DSA_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(o, 16) || !aligned(idx, 4) ||
      !aligned(kv_scale, 4) || (q_scale && !aligned(q_scale, 4)) || (sink && !aligned(sink, 4)))
    return DSA_ERR_INVALID_VALUE;
  if (K > 4096 || !dsa::attn_fp8_supported(Hq, Dqk, Dv)) return DSA_ERR_NOT_SUPPORTED;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_attn_fp8_workspace_size(int64_t B, int64_t M, int32_t Hq, int32_t Dqk,
                                              int32_t Dv, int32_t K, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_VALUE;
  alignas(16) static const int64_t dummy[2] = {0, 0};  // stand-in pointers: never dereferenced
  const float* fdummy = reinterpret_cast<const float*>(dummy);
  const dsa_status st = check_attn_fp8(dummy, nullptr, dummy, fdummy, nullptr,
                                       reinterpret_cast<const int32_t*>(dummy), dummy, B, M, 1,
                                       Hq, Dqk, Dv, K);
  if (st != DSA_OK) return st;
  const dsa::AttnFp8Args a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           B, M, 1, Hq, Dqk, Dv, K, 0.f};
  *bytes = dsa::attn_fp8_workspace_bytes(a);
  return DSA_OK;
}

dsa_status dsa_sparse_attn_fwd_fp8(const void* q, const float* q_scale, const void* kv,
                                   const float* kv_scale, const float* attn_sink,
                                   const int32_t* topk_idxs, void* o, int64_t B, int64_t M,
                                   int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K,
                                   float sm_scale, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  dsa_status st = check_attn_fp8(q, q_scale, kv, kv_scale, attn_sink, topk_idxs, o, B, M, N, Hq,
                                 Dqk, Dv, K);
  if (st != DSA_OK) return st;
  const dsa::AttnFp8Args a{q, q_scale, kv, kv_scale, attn_sink, topk_idxs, o,
                           B, M, N, Hq, Dqk, Dv, K, sm_scale};
  st = check_workspace(workspace, workspace_bytes, dsa::attn_fp8_workspace_bytes(a));
  if (st != DSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_attn_fp8(a, dsa::Workspace{workspace, workspace_bytes}, s), s);
}

}  // extern "C"

namespace {

// ---- indexer + top-k in slabs of rows -------------------------------------
// The [B, M, N] logits never exist: rows are scored and selected in slabs
// whose logits live in the workspace.  A slab is a group of whole batch
// entries (M <= slab rows) or a run of tokens of one batch entry; a tail run
// too short for the indexer's prefill layout joins the previous run, so
// every token is scored with the same layout (same summation order) as by
// one dsa_indexer_logits call over all rows, and the selection, exact by
// definition, is the same as dsa_topk's on those logits.
constexpr int64_t kDefaultSlabRows = 2048;

struct Slab {
  int64_t b0, nb;  // batch entries [b0, b0 + nb)
  int64_t t0, nt;  // tokens [t0, t0 + nt) of each
};

// Calls f(slab) for every slab, in row order.
template <class F>
void for_each_slab(int64_t B, int64_t M, int H, int64_t slab_rows, F&& f) {
  if (M <= slab_rows) {
    const int64_t per = slab_rows / M;
    for (int64_t b0 = 0; b0 < B; b0 += per) f(Slab{b0, per < B - b0 ? per : B - b0, 0, M});
    return;
  }
  const int64_t tmin = dsa::indexer_prefill_min_tokens(H);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t0 = 0; t0 < M;) {
      int64_t nt = M - t0 < slab_rows ? M - t0 : slab_rows;
      if (M - (t0 + nt) > 0 && M - (t0 + nt) < tmin) nt = M - t0;  // short tail joins
      f(Slab{b, 1, t0, nt});
      t0 += nt;
    }
}

struct SlabPlan {
  size_t logits_bytes;  // the largest slab's logits, 256-byte aligned
  size_t topk_bytes;    // the largest slab's top-k scratch
  size_t bytes() const { return logits_bytes + topk_bytes; }
};

int64_t slab_rows_or_default(int64_t slab_rows) {
  return slab_rows > 0 ? slab_rows : kDefaultSlabRows;
}

SlabPlan plan_slabs(int64_t B, int64_t M, int64_t N, int H, int K, int64_t slab_rows) {
  SlabPlan plan{0, 0};
  for_each_slab(B, M, H, slab_rows, [&](const Slab& sl) {
    const size_t lb = ((size_t)(sl.nb * sl.nt) * (size_t)N * sizeof(float) + 255) & ~(size_t)255;
    if (lb > plan.logits_bytes) plan.logits_bytes = lb;
    const size_t tb = dsa::topk_workspace_bytes(
        dsa::TopkArgs{nullptr, nullptr, nullptr, nullptr, sl.nb, sl.nt, N, K});
    if (tb > plan.topk_bytes) plan.topk_bytes = tb;
  });
  return plan;
}

// Every slab: indexer into the workspace's logits, top-k from it.
dsa_status run_indexer_topk(const dsa::IndexerArgs& ia, int32_t* topk_idxs, int K,
                            int64_t slab_rows, const SlabPlan& plan, dsa::Workspace ws,
                            hipStream_t s) {
  float* slab_logits = static_cast<float*>(ws.ptr);
  const dsa::Workspace tws{static_cast<char*>(ws.ptr) + plan.logits_bytes,
                           ws.bytes - plan.logits_bytes};
  const int64_t M = ia.M, N = ia.N;
  const int H = ia.H, D = ia.D;
  dsa_status st = DSA_OK;
  for_each_slab(ia.B, M, H, slab_rows, [&](const Slab& sl) {
    if (st != DSA_OK) return;
    const int64_t r0 = sl.b0 * M + sl.t0;  // first row of the slab
    dsa::IndexerArgs a = ia;
    a.q = static_cast<const uint8_t*>(ia.q) + r0 * H * D;
    a.q_scale = ia.q_scale ? ia.q_scale + r0 * H : nullptr;
    a.k = static_cast<const uint8_t*>(ia.k) + sl.b0 * N * D;
    a.k_scale = ia.k_scale + sl.b0 * N;
    a.w = ia.w + r0 * H;
    a.ks = ia.ks + r0;
    a.ke = ia.ke + r0;
    a.logits = slab_logits;
    a.B = sl.nb;
    a.M = sl.nt;
    st = finish(dsa::launch_indexer(a, s), s);
    if (st != DSA_OK) return;
    const dsa::TopkArgs t{slab_logits, a.ks, a.ke, topk_idxs + r0 * K, sl.nb, sl.nt, N, K};
    st = finish(dsa::launch_topk(t, tws, s), s);
  });
  return st;
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_topk_workspace_size(int64_t B, int64_t M, int64_t N, int32_t H, int32_t D,
                                           int32_t K, int64_t slab_rows, size_t* bytes) {
  if (!bytes || slab_rows < 0) return DSA_ERR_INVALID_VALUE;
  alignas(16) static const int64_t dummy[2] = {0, 0};  // stand-in pointers: never dereferenced
  const float* f = reinterpret_cast<const float*>(dummy);
  const int32_t* i = reinterpret_cast<const int32_t*>(dummy);
  dsa_status st = check_indexer(dummy, nullptr, dummy, f, f, i, i, f, B, M, N, H, D);
  if (st == DSA_OK) st = check_topk(f, i, i, i, B, M, N, K);
  if (st != DSA_OK) return st;
  *bytes = plan_slabs(B, M, N, H, K, slab_rows_or_default(slab_rows)).bytes();
  return DSA_OK;
}

dsa_status dsa_indexer_topk(const void* q, const float* q_scale, const void* k,
                            const float* k_scale, const float* weights, const int32_t* ks,
                            const int32_t* ke, int32_t* topk_idxs, int64_t B, int64_t M,
                            int64_t N, int32_t H, int32_t D, int32_t K, int64_t slab_rows,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (slab_rows < 0) return DSA_ERR_INVALID_VALUE;
  const float* dummy = k_scale;  // any non-NULL aligned pointer for the logits check
  dsa_status st = check_indexer(q, q_scale, k, k_scale, weights, ks, ke, dummy, B, M, N, H, D);
  if (st == DSA_OK) st = check_topk(dummy, ks, ke, topk_idxs, B, M, N, K);
  if (st != DSA_OK) return st;
  const int64_t rows = slab_rows_or_default(slab_rows);
  const SlabPlan plan = plan_slabs(B, M, N, H, K, rows);
  if (workspace == nullptr || workspace_bytes < plan.bytes()) return DSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSA_ERR_INVALID_VALUE;
  const dsa::IndexerArgs ia{q, q_scale, k, k_scale, weights, ks, ke, nullptr, B, M, N, H, D};
  return run_indexer_topk(ia, topk_idxs, K, rows, plan,
                          dsa::Workspace{workspace, workspace_bytes},
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

dsa_status check_prefill(const dsa_prefill_args* p) {
  if (!p) return DSA_ERR_INVALID_VALUE;
  // logits == NULL selects the slab mode: any non-NULL stand-in passes the
  // pointer checks below (it is never used)
  const float* lg = p->logits ? p->logits : p->index_k_scale;
  dsa_status st = check_indexer(p->index_q, p->index_q_scale, p->index_k, p->index_k_scale,
                                p->index_weights, p->ks, p->ke, lg, p->batch, p->seq_q,
                                p->seq_kv, p->index_heads, p->index_dim);
  if (st == DSA_OK)
    st = check_topk(lg, p->ks, p->ke, p->topk_idxs, p->batch, p->seq_q, p->seq_kv, p->topk);
  if (st == DSA_OK)
    st = check_attn(p->q, p->kv, (int)p->kv_dtype, p->kv_scale, p->attn_sink, p->topk_idxs, p->o,
                    p->batch, p->seq_q, p->seq_kv, p->heads, p->dqk, p->dv, p->topk);
  return st;
}

dsa::TopkArgs prefill_topk_args(const dsa_prefill_args* p) {
  return dsa::TopkArgs{p->logits, p->ks, p->ke, p->topk_idxs, p->batch, p->seq_q, p->seq_kv,
                       p->topk};
}

dsa::AttnArgs prefill_attn_args(const dsa_prefill_args* p) {
  return attn_args(p->q, p->kv, (int)p->kv_dtype, p->kv_scale, p->attn_sink, p->topk_idxs, p->o,
                   p->batch, p->seq_q, p->seq_kv, p->heads, p->dqk, p->dv, p->topk, p->sm_scale);
}

SlabPlan prefill_slab_plan(const dsa_prefill_args* p) {
  return plan_slabs(p->batch, p->seq_q, p->seq_kv, p->index_heads, p->topk, kDefaultSlabRows);
}

// The stages run one after the other on the stream, so they share one
// workspace: the larger of the top-k's (or, without a logits buffer, the
// slabs') and the attention's needs.
size_t prefill_workspace_bytes(const dsa_prefill_args* p) {
  const size_t a = p->logits ? dsa::topk_workspace_bytes(prefill_topk_args(p))
                             : prefill_slab_plan(p).bytes();
  const size_t b = dsa::attn_workspace_bytes(prefill_attn_args(p));
  return a > b ? a : b;
}

// The three stages on one stream with the given scratch.
dsa_status run_prefill(const dsa_prefill_args* p, dsa::Workspace ws, hipStream_t s) {
  dsa::IndexerArgs ia{p->index_q, p->index_q_scale, p->index_k, p->index_k_scale,
                      p->index_weights, p->ks, p->ke, p->logits, p->batch, p->seq_q,
                      p->seq_kv, p->index_heads, p->index_dim};
  dsa_status st;
  if (p->logits) {
    st = finish(dsa::launch_indexer(ia, s), s);
    if (st != DSA_OK) return st;
    st = finish(dsa::launch_topk(prefill_topk_args(p), ws, s), s);
  } else {
    st = run_indexer_topk(ia, p->topk_idxs, p->topk, kDefaultSlabRows, prefill_slab_plan(p), ws,
                          s);
  }
  if (st != DSA_OK) return st;
  return finish(dsa::launch_attn(prefill_attn_args(p), ws, s), s);
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_attn_bwd(const void* q, const void* kv, const float* attn_sink,
                               const int32_t* topk_idxs, const void* o, const void* dO,
                               float* dq, float* dkv, float* dsink, int64_t B, int64_t M,
                               int64_t N, int32_t Hq, int32_t Dqk, int32_t Dv, int32_t K,
                               float sm_scale, void* stream) {
  if (!q || !kv || !topk_idxs || !o || !dO || !dq || !dkv) return DSA_ERR_INVALID_VALUE;
  if ((attn_sink == nullptr) != (dsink == nullptr)) return DSA_ERR_INVALID_VALUE;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Dqk <= 0 || Dv <= 0 || K <= 0 || Dv > Dqk)
    return DSA_ERR_INVALID_VALUE;
  if (B * M > kMaxI32 || N > kMaxI32 || B > kMaxI32 / N) return DSA_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dkv, 16) || !aligned(topk_idxs, 4) ||
      (attn_sink && !aligned(attn_sink, 4)) || (dsink && !aligned(dsink, 4)))
    return DSA_ERR_INVALID_VALUE;
  if (K > 4096 || !dsa::attn_bwd_supported(Hq, Dqk, Dv)) return DSA_ERR_NOT_SUPPORTED;
  const dsa::AttnBwdArgs a{q, kv, attn_sink, topk_idxs, o, dO, dq, dkv, dsink,
                           B, M, N, Hq, Dqk, Dv, K, sm_scale};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(dsa::launch_attn_bwd(a, s), s);
}

dsa_status dsa_prefill_workspace_size(const dsa_prefill_args* p, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_VALUE;
  const dsa_status st = check_prefill(p);
  if (st != DSA_OK) return st;
  *bytes = prefill_workspace_bytes(p);
  return DSA_OK;
}

dsa_status dsa_prefill(const dsa_prefill_args* p, void* stream) {
  dsa_status st = check_prefill(p);
  if (st != DSA_OK) return st;
  if (!p->logits && (p->workspace == nullptr || !aligned(p->workspace, 256)))
    return p->workspace == nullptr ? DSA_ERR_WORKSPACE : DSA_ERR_INVALID_VALUE;
  st = check_workspace(p->workspace, p->workspace_bytes, prefill_workspace_bytes(p));
  if (st != DSA_OK) return st;
  return run_prefill(p, dsa::Workspace{p->workspace, p->workspace_bytes},
                     static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Scratch of dsa_prefill_noalloc: one copy per device, for the life of the
// process.  In host code `scratch` only names the symbol; the device address
// of each device's copy comes from hipGetSymbolAddress with that device
// current, and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

// Device address of this device's scratch (looked up once per device), or
// nullptr if the lookup failed.
void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

dsa_status dsa_prefill_noalloc(const dsa_prefill_args* p, void* stream) {
  dsa_status st = check_prefill(p);
  if (st != DSA_OK) return st;
  if (p->workspace != nullptr || p->workspace_bytes != 0) return DSA_ERR_INVALID_VALUE;
  const size_t need = prefill_workspace_bytes(p);
  if (need > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return DSA_ERR_LAUNCH;
    }
    ws = scratch_address(dev);
    if (ws == nullptr) return DSA_ERR_LAUNCH;
  }
  return run_prefill(p, dsa::Workspace{ws, need}, static_cast<hipStream_t>(stream));
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_VALUE: return "DSA_ERR_INVALID_VALUE: invalid argument";
    case DSA_ERR_NOT_SUPPORTED: return "DSA_ERR_NOT_SUPPORTED: no kernel for this shape";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: kernel launch or execution failed";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace smaller than the call needs";
    default: break;
  }
  return "unknown dsa_status";
}

int dsa_version(void) { return DSA_VERSION; }

}  // extern "C"
