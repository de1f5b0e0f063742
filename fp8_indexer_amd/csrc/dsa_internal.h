// dsa_internal.h -- host-side launch interfaces between the C ABI (api.hip)
// and the kernel translation units.  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct IndexerArgs {
  const void* q;
  const float* q_scale;
  const void* k;
  const float* k_scale;
  const float* w;
  const int32_t* ks;
  const int32_t* ke;
  float* logits;
  int64_t B, M, N;
  int H, D;
};

struct TopkArgs {
  const float* logits;
  const int32_t* ks;
  const int32_t* ke;
  int32_t* topk_idxs;
  int64_t B, M, N;
  int K;
};

struct AttnArgs {
  const void* q;
  const void* kv;
  bool fp8;
  const float* kv_scale;
  const float* attn_sink;
  const int32_t* topk_idxs;
  void* o;
  int64_t B, M, N;
  int Hq, Dqk, Dv, K;
  float sm_scale;
};

bool indexer_supported(int H, int D);
bool attn_supported(int Hq, int Dqk, int Dv, bool fp8);

// Stream-ordered temporaries (hipMallocAsync) come from the current device's
// default memory pool; keep freed blocks in the pool between calls.
inline void keep_pool_memory() {
  static bool done[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || done[dev]) return;
  hipMemPool_t pool;
  if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
    uint64_t thr = UINT64_MAX;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
  }
  (void)hipGetLastError();
  done[dev] = true;
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace dsa
