// dsa_internal.h -- host-side launch interfaces between the C ABI (api.hip)
// and the kernel translation units.  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
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

// Caller-provided device scratch (may be NULL / 0 bytes: the calls then take
// their paths that need none).
struct Workspace {
  void* ptr;
  size_t bytes;
};

struct AttnBwdArgs {
  const void* q;
  const void* kv;
  const float* attn_sink;
  const int32_t* topk_idxs;
  const void* o;
  const void* dO;
  float* dq;
  float* dkv;
  float* dsink;
  int64_t B, M, N;
  int Hq, Dqk, Dv, K;
  float sm_scale;
};

// Full-FP8 attention: q and kv hold e4m3fn codes.
struct AttnFp8Args {
  const void* q;
  const float* q_scale;   // [B, M, Hq] or NULL (= 1)
  const void* kv;
  const float* kv_scale;  // [B, N]
  const float* attn_sink;
  const int32_t* topk_idxs;
  void* o;
  int64_t B, M, N;
  int Hq, Dqk, Dv, K;
  float sm_scale;
};

bool indexer_supported(int H, int D);
bool attn_bwd_supported(int Hq, int Dqk, int Dv);

// Fewest query tokens per batch entry for which the indexer uses its
// prefill layout (fewer: the key-parallel decode layout, whose head sums
// are added in another order).
inline int64_t indexer_prefill_min_tokens(int H) { return 128 / H + 1; }
bool attn_supported(int Hq, int Dqk, int Dv, bool fp8);

// Compute units of the current device (cached per device, thread-safe).
int device_cus();

// Scratch bytes the fastest path of a call needs (0: none).  The launch
// functions take that path only when the workspace holds at least as many
// bytes, and a path without scratch otherwise.
size_t topk_workspace_bytes(const TopkArgs& a);
size_t attn_workspace_bytes(const AttnArgs& a);

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, Workspace ws, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, Workspace ws, hipStream_t stream);
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);

bool attn_fp8_supported(int Hq, int Dqk, int Dv);
size_t attn_fp8_workspace_bytes(const AttnFp8Args& a);
hipError_t launch_attn_fp8(const AttnFp8Args& a, Workspace ws, hipStream_t stream);

// Merge of split partial results (bf16 O_s / l_s [rows, S, Hq, Dv], then
// fp32 (m_s, l_s) [rows, S, Hq], m in log2 units) into bf16 o.
hipError_t launch_attn_merge(const uint16_t* wso, const float2* wsml, const float* sink,
                             uint16_t* o, long long rows, int Hq, int Dv, int S,
                             hipStream_t stream);

}  // namespace dsa
