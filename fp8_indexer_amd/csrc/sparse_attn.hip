// sparse_attn.hip -- gathered sparse attention forward with a sink, gfx950.
//
// Semantics (DeepSeek V4.1 atlas page, sparse_attn_kernel / sparse_attn):
// for each query token, gather the KV rows named by its top-k indices, run an
// online softmax over q.kv * sm_scale, add exp(attn_sink[h]) to the
// denominator only, mask -1 indices, and give zero output when no index is
// valid.  The value is the first Dv columns of the same latent row.
//
// Design (MI355X-first):
//  * One workgroup per query token; wave w owns 16 heads.  Its q rows live in
//    VGPRs for the whole token as MFMA B-fragments.
//  * The product is formed transposed, S^T[j, h] = kv_j . q_h, on
//    v_mfma_f32_16x16x32_bf16.  In the C layout each lane then holds one head
//    and 8 consecutive gathered rows, which is exactly the B-fragment layout
//    of the next product O^T[c, h] += V^T[c, j] P^T[j, h]: P never leaves
//    registers, and the per-head rescale by exp2(m_old - m_new) is a
//    lane-local multiply of the fp32 O accumulators.
//  * KV rows are gathered 32 at a time straight from HBM/L2 into a row-major
//    LDS tile with gfx950's 16-byte direct-to-LDS loads (global_load_lds_
//    dwordx4; one row is 1152 contiguous bytes, so each wavefront instruction
//    moves 1 KiB of whole rows).  The tile is double buffered: the loads of
//    tile i+1 are in flight while tile i is computed, no VGPRs are spent on
//    staging, and there is one barrier per tile.  QK^T reads its A operand
//    from the tile with 16-byte LDS loads; PV needs V with the gathered-row axis innermost, and
//    gets it from the same row-major tile through gfx950's transposing LDS
//    load (ds_read_b64_tr_b16: each lane of a 16-lane group receives one
//    column of a 4x16 block).  This is the AMD answer to the K-major-V
//    problem the TileLang FP8 page describes: no second copy and no
//    transpose pass.
//  * Softmax in base 2 with sm_scale*log2(e) folded into one multiply,
//    running max initialised to -1e30 (finite), fp32 state.
//  * Tiles whose 32 indices are all invalid are skipped entirely.
//  * FP8 KV (e4m3fn + per-row fp32 scale): rows are prefetched into VGPRs
//    one tile ahead and widened to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8)
//    on the way into LDS; the row scale multiplies the score of that row and
//    its probability before the bf16 cast.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kBI = 32;      // gathered rows per tile
constexpr int kKVPad = 8;    // row padding (elements): odd 16-byte stride
constexpr int kMaxK = 4096;  // largest supported top-k
constexpr float kLog2e = 1.4426950408889634f;

template <int DQK, int DV, bool FP8, int NW>
struct AttnCfg {
  static_assert(DQK % 32 == 0 && DV % 16 == 0 && DV <= DQK, "dims");
  static constexpr int THREADS = NW * kWave;
  static constexpr int RS = DQK + kKVPad;          // LDS row stride (elements)
  static constexpr int TILE = kBI * RS;            // LDS tile (elements)
  static constexpr int UPR = RS / 8;               // 16-byte units per padded row
  static constexpr int UNITS = kBI * UPR;
  static constexpr int DMA_INSTR = (UNITS + kWave - 1) / kWave;
  static constexpr int CPR = DQK / 8;              // FP8 path: 8-code chunks per row
  static constexpr int CHUNKS = kBI * CPR;
  static constexpr int CPT = (CHUNKS + THREADS - 1) / THREADS;
  static constexpr int QC = DQK / 32;              // 32-deep k-steps of QK
  static constexpr int OT = DV / 16;               // 16-wide output tiles
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read: within each 16-lane group, lane i supplies the
// address of 4 consecutive bf16 of row i/4 (columns 4*(i%4)..+3) of a 4x16
// block and receives column i (rows 0..3) of that block.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), lgkm/exp untouched
}

template <int DQK, int DV, bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv_, const float* __restrict__ kv_scale,
    const float* __restrict__ sink, const int* __restrict__ idx, uint16_t* __restrict__ o, int M,
    int N, int Hq, int K, float scale_log2) {
  using C = AttnCfg<DQK, DV, FP8, NW>;
  __shared__ __align__(16) uint16_t sKV0[C::TILE];
  __shared__ __align__(16) uint16_t sKV1[C::TILE];
  __shared__ int sIdx[kMaxK];           // sanitised indices (-1 = invalid), padded
  __shared__ int sFirst[kMaxK / kBI];   // a valid index of each tile, or -1
  __shared__ int sList[kMaxK / kBI];    // tiles with a valid index, ascending
  __shared__ float sSc0[kBI], sSc1[kBI];  // FP8: per-row scales of a tile
  __shared__ int sNvt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int rtok = (int)(gridDim.x - 1 - blockIdx.x);  // (b, t) row, latest first
  const int b = rtok / M;
  const int ntiles = (K + kBI - 1) / kBI;

  // ---- indices -> LDS, list of tiles holding a valid index -----------------
  {
    const int* ridx = idx + (size_t)rtok * K;
    for (int p = tid; p < ntiles * kBI; p += C::THREADS) {
      const int v = p < K ? ridx[p] : -1;
      sIdx[p] = (v >= 0 && v < N) ? v : -1;
    }
  }
  __syncthreads();
  for (int t = tid; t < ntiles; t += C::THREADS) {
    int first = -1;
    for (int r = kBI - 1; r >= 0; --r) {
      const int v = sIdx[t * kBI + r];
      first = v >= 0 ? v : first;
    }
    sFirst[t] = first;
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += kWave) {
      const int t = t0 + lane;
      const bool f = t < ntiles && sFirst[t] >= 0;
      const uint64_t m = __ballot(f);
      if (f) sList[base + __popcll(m & lt)] = t;
      base += __popcll(m);
    }
    if (lane == 0) sNvt = base;
  }

  // ---- q fragments for this wave's 16 heads --------------------------------
  const int h = wave * 16 + col;
  bf16x8 qf[C::QC];
  {
    const uint16_t* qrow = q + ((size_t)rtok * Hq + h) * DQK;
#pragma unroll
    for (int c = 0; c < C::QC; ++c)
      qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 32 + g * 8);
  }
  f32x4 oacc[C::OT];
#pragma unroll
  for (int t = 0; t < C::OT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, lsum = 0.f;
  __syncthreads();
  const int nvt = sNvt;

  // ---- tile staging ---------------------------------------------------------
  // bf16: direct-to-LDS gather.  Rows of invalid slots load a valid row of the
  // same tile instead (finite data; their scores are masked to -inf).
  auto dma = [&](uint16_t* dst, int tile) {
    const uint16_t* kvb = static_cast<const uint16_t*>(kv_) + (size_t)b * N * DQK;
    const int first = sFirst[tile];
    for (int k = wave; k < C::DMA_INSTR; k += NW) {
      const int u = k * kWave + lane;
      const int r = u / C::UPR, c = u % C::UPR;
      if (u < C::UNITS && c < C::UPR - 1) {
        int row = sIdx[tile * kBI + r];
        row = row >= 0 ? row : first;
        __builtin_amdgcn_global_load_lds(kvb + (size_t)row * DQK + c * 8,
                                         (lds_void*)(dst + k * kWave * 8), 16, 0, 0);
      }
    }
  };
  // FP8: register prefetch one tile ahead, widened to bf16 when stored.
  typedef typename std::conditional<FP8, uint2, int>::type chunk_t;
  constexpr int CPT = FP8 ? C::CPT : 1;
  chunk_t pre[CPT];
  float pscale = 0.f;
  auto gload = [&](int tile) {
    if constexpr (FP8) {
      const uint8_t* kvb = static_cast<const uint8_t*>(kv_) + (size_t)b * N * DQK;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int ch = tid + j * C::THREADS;
        uint2 v = {0u, 0u};
        if (ch < C::CHUNKS) {
          const int row = sIdx[tile * kBI + ch / C::CPR];
          if (row >= 0)
            v = *reinterpret_cast<const uint2*>(kvb + (size_t)row * DQK + (ch % C::CPR) * 8);
        }
        pre[j] = v;
      }
      if (tid < kBI) {
        const int row = sIdx[tile * kBI + tid];
        pscale = row >= 0 ? kv_scale[(size_t)b * N + row] : 0.f;
      }
    }
  };
  auto lstore = [&](uint16_t* dst, float* dsc) {
    if constexpr (FP8) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int ch = tid + j * C::THREADS;
        if (ch < C::CHUNKS) {
          const uint2 raw = pre[j];
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true);
          *reinterpret_cast<i32x4*>(dst + (ch / C::CPR) * C::RS + (ch % C::CPR) * 8) =
              i32x4{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1),
                    __builtin_bit_cast(int, p2), __builtin_bit_cast(int, p3)};
        }
      }
      if (tid < kBI) dsc[tid] = pscale;
    }
  };

  // ---- one tile: S^T = KV.Q^T, online softmax, O^T += V^T.P^T ----------------
  auto compute = [&](const uint16_t* sK, const float* sSc, int tile) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      // MFMA tile tau, A-row r -> gathered row 8*(r/4) + 4*tau + r%4, so that
      // lane (h, g) ends up with rows 8g .. 8g+7.
      const uint16_t* a0 = sK + (8 * (col >> 2) + (col & 3)) * C::RS + g * 8;
      const uint16_t* a1 = a0 + 4 * C::RS;
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(a0 + c * 32);
        const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(a1 + c * 32);
        s0 = mfma_bf16_16x16x32(x0, qf[c], s0);
        s1 = mfma_bf16_16x16x32(x1, qf[c], s1);
      }
    }
    const int* ti = sIdx + tile * kBI + 8 * g;
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float raw = i < 4 ? s0[i] : s1[i - 4];
      float x = raw * scale_log2;
      if constexpr (FP8) x *= sSc[8 * g + i];
      x = ti[i] >= 0 ? x : -INFINITY;
      sv[i] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, wave_xor(tmax, 16));
    tmax = fmaxf(tmax, wave_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float alpha = exp2f(m - mnew);
    m = mnew;
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float p0 = exp2f(sv[i] - m), p1 = exp2f(sv[i + 1] - m);
      psum += p0 + p1;
      if constexpr (FP8) {
        p0 *= sSc[8 * g + i];
        p1 *= sSc[8 * g + i + 1];
      }
      pk[i >> 1] = pack_bf16x2(p0, p1);
    }
    lsum = lsum * alpha + psum;
    const bf16x8 pb =
        __builtin_bit_cast(bf16x8, i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
    // A operand: lane (c = 16t + col, g) needs V[8g .. 8g+7][c]: two
    // transposing reads of the 4x16 blocks at rows 8g and 8g+4.
    const uint16_t* vb = sK + (8 * g + (col >> 2)) * C::RS + 4 * (col & 3);
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
      const i16x4 lo = lds_read_tr16(vb + t * 16);
      const i16x4 hi = lds_read_tr16(vb + 4 * C::RS + t * 16);
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      oacc[t] = mfma_bf16_16x16x32(va, pb, oacc[t] * alpha);
    }
  };

  auto step = [&](int it, const uint16_t* cur, const float* curS, uint16_t* nxt, float* nxtS) {
    if constexpr (!FP8) wait_vmem_all();  // this wave's loads of tile `it`
    __syncthreads();  // tile `it` complete; everyone is done with `nxt`
    if (it + 1 < nvt) {
      if constexpr (FP8) {
        lstore(nxt, nxtS);
        if (it + 2 < nvt) gload(sList[it + 2]);
      } else {
        dma(nxt, sList[it + 1]);
      }
    }
    compute(cur, curS, sList[it]);
  };

  if (nvt > 0) {
    if constexpr (FP8) {
      gload(sList[0]);
      lstore(sKV0, sSc0);
      if (nvt > 1) gload(sList[1]);
    } else {
      dma(sKV0, sList[0]);
    }
  }
#pragma unroll 1
  for (int it = 0; it < nvt; it += 2) {
    step(it, sKV0, sSc0, sKV1, sSc1);
    if (it + 1 < nvt) step(it + 1, sKV1, sSc1, sKV0, sSc0);
  }

  // ---- sink, normalise, store ------------------------------------------------
  float l = lsum;
  l += wave_xor(l, 16);
  l += wave_xor(l, 32);
  if (sink) l += exp2f(sink[h] * kLog2e - m);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = o + ((size_t)rtok * Hq + h) * DV + g * 4;
#pragma unroll
  for (int t = 0; t < C::OT; ++t) {
    const f32x4 v = oacc[t] * inv;
    uint2 pk2;
    pk2.x = pack_bf16x2(v[0], v[1]);
    pk2.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(orow + t * 16) = pk2;
  }
}

template <int DQK, int DV, bool FP8, int NW>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using C = AttnCfg<DQK, DV, FP8, NW>;
  const long long rows = a.B * a.M;
  if (rows > 0x7fffffffLL || a.K > kMaxK) return hipErrorInvalidValue;
  const float scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / sqrtf((float)DQK);
  hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, FP8, NW>), dim3((unsigned)rows),
                     dim3(C::THREADS), 0, stream, (const uint16_t*)a.q, a.kv, a.kv_scale,
                     a.attn_sink, a.topk_idxs, (uint16_t*)a.o, (int)a.M, (int)a.N, a.Hq, a.K,
                     (float)((double)scale * 1.4426950408889634));
  return hipGetLastError();
}

}  // namespace

bool attn_supported(int Hq, int Dqk, int Dv, bool fp8) {
  const int nw = Hq / 16;
  if (Hq % 16 != 0 || !(nw == 1 || nw == 2 || nw == 4 || nw == 8)) return false;
  if (Dqk == 64 && Dv == 64) return !fp8;
  if (Dqk == 576 && Dv == 512) return true;
  return false;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int nw = a.Hq / 16;
#define DSA_ATT_NW(DQK, DV, F8)                       \
  switch (nw) {                                       \
    case 1: return launch<DQK, DV, F8, 1>(a, stream); \
    case 2: return launch<DQK, DV, F8, 2>(a, stream); \
    case 4: return launch<DQK, DV, F8, 4>(a, stream); \
    case 8: return launch<DQK, DV, F8, 8>(a, stream); \
    default: return hipErrorInvalidValue;             \
  }
  if (a.Dqk == 64 && a.Dv == 64 && !a.fp8) { DSA_ATT_NW(64, 64, false) }
  if (a.Dqk == 576 && a.Dv == 512 && !a.fp8) { DSA_ATT_NW(576, 512, false) }
  if (a.Dqk == 576 && a.Dv == 512 && a.fp8) { DSA_ATT_NW(576, 512, true) }
#undef DSA_ATT_NW
  return hipErrorInvalidValue;
}

}  // namespace dsa
