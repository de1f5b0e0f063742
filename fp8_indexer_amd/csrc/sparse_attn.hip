// sparse_attn.hip -- gathered sparse attention forward with a sink, gfx950.
//
// Semantics (DeepSeek V4.1 atlas page, sparse_attn_kernel / sparse_attn):
// for each query token, gather the KV rows named by its top-k indices, run an
// online softmax over q.kv * sm_scale, add exp(attn_sink[h]) to the
// denominator only, mask -1 indices, and give zero output when no index is
// valid.  The value is the first Dv columns of the same latent row.
//
// Design (MI355X-first):
//  * One workgroup per query token; each wave owns HPW heads (32 at 128
//    heads: 4 waves, one per SIMD).  Its q rows live in registers for the
//    whole token as MFMA B-fragments, and every KV fragment read from LDS
//    feeds HPW/16 MFMAs, so LDS bytes per flop fall with HPW.
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
//  * Softmax in base 2 with sm_scale*log2(e) folded into one multiply, fp32
//    state, max started at -1e30 (finite).  The reference of the exponent is
//    fixed per head at the max of the first tile and never moved: o = O/l
//    is exact for any reference, and p = 2^(s - ref) stays <= 2^16 as long
//    as no later score exceeds the reference by more than 16 (log2 units).
//    If one does, the whole workgroup restarts the token with a max-only
//    pre-pass and a second pass at the exact max.  The fp32 O accumulators
//    are thus only ever touched by MFMA inside the loop (no per-tile rescale),
//    which is what lets 32 heads per wave keep q and O in registers.
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
constexpr int kKVPad = 16;   // row padding (elements): see the LDS layout note
constexpr int kMaxK = 4096;  // largest supported top-k
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRefSlack = 16.f;  // scores may exceed the reference by 2^16

// LDS operand lookahead (k-steps) and scheduling barriers in the MFMA loops
// (tuning knobs).
#ifndef DSA_ATTN_LA
#define DSA_ATTN_LA 2
#endif
#ifndef DSA_ATTN_SB
#define DSA_ATTN_SB 1
#endif
constexpr int kLA = DSA_ATTN_LA;
constexpr bool kSchedBarrier = DSA_ATTN_SB != 0;

template <int DQK, int DV, bool FP8, int NW, int HPW>
struct AttnCfg {
  static_assert(DQK % 32 == 0 && DV % 16 == 0 && DV <= DQK, "dims");
  static_assert(HPW == 16 || HPW == 32, "heads per wave");
  static constexpr int THREADS = NW * kWave;
  static constexpr int HT = HPW / 16;              // 16-head MFMA tiles per wave
  static constexpr int RS = DQK + kKVPad;          // LDS row stride (elements)
  static constexpr int TILE = kBI * RS;            // LDS tile (elements)
  static constexpr int UPR = RS / 8;               // 16-byte units per padded row
  static_assert(UPR % 4 == 2, "row stride must be an odd number of 32-byte pairs");
  static constexpr int UNITS = kBI * UPR;
  static constexpr int DMA_INSTR = (UNITS + kWave - 1) / kWave;
  // DMA instructions issued per tile by waves [0, DMA_HI_WAVES) and the rest
  static constexpr int DMA_HI = (DMA_INSTR + NW - 1) / NW;
  static constexpr int DMA_LO = DMA_INSTR / NW;
  static constexpr int DMA_HI_WAVES = DMA_INSTR - DMA_LO * NW;  // waves issuing DMA_HI
  // LDS tiles: bf16 gathers run two tiles ahead, fp8 stages through VGPRs
  static constexpr int NBUF = FP8 ? 2 : 3;
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

// s_waitcnt vmcnt(n) (6-bit count: bits 3:0 and 15:14), lgkm/exp untouched.
template <int n>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// 16-byte direct-to-LDS load: lane i's 16 bytes at `g` land at LDS byte
// address lds_base + 16*i (lds_base is wave-uniform).  Issued through inline
// asm so that the compiler does not order it against LDS reads of the other
// buffer; completion is awaited explicitly with wait_vmem_all().
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS tile layout.  Row r of a tile starts at r*RS elements; RS is an odd
// number of 32-byte pairs (74 16-byte units for 576-wide rows), so the
// 4x16 blocks read by 32 lanes of a transposing load (8 rows x 32 bytes) fill
// the 64 banks exactly.  Inside a row, 16-byte unit u is stored at position
// u ^ ((r >> 3) & 1): rows r and r+8 would otherwise share banks, and the
// QK^T operand read (16 lanes = 16 consecutive rows, same unit) would
// conflict two ways.
__device__ __forceinline__ int unit_swz(int r) { return (r >> 3) & 1; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_void*)p);
}

template <int DQK, int DV, bool FP8, int NW, int HPW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv_, const float* __restrict__ kv_scale,
    const float* __restrict__ sink, const int* __restrict__ idx, uint16_t* __restrict__ o, int M,
    int N, int Hq, int K, float scale_log2) {
  using C = AttnCfg<DQK, DV, FP8, NW, HPW>;
  constexpr int HT = C::HT;
  __shared__ __align__(16) uint16_t sKV[C::NBUF][C::TILE];
  __shared__ int sIdx[kMaxK];           // sanitised indices (-1 = invalid), padded
  __shared__ int sFirst[kMaxK / kBI];   // a valid index of each tile, or -1
  __shared__ int sList[kMaxK / kBI];    // tiles with a valid index, ascending
  __shared__ float sSc0[kBI], sSc1[kBI];  // FP8: per-row scales of a tile
  __shared__ int sNvt;
  __shared__ int sFlag;  // a wave saw a score above its reference + slack

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

  // ---- q fragments for this wave's heads -----------------------------------
  const int h0 = wave * HPW + col;  // head of head-tile ht: h0 + 16*ht
  bf16x8 qf[HT][C::QC];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = q + ((size_t)rtok * Hq + h0 + 16 * ht) * DQK;
#pragma unroll
    for (int c = 0; c < C::QC; ++c)
      qf[ht][c] = *reinterpret_cast<const bf16x8*>(qrow + c * 32 + g * 8);
  }
  f32x4 oacc[HT][C::OT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int t = 0; t < C::OT; ++t) oacc[ht][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HT], lsum[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m[ht] = -1e30f;
    lsum[ht] = 0.f;
  }
  // Complete the q loads here: the gathers below are issued through inline
  // asm, invisible to the compiler's vmcnt bookkeeping, and a q wait left
  // inside the tile loop would also wait for every gather in flight.
  wait_vmem_all();
  __syncthreads();
  const int nvt = sNvt;

  // ---- tile staging ---------------------------------------------------------
  // bf16: direct-to-LDS gather.  Rows of invalid slots load a valid row of the
  // same tile instead (finite data; their scores are masked to -inf).
  auto dma = [&](uint16_t* dst, int tile) {
    const uint16_t* kvb = static_cast<const uint16_t*>(kv_) + (size_t)b * N * DQK;
    const int first = sFirst[tile];
    const uint32_t base = lds_addr(dst);
    for (int k = wave; k < C::DMA_INSTR; k += NW) {
      const int u = k * kWave + lane;
      const int r = u / C::UPR, p = u % C::UPR;
      if (u < C::UNITS && p < C::CPR) {
        int row = sIdx[tile * kBI + r];
        row = row >= 0 ? row : first;
        dma16(kvb + (size_t)row * DQK + (p ^ unit_swz(r)) * 8,
              __builtin_amdgcn_readfirstlane(base + k * kWave * 16));
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
          const int r = ch / C::CPR;
          *reinterpret_cast<i32x4*>(dst + r * C::RS + ((ch % C::CPR) ^ unit_swz(r)) * 8) =
              i32x4{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1),
                    __builtin_bit_cast(int, p2), __builtin_bit_cast(int, p3)};
        }
      }
      if (tid < kBI) dsc[tid] = pscale;
    }
  };

  // ---- one tile: S^T = KV.Q^T, online softmax, O^T += V^T.P^T ----------------
  // MFMA tile tau covers gathered rows 16*tau .. 16*tau+15 (A-row r = row
  // 16*tau + r: with the odd 73-unit row stride the 16 rows of one read hit
  // 16 different bank groups).  In the C layout lane (h, g) then holds rows
  // 4g+i (tau=0) and 16+4g+i (tau=1); those 8 rows, in that order, are the
  // k-slots of its P^T B-fragment, and the V^T A-fragment is read to match
  // with two transposing reads of the 4-row blocks at rows 4g and 16+4g.
  // mode 0: reference = max of the first tile; 1: max-only pre-pass;
  // 2: reference = exact max from the pre-pass.
  auto compute = [&](const uint16_t* sK, const float* sSc, int tile, int it, int mode,
                     auto&& after_qk) {
    f32x4 s[2][HT];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) s[tau][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // LA k-steps of A fragments in flight: step c+LA is loaded before the
      // MFMAs of step c are issued, and a scheduling barrier keeps the
      // compiler from hoisting every LDS read (which would cost registers).
      // Rows col and 16+col, unit 4c+g (rows 8..15 and 24..31 flip bit 0).
      const uint16_t* a0 = sK + col * C::RS + (g ^ unit_swz(col)) * 8;
      const uint16_t* a1 = a0 + 16 * C::RS;
      constexpr int R = kLA + 1;
      bf16x8 xa[R][2];
#pragma unroll
      for (int c = 0; c < kLA && c < C::QC; ++c) {
        xa[c % R][0] = *reinterpret_cast<const bf16x8*>(a0 + c * 32);
        xa[c % R][1] = *reinterpret_cast<const bf16x8*>(a1 + c * 32);
      }
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        if (c + kLA < C::QC) {
          xa[(c + kLA) % R][0] = *reinterpret_cast<const bf16x8*>(a0 + (c + kLA) * 32);
          xa[(c + kLA) % R][1] = *reinterpret_cast<const bf16x8*>(a1 + (c + kLA) * 32);
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          s[0][ht] = mfma_bf16_16x16x32(xa[c % R][0], qf[ht][c], s[0][ht]);
          s[1][ht] = mfma_bf16_16x16x32(xa[c % R][1], qf[ht][c], s[1][ht]);
        }
        if (kSchedBarrier) __builtin_amdgcn_sched_barrier(0);
      }
    }
    after_qk();
    const int* ti = sIdx + tile * kBI + 4 * g;
    bool valid[8];
    float scl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int jj = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
      valid[i] = ti[(i < 4 ? 0 : 16) + (i & 3)] >= 0;
      scl[i] = FP8 ? sSc[jj] * scale_log2 : scale_log2;
    }
    float sv[HT][8];
    float tmax[HT];
    bool over = false;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float raw = s[i >> 2][ht][i & 3];
        const float x = valid[i] ? raw * scl[i] : -INFINITY;
        sv[ht][i] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, wave_xor(mx, 16));
      mx = fmaxf(mx, wave_xor(mx, 32));
      tmax[ht] = mx;
      if (mode == 1) {
        m[ht] = fmaxf(m[ht], mx);
      } else if (mode == 0) {
        if (it == 0) m[ht] = mx;  // every head sees a valid index in the first tile
        over = over || (mx > m[ht] + kRefSlack);
      }
    }
    if (mode == 1) return;
    if (__ballot(over) != 0ull && lane == 0) sFlag = 1;
    bf16x8 pb[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float p0 = fast_exp2(sv[ht][i] - m[ht]), p1 = fast_exp2(sv[ht][i + 1] - m[ht]);
        psum += p0 + p1;
        if constexpr (FP8) {
          p0 *= sSc[(i < 4 ? 0 : 16) + 4 * g + (i & 3)];
          p1 *= sSc[(i < 4 ? 0 : 16) + 4 * g + ((i + 1) & 3)];
        }
        pk[i >> 1] = pack_bf16x2(p0, p1);
      }
      lsum[ht] += psum;
      pb[ht] = __builtin_bit_cast(bf16x8, i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
    }
    // A operand: lane (c = 16t + col, g) needs V[4g..4g+3][c] and
    // V[16+4g..16+4g+3][c]: two transposing reads.
    const int vr = 4 * g + (col >> 2);  // and vr + 16
    const uint16_t* vb =
        sK + vr * C::RS + (((col & 3) >> 1) ^ unit_swz(vr)) * 8 + 4 * (col & 1);
    auto vload = [&](int t) {
      const i16x4 lo = lds_read_tr16(vb + t * 16);
      const i16x4 hi = lds_read_tr16(vb + 16 * C::RS + t * 16);
      return __builtin_bit_cast(bf16x8,
                                i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    constexpr int R = kLA + 1;
    bf16x8 va[R];
#pragma unroll
    for (int t = 0; t < kLA && t < C::OT; ++t) va[t % R] = vload(t);
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
      if (t + kLA < C::OT) va[(t + kLA) % R] = vload(t + kLA);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        oacc[ht][t] = mfma_bf16_16x16x32(va[t % R], pb[ht], oacc[ht][t]);
      if (kSchedBarrier) __builtin_amdgcn_sched_barrier(0);
    }
  };


  // Waits until this wave's gathers of tile `it` have landed, leaving those of
  // tile it+1 (issued one iteration later) in flight.
  auto wait_tile = [&](bool next_in_flight) {
    if constexpr (!FP8) {
      if (!next_in_flight) {
        wait_vmem_all();
      } else if (wave < C::DMA_HI_WAVES) {
        wait_vmem_le<C::DMA_HI>();
      } else {
        wait_vmem_le<C::DMA_LO>();
      }
    }
  };

  // A direct-to-LDS load holds up its own wave's instruction issue, so the
  // two waves that share a SIMD (w and w+4) issue theirs at different times:
  // one right after the barrier, the other after its QK^T, while its partner
  // keeps the MFMA pipe busy.
  const bool dma_early = ((wave >> 2) & 1) == 0;

#pragma unroll 1
  for (int mode = 0;;) {
    if (tid == 0) sFlag = 0;
    if (nvt > 0) {
      if constexpr (FP8) {
        gload(sList[0]);
        lstore(sKV[0], sSc0);
        if (nvt > 1) gload(sList[1]);
      } else {
        dma(sKV[0], sList[0]);
        if (nvt > 1) dma(sKV[1], sList[1]);
      }
    }
    bool restart = false;
#pragma unroll 1
    for (int it = 0; it < nvt; ++it) {
      const int cb = it % C::NBUF;
      const uint16_t* cur = sKV[cb];
      const bool odd = it & 1;
      const float* curS = odd ? sSc1 : sSc0;
      float* nxtS = odd ? sSc0 : sSc1;
      wait_tile(it + 1 < nvt);  // gathers of tile `it` done (bf16)
      __syncthreads();  // tile `it` complete; everyone is done with tile it-1's buffer
      if (sFlag) {      // uniform: written before the barrier
        restart = true;
        break;
      }
      if constexpr (FP8) {
        if (it + 1 < nvt) {
          lstore(sKV[(it + 1) % C::NBUF], nxtS);
          if (it + 2 < nvt) gload(sList[it + 2]);
        }
      } else {
        if (it + 2 < nvt && dma_early) dma(sKV[(it + 2) % C::NBUF], sList[it + 2]);
      }
      compute(cur, curS, sList[it], it, mode, [&] {
        if constexpr (!FP8) {
          if (it + 2 < nvt && !dma_early) dma(sKV[(it + 2) % C::NBUF], sList[it + 2]);
        }
      });
    }
    wait_vmem_all();  // no gather may still be landing in LDS
    __syncthreads();
    restart = restart || sFlag;
    if (mode == 1 || restart) {
      // pre-pass done -> final pass; or restart: pre-pass from scratch
      mode = mode == 1 ? 2 : 1;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if (mode == 1) m[ht] = -INFINITY;
        lsum[ht] = 0.f;
#pragma unroll
        for (int t = 0; t < C::OT; ++t) oacc[ht][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();  // sFlag reset below is not seen early
      continue;
    }
    break;
  }

  // ---- sink, normalise, store ------------------------------------------------
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = h0 + 16 * ht;
    float l = lsum[ht];
    l += wave_xor(l, 16);
    l += wave_xor(l, 32);
    if (sink) l += fast_exp2(sink[h] * kLog2e - m[ht]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = o + ((size_t)rtok * Hq + h) * DV + g * 4;
#pragma unroll
    for (int t = 0; t < C::OT; ++t) {
      const f32x4 v = oacc[ht][t] * inv;
      uint2 pk2;
      pk2.x = pack_bf16x2(v[0], v[1]);
      pk2.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(orow + t * 16) = pk2;
    }
  }
}

template <int DQK, int DV, bool FP8, int NW, int HPW>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  using C = AttnCfg<DQK, DV, FP8, NW, HPW>;
  const long long rows = a.B * a.M;
  if (rows > 0x7fffffffLL || a.K > kMaxK || a.Hq != NW * HPW) return hipErrorInvalidValue;
  const float scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / sqrtf((float)DQK);
  hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, FP8, NW, HPW>), dim3((unsigned)rows),
                     dim3(C::THREADS), 0, stream, (const uint16_t*)a.q, a.kv, a.kv_scale,
                     a.attn_sink, a.topk_idxs, (uint16_t*)a.o, (int)a.M, (int)a.N, a.Hq, a.K,
                     (float)((double)scale * 1.4426950408889634));
  return hipGetLastError();
}

// Heads per wave at 128 heads (tuning knob: 32 -> 4 waves, 16 -> 8 waves).
#ifndef DSA_ATTN_HPW128
#define DSA_ATTN_HPW128 16
#endif

template <int DQK, int DV, bool FP8>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
  switch (a.Hq) {
    case 16: return launch<DQK, DV, FP8, 1, 16>(a, stream);
    case 32: return launch<DQK, DV, FP8, 2, 16>(a, stream);
    case 64: return launch<DQK, DV, FP8, 4, 16>(a, stream);
    case 128: return launch<DQK, DV, FP8, 128 / DSA_ATTN_HPW128, DSA_ATTN_HPW128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported(int Hq, int Dqk, int Dv, bool fp8) {
  if (!(Hq == 16 || Hq == 32 || Hq == 64 || Hq == 128)) return false;
  if (Dqk == 64 && Dv == 64) return !fp8;
  if (Dqk == 576 && Dv == 512) return true;
  return false;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.Dqk == 64 && a.Dv == 64 && !a.fp8) return launch_heads<64, 64, false>(a, stream);
  if (a.Dqk == 576 && a.Dv == 512 && !a.fp8) return launch_heads<576, 512, false>(a, stream);
  if (a.Dqk == 576 && a.Dv == 512 && a.fp8) return launch_heads<576, 512, true>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
