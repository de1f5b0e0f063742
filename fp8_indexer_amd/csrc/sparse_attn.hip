// sparse_attn.hip -- gathered sparse attention forward with a sink, gfx950.
//
// Semantics (DeepSeek V4.1 atlas page, sparse_attn_kernel / sparse_attn):
// for each query token, gather the KV rows named by its top-k indices, run an
// online softmax over q.kv * sm_scale, add exp(attn_sink[h]) to the
// denominator only, mask -1 indices, and give zero output when no index is
// valid.  The value is the first Dv columns of the same latent row.
//
// Design (MI355X-first):
//  * One workgroup per query token.  With 128 heads it has 4 waves (one per
//    SIMD) of 32 heads each; fewer heads use 16 per wave and fewer waves.  A
//    wave's q rows are MFMA B-fragments held in registers for the whole
//    token, except for the last few 32-deep k-steps, which sit in LDS: the
//    O accumulators (128 heads x 128 columns, fp32) fill the 256 AGPRs and
//    q, the score accumulators and the staged KV chunks share the 256
//    VGPRs.
//  * The product is formed transposed, S^T[j, h] = kv_j . q_h, on
//    v_mfma_f32_16x16x32_bf16.  In the C layout each lane then holds one head
//    and 8 gathered rows, which is the B-fragment layout of the next product
//    O^T[c, h] += V^T[c, j] P^T[j, h].  P is packed to bf16 and written to
//    LDS; groups of PG waves read each other's P and split the Dv columns,
//    so each wave multiplies V for PG*16 heads over Dv/PG columns and every
//    V fragment read from LDS feeds PG MFMAs.
//  * KV rows are gathered 32 at a time: each thread loads its share of the
//    next tile (16 threads per 1152-byte row, 16-byte loads) into VGPRs while
//    PV of the current tile runs, then writes it to the other LDS buffer
//    (double buffering, two barriers per tile).  QK^T reads its A operand
//    from the row-major tile with 16-byte LDS loads; PV needs V with the
//    gathered-row axis innermost and gets it from the same tile through
//    gfx950's transposing LDS load (ds_read_b64_tr_b16: each lane of a
//    16-lane group receives one column of a 4x16 block), with no second copy
//    and no transpose pass, which is the problem the TileLang FP8 page's
//    K-major V layout addresses on its hardware.
//  * Softmax in base 2 with sm_scale*log2(e) folded into one multiply, fp32
//    state.  The reference of the exponent is fixed per head at the max of
//    the first tile and never moved: o = O/l is exact for any reference, and
//    bf16 P and fp32 O and l carry p = 2^(s - ref) > 1 exactly as long as
//    nothing overflows.  At the end of the token, a head whose per-lane sum
//    of p passed 2^40 (so every p <= 2^40, far from the fp32 range) makes
//    the whole workgroup restart the token with a max-only pre-pass and a
//    second pass at the exact max.  The fp32 O accumulators are thus only
//    ever touched by MFMA inside the loop (no per-tile rescale).
//  * Tiles whose 32 indices are all invalid are skipped entirely.
//  * FP8 KV (e4m3fn + per-row fp32 scale): the staged codes are widened to
//    bf16 exactly (v_cvt_scalef32_pk_bf16_fp8) on the way into LDS; the row
//    scale multiplies the score of that row and its probability before the
//    bf16 cast.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kBI = 32;      // gathered rows per tile
constexpr int kKVPad = 16;   // row padding (elements): see the LDS layout note
constexpr int kMaxK = 4096;  // largest supported top-k
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPLimit = 0x1p40f;  // largest per-lane l (hence p) without a restart

// LDS operand lookahead (k-steps) and scheduling barriers in the MFMA loops
// (tuning knobs).
#ifndef DSA_ATTN_LA
#define DSA_ATTN_LA 1
#endif
#ifndef DSA_ATTN_SB
#define DSA_ATTN_SB 1
#endif
constexpr int kLA = DSA_ATTN_LA;
// P group size (tuning knob): with 16 heads per wave, groups of this many
// waves share P and split the output columns for PV.
#ifndef DSA_ATTN_PG
#define DSA_ATTN_PG 4
#endif
constexpr int kPG = DSA_ATTN_PG;
// q k-steps read from LDS instead of registers (tuning knob; the last ones).
#ifndef DSA_ATTN_QL
#define DSA_ATTN_QL 6
#endif
#ifndef DSA_ATTN_QL32
#define DSA_ATTN_QL32 5
#endif
#ifndef DSA_ATTN_SQKEND
#define DSA_ATTN_SQKEND 0
#endif
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
  static constexpr int CPR = DQK / 8;              // 8-element chunks per row
  // Staging: TPR threads per row; in pass p thread tid takes row slot
  // p*RPP + tid/TPR, chunks tid%TPR + TPR*j: NC chunks per thread and tile.
  static constexpr int TPR = CPR < 16 ? CPR : 16;
  static constexpr int RPP = THREADS / TPR;
  static constexpr int PASSES = (kBI + RPP - 1) / RPP;
  static constexpr int CPT = (CPR + TPR - 1) / TPR;
  static constexpr int NC = PASSES * CPT;
  static constexpr int QC = DQK / 32;              // 32-deep k-steps of QK
  // The last QL k-steps of q come from LDS (registers for 8 waves x 16 heads
  // hold O and the rest of q); only with 16 heads per wave.
  static constexpr int QL = (HPW == 16 && NW == 8 && DSA_ATTN_QL < QC)   ? DSA_ATTN_QL
                            : (HPW == 32 && NW == 4 && DSA_ATTN_QL32 < QC) ? DSA_ATTN_QL32
                                                                            : 0;
  static constexpr int QR = QC - QL;               // k-steps of q kept in registers
  static constexpr int OT = DV / 16;               // 16-wide output tiles
  // P groups: PG waves (16 heads each) share their P fragments through LDS and
  // split the Dv columns, so each wave multiplies V for PG*16 heads over
  // DV/PG columns: OH head tiles x OTW column tiles of O per wave.
  static constexpr int PG = (NW % kPG == 0 && OT % kPG == 0) ? kPG : 1;
  static constexpr int OH = PG * HT;
  static constexpr int OTW = OT / PG;
};

// QK^T MFMAs with the accumulator pinned to VGPRs.  The O accumulators of PV
// (compiler-scheduled MFMAs) then fill the AGPRs, which is what lets 32 heads
// per wave fit: with every MFMA result in AGPRs, O and S together need more
// than the 256 AGPRs of a wave.  Hazards the compiler cannot see through the
// asm: the accumulator is tied (vdst = srcC, no register to reuse while the
// MFMA still reads it), each MFMA is preceded by 2 wait states (VALU write ->
// MFMA read), and qk_drain() gives the MFMA results 24 wait states before
// any VALU reads them.
#ifndef DSA_ATTN_QKASM
#define DSA_ATTN_QKASM 1
#endif
__device__ __forceinline__ void qk_mfma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if (DSA_ATTN_QKASM) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  } else {
    acc = mfma_bf16_16x16x32(a, b, acc);
  }
}
__device__ __forceinline__ void qk_drain(f32x4& x0, f32x4& x1) {
  if (DSA_ATTN_QKASM) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x0), "+v"(x1));
}

// Lane index computed afresh (an asm the compiler cannot merge with an
// earlier copy of the same value).
__device__ __forceinline__ int fresh_lane_id() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read: within each 16-lane group, lane i supplies the
// address of 4 consecutive bf16 of row i/4 (columns 4*(i%4)..+3) of a 4x16
// block and receives column i (rows 0..3) of that block.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// LDS tile layout: row r of a tile starts at r*RS elements, units in natural
// order.  RS is an odd number of 32-byte pairs (74 16-byte units for
// 576-wide rows), so the 4x16 blocks read by 32 lanes of a transposing load
// (8 rows x 32 bytes) fill the 64 banks exactly; the QK^T operand read (16
// consecutive rows, one unit each) also runs at full rate with this stride
// (measured on gfx950: ~190 B/clk per CU; XOR-swizzling the units by row
// halves it, and slows the transposing read by a quarter).

template <int DQK, int DV, bool FP8, int NW, int HPW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv_, const float* __restrict__ kv_scale,
    const float* __restrict__ sink, const int* __restrict__ idx, uint16_t* __restrict__ o, int M,
    int N, int Hq, int K, float scale_log2, int S, int kspan, uint16_t* __restrict__ wso,
    float2* __restrict__ wsml) {
  using C = AttnCfg<DQK, DV, FP8, NW, HPW>;
  constexpr int HT = C::HT, PG = C::PG, OH = C::OH, OTW = C::OTW;
  __shared__ __align__(16) uint16_t sKV[2][C::TILE];
  __shared__ int sIdx[kMaxK];           // sanitised indices (-1 = invalid), padded
  __shared__ int sList[kMaxK / kBI];    // tiles with a valid index, ascending
  __shared__ int sFirst[kMaxK / kBI];   // first valid index of each tile, or -1
  __shared__ int sFull[kMaxK / kBI];    // all 32 indices of the tile are valid
  __shared__ float sSc[2][kBI];         // FP8: per-row scales of a tile
  __shared__ int sNvt;
  __shared__ int sFlag[1];  // a head's sum passed kPLimit: restart
  __shared__ __align__(16) bf16x8 sP[NW][HT][kWave];  // P B-fragments
  __shared__ float sL[PG > 1 ? NW : 1][HT][16], sM[PG > 1 ? NW : 1][HT][16];
  __shared__ float sSink[NW * HPW];     // attn_sink of each head
  __shared__ __align__(16) bf16x8 sQ[C::QL > 0 ? C::QL : 1][NW][HT][kWave];  // q B-fragments

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: an SGPR
  const int g = lane >> 4, col = lane & 15;
  // workgroup -> (b, t) row, latest first, and split s of its K indices:
  // [s*kspan, s*kspan + klen) (S = 1: the whole row)
  int rtok = (int)(gridDim.x / S - 1 - blockIdx.x / S);
  int split = (int)(blockIdx.x % S);
  if constexpr (SPLIT) {
    int rrow = (int)(blockIdx.x / S);
    split_to_xcd(rrow, split, S);
    rtok = (int)(gridDim.x / S) - 1 - rrow;
  }
  const int b = rtok / M;
  const int kbeg = split * kspan;
  const int klen = max(0, min(K - kbeg, kspan));
  const int ntiles = (klen + kBI - 1) / kBI;

  // ---- prologue: every global load is issued before anything waits on one --
  // indices (the first IB per thread; more for K > IB * THREADS)
  const int* ridx = idx + (size_t)rtok * K + kbeg;
  const int nidx = ntiles * kBI;
  constexpr int IB = 8;
  int iv[IB];
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int p = tid + j * C::THREADS;
    iv[j] = p < klen ? ridx[p] : -1;
  }
  // q fragments of this wave's heads; the last QL k-steps go to LDS below
  const int h0 = wave * HPW + col;  // head of head-tile ht: h0 + 16*ht
  bf16x8 qf[HT][C::QR];
  bf16x8 ql[C::QL > 0 ? C::QL : 1][HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = q + ((size_t)rtok * Hq + h0 + 16 * ht) * DQK;
#pragma unroll
    for (int c = 0; c < C::QR; ++c)
      qf[ht][c] = *reinterpret_cast<const bf16x8*>(qrow + c * 32 + g * 8);
#pragma unroll
    for (int c = C::QR; c < C::QC; ++c)
      ql[c - C::QR][ht] = *reinterpret_cast<const bf16x8*>(qrow + c * 32 + g * 8);
  }
  const float skv = (sink && tid < Hq) ? sink[tid] : 0.f;
  const int c0 = (wave % PG) * (DV / PG);  // first output column of this wave
  f32x4 oacc[OH][OTW];
#pragma unroll
  for (int oh = 0; oh < OH; ++oh)
#pragma unroll
    for (int t = 0; t < OTW; ++t) oacc[oh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HT], lsum[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m[ht] = -1e30f;
    lsum[ht] = 0.f;
  }
  // indices -> LDS (sanitised: -1 = invalid), sink -> LDS.  Per tile, the
  // first valid index (invalid slots gather that row: finite data whose p is
  // exactly 0) and whether all 32 are valid: for the first IB*THREADS
  // indices a half-wave holds one tile in iv[j], so two ballots give both.
  auto sanitise = [&](int v) { return (v >= 0 && v < N) ? v : -1; };
  static_assert(kBI == 32, "a tile is one half-wave of iv[j]");
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int p = tid + j * C::THREADS;
    const int v = sanitise(iv[j]);
    if (p < nidx) sIdx[p] = v;
    const uint64_t mk = __ballot(v >= 0);
    const uint32_t mh = (uint32_t)(mk >> (lane & 32));
    const int fl = mh ? __builtin_ctz(mh) : 0;
    const int first = __shfl(v, (lane & 32) + fl, kWave);
    const int t = p / kBI;
    if ((lane & 31) == 0 && t < ntiles) {
      sFirst[t] = mh ? first : -1;
      sFull[t] = mh == 0xffffffffu;
    }
  }
  for (int p = tid + IB * C::THREADS; p < nidx; p += C::THREADS)
    sIdx[p] = sanitise(p < klen ? ridx[p] : -1);
  if (tid < Hq) sSink[tid] = skv;
  __syncthreads();
  // tiles beyond the first IB*THREADS indices: one lane per tile scans it
  constexpr int T0 = IB * C::THREADS / kBI;
  for (int t = T0 + tid; t < ntiles; t += C::THREADS) {
    int first = -1;
    bool full = true;
    for (int r = kBI - 1; r >= 0; --r) {
      const int v = sIdx[t * kBI + r];
      first = v >= 0 ? v : first;
      full = full && v >= 0;
    }
    sFirst[t] = first;
    sFull[t] = full;
  }
  if (ntiles > T0) __syncthreads();  // uniform
  // ---- tile staging: VGPRs, then LDS ----------------------------------------
  // Each thread moves NC chunks of a tile (chunk = 8 elements of one row: 16
  // bytes of bf16 or 8 fp8 codes).  The loads of tile it+1 are issued one by
  // one between the QK^T k-steps of tile it and written to the other LDS
  // buffer one by one between the PV column steps: a burst of gathers would
  // hold up the issuing wave (the vector memory unit takes about 16 cycles
  // per 64-lane 16-byte load) and, at one wave per SIMD, the SIMD with it.
  typedef typename std::conditional<FP8, uint2, i32x4>::type chunk_t;
  typedef typename std::conditional<FP8, uint8_t, uint16_t>::type elem_t;
  constexpr int NC = C::NC;
  chunk_t pre[NC];
  int grow[C::PASSES];
  float pscale = 0.f;
  const int srow = tid / C::TPR, sch = tid % C::TPR;
  const elem_t* kvb = static_cast<const elem_t*>(kv_) + (size_t)b * N * DQK + sch * 8;
  // chunk k: pass k / CPT (row slot p*RPP + srow), 16-byte unit sch + TPR*(k % CPT)
  auto chunk_ok = [&](int k) {
    const int r = (k / C::CPT) * C::RPP + srow, u = sch + C::TPR * (k % C::CPT);
    return (kBI % C::RPP == 0 || r < kBI) && (C::CPR % C::TPR == 0 || u < C::CPR);
  };
  // rows of a tile's staging passes; invalid slots load the tile's first
  // valid row (finite data; the slot's score is masked and its p is exactly 0)
  auto gather_rows = [&](int tile) {
    const int* ti = sIdx + tile * kBI;
    const int first = sFirst[tile];
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int r = p * C::RPP + srow;
      const int row = (kBI % C::RPP == 0 || r < kBI) ? ti[r] : 0;
      grow[p] = row >= 0 ? row : first;
    }
    if constexpr (FP8) {
      if (tid < kBI) {
        const int row = ti[tid];
        pscale = row >= 0 ? kv_scale[(size_t)b * N + row] : 0.f;
      }
    }
  };
  auto gather_chunk = [&](int k) {
    chunk_t v{};
    if (chunk_ok(k))
      v = *reinterpret_cast<const chunk_t*>(kvb + (size_t)grow[k / C::CPT] * DQK +
                                            C::TPR * (k % C::CPT) * 8);
    pre[k] = v;
  };
  auto store_chunk = [&](uint16_t* dst, int k) {
    if (!chunk_ok(k)) return;
    const int r = (k / C::CPT) * C::RPP + srow, u = sch + C::TPR * (k % C::CPT);
    i32x4 v;
    if constexpr (FP8) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const uint2 raw = pre[k];
      const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false);
      const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true);
      const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false);
      const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true);
      v = i32x4{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1),
                __builtin_bit_cast(int, p2), __builtin_bit_cast(int, p3)};
    } else {
      v = pre[k];
    }
    *reinterpret_cast<i32x4*>(dst + r * C::RS + u * 8) = v;
  };
  auto store_scale = [&](float* dsc) {
    if constexpr (FP8) {
      if (tid < kBI) dsc[tid] = pscale;
    }
  };
  auto gload = [&](int tile) {
    gather_rows(tile);
#pragma unroll
    for (int k = 0; k < NC; ++k) gather_chunk(k);
  };
  auto lstore = [&](uint16_t* dst, float* dsc) {
#pragma unroll
    for (int k = 0; k < NC; ++k) store_chunk(dst, k);
    store_scale(dsc);
  };
  // Tile 0 -- the first tile of nearly every row -- is gathered while the
  // tile list is built; invalid slots load nothing (zeros: finite, masked,
  // p exactly 0).  Used by the first pass if tile 0 holds a valid index.
  {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int r = p * C::RPP + srow;
      grow[p] = (kBI % C::RPP == 0 || r < kBI) && r < nidx ? sIdx[r] : -1;
    }
    if constexpr (FP8) {
      if (tid < kBI) {
        const int row = tid < nidx ? sIdx[tid] : -1;
        pscale = row >= 0 ? kv_scale[(size_t)b * N + row] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      chunk_t v{};
      if (chunk_ok(k) && grow[k / C::CPT] >= 0)
        v = *reinterpret_cast<const chunk_t*>(kvb + (size_t)grow[k / C::CPT] * DQK +
                                              C::TPR * (k % C::CPT) * 8);
      pre[k] = v;
    }
  }
  // list of tiles holding a valid index, ascending
  if (wave == 0) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += kWave) {
      const int t = t0 + lane;
      const bool f = t < ntiles && sFirst[t] >= 0;
      const uint64_t mk = __ballot(f);
      if (f) sList[base + __popcll(mk & lt)] = t;
      base += __popcll(mk);
    }
    if (lane == 0) sNvt = base;
  }
#pragma unroll
  for (int c = C::QR; c < C::QC; ++c)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) sQ[c - C::QR][wave][ht][lane] = ql[c - C::QR][ht];
  __syncthreads();
  const int nvt = sNvt;

  // Staging schedule (at most half the chunks in registers at a time): the
  // first GH chunks are loaded over the first half of the QK^T k-steps and
  // written to LDS over the second half (the other buffer is free since the
  // barrier that started this tile); the others are loaded over the second
  // half and written during the first half of PV, so that the stores have
  // drained by the next barrier.
  constexpr int GH = (NC + 1) / 2, QH = C::QC / 2;
  // QK^T k-step after which chunk k is loaded
  auto gstep = [](int k) {
    return k < GH ? (k * QH) / GH : QH + ((k - GH) * (C::QC - QH)) / (NC - GH > 0 ? NC - GH : 1);
  };
  // QK^T k-step after which chunk k is stored (chunks k < GH; QC: after the
  // last k-step, beside the softmax, whose VALU work leaves LDS idle), PV
  // column step (others)
  auto sqk = [](int k) { return DSA_ATTN_SQKEND ? C::QC : QH + (k * (C::QC - QH)) / GH; };
  auto spv = [](int k) { return ((k - GH) * ((OTW + 1) / 2)) / (NC - GH > 0 ? NC - GH : 1); };

  // ---- one tile: S^T = KV.Q^T, softmax, O^T += V^T.P^T -----------------------
  // MFMA tile tau covers gathered rows 16*tau .. 16*tau+15 (A-row r = row
  // 16*tau + r).  In the C layout lane (h, g) then holds rows 4g+i (tau=0)
  // and 16+4g+i (tau=1); those 8 rows, in that order, are the k-slots of its
  // P^T B-fragment, and the V^T A-fragment is read to match with two
  // transposing reads of the 4-row blocks at rows 4g and 16+4g.
  // mode 0: reference = max of the first tile; 1: max-only pre-pass;
  // 2: reference = exact max from the pre-pass.  P goes to LDS (sP).
  // With `gat`, the gather chunks of the tile whose rows are in grow are
  // loaded between the k-steps, and the first GH of them stored to dst.
  // This wave's own P fragments stay in pown.
  bf16x8 pown[HT];
  auto qk_softmax = [&](const uint16_t* sK, const float* sS, int tile, int it, int mode,
                        bool gat, uint16_t* dst) {
    f32x4 s[2][HT];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) s[tau][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // LA k-steps of A fragments in flight: step c+LA is loaded before the
      // MFMAs of step c are issued, and a scheduling barrier keeps the
      // compiler from hoisting every LDS read (which would cost registers).
      // Rows col and 16+col, unit 4c+g.
      const uint16_t* a0 = sK + col * C::RS + g * 8;
      const uint16_t* a1 = a0 + 16 * C::RS;
      constexpr int R = kLA + 1;
      bf16x8 xa[R][2], xq[R][HT];
      auto ld = [&](int c) {
        xa[c % R][0] = *reinterpret_cast<const bf16x8*>(a0 + c * 32);
        xa[c % R][1] = *reinterpret_cast<const bf16x8*>(a1 + c * 32);
        if (c >= C::QR) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) xq[c % R][ht] = sQ[c - C::QR][wave][ht][lane];
        }
      };
#pragma unroll
      for (int c = 0; c < kLA && c < C::QC; ++c) ld(c);
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        if (c + kLA < C::QC) ld(c + kLA);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const bf16x8 qb = c < C::QR ? qf[ht][c < C::QR ? c : 0] : xq[c % R][ht];
          qk_mfma(s[0][ht], xa[c % R][0], qb);
          qk_mfma(s[1][ht], xa[c % R][1], qb);
        }
        if (gat) {
#pragma unroll
          for (int k = 0; k < GH; ++k)
            if (sqk(k) == c) store_chunk(dst, k);
#pragma unroll
          for (int k = 0; k < NC; ++k)
            if (gstep(k) == c) gather_chunk(k);
        }
        if (kSchedBarrier) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) qk_drain(s[0][ht], s[1][ht]);
      if (gat) {
#pragma unroll
        for (int k = 0; k < GH; ++k)
          if (sqk(k) == C::QC) store_chunk(dst, k);
      }
    }
    // tv = score * sm_scale * log2(e) - reference (log2 units), -inf when masked
    float tv[HT][8];
    if ((mode == 2 || (mode == 0 && it > 0)) && sFull[tile]) {
      // steady state on a tile whose 32 indices are all valid: no masking
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int jj = (i < 4 ? 0 : 16) + (i & 3);
          const float scl = FP8 ? sS[jj + 4 * g] * scale_log2 : scale_log2;
          tv[ht][i] = fmaf(s[i >> 2][ht][i & 3], scl, -m[ht]);
        }
    } else {
      const int* ti = sIdx + tile * kBI + 4 * g;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int jj = (i < 4 ? 0 : 16) + (i & 3);
          const float scl = FP8 ? sS[jj + 4 * g] * scale_log2 : scale_log2;
          const float raw = s[i >> 2][ht][i & 3];
          const float x = ti[jj] >= 0 ? raw * scl : -INFINITY;
          sv[i] = x;
          mx = fmaxf(mx, x);
        }
        if (mode == 1 || (mode == 0 && it == 0)) {
          mx = fmaxf(mx, wave_xor(mx, 16));
          mx = fmaxf(mx, wave_xor(mx, 32));
          // the first tile holds a valid index, so every head's max is finite
          m[ht] = mode == 1 ? fmaxf(m[ht], mx) : mx;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tv[ht][i] = sv[i] - m[ht];
      }
    }
    if (mode == 1) return;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float p0 = fast_exp2(tv[ht][i]), p1 = fast_exp2(tv[ht][i + 1]);
        psum += p0 + p1;
        if constexpr (FP8) {
          p0 *= sS[(i < 4 ? 0 : 16) + 4 * g + (i & 3)];
          p1 *= sS[(i < 4 ? 0 : 16) + 4 * g + ((i + 1) & 3)];
        }
        pk[i >> 1] = pack_bf16x2(p0, p1);
      }
      lsum[ht] += psum;
      pown[ht] = __builtin_bit_cast(bf16x8, i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
      if constexpr (PG > 1) sP[wave][ht][lane] = pown[ht];
    }
  };
  // PV of a tile: O^T += V^T P^T over this wave's heads (PG = 1), or over
  // the whole P group's heads for this wave's Dv/PG columns.  O tile oh
  // belongs to the group's wave (wave + oh/HT) % PG, head tile oh % HT: the
  // first HT are this wave's own, whose P is still in registers, so the
  // first MFMAs need no LDS read.  The staged chunks go to dst between the
  // column steps.  The first kLA V fragments are read by pv_prefetch, which
  // can run before the barrier that publishes P.
  auto pgrp = [&](int oh) { return (wave % PG + oh / HT) % PG; };
  // A operand: lane (c = c0 + 16t + col, g) needs V[4g..4g+3][c] and
  // V[16+4g..16+4g+3][c]: two transposing reads.
  const int voff = (4 * g + (col >> 2)) * C::RS + ((col & 3) >> 1) * 8 + 4 * (col & 1) + c0;
  auto vload = [&](const uint16_t* sK, int t) {
    const i16x4 lo = lds_read_tr16(sK + voff + t * 16);
    const i16x4 hi = lds_read_tr16(sK + voff + 16 * C::RS + t * 16);
    return __builtin_bit_cast(bf16x8,
                              i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  constexpr int RV = kLA + 1;
  bf16x8 va[RV];
  auto pv_prefetch = [&](const uint16_t* sK) {
#pragma unroll
    for (int t = 0; t < kLA && t < OTW; ++t) va[t % RV] = vload(sK, t);
  };
  auto pv_tile = [&](const uint16_t* sK, uint16_t* dst) {
    bf16x8 pv[OH];
#pragma unroll
    for (int oh = 0; oh < OH; ++oh)
      pv[oh] = oh < HT ? pown[oh % HT] : sP[(wave / PG) * PG + pgrp(oh)][oh % HT][lane];
#pragma unroll
    for (int t = 0; t < OTW; ++t) {
      if (t + kLA < OTW) va[(t + kLA) % RV] = vload(sK, t + kLA);
#pragma unroll
      for (int oh = 0; oh < OH; ++oh)
        oacc[oh][t] = mfma_bf16_16x16x32(va[t % RV], pv[oh], oacc[oh][t]);
#pragma unroll
      for (int k = GH; k < NC; ++k)
        if (spv(k) == t) store_chunk(dst, k);
      if (kSchedBarrier) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile schedule.  Iteration `it`: QK^T + softmax of tile it, with this
  // thread's share of tile it+1 loaded into VGPRs in between; the first V
  // fragments of tile it | barrier | PV of tile it, with the share written
  // to the other LDS buffer (last read in iteration it-1) in between.  The
  // last iteration re-gathers its own tile (L2-warm, never read) so that the
  // loop body has no branches.
  //
  // With the reference fixed at the first tile's max, p = 2^(s - ref) grows
  // past 1 when a later score exceeds it; bf16 P and fp32 O and l represent
  // that exactly as long as nothing overflows, so the check is made once, at
  // the end: a head whose partial sum passed 2^40 (every p <= 2^40, far from
  // the fp32 range) restarts the token with a max-only pre-pass and a final
  // pass at the exact max.
#pragma unroll 1
  for (int mode = 0;;) {
    if (tid == 0) sFlag[0] = 0;
    if (nvt > 0) {
      if (mode != 0 || sList[0] != 0) gload(sList[0]);  // else: tile 0, gathered above
      lstore(sKV[0], sSc[0]);
    }
#pragma unroll 1
    for (int it = 0; it < nvt; ++it) {
      const uint16_t* cur = sKV[it & 1];
      uint16_t* nxt = sKV[(it + 1) & 1];
      const float* curS = sSc[it & 1];
      float* nxtS = sSc[(it + 1) & 1];
      __syncthreads();  // tile it complete
      const bool more = it + 1 < nvt;
      gather_rows(sList[more ? it + 1 : it]);
      qk_softmax(cur, curS, sList[it], it, mode, true, nxt);
      pv_prefetch(cur);
      __syncthreads();  // P of the whole P group visible
      // (in the max-only pre-pass P is stale and O is discarded; PV still
      // runs, for the staging stores between its steps)
      pv_tile(cur, nxt);
      store_scale(nxtS);
    }
    if (mode == 0) {
      bool bad = false;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) bad = bad || !(lsum[ht] <= kPLimit);
      if (__ballot(bad) != 0ull && lane == 0) sFlag[0] = 1;
    }
    // l and m of each head to the P group (read after the final pass)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float l = lsum[ht];
      l += wave_xor(l, 16);
      l += wave_xor(l, 32);
      lsum[ht] = l;
      if (PG > 1 && g == 0) {
        sL[PG > 1 ? wave : 0][ht][col] = l;
        sM[PG > 1 ? wave : 0][ht][col] = m[ht];
      }
    }
    __syncthreads();
    const bool restart = sFlag[0] != 0;
    if (mode == 1 || restart) {
      // pre-pass done -> final pass; or restart: pre-pass from scratch
      mode = mode == 1 ? 2 : 1;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if (mode == 1) m[ht] = -INFINITY;
        lsum[ht] = 0.f;
      }
#pragma unroll
      for (int oh = 0; oh < OH; ++oh)
#pragma unroll
        for (int t = 0; t < OTW; ++t) oacc[oh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();  // the flag reset below is not seen early
      continue;
    }
    break;
  }

  // ---- sink, normalise, store ------------------------------------------------
  // l and m of the heads of this wave's O tiles (P groups: exchanged via LDS)
  float lf[OH], mf[OH];
  if constexpr (PG == 1) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      lf[ht] = lsum[ht];
      mf[ht] = m[ht];
    }
  } else {
#pragma unroll
    for (int oh = 0; oh < OH; ++oh) {
      lf[oh] = sL[(wave / PG) * PG + pgrp(oh)][oh % HT][col];
      mf[oh] = sM[(wave / PG) * PG + pgrp(oh)][oh % HT][col];
    }
  }
  if constexpr (SPLIT) {
    // split: this split's normalised O in bf16 (O / l; 0 without a valid
    // index) into the workspace, staged through LDS as in the unsplit
    // epilogue below (whole 16-byte lanes of each head row), and (m, l) of
    // each head, for the merge kernel
    const size_t part = (size_t)rtok * S + split;
    constexpr int OS = DV + 8;
    constexpr int OP = (NW * HPW * OS * 2 + (int)sizeof(sKV) - 1) / (int)sizeof(sKV);
    constexpr int ORP = NW * HPW / OP;  // head rows per pass
    static_assert((NW * HPW) % OP == 0 && ORP * OS * 2 <= (int)sizeof(sKV), "O staging");
    uint16_t* so = &sKV[0][0];
    const int ln = fresh_lane_id(), colx = ln & 15, gx = ln >> 4;
    float inv[OH];
#pragma unroll
    for (int oh = 0; oh < OH; ++oh) {
      const int h = ((wave / PG) * PG + pgrp(oh)) * HPW + (oh % HT) * 16 + colx;
      if (gx == 0 && wave % PG == 0) wsml[part * Hq + h] = float2{mf[oh], lf[oh]};
      inv[oh] = lf[oh] > 0.f ? __builtin_amdgcn_rcpf(lf[oh]) : 0.f;
    }
#pragma unroll
    for (int pass = 0; pass < OP; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's rows are read
#pragma unroll
      for (int oh = 0; oh < OH; ++oh) {
        const int hr = ((wave / PG) * PG + pgrp(oh)) * HPW + (oh % HT) * 16 - pass * ORP;
        if (hr >= 0 && hr < ORP) {  // uniform over the wave
          uint16_t* srow = so + (hr + colx) * OS + c0 + gx * 4;
#pragma unroll
          for (int t = 0; t < OTW; ++t) {
            const f32x4 v = oacc[oh][t] * inv[oh];
            uint2 pk2;
            pk2.x = pack_bf16x2(v[0], v[1]);
            pk2.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(srow + t * 16) = pk2;
          }
        }
      }
      __syncthreads();
      uint16_t* obase = wso + (part * Hq + pass * ORP) * DV;
      for (int u = tid; u < ORP * (DV / 8); u += C::THREADS) {
        const int r = u / (DV / 8), c8 = u % (DV / 8);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * DV + c8 * 8) =
            *reinterpret_cast<const i32x4*>(so + r * OS + c8 * 8);
      }
    }
  } else {
    // Normalised bf16 O goes through LDS (the KV tile buffers, free now) in
    // OP passes over the heads, so that every head row of o is written whole
    // with 16-byte lanes: stored straight from the MFMA layout, each store
    // instruction would write 16 separate 32-byte pieces.  Row stride OS =
    // DV + 8 elements keeps the 8-byte LDS writes of 32 lanes on distinct
    // banks.  The lane's position is recomputed here rather than kept live
    // (and spilled) across the tile loop.
    constexpr int OS = DV + 8;
    constexpr int OP = (NW * HPW * OS * 2 + (int)sizeof(sKV) - 1) / (int)sizeof(sKV);
    constexpr int ORP = NW * HPW / OP;  // head rows per pass
    static_assert((NW * HPW) % OP == 0 && ORP * OS * 2 <= (int)sizeof(sKV), "O staging");
    uint16_t* so = &sKV[0][0];
    const int ln = fresh_lane_id(), colx = ln & 15, gx = ln >> 4;
    float inv[OH];
#pragma unroll
    for (int oh = 0; oh < OH; ++oh) {
      const int h = ((wave / PG) * PG + pgrp(oh)) * HPW + (oh % HT) * 16 + colx;
      float l = lf[oh];
      if (sink) l += fast_exp2(sSink[h] * kLog2e - mf[oh]);
      inv[oh] = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
    }
#pragma unroll
    for (int pass = 0; pass < OP; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's rows are read
#pragma unroll
      for (int oh = 0; oh < OH; ++oh) {
        const int hr = ((wave / PG) * PG + pgrp(oh)) * HPW + (oh % HT) * 16 - pass * ORP;
        if (hr >= 0 && hr < ORP) {  // uniform over the wave
          uint16_t* srow = so + (hr + colx) * OS + c0 + gx * 4;
#pragma unroll
          for (int t = 0; t < OTW; ++t) {
            const f32x4 v = oacc[oh][t] * inv[oh];
            uint2 pk2;
            pk2.x = pack_bf16x2(v[0], v[1]);
            pk2.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(srow + t * 16) = pk2;
          }
        }
      }
      __syncthreads();
      uint16_t* obase = o + ((size_t)rtok * Hq + pass * ORP) * DV;
      for (int u = tid; u < ORP * (DV / 8); u += C::THREADS) {
        const int r = u / (DV / 8), c8 = u % (DV / 8);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * DV + c8 * 8) =
            *reinterpret_cast<const i32x4*>(so + r * OS + c8 * 8);
      }
    }
  }
}

// Merge of the splits of one row (one thread per head and 4 output
// columns): o = sum_s 2^(m_s - M) O_s / (sum_s 2^(m_s - M) l_s + e^sink 2^-M)
// with M = max_s m_s -- the same value as one pass over all K indices,
// since every split's O_s and l_s share its reference m_s.
template <int DV, int CW>
__global__ __launch_bounds__(256) void attn_merge_kernel(const uint16_t* __restrict__ wso,
                                                         const float2* __restrict__ wsml,
                                                         const float* __restrict__ sink,
                                                         uint16_t* __restrict__ o, int Hq, int S) {
  // CW output columns per thread (8: one 16-byte load per split)
  static_assert(CW == 4 || CW == 8, "columns per thread");
  constexpr int TPH = DV / CW;       // threads per head
  constexpr int HPB = 256 / TPH;     // heads per workgroup
  static_assert(256 % TPH == 0, "DV");
  using pk_t = std::conditional_t<CW == 8, uint4, uint2>;
  const int hblocks = Hq / HPB;
  const int row = blockIdx.x / hblocks;
  const int h = (blockIdx.x % hblocks) * HPB + threadIdx.x / TPH;
  const int cq = (threadIdx.x % TPH) * CW;
  const size_t p0 = (size_t)row * S;
  float mmax = -INFINITY;
  for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, wsml[(p0 + s) * Hq + h].x);
  float l = 0.f;
  float acc[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) acc[j] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float2 ml = wsml[(p0 + s) * Hq + h];
    const float wgt = fast_exp2(ml.x - mmax) * ml.y;  // the split's share of l
    l += wgt;
    const pk_t pk = *reinterpret_cast<const pk_t*>(wso + ((p0 + s) * Hq + h) * DV + cq);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&pk);
#pragma unroll
    for (int j = 0; j < CW / 2; ++j) {
      acc[2 * j] += wgt * __uint_as_float(w[j] << 16);
      acc[2 * j + 1] += wgt * __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  if (sink) l += fast_exp2(sink[h] * kLog2e - mmax);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  pk_t out;
  uint32_t* w = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
  for (int j = 0; j < CW / 2; ++j) w[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *reinterpret_cast<pk_t*>(o + ((size_t)row * Hq + h) * DV + cq) = out;
}

// Splits of each row's K indices: with few rows (decode: B*M at most half
// the compute units) each row is split over S workgroups, at least 4 tiles
// each, so that the device is filled.  Returns S (1: unsplit) and the span.
int attn_splits(const AttnArgs& a, int& kspan) {
  const long long rows = a.B * a.M;
  const int cus = device_cus();
  int S = 1;
  kspan = a.K;
  if (rows * 2 <= cus) {
    const int want = (int)((cus + rows - 1) / rows);
    const int max_s = max(1, a.K / (4 * kBI));
    S = min(want, max_s);
    kspan = (a.K + S - 1) / S;
    kspan = (kspan + kBI - 1) / kBI * kBI;
    S = (a.K + kspan - 1) / kspan;
  }
  return S;
}

// Partial results of the splits: bf16 O_s / l_s [rows, S, Hq, Dv], then
// fp32 (m_s, l_s) [rows, S, Hq].
size_t attn_split_bytes(const AttnArgs& a, int S) {
  if (S <= 1) return 0;
  return (size_t)(a.B * a.M) * S * a.Hq * (a.Dv * sizeof(uint16_t) + sizeof(float2));
}

template <int DQK, int DV, bool FP8, int NW, int HPW>
hipError_t launch(const AttnArgs& a, Workspace ws, hipStream_t stream) {
  using C = AttnCfg<DQK, DV, FP8, NW, HPW>;
  const long long rows = a.B * a.M;
  if (rows > 0x7fffffffLL || a.K > kMaxK || a.Hq != NW * HPW) return hipErrorInvalidValue;
  const float scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / sqrtf((float)DQK);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  // Few rows: split with a merge when the caller's workspace holds the
  // partials; otherwise the rows run unsplit (same result).
  int kspan;
  int S = attn_splits(a, kspan);
  const size_t need = attn_split_bytes(a, S);
  if (S > 1 && (ws.ptr == nullptr || ws.bytes < need)) {
    S = 1;
    kspan = a.K;
  }
  if (S == 1) {
    hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, FP8, NW, HPW, false>), dim3((unsigned)rows),
                       dim3(C::THREADS), 0, stream, (const uint16_t*)a.q, a.kv, a.kv_scale,
                       a.attn_sink, a.topk_idxs, (uint16_t*)a.o, (int)a.M, (int)a.N, a.Hq, a.K,
                       scale_log2, 1, a.K, nullptr, nullptr);
    return hipGetLastError();
  }
  uint16_t* wso = static_cast<uint16_t*>(ws.ptr);
  float2* wsml = reinterpret_cast<float2*>(wso + (size_t)rows * S * a.Hq * DV);
  hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, FP8, NW, HPW, true>),
                     dim3((unsigned)(rows * S)), dim3(C::THREADS), 0, stream,
                     (const uint16_t*)a.q, a.kv, a.kv_scale, a.attn_sink, a.topk_idxs,
                     (uint16_t*)a.o, (int)a.M, (int)a.N, a.Hq, a.K, scale_log2, S, kspan, wso,
                     wsml);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_attn_merge(wso, wsml, a.attn_sink, (uint16_t*)a.o, rows, a.Hq, DV, S, stream);
}

// Heads per wave at 128 heads (tuning knob: 32 -> 4 waves, 16 -> 8 waves).
#ifndef DSA_ATTN_HPW128
#define DSA_ATTN_HPW128 32
#endif

template <int DQK, int DV, bool FP8>
hipError_t launch_heads(const AttnArgs& a, Workspace ws, hipStream_t stream) {
  switch (a.Hq) {
    case 16: return launch<DQK, DV, FP8, 1, 16>(a, ws, stream);
    case 32: return launch<DQK, DV, FP8, 2, 16>(a, ws, stream);
    case 64: return launch<DQK, DV, FP8, 4, 16>(a, ws, stream);
    case 128: return launch<DQK, DV, FP8, 128 / DSA_ATTN_HPW128, DSA_ATTN_HPW128>(a, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_merge(const uint16_t* wso, const float2* wsml, const float* sink,
                             uint16_t* o, long long rows, int Hq, int Dv, int S,
                             hipStream_t stream) {
  if (Dv == 512) {
    constexpr int HPB = 256 / (512 / 8);
    if (Hq % HPB != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_merge_kernel<512, 8>), dim3((unsigned)(rows * (Hq / HPB))), dim3(256),
                       0, stream, wso, wsml, sink, o, Hq, S);
  } else if (Dv == 64) {
    constexpr int HPB = 256 / (64 / 4);
    if (Hq % HPB != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_merge_kernel<64, 4>), dim3((unsigned)(rows * (Hq / HPB))), dim3(256),
                       0, stream, wso, wsml, sink, o, Hq, S);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool attn_supported(int Hq, int Dqk, int Dv, bool fp8) {
  if (!(Hq == 16 || Hq == 32 || Hq == 64 || Hq == 128)) return false;
  if (Dqk == 64 && Dv == 64) return !fp8;
  if (Dqk == 576 && Dv == 512) return true;
  return false;
}

size_t attn_workspace_bytes(const AttnArgs& a) {
  int kspan;
  return attn_split_bytes(a, attn_splits(a, kspan));
}

hipError_t launch_attn(const AttnArgs& a, Workspace ws, hipStream_t stream) {
  if (a.Dqk == 64 && a.Dv == 64 && !a.fp8) return launch_heads<64, 64, false>(a, ws, stream);
  if (a.Dqk == 576 && a.Dv == 512 && !a.fp8) return launch_heads<576, 512, false>(a, ws, stream);
  if (a.Dqk == 576 && a.Dv == 512 && a.fp8) return launch_heads<576, 512, true>(a, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
