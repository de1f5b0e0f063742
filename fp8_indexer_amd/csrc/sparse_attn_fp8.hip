// sparse_attn_fp8.hip -- full-FP8 gathered sparse attention forward with a
// sink, gfx950.
//
// Semantics: the sparse attention of the DeepSeek V4.1 atlas page
// (sparse_attn_kernel / sparse_attn: gather the top-k KV rows by index, online
// softmax, attn_sink in the denominator only, -1 masked, zero output for a row
// without a valid index) with an e4m3 query and KV cache and a bf16 output,
// as in the TileLang "deepseek_v32" page, section "Sparse MLA Forward (FP8)".
// Values: q = code * q_scale[b,t,h], kv = code * kv_scale[b,j].  Both
// products run on fp8 MFMA; the probabilities enter PV as e4m3, scaled up
// before the cast so that they use the format's range (the scaling by the
// e4m3 maximum, 448, proposed in the FlashInfer MLA pull-request discussion,
// with the output divided by the same factor).
//
// Design (MI355X-first):
//  * v_mfma_f32_32x32x64_f8f6f4 for both products (measured on gfx950: 4.7
//    of the 5.0 PFLOP/s fp8 peak; the older 16x16x32 fp8 MFMA runs at only
//    the bf16 rate).  Lane l holds A row l%32 / B column l%32 and bytes
//    [32*(l/32), +32) of the 64-deep k-step; C lane l holds column l%32, rows
//    8i + 4*(l/32) + j in register 4i + j.
//  * One workgroup of 4 waves per query token (per split of its indices).
//    QK^T is formed transposed, S^T[j, h] = kv_j . q_h, with q as the B
//    operand in registers (72 VGPRs for 32 heads and 576 dims).  With 128
//    heads each wave owns a 32-head tile and both 32-row halves of a 64-row
//    KV tile; with 64 heads two waves share a head tile and take one half
//    each.
//  * PV contracts over 64 gathered rows per MFMA: O^T[c, h] += V^T[c, k]
//    P^T[k, h].  The P^T B-fragment is the QK^T C-fragment itself (lane (h,
//    g) holds its 32 rows' probabilities as 32 e4m3 bytes) once the MFMA row
//    of each gathered row is chosen so that the V^T A-fragment can be read
//    with gfx950's 8-bit transposing LDS load (ds_read_b64_tr_b8: in each
//    16-lane group, lanes 2r and 2r+1 give the address of row r's 16 bytes
//    and lane i receives byte i of all 8 rows; the row order is given at
//    vfrag below).  This replaces the K-major V copy that the TileLang page
//    builds in shared memory.
//  * All 4 waves share P through LDS and split the 512 output columns, so
//    each V fragment feeds one MFMA per 32-head tile and O (128 heads x 128
//    columns per wave) fills the AGPRs.
//  * KV tiles of 64 gathered rows go straight from global memory to LDS
//    (one 64-lane direct load per 16-byte unit of the row, lane = row) in
//    a unit-major layout, three tile buffers deep.  Software pipeline, one
//    iteration per tile: the PV of tile i-1 interleaved MFMA by MFMA with
//    the softmax of tile i, then the QK^T of tile i+1 with the loads of
//    tile i+2 issued between its k-steps; two barriers per iteration.
//  * Softmax in base 2 with sm_scale*log2(e) and q_scale folded into one
//    per-head factor.  The exponent reference of each head is the first
//    tile's max and is never moved, so O is only ever touched by MFMA; P is
//    2^(x - ref) * 16 * kv_scale_j / sigma (sigma = the largest kv_scale of
//    the row's indices) before the e4m3 cast.  If some score exceeds its
//    reference by more than log2(28) (P could pass the e4m3 maximum), the
//    workgroup restarts the token with a max-only pre-pass and a final pass
//    at the exact max with P = 2^(x - max) * 448 * kv_scale_j / sigma.  The
//    denominator sums the unrounded 2^(x - ref).
#include <type_traits>
#include <utility>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kDqk = 576, kDv = 512;
constexpr int kBI = 64;                  // gathered rows per tile
constexpr int kUnits = kDqk / 16;        // 16-byte units per row
constexpr int kBlocks = kUnits;          // LDS blocks per tile: 9 64-byte chunks x 4 row groups
constexpr int kBS = 16 * 64 + 64;        // LDS stride of a block (bytes): 16 rows x 64 + 64 pad
constexpr int kTile = kBlocks * kBS;     // LDS tile (bytes)
constexpr int kKS = kDqk / 64;           // 64-deep k-steps of QK^T
constexpr int kThreads = 256;
constexpr int kMaxK = 4096;
constexpr int kMaxTiles = kMaxK / kBI;
constexpr int kOTW = kDv / 32 / 4;       // 32-column O tiles per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kP0 = 16.f;              // P factor of the first pass
constexpr float kPMax = 448.f;           // P factor of the exact-max pass
constexpr float kHeadroom = 4.8f;        // < log2(448 / kP0)
static_assert(kUnits % 4 == 0, "units per wave");
static_assert(kBI == 64, "a 64-lane load fills one unit of a tile");

__device__ __forceinline__ f32x16 mfma_f8_32x32x64(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// QK^T MFMAs with the accumulator pinned to VGPRs, so that the O
// accumulators of PV (compiler-scheduled MFMAs) have the AGPRs to
// themselves: with both in AGPRs, 128 heads need more than a wave's 256.
// Hazards the compiler cannot see through the asm: the accumulator is tied
// (vdst = srcC), each MFMA is preceded by 2 wait states (VALU write -> MFMA
// read), and qk_drain() gives the results 24 wait states before any VALU
// reads them.
__device__ __forceinline__ void qk_mfma(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0"
               : "+v"(acc)
               : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_drain(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}

// LDS tile layout: block (c, G) holds bytes [64c, 64c+64) (chunk c) of tile
// rows [16G, 16G+16) at (4c + G) * kBS; inside it, the 16-byte unit p of
// row r (0..15) sits at slot 4r + (p ^ sw(r)), sw(r) = (r >> 2) & 3.  One
// 64-lane direct load fills one block, 4 lanes per row: 16 rows x 64
// contiguous bytes, i.e. 16 cache lines (one 16-byte unit of 64 rows per
// load touched 64, and the memory pipeline takes a gather load at about
// one line per cycle).  The swizzle keeps the QK^T operand read (16 rows,
// one unit each, per 16 lanes) and the transposing V read (8 rows x 16
// bytes per 16 lanes, 32 lanes per pass) free of bank conflicts.
__device__ __forceinline__ int unit_slot(int r, int p) { return 4 * r + (p ^ ((r >> 2) & 3)); }

// Workgroup barriers without the release fence of __syncthreads(), which
// waits for every outstanding global load, the direct-to-LDS loads of a
// tile still in flight included.  bar_lds(): this wave's LDS accesses are
// done (its LDS writes are visible to the workgroup after the barrier);
// bar_all(): its global loads (direct-to-LDS ones included) too.  The
// memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void bar_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void bar_all() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
using IC = std::integral_constant<int, N>;

// One direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4:
// lane l's bytes go to LDS address M0 + 16 l).  Written as inline asm so
// that the compiler, which cannot tell which LDS buffer such a load writes,
// does not make every later LDS read wait for it; the waits these loads
// need are explicit (bar_all()).  The compiler's own vmcnt waits stay
// correct: loads it does not know of only make them more conservative.
// One wait state separates the M0 write from the load that reads it.
// OFF is the instruction's offset, added to both the global and the LDS
// address.
template <int OFF>
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(src), "s"(lds_addr), "i"(OFF)
               : "memory", "m0");
}

// f(IC<0>{}), ..., f(IC<N-1>{}): a loop whose index is a compile-time
// constant in the body (register arrays indexed by it stay in registers
// however large the body grows).
template <class F, int... Ns>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Ns...>) {
  (f(IC<Ns>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct f32x8_pair {
  float4 a, b;
};

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

// Four fp32 -> four e4m3fn bytes (round to nearest even, a in byte 0; a
// value above 464 gives the NaN code).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int HQ, bool SPLIT>
__global__ __launch_bounds__(kThreads) void sparse_attn_fp8_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale,
    const float* __restrict__ sink, const int* __restrict__ idx, uint16_t* __restrict__ o,
    int M, int N, int K, float scale_log2, int S, int kspan, uint16_t* __restrict__ wso,
    float2* __restrict__ wsml) {
  static_assert(HQ == 64 || HQ == 128, "heads");
  constexpr int TS = 128 / HQ;   // waves per head tile (each takes 2/TS row halves)
  constexpr int NT = 2 / TS;     // 32-row halves per wave
  constexpr int NHT = HQ / 32;   // 32-head tiles
  __shared__ __align__(16) uint8_t sKV[3][kTile];
  __shared__ int sIdx[kMaxK];
  __shared__ int sList[kMaxTiles], sFirst[kMaxTiles];
  // per tile row: (kv_scale, score bias): (scale, 0) or (0, -inf) for an invalid slot
  __shared__ __align__(16) float2 sSB[3][kBI];
  // P^T fragments of tile i in buffer i % 2: [head tile][row half][lane]
  __shared__ __align__(16) i32x4 sP[2][NHT][2][kWave];
  __shared__ float sMx[TS][HQ], sLs[TS][HQ], sMf[HQ];
  __shared__ float sRed[kThreads / kWave];
  __shared__ int sNvt, sFlag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, hl = lane & 31;
  const int qht = wave / TS;                 // head tile of this wave's QK^T
  const int tau0 = TS == 2 ? wave % 2 : 0;   // first row half of this wave
  const int hq = qht * 32 + hl;              // this lane's head in QK^T / softmax
  const int c0 = wave * (kDv / 4);           // first output column of this wave's PV

  // workgroup -> (b, t) row, latest first, and split s of its K indices
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
  const int nidx = ntiles * kBI;

  // ---- prologue -------------------------------------------------------------
  // q fragments: lane (h, g) holds bytes [64s + 32g, +32) of its head's row
  i32x8 qf[kKS];
  {
    const uint8_t* qrow = q + ((size_t)rtok * HQ + hq) * kDqk + 32 * g;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(qrow + 64 * s);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(qrow + 64 * s + 16);
      qf[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  const float qsl = (q_scale ? q_scale[(size_t)rtok * HQ + hq] : 1.f) * scale_log2;
  // Indices: wave w takes tiles w, w+4, ... (a tile is 64 indices, one per
  // lane), all loaded before any is used.  Invalid indices (-1 or outside
  // [0, N)) become ~first, first = the tile's first valid index (negative:
  // still invalid; the row such a slot gathers, finite data whose
  // probability is exactly 0, is v ^ (v >> 31)).  sigma = the largest
  // kv_scale of the valid indices.
  const int* ridx = idx + (size_t)rtok * K + kbeg;
  const float* ksb = kv_scale + (size_t)b * N;
  constexpr int kTPW = kMaxTiles / 4;  // tiles per wave at most
  int vv[kTPW];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int p = (wave + 4 * j) * kBI + lane;
    vv[j] = p < klen ? ridx[p] : -1;
  }
  float smax = 0.f;
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int t = wave + 4 * j;
    int v = vv[j];
    v = (v >= 0 && v < N) ? v : -1;
    vv[j] = v;
    if (t < ntiles) {  // uniform over the wave
      const uint64_t mk = __ballot(v >= 0);
      const int first = mk ? __shfl(v, (int)__builtin_ctzll(mk), kWave) : -1;
      sIdx[t * kBI + lane] = v >= 0 ? v : (first >= 0 ? ~first : -1);
      if (lane == 0) sFirst[t] = first;
    }
  }
#pragma unroll
  for (int j = 0; j < kTPW; ++j)
    if (vv[j] >= 0) smax = fmaxf(smax, ksb[vv[j]]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) smax = fmaxf(smax, __shfl_xor(smax, sh, kWave));
  if (lane == 0) sRed[wave] = smax;
  if (tid == 0) sFlag = 0;
  __syncthreads();
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
  __syncthreads();
  float sigma = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) sigma = fmaxf(sigma, sRed[w]);
  const float inv_sigma = sigma > 0.f ? 1.f / sigma : 1.f;
  const int nvt = sNvt;

  // ---- staging: direct global -> LDS loads ---------------------------------
  // A tile buffer is 36 units; wave w fills units w, w+4, ... (9 each), one
  // 64-lane direct load per unit with lane l loading row l.  No VGPRs hold
  // the tile on its way; the wait for the loads comes right before the
  // barrier that publishes the tile.
  float2 psb = float2{0.f, -INFINITY};
  const uint8_t* kvb = kv + (size_t)b * N * kDqk;
  constexpr int kUPW = kUnits / 4;  // units per wave
  auto issue_sb_to = [&](int tile, float2& dst) __attribute__((always_inline)) {
    if (tid < kBI) {
      const int row = sIdx[tile * kBI + tid];
      dst = row >= 0 ? float2{ksb[row], 0.f} : float2{0.f, -INFINITY};
    }
  };
  auto issue_sb = [&](int tile) __attribute__((always_inline)) { issue_sb_to(tile, psb); };
  // LDS address of tile buffer 0 (the others follow at kTile-byte steps)
  const uint32_t kv_lds =
      (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)(&sKV[0][0]);
  // Wave w fills row group w (rows 16w..16w+15), chunks 0..8: lane l
  // writes slot l of the block, i.e. unit (l & 3) ^ sw(l >> 2) of row
  // 16w + (l >> 2) (invalid slots: the tile's first valid row).
  auto row_src = [&](int tile) __attribute__((always_inline)) {
    const int v = sIdx[tile * kBI + 16 * wave + (lane >> 2)];
    return kvb + (size_t)(v ^ (v >> 31)) * kDqk + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
  };
  // chunk k of this wave's row group, for the tile whose row addresses are in src
  auto issue_unit = [&](const uint8_t* src, int k, int buf) __attribute__((always_inline)) {
    const uint32_t lds = kv_lds + buf * kTile + wave * kBS;
    switch (k) {  // the global offset 64 k is an immediate (added to the LDS address too)
#define DSA_F8_UNIT(K) \
  case K: lds_dma16<64 * K>(src, __builtin_amdgcn_readfirstlane(lds + K * (4 * kBS - 64))); break;
      DSA_F8_UNIT(0) DSA_F8_UNIT(1) DSA_F8_UNIT(2) DSA_F8_UNIT(3) DSA_F8_UNIT(4)
      DSA_F8_UNIT(5) DSA_F8_UNIT(6) DSA_F8_UNIT(7) DSA_F8_UNIT(8)
#undef DSA_F8_UNIT
      default: break;
    }
  };
  auto issue_all = [&](int tile, int buf) __attribute__((always_inline)) {
    issue_sb(tile);
    const uint8_t* src = row_src(tile);
#pragma unroll
    for (int k = 0; k < kUPW; ++k) issue_unit(src, k, buf);
  };
  auto commit = [&](int buf) __attribute__((always_inline)) {
    if (tid < kBI) sSB[buf][tid] = psb;
  };
  // vmcnt(0): every global load of this wave, the direct-to-LDS ones
  // included, has landed
  auto wait_loads = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0f70); };

  // ---- per-tile pieces --------------------------------------------------------
  f32x16 oacc[NHT][kOTW];
  auto zero_o = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int oh = 0; oh < NHT; ++oh)
#pragma unroll
      for (int t = 0; t < kOTW; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[oh][t][e] = 0.f;
  };
  zero_o();
  float m = -1e30f;        // exponent reference of head hq (log2 units)
  float lsum = 0.f;        // this lane's share of sum 2^(x - m)
  float xmax = -INFINITY;  // largest x - m seen (first pass: overflow check)
  f32x16 sacc[NT];         // S^T of the tile in flight

  // QK^T operand: lane (r, g) of row half tau reads row 32 tau + r, units
  // 2g and 2g + 1 of chunk s (k-step s): row group 2 tau + r / 16
  const int aoff0 = (2 * tau0 + (hl >> 4)) * kBS + 16 * unit_slot(hl & 15, 2 * g);
  const int aoff1 = (2 * tau0 + (hl >> 4)) * kBS + 16 * unit_slot(hl & 15, 2 * g + 1);
  auto lda = [&](const uint8_t* sK, int s, int u) __attribute__((always_inline)) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(sK + aoff0 + (4 * s + 2 * u) * kBS);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(sK + aoff1 + (4 * s + 2 * u) * kBS);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // QK^T of a tile, one k-step at a time (the next step's operands are read
  // before this step's MFMAs; a scheduling barrier between steps keeps the
  // compiler from hoisting every read).  `extra(s)` runs after the MFMAs of
  // step s: the issue of the next tile's loads, spread over the k-steps.
  auto qk = [&](const uint8_t* sK, auto&& extra) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[u][e] = 0.f;
    i32x8 a[2][NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) a[0][u] = lda(sK, 0, u);
    static_for<kKS>([&](auto ss) __attribute__((always_inline)) {
      constexpr int s = decltype(ss)::value;
      if constexpr (s + 1 < kKS) {
#pragma unroll
        for (int u = 0; u < NT; ++u) a[(s + 1) & 1][u] = lda(sK, s + 1, u);
      }
#pragma unroll
      for (int u = 0; u < NT; ++u) qk_mfma(sacc[u], a[s & 1][u], qf[s]);
      extra(s);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int u = 0; u < NT; ++u) qk_drain(sacc[u]);
  };
  auto no_extra = [](int) __attribute__((always_inline)) {};
  // C registers 4i..4i+3 of row half tau hold rows 32 tau + 8i + 4g + 0..3:
  // their (scale, bias) pairs are two 16-byte reads
  auto rowsb = [&](const float2* sb, int tau, int i) __attribute__((always_inline)) {
    const float4* p4 = reinterpret_cast<const float4*>(sb + 32 * tau + 8 * i + 4 * g);
    return f32x8_pair{p4[0], p4[1]};
  };
  // largest x of the tile in flight for this lane's head (masked: -inf)
  auto tile_max = [&](const float2* sb) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x8_pair v = rowsb(sb, tau0 + u, i);
        mx = fmaxf(mx, fmaf(sacc[u][4 * i + 0], qsl * v.a.x, v.a.y));
        mx = fmaxf(mx, fmaf(sacc[u][4 * i + 1], qsl * v.a.z, v.a.w));
        mx = fmaxf(mx, fmaf(sacc[u][4 * i + 2], qsl * v.b.x, v.b.y));
        mx = fmaxf(mx, fmaf(sacc[u][4 * i + 3], qsl * v.b.z, v.b.w));
      }
    return fmaxf(mx, wave_xor(mx, 32));
  };

  // V^T A-fragment of output column tile t: slot 8q + r of lane half g is
  // row 16q + rr, rr = 8(r>>2) + 4g + (r&3), r = the row the lane pair (2r,
  // 2r+1) of each 16-lane group addresses; the lane's 8 bytes are half
  // l16 & 1 of unit c0/16 + 2t + ch: chunk c0/64 + t/2, unit 2(t&1) + ch,
  // row group q.
  const int l16 = lane & 15, trr = l16 >> 1, ch = (lane >> 4) & 1;
  int vo[2];  // read 0 of an even / odd column tile, within chunk c0/64
  {
    const int rr = 8 * (trr >> 2) + 4 * g + (trr & 3);
    vo[0] = (c0 / 64) * 4 * kBS + 16 * unit_slot(rr, ch) + 8 * (l16 & 1);
    vo[1] = (c0 / 64) * 4 * kBS + 16 * unit_slot(rr, 2 + ch) + 8 * (l16 & 1);
  }
  auto vfrag = [&](const uint8_t* sK, int t) __attribute__((always_inline)) {
    const uint8_t* vp = sK + vo[t & 1] + 4 * kBS * (t >> 1);
    const i32x2 r0 = lds_read_tr8(vp);
    const i32x2 r1 = lds_read_tr8(vp + kBS);
    const i32x2 r2 = lds_read_tr8(vp + 2 * kBS);
    const i32x2 r3 = lds_read_tr8(vp + 3 * kBS);
    return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  };

  // Phase 1 of an iteration: PV of the previous tile (WITH_PV) interleaved
  // with the softmax of the tile in flight, EPM softmax elements after each
  // MFMA, so that the VALU work issues while the MFMAs run.  P = 2^(x - m) *
  // kv_scale * pf goes to this wave's halves of the P^T fragments in dst.
  constexpr int NM = NHT * kOTW;     // PV MFMAs per wave and tile
  constexpr int NE = NT * 16;        // softmax elements per lane and tile
  constexpr int EPM = NE / NM;       // elements per MFMA
  static_assert(NE % NM == 0 && 4 % EPM == 0, "interleave");
  // PV runs over pairs of head tiles: the two P fragments of a pair stay in
  // registers for its kOTW column tiles (the V fragments are read once per
  // pair), which keeps 16 VGPRs of P live instead of 32.
  constexpr int OHG = NHT;  // head tiles per pair
  constexpr int NPAIR = NM / OHG;        // (pair, column tile) steps
  auto phase1 = [&](auto with_pv, const uint8_t* sKp, i32x4 (*sPp)[2][kWave],
                    const float2* sb, i32x4 (*sPc)[2][kWave], float pf) {
    constexpr bool WPV = decltype(with_pv)::value;
    i32x8 pb[OHG];
    i32x8 va[2];
    auto load_pb = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < OHG; ++k) {
        const i32x4 lo = sPp[grp * OHG + k][0][lane], hi = sPp[grp * OHG + k][1][lane];
        pb[k] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    if constexpr (WPV) {
      load_pb(0);
      va[0] = vfrag(sKp, 0);
    }
    f32x8_pair sbv[2];
    sbv[0] = rowsb(sb, tau0, 0);
    float p[4];
    int pk[4];
    static_for<NM>([&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (WPV) {
        constexpr int st = n / OHG, k = n % OHG;  // step (pair, column tile)
        constexpr int grp = st / kOTW, t = st % kOTW;
        if constexpr (k == 0 && st + 1 < NPAIR) va[(st + 1) & 1] = vfrag(sKp, (st + 1) % kOTW);
        oacc[grp * OHG + k][t] = mfma_f8_32x32x64(va[st & 1], pb[k], oacc[grp * OHG + k][t]);
        if constexpr (k == OHG - 1 && t == kOTW - 1 && grp + 1 < NHT / OHG) load_pb(grp + 1);
      }
      static_for<EPM>([&](auto kk) __attribute__((always_inline)) {
        constexpr int e = n * EPM + decltype(kk)::value, gi = e / 4, j = e % 4, u = gi / 4,
                      i = gi % 4;
        if constexpr (j == 0 && gi + 1 < NT * 4)
          sbv[(gi + 1) & 1] = rowsb(sb, tau0 + (gi + 1) / 4, (gi + 1) % 4);
        const f32x8_pair& v = sbv[gi & 1];
        const float ks = j == 0 ? v.a.x : j == 1 ? v.a.z : j == 2 ? v.b.x : v.b.z;
        const float bias = j == 0 ? v.a.y : j == 1 ? v.a.w : j == 2 ? v.b.y : v.b.w;
        const float tt = fmaf(sacc[u][4 * i + j], qsl * ks, bias) - m;
        xmax = fmaxf(xmax, tt);
        const float ex = fast_exp2(tt);
        lsum += ex;
        p[j] = ex * (ks * pf);
        if constexpr (j == 3) {
          pk[i] = pack_fp8x4(p[0], p[1], p[2], p[3]);
          if constexpr (i == 3) sPc[qht][tau0 + u][lane] = i32x4{pk[0], pk[1], pk[2], pk[3]};
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // PV alone (the last tile)
  auto pv_only = [&](const uint8_t* sKp, i32x4 (*sPp)[2][kWave]) {
    i32x8 pb[NHT];
#pragma unroll
    for (int oh = 0; oh < NHT; ++oh) {
      const i32x4 lo = sPp[oh][0][lane], hi = sPp[oh][1][lane];
      pb[oh] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int t = 0; t < kOTW; ++t) {
      const i32x8 va = vfrag(sKp, t);
#pragma unroll
      for (int oh = 0; oh < NHT; ++oh) oacc[oh][t] = mfma_f8_32x32x64(va, pb[oh], oacc[oh][t]);
    }
  };

  // Pipelined pass (mode 0: reference = the first tile's max, P factor 16;
  // mode 2: the exact max, P factor 448).  Iteration it: | PV of tile it-1
  // beside the softmax of tile it | QK^T of tile it+1 beside the issue of
  // tile it+2's loads |.  Three LDS tile buffers: tile i lives in buffer
  // i % 3 from its load (issued in iteration i-2) to its PV (iteration
  // i+1); the buffer tile it+2 goes to held tile it-1, whose PV ends before
  // the barrier that opens the second half.
  auto pipelined = [&]() __attribute__((always_inline)) {
    const float pf = kP0 * inv_sigma;
    if (nvt == 0) return;
    __syncthreads();  // every wave is past its previous use of the buffers
    // tiles 0 and 1 together: one wait
    float2 psb1 = float2{0.f, -INFINITY};
    issue_all(sList[0], 0);
    if (nvt > 1) {
      issue_sb_to(sList[1], psb1);
      const uint8_t* src = row_src(sList[1]);
#pragma unroll
      for (int k = 0; k < kUPW; ++k) issue_unit(src, k, 1);
    }
    wait_loads();
    commit(0);
    if (tid < kBI) sSB[1][tid] = psb1;
    __syncthreads();
    qk(sKV[0], no_extra);
    {
      float mx = tile_max(sSB[0]);
      if constexpr (TS == 2) {
        if (g == 0) sMx[tau0][hq] = mx;
        __syncthreads();
        mx = fmaxf(sMx[0][hq], sMx[1][hq]);
      }
      m = mx;  // the first tile holds a valid index: finite
    }
    // iteration it with tile it in buffer bc = it % 3 (its P goes to P
    // buffer bc as well)
    int bc = 0;
    auto step = [&](int it, auto later) __attribute__((always_inline)) {
      const int bp = bc == 0 ? 2 : bc - 1, bn = bc == 2 ? 0 : bc + 1;
      bar_lds();  // P of tile it-1 visible (tile it+2's loads stay in flight)
      phase1(later, sKV[bp], sP[(it - 1) & 1], sSB[bc], sP[it & 1], pf);
      if constexpr (decltype(later)::value) {
        if (it + 1 < nvt) commit(bn);  // row scales of tile it+1, loaded in the last iteration
      }
      bar_all();  // tile it+1 landed; P of tile it visible; tile it-1's buffer free
      if (it + 2 < nvt) {
        const int tile = sList[it + 2];
        issue_sb(tile);
        const uint8_t* src = row_src(tile);
        qk(sKV[bn], [&](int s) __attribute__((always_inline)) {
          if (s < kUPW) issue_unit(src, s, bp);
        });
      } else {
        qk(sKV[bn], no_extra);  // tile it+1 (past the last tile: unused)
      }
      bc = bn;
    };
    step(0, std::false_type{});
#pragma unroll 1
    for (int it = 1; it < nvt; ++it) step(it, std::true_type{});
    bar_all();  // P of the last tile visible
    const int bl = bc == 0 ? 2 : bc - 1;
    pv_only(sKV[bl], sP[(nvt - 1) & 1]);
  };
  // Max-only pass: the exact max of each head (one tile at a time).
  auto prepass = [&]() __attribute__((always_inline)) {
    m = -INFINITY;
#pragma unroll 1
    for (int it = 0; it < nvt; ++it) {
      __syncthreads();  // the previous tile's QK^T is done
      issue_all(sList[it], 0);
      wait_loads();
      commit(0);
      __syncthreads();
      qk(sKV[0], no_extra);
      m = fmaxf(m, tile_max(sSB[0]));
    }
    if constexpr (TS == 2) {
      if (g == 0) sMx[tau0][hq] = m;
      __syncthreads();
      m = fmaxf(sMx[0][hq], sMx[1][hq]);
    }
  };

  // Pass at the exact max (after a restart): one tile at a time.
  auto exact_pass = [&]() __attribute__((always_inline)) {
    const float pf = kPMax * inv_sigma;
#pragma unroll 1
    for (int it = 0; it < nvt; ++it) {
      __syncthreads();  // the previous tile's PV is done
      issue_all(sList[it], 0);
      wait_loads();
      commit(0);
      __syncthreads();
      qk(sKV[0], no_extra);
      phase1(std::false_type{}, sKV[0], sP[0], sSB[0], sP[1], pf);
      __syncthreads();
      pv_only(sKV[0], sP[1]);
    }
  };

  int mode = 0;
  pipelined();
  if (__ballot(xmax > kHeadroom) != 0ull && lane == 0) sFlag = 1;
  __syncthreads();
  if (sFlag != 0) {
    // some P could have passed the e4m3 range: exact max, then again
    zero_o();
    lsum = 0.f;
    __syncthreads();  // every wave is past its last tile
    prepass();
    mode = 2;
    exact_pass();
  }

  // ---- sink, normalise, store -------------------------------------------------
  // l of each head: this lane's share, both lane halves, both row halves
  {
    const float l = lsum + wave_xor(lsum, 32);
    if (g == 0) {
      sLs[tau0][hq] = l;
      if (tau0 == 0) sMf[hq] = m;
    }
  }
  __syncthreads();
  // O holds sum_j e4m3(2^(x_j - m) kv_scale_j pf) * code_j: o = O / (pf l)
  const float pf_out = (mode == 2 ? kPMax : kP0) * inv_sigma;
  float inv[NHT];
#pragma unroll
  for (int oh = 0; oh < NHT; ++oh) {
    const int h = oh * 32 + hl;
    float l = sLs[0][h];
    if constexpr (TS == 2) l += sLs[1][h];
    const float mh = sMf[h];
    if constexpr (SPLIT) {
      if (wave == 0 && g == 0) wsml[((size_t)rtok * S + split) * HQ + h] = float2{mh, l};
    } else {
      if (sink) l += fast_exp2(sink[h] * kLog2e - mh);
    }
    inv[oh] = l > 0.f ? __builtin_amdgcn_rcpf(l * pf_out) : 0.f;
  }
  if constexpr (SPLIT) {
    // this split's O / l in bf16 (0 without a valid index) into the
    // workspace, staged through LDS as in the unsplit epilogue below
    const size_t part = (size_t)rtok * S + split;
    constexpr int OS = kDv + 8;
    constexpr int ORP = 64;
    static_assert(ORP * OS * 2 <= 2 * kTile, "O staging");
    uint16_t* so = reinterpret_cast<uint16_t*>(&sKV[0][0]);
#pragma unroll
    for (int pass = 0; pass < HQ / ORP; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's rows are read
#pragma unroll
      for (int oh = 0; oh < NHT; ++oh) {
        const int hr = oh * 32 - pass * ORP;
        if (hr >= 0 && hr < ORP) {
          uint16_t* srow = so + (hr + hl) * OS + c0 + 4 * g;
#pragma unroll
          for (int t = 0; t < kOTW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& v = oacc[oh][t];
              uint2 pk2;
              pk2.x = pack_bf16x2(v[4 * i] * inv[oh], v[4 * i + 1] * inv[oh]);
              pk2.y = pack_bf16x2(v[4 * i + 2] * inv[oh], v[4 * i + 3] * inv[oh]);
              *reinterpret_cast<uint2*>(srow + 32 * t + 8 * i) = pk2;
            }
        }
      }
      __syncthreads();
      uint16_t* obase = wso + (part * HQ + pass * ORP) * kDv;
      for (int u = tid; u < ORP * (kDv / 8); u += kThreads) {
        const int r = u / (kDv / 8), c8 = u % (kDv / 8);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * kDv + c8 * 8) =
            *reinterpret_cast<const i32x4*>(so + r * OS + c8 * 8);
      }
    }
  } else {
    // bf16 O through LDS (the KV buffers, free now) in passes of 64 heads so
    // that each head row of o is written whole with 16-byte lanes
    constexpr int OS = kDv + 8;  // row stride (elements): 16-byte aligned rows
    constexpr int ORP = 64;      // head rows per pass (tile buffers 0 and 1)
    static_assert(ORP * OS * 2 <= 2 * kTile, "O staging");
    uint16_t* so = reinterpret_cast<uint16_t*>(&sKV[0][0]);
#pragma unroll
    for (int pass = 0; pass < HQ / ORP; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's rows are read
#pragma unroll
      for (int oh = 0; oh < NHT; ++oh) {
        const int hr = oh * 32 - pass * ORP;
        if (hr >= 0 && hr < ORP) {
          uint16_t* srow = so + (hr + hl) * OS + c0 + 4 * g;
#pragma unroll
          for (int t = 0; t < kOTW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x16& v = oacc[oh][t];
              uint2 pk2;
              pk2.x = pack_bf16x2(v[4 * i] * inv[oh], v[4 * i + 1] * inv[oh]);
              pk2.y = pack_bf16x2(v[4 * i + 2] * inv[oh], v[4 * i + 3] * inv[oh]);
              *reinterpret_cast<uint2*>(srow + 32 * t + 8 * i) = pk2;
            }
        }
      }
      __syncthreads();
      uint16_t* obase = o + ((size_t)rtok * HQ + pass * ORP) * kDv;
      for (int u = tid; u < ORP * (kDv / 8); u += kThreads) {
        const int r = u / (kDv / 8), c8 = u % (kDv / 8);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * kDv + c8 * 8) =
            *reinterpret_cast<const i32x4*>(so + r * OS + c8 * 8);
      }
    }
  }
}

// Splits of each row's K indices (decode: B*M at most half the compute
// units): S workgroups per row, at least 4 tiles each.  Returns S (1:
// unsplit) and the span of each split.
int fp8_splits(const AttnFp8Args& a, int& kspan) {
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

size_t fp8_split_bytes(const AttnFp8Args& a, int S) {
  if (S <= 1) return 0;
  return (size_t)(a.B * a.M) * S * a.Hq * (a.Dv * sizeof(uint16_t) + sizeof(float2));
}

template <int HQ>
hipError_t launch_fp8(const AttnFp8Args& a, Workspace ws, hipStream_t stream) {
  const long long rows = a.B * a.M;
  if (rows > 0x7fffffffLL || a.K > kMaxK || a.Hq != HQ) return hipErrorInvalidValue;
  const float scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / sqrtf((float)kDqk);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  int kspan;
  int S = fp8_splits(a, kspan);
  if (S > 1 && (ws.ptr == nullptr || ws.bytes < fp8_split_bytes(a, S))) {
    S = 1;
    kspan = a.K;
  }
  const uint8_t* q = static_cast<const uint8_t*>(a.q);
  const uint8_t* kv = static_cast<const uint8_t*>(a.kv);
  if (S == 1) {
    hipLaunchKernelGGL((sparse_attn_fp8_kernel<HQ, false>), dim3((unsigned)rows), dim3(kThreads),
                       0, stream, q, a.q_scale, kv, a.kv_scale, a.attn_sink, a.topk_idxs,
                       (uint16_t*)a.o, (int)a.M, (int)a.N, a.K, scale_log2, 1, a.K, nullptr,
                       nullptr);
    return hipGetLastError();
  }
  uint16_t* wso = static_cast<uint16_t*>(ws.ptr);
  float2* wsml = reinterpret_cast<float2*>(wso + (size_t)rows * S * HQ * kDv);
  hipLaunchKernelGGL((sparse_attn_fp8_kernel<HQ, true>), dim3((unsigned)(rows * S)),
                     dim3(kThreads), 0, stream, q, a.q_scale, kv, a.kv_scale, a.attn_sink,
                     a.topk_idxs, (uint16_t*)a.o, (int)a.M, (int)a.N, a.K, scale_log2, S, kspan,
                     wso, wsml);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_attn_merge(wso, wsml, a.attn_sink, (uint16_t*)a.o, rows, HQ, kDv, S, stream);
}

}  // namespace

bool attn_fp8_supported(int Hq, int Dqk, int Dv) {
  return (Hq == 64 || Hq == 128) && Dqk == kDqk && Dv == kDv;
}

size_t attn_fp8_workspace_bytes(const AttnFp8Args& a) {
  int kspan;
  return fp8_split_bytes(a, fp8_splits(a, kspan));
}

hipError_t launch_attn_fp8(const AttnFp8Args& a, Workspace ws, hipStream_t stream) {
  if (a.Dqk != kDqk || a.Dv != kDv) return hipErrorInvalidValue;
  if (a.Hq == 128) return launch_fp8<128>(a, ws, stream);
  if (a.Hq == 64) return launch_fp8<64>(a, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
