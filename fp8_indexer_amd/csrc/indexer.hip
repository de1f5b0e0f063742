// indexer.hip -- FP8 lightning-indexer scores on gfx950.
//
// Computes, for every query token t and every key in its window [s, e)
// (Modular "sparse_index_fp8_sm100_prefill" page, score formula; TileLang
// "deepseek_v32" page, "Lightning Indexer"):
//   logits[b,t,key] = k_scale[key] * sum_h relu(q[t,h,:].k[key,:]) * w[t,h] * q_scale[t,h]
//
// Design (MI355X-first):
//  * Q-resident: a workgroup owns a block of TB query tokens; each of its 8
//    waves keeps 128 (token, head) rows of q as MFMA A-fragments in VGPRs for
//    the whole launch.  Keys stream through LDS in 64-key tiles, double
//    buffered with a register prefetch, and every tile is shared by the 8
//    waves.  The product S[(t,h), key] = q . k runs on the OCP-fp8 MFMA
//    v_mfma_f32_16x16x128_f8f6f4 (one instruction covers a 128-deep dot).
//  * The MFMA C layout puts 4 consecutive (t,h) rows of one token in each
//    lane, so relu * w and most of the head sum are lane-local; the remaining
//    sum over the 4 lane groups is two cross-lane butterflies per (token, key).
//  * Work items are (token block, key chunk): a block only visits the chunks
//    of its clamped window union [min s, max e) (range skipping for causal and
//    packed variable-length inputs), and late token blocks, which have the
//    longest windows, are dispatched first.  Item ids are laid out so that all
//    chunks of one token block land on the same XCD, which keeps that block's
//    q in one L2.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

// Waves per workgroup (tuning knob): 4 lets two workgroups share a CU, so
// one's start-up (q loads, window reduction, first key tile) overlaps the
// other's tiles; 8 shares each key tile among more waves.
#ifndef DSA_IDX_WAVES
#define DSA_IDX_WAVES 4
#endif
constexpr int kIdxWaves = DSA_IDX_WAVES;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kRowsPerWave = 128;               // (token, head) rows per wave
constexpr int kRT = kRowsPerWave / 16;          // 16-row MFMA tiles per wave
#ifndef DSA_IDX_KT
#define DSA_IDX_KT 64
#endif
constexpr int kKT = DSA_IDX_KT;                 // keys per LDS tile (tuning knob)
constexpr int kXcds = 8;
constexpr int kMinChunk = 64;   // keys per chunk, at least (one key tile)
constexpr int kBalBlocks = 1024;  // key-parallel: token blocks of the balanced schedule, at most
#ifndef DSA_IDX_PIECE_OV
#define DSA_IDX_PIECE_OV 512
#endif
constexpr int kPieceOv = DSA_IDX_PIECE_OV;  // balanced schedule: start-up cost of a piece, in keys
// VALU instructions scheduled after each MFMA of the next sub-tile (tuning knob)
#ifndef DSA_IDX_VPM
#define DSA_IDX_VPM 10
#endif
constexpr int kIdxVpm = DSA_IDX_VPM;

// KP (key-parallel, for decode-like inputs with at most TW tokens per batch
// entry): all waves of a workgroup hold the same tokens and each takes one
// 16-key sub-tile of every key tile, instead of each wave owning its tokens.
// RT: 16-row MFMA tiles per wave (kRT; H / 16 for one token per wave, so
// that a single decode token fills every MFMA row).
template <int H, int D, bool KP, int RT_ = kRT>
struct IdxCfg {
  static_assert(H == 4 || H == 8 || H == 16 || H == 32 || H == 64 || H == 128, "H");
  static_assert(D == 64 || D == 128 || D == 256, "D");
  static_assert(RT_ == kRT || (KP && RT_ * 16 == H), "row tiles");
  static constexpr int RT = RT_;
  static constexpr int GR = 4 * RT;            // rows per lane group
  static constexpr int TW = 16 * RT / H;       // tokens per wave
  static constexpr int TB = KP ? TW : TW * kIdxWaves;  // tokens per workgroup
  static constexpr int KS = (D + 127) / 128;   // 128-deep MFMA steps
  static constexpr int CPR = D / 16;           // 16-byte chunks per key row
  // keys per LDS tile: larger when streaming a long key range per token
  // (more bytes in flight per workgroup), NS 16-key sub-tiles per wave
  static constexpr int KT = KP ? 256 : kKT;
  static constexpr int NS = KP ? KT / 16 / kIdxWaves : KT / 16;
  static constexpr int TILE_BYTES = KT * D;
  static constexpr int CHUNKS = KT * CPR;
  static constexpr int CPT = (CHUNKS + kIdxThreads - 1) / kIdxThreads;
  // Row placement: C element (row tile rt, lane group g, i) holds the row
  // with group-major index L = GR*g + 4*rt + i, i.e. token L / H, head L % H.
  // A lane group then holds whole tokens (H <= GR: TPL tokens per lane, no
  // cross-lane sum) or 1/GPT of one token (H > GR: GPT lane groups are
  // summed with 1 or 2 lane swaps).
  static constexpr int TPL = H < GR ? GR / H : 1;  // tokens per lane
  static constexpr int GPT = H > GR ? H / GR : 1;  // lane groups per token
};

// Sum of v over the lanes l and l^16 (S = 16) or l and l^32 (S = 32), using
// gfx950's row-swap permutes (no LDS round trip).  With both inputs equal,
// the two results are the two halves of the butterfly; the empty asm keeps
// the compiler from folding their sum as if they were the same value (it
// emits r0 + r0 without it).
template <int S>
__device__ __forceinline__ float lane_swap_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  unsigned a, c;
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = r[0];
    c = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = r[0];
    c = r[1];
  }
  asm volatile("" : "+v"(a), "+v"(c));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, c);
}

// Minimum over the 64 lanes of a wave: DPP within each 16-lane row, then
// the two row-swap permutes (no LDS round trip).
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  unsigned a, c;
  {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    a = r[0];
    c = r[1];
  }
  asm volatile("" : "+v"(a), "+v"(c));  // see lane_swap_sum
  v = min((int)a, (int)c);
  {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    a = r[0];
    c = r[1];
  }
  asm volatile("" : "+v"(a), "+v"(c));
  return min((int)a, (int)c);
}

// max(x, 0) for a non-NaN float as one integer max on its bits (negative
// floats are negative integers; -0 becomes +0), without the NaN-quieting
// canonicalisation that fmaxf costs.
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Byte offset of logical 16-byte chunk c of key row kk inside an LDS tile:
// chunks are XOR-swizzled by the row so that 16 lanes reading the same
// logical chunk of 16 consecutive rows hit different banks.
template <int D>
__device__ __forceinline__ int tile_off(int kk, int c) {
  constexpr int CPR = D / 16;
  return kk * D + ((c ^ (kk % CPR)) << 4);
}

template <int H, int D, bool KP, int RT>
__global__ __launch_bounds__(kIdxThreads) void indexer_logits_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale,
    const float* __restrict__ w, const int* __restrict__ ks,
    const int* __restrict__ ke, float* __restrict__ logits, int M, int N, int B,
    int n_tblocks, int n_chunks, int chunk_keys) {
  using C = IdxCfg<H, D, KP, RT>;
  static_assert(!KP || (C::KT / 16) % kIdxWaves == 0, "key-parallel: whole sub-tiles per wave");
  static_assert(C::KT <= kIdxThreads, "one key scale per thread");
  __shared__ __align__(16) uint8_t sK[2][C::TILE_BYTES];
  __shared__ float sKs[2][C::KT];
  __shared__ int sRed[2][kIdxWaves];
  __shared__ int sCum[KP ? kBalBlocks + 1 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;

  // ---- one item: (batch b, token block tb, keys [off0, off1) of the
  // block's window union, counted from its start) -------------------------
  auto process = [&](const int b, const int tb, const int off0, const int off1) {
  const int t0 = tb * C::TB;

  // ---- this wave's tokens: q fragments and effective weights (issued
  // before the window reduction, which they do not depend on) ------------
  const int tw0 = KP ? t0 : t0 + wave * C::TW;
  i32x8 qf[RT][C::KS];
  float weff[RT][4], qsc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // A row col of tile rt is C row (g', i') = (col / 4, col % 4)
    const int L = C::GR * (col >> 2) + 4 * rt + (col & 3);
    const int t = tw0 + L / H, h = L % H;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int d0 = s * 128 + g * 32;
      i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t < M && d0 < D) {
        const i32x4* p = reinterpret_cast<const i32x4*>(q + ((size_t)(b * M + t) * H + h) * D + d0);
        const i32x4 lo = p[0], hi = p[1];
        v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      qf[rt][s] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int L2 = C::GR * g + 4 * rt + i;
      const int t2 = tw0 + L2 / H, h2 = L2 % H;
      float we = 0.f, qs = 1.f;
      if (t2 < M) {
        const size_t o = (size_t)(b * M + t2) * H + h2;
        we = w[o];
        if (q_scale) qs = q_scale[o];
      }
      weff[rt][i] = we;  // times qsc once the loads are in (below)
      qsc[rt][i] = qs;
    }
  }
  // ---- window union of the block: [kmin, kmax) ---------------------------
  int smin = N, emax = 0;
  for (int i = tid; i < C::TB; i += kIdxThreads) {
    const int t = t0 + i;
    if (t < M) {
      const int r = b * M + t;
      const int s = clampi(ks[r], 0, N);
      const int e = clampi(ke[r], s, N);
      if (e > s) {
        smin = min(smin, s);
        emax = max(emax, e);
      }
    }
  }
  smin = wave_min(smin);
  emax = -wave_min(-emax);
  if (lane == 0) {
    sRed[0][wave] = smin;
    sRed[1][wave] = emax;
  }
  __syncthreads();
  int kmin = sRed[0][0], kmax = sRed[1][0];
#pragma unroll
  for (int i = 1; i < kIdxWaves; ++i) {
    kmin = min(kmin, sRed[0][i]);
    kmax = max(kmax, sRed[1][i]);
  }
  const int c0 = kmin + off0;
  if (kmin >= kmax || c0 >= kmax) return;  // uniform across the workgroup
  const int c1 = min(kmax, kmin + off1);

  // windows of the wave (for tile skipping) and of this lane's tokens
  // (token of slot j: (32*g)/H + j), clipped to the chunk so that
  // zero-filled keys are never written
  int wmin = N, wmax = 0;
  for (int tl = 0; tl < C::TW; ++tl) {
    const int t = tw0 + tl;
    if (t < M) {
      const int r = b * M + t;
      const int s = max(clampi(ks[r], 0, N), c0);
      const int e = min(clampi(ke[r], 0, N), c1);
      if (e > s) {
        wmin = min(wmin, s);
        wmax = max(wmax, e);
      }
    }
  }
  int ls[C::TPL], le[C::TPL];
  float* orow[C::TPL];
#pragma unroll
  for (int j = 0; j < C::TPL; ++j) {
    const int t = tw0 + (C::GR * g) / H + j;
    int s = 0, e = 0;
    if (t < M) {
      const int r = b * M + t;
      s = clampi(ks[r], 0, N);
      e = clampi(ke[r], s, N);
    }
    ls[j] = max(s, c0);
    le[j] = min(e, c1);
    orow[j] = logits + (size_t)(b * M + min(t, M - 1)) * N;
  }
  // a lane stores the sums of its tokens if it is the first of their groups
  const bool store_lane = (g % C::GPT) == 0;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) weff[rt][i] *= qsc[rt][i];

  // ---- K tile staging -----------------------------------------------------
  // Two register sets: the loads of tile t+2 are issued while tile t is
  // computed and stored to LDS at the end of tile t+1, so each load has two
  // tiles of compute to arrive.
  const int ntiles = (c1 - c0 + C::KT - 1) / C::KT;
  i32x4 pre2[2][C::CPT];
  float pks2[2] = {0.f, 0.f};
  // register set / LDS buffer of tile t: t & 1, a compile-time SETC below
  auto gload = [&](int tile, auto setc) {
    constexpr int SET = decltype(setc)::value;
    i32x4* pre = pre2[SET];
    float& pks = pks2[SET];
    const int kb = c0 + tile * C::KT;
    // Every load is issued and its data used as loaded: a key past the
    // range reads the range's last key, whose score column is computed but
    // never stored.  So nothing waits on a load before the tile's LDS store,
    // and the number of loads in flight does not depend on the data (the
    // wait before that store leaves the next tile's loads outstanding).
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int ch = tid + j * kIdxThreads;
      i32x4 v = {0, 0, 0, 0};
      if (C::CHUNKS % kIdxThreads == 0 || ch < C::CHUNKS) {
        const int key = min(kb + ch / C::CPR, c1 - 1);
        v = *reinterpret_cast<const i32x4*>(k + ((size_t)b * N + key) * D + (ch % C::CPR) * 16);
      }
      pre[j] = v;
    }
    if (C::KT >= kIdxThreads || tid < C::KT) pks = k_scale[(size_t)b * N + min(kb + tid, c1 - 1)];
  };
  auto lstore = [&](auto setc) {
    constexpr int SET = decltype(setc)::value;
    constexpr int buf = SET;
    const i32x4* pre = pre2[SET];
    const float pks = pks2[SET];
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int ch = tid + j * kIdxThreads;
      if (C::CHUNKS % kIdxThreads == 0 || ch < C::CHUNKS)
        *reinterpret_cast<i32x4*>(&sK[buf][tile_off<D>(ch / C::CPR, ch % C::CPR)]) = pre[j];
    }
    if (C::KT >= kIdxThreads || tid < C::KT) sKs[buf][tid] = pks;
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  gload(0, Set0{});
  gload(ntiles > 1 ? 1 : 0, Set1{});
  lstore(Set0{});
  __syncthreads();

  auto tile_step = [&](const int tile, auto setc) {
    constexpr int SET = decltype(setc)::value;
    constexpr int buf = SET;
    const int kb = c0 + tile * C::KT;
    gload(tile + 2 < ntiles ? tile + 2 : ntiles - 1, setc);  // the last tile again at the end
    // skip waves whose tokens do not see this tile
    if (wmax > kb && wmin < kb + C::KT) {
      // 16-key sub-tiles, software pipelined (128-deep keys): the MFMAs of
      // sub-tile n+1 are issued before the epilogue of sub-tile n
      constexpr int NB = C::KS == 1 ? 2 : 1;
      f32x4 acc[NB][RT];
      auto mm = [&](int n, f32x4* a) {
        const int kk = n * 16 + col;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          i32x8 bf = {0, 0, 0, 0, 0, 0, 0, 0};
          if (D % 128 == 0 || s * 128 + g * 32 < D) {
            const int c = s * 8 + g * 2;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(&sK[buf][tile_off<D>(kk, c)]);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(&sK[buf][tile_off<D>(kk, c + 1)]);
            bf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) a[rt] = mfma_f8_16x16x128(qf[rt][s], bf, a[rt]);
        }
      };
      // epilogue: relu * weight, sum over heads, * k_scale (epi_sum), masked
      // store (epi_store)
      auto epi_sum = [&](const f32x4* a, float* sum) {
        // 4 independent partial sums per token (short dependency chains)
        float part[C::TPL][4];
#pragma unroll
        for (int j = 0; j < C::TPL; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) part[j][i] = 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            part[(4 * rt + i) / (C::GR / C::TPL)][i] =
                fmaf(relu(a[rt][i]), weff[rt][i], part[(4 * rt + i) / (C::GR / C::TPL)][i]);
#pragma unroll
        for (int j = 0; j < C::TPL; ++j) sum[j] = (part[j][0] + part[j][1]) + (part[j][2] + part[j][3]);
        if constexpr (C::GPT >= 2) sum[0] = lane_swap_sum<16>(sum[0]);
        if constexpr (C::GPT >= 4) sum[0] = lane_swap_sum<32>(sum[0]);
      };
      auto epi_store = [&](int n, const float* sum) {
        const int kk = n * 16 + col;
        const float ksc = sKs[buf][kk];
        const int key = kb + kk;
#pragma unroll
        for (int j = 0; j < C::TPL; ++j)
          if (store_lane && key >= ls[j] && key < le[j]) orow[j][key] = sum[j] * ksc;
      };
      auto epi = [&](int n, const f32x4* a) {
        float sum[C::TPL];
        epi_sum(a, sum);
        epi_store(n, sum);
      };
      // this wave's sub-tiles: all of them, or (key-parallel) every
      // kIdxWaves-th one
      auto sub = [&](int j) { return KP ? j * kIdxWaves + wave : j; };
      if constexpr (NB == 2) {
        mm(sub(0), acc[0]);
#pragma unroll
        for (int j = 0; j < C::NS; ++j) {
          float sum[C::TPL];
          if (j + 1 < C::NS) {
            mm(sub(j + 1), acc[(j + 1) & 1]);
            epi_sum(acc[j & 1], sum);
            // interleave: the B-fragment LDS reads, then each MFMA of
            // sub-tile j+1 followed by a share of sub-tile j's VALU
            // epilogue, which the fp8 MFMA (32 cycles) hides
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
#pragma unroll
            for (int i = 0; i < RT * C::KS; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, kIdxVpm, 0);  // VALU
            }
          } else {
            epi_sum(acc[j & 1], sum);
          }
          epi_store(sub(j), sum);
        }
      } else {
#pragma unroll 1
        for (int j = 0; j < C::NS; ++j) {
          mm(sub(j), acc[0]);
          epi(sub(j), acc[0]);
        }
      }
    }
    if (tile + 1 < ntiles) lstore(std::integral_constant<int, SET ^ 1>{});
    __syncthreads();
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    tile_step(tile, Set0{});
    if (tile + 1 < ntiles) tile_step(tile + 1, Set1{});
  }
  };

  if constexpr (KP) {
    if (n_chunks > 0) {
      // one item per workgroup, items in id order (chunks of a batch entry
      // spread over the XCDs)
      const int per_batch = n_tblocks * n_chunks;
      const int id = blockIdx.x % per_batch;
      const int off = (id % n_chunks) * chunk_keys;
      process(blockIdx.x / per_batch, n_tblocks - 1 - id / n_chunks, off, off + chunk_keys);
      return;
    }
    // Balanced (n_chunks == 0; at most kBalBlocks token blocks): the window
    // unions of all blocks, laid end to end, are cut into gridDim.x equal
    // ranges of whole key tiles, one per workgroup, each processed as the
    // pieces it covers in every block it spans.  The host cannot size
    // chunks by the windows (they are in device memory); decode windows
    // differ by an order of magnitude between batch entries.
    const int nblk = B * n_tblocks;
    constexpr int kPer = kBalBlocks / kIdxThreads;  // blocks per thread
    int len[kPer], tsum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid * kPer + j;
      int smin = N, emax = 0;
      if (i < nblk) {
        const int bb = i / n_tblocks, tb = i % n_tblocks;
        for (int tl = 0; tl < C::TB; ++tl) {
          const int t = tb * C::TB + tl;
          if (t < M) {
            const int r = bb * M + t;
            const int s0 = clampi(ks[r], 0, N);
            const int e0 = clampi(ke[r], s0, N);
            if (e0 > s0) {
              smin = min(smin, s0);
              emax = max(emax, e0);
            }
          }
        }
      }
      // a piece costs its keys plus a start-up (q, weights, the first key
      // tiles' latency) worth about kPieceOv keys: the schedule counts it
      len[j] = emax > smin ? emax - smin + kPieceOv : 0;
      tsum += len[j];
    }
    // exclusive prefix of the block lengths in sCum[0..nblk], sCum[nblk] =
    // total (lane scan by shuffles, then the wave totals)
    int incl = tsum;
#pragma unroll
    for (int sh = 1; sh < kWave; sh <<= 1) {
      const int y = __shfl_up(incl, sh, kWave);
      if (lane >= sh) incl += y;
    }
    if (lane == kWave - 1) sRed[0][wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kIdxWaves; ++i) {
      before += i < wave ? sRed[0][i] : 0;
      total += sRed[0][i];
    }
    int run = before + incl - tsum;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid * kPer + j;
      if (i < nblk) sCum[i] = run;
      run += len[j];
    }
    if (tid == 0) sCum[nblk] = total;
    __syncthreads();
    const int G = (int)gridDim.x;
    const int per = (int)(((long long)total + G - 1) / G + C::KT - 1) / C::KT * C::KT;
    int pos = (int)min((long long)blockIdx.x * per, (long long)total);
    const int end = (int)min((long long)pos + per, (long long)total);
    // the block holding pos: the last i with sCum[i] <= pos (binary search)
    int lo = 0, hi = nblk - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sCum[mid] <= pos) lo = mid;
      else hi = mid - 1;
    }
    for (int i = lo; pos < end && i < nblk; ++i) {
      const int b0 = sCum[i], b1 = sCum[i + 1];
      if (b1 <= pos) continue;  // an empty block
      const int stop = min(end, b1);
      // the block's keys follow its start-up share [b0, b0 + kPieceOv)
      const int k0 = max(pos - b0 - kPieceOv, 0), k1 = stop - b0 - kPieceOv;
      if (k1 > k0) {
        __syncthreads();  // the previous piece's LDS reads are complete
        process(i / n_tblocks, i % n_tblocks, k0, k1);
      }
      pos = stop;
    }
  } else {
    // Persistent, per XCD: token blocks are numbered latest first
    // (descending work for causal-like windows) and block j belongs to XCD
    // j % 8, the XCD that runs workgroups g with g % 8 == j % 8 (workgroups
    // are dispatched to the XCDs round-robin).  Inside an XCD, its blocks'
    // items are numbered block-major (the chunks of a block are consecutive
    // items) and its L workgroups take them as a snake over rounds (local
    // workgroup l: items l, 2L-1-l, 2L+l, ...), which pairs long items with
    // short ones.  The chunks of a block then run at the same time on the
    // block's XCD, so its q comes from HBM once and from that XCD's L2 for
    // the other chunks.
    const int G = (int)gridDim.x, per_chunk = B * n_tblocks;
    const int nx = (G % kXcds == 0 && per_chunk >= 2 * kXcds) ? kXcds : 1;  // else one group
    const int x = (int)blockIdx.x % nx, l = (int)blockIdx.x / nx, L = G / nx;
    const int nbx = (per_chunk - x + nx - 1) / nx;  // blocks of this XCD
    const int n_items = nbx * n_chunks;
    for (int rnd = 0;; ++rnd) {
      const int item = rnd * L + ((rnd & 1) ? L - 1 - l : l);
      if (item >= n_items) break;
      __syncthreads();  // the previous item's LDS reads are complete
      const int rem = (item / n_chunks) * nx + x;  // block number, latest first
      const int off = (item % n_chunks) * chunk_keys;
      process(rem % B, n_tblocks - 1 - rem / B, off, off + chunk_keys);
    }
  }
}

template <int H, int D, bool KP, int RT = kRT>
hipError_t launch_kp(const IndexerArgs& a, hipStream_t stream) {
  using C = IdxCfg<H, D, KP, RT>;
  const int n_tblocks = (int)((a.M + C::TB - 1) / C::TB);
  // Key chunks: a chunk reloads its token block's q, so blocks are split
  // only as far as needed to give every workgroup slot of the device an item
  // (decode-like and small inputs with few token blocks), with chunks of at
  // least one key tile.
  // The persistent layout wants two items per workgroup, so that the snake
  // schedule can pair long windows with short ones.
  const int cus = device_cus();
  const long long slots = (long long)cus * (8 / kIdxWaves);  // 2 waves per SIMD, 4 SIMDs
  const long long tblocks = (long long)a.B * n_tblocks;
  const long long max_chunks = (a.N + kMinChunk - 1) / kMinChunk;
  const long long want = ((KP ? 1 : 2) * slots + tblocks - 1) / tblocks;
  const int n_chunks0 = (int)(want < 1 ? 1 : (want > max_chunks ? max_chunks : want));
  int chunk_keys = (int)((a.N + n_chunks0 - 1) / n_chunks0);
  chunk_keys = (chunk_keys + C::KT - 1) / C::KT * C::KT;
  const int n_chunks = (int)((a.N + chunk_keys - 1) / chunk_keys);
  const long long items = tblocks * n_chunks;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  if (KP && tblocks <= kBalBlocks && tblocks * (a.N + kPieceOv) <= 0x7fffffffLL) {
    // key-parallel, balanced over the device-side windows (n_chunks = 0)
    hipLaunchKernelGGL((indexer_logits_kernel<H, D, KP, RT>), dim3((unsigned)slots),
                       dim3(kIdxThreads), 0, stream, (const uint8_t*)a.q, a.q_scale,
                       (const uint8_t*)a.k, a.k_scale, a.w, a.ks, a.ke, a.logits, (int)a.M,
                       (int)a.N, (int)a.B, n_tblocks, 0, 0);
    return hipGetLastError();
  }
  const long long blocks = KP ? items : (items < slots ? items : slots);
  hipLaunchKernelGGL((indexer_logits_kernel<H, D, KP, RT>), dim3((unsigned)blocks), dim3(kIdxThreads), 0,
                     stream, (const uint8_t*)a.q, a.q_scale, (const uint8_t*)a.k, a.k_scale, a.w,
                     a.ks, a.ke, a.logits, (int)a.M, (int)a.N, (int)a.B, n_tblocks, n_chunks,
                     chunk_keys);
  return hipGetLastError();
}

// Few tokens per batch entry (decode): the key-parallel layout; one token
// per batch entry with fewer than 128 heads: H / 16 row tiles, no empty rows.
template <int H, int D>
hipError_t launch(const IndexerArgs& a, hipStream_t stream) {
  static_assert(kRowsPerWave == 128, "indexer_prefill_min_tokens assumes 128 rows per wave");
  if constexpr (H >= 16 && H < kRowsPerWave) {
    if (a.M == 1) return launch_kp<H, D, true, H / 16>(a, stream);
  }
  if (a.M < indexer_prefill_min_tokens(H)) return launch_kp<H, D, true>(a, stream);
  return launch_kp<H, D, false>(a, stream);
}

}  // namespace

bool indexer_supported(int H, int D) {
  const bool h = H == 4 || H == 8 || H == 16 || H == 32 || H == 64 || H == 128;
  const bool d = D == 64 || D == 128 || D == 256;
  return h && d;
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream) {
#define DSA_IDX_CASE(HH, DD) \
  if (a.H == HH && a.D == DD) return launch<HH, DD>(a, stream);
#define DSA_IDX_H(HH) DSA_IDX_CASE(HH, 64) DSA_IDX_CASE(HH, 128) DSA_IDX_CASE(HH, 256)
  DSA_IDX_H(4) DSA_IDX_H(8) DSA_IDX_H(16) DSA_IDX_H(32) DSA_IDX_H(64) DSA_IDX_H(128)
#undef DSA_IDX_H
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
