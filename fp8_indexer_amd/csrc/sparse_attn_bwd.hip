// sparse_attn_bwd.hip -- gradients of the gathered sparse attention with a
// sink, gfx950.
//
// Method (TileLang "deepseek_v32" page, "Sparse MLA Backward"), for each query
// token and head, over the gathered rows j of its top-k list:
//   p_j   = exp(s_j - lse)           (lse of the forward, sink included)
//   dp_j  = dO . V_j                 (V_j: the first Dv columns of row j)
//   Delta = dO . o                   (o: the forward output)
//   ds_j  = p_j (dp_j - Delta)
//   dq    = sm_scale sum_j ds_j kv_j
//   dkv_j += sm_scale ds_j q + p_j dO (first Dv columns), scattered to row j
//   dsink -= p_sink Delta
//
// Design (MI355X-first):
//  * One workgroup per (query token, group of 16 heads).  The token's
//    indices go to LDS once, with the list of its 16-row tiles that hold a
//    valid index (the others are skipped); 4 waves take the listed tiles in
//    turn (wave w: entries w, w+4, ...), each gathering its own tiles into
//    its own LDS buffer, so the waves never wait for each other inside the
//    loops.  The rows of a wave's next tile are loaded into registers while
//    it computes the current one.
//  * Pass 1 recomputes lse: S^T = KV.Q^T on v_mfma_f32_16x16x32_bf16 (q
//    B-fragments in VGPRs), an online max / sum per head, combined over the
//    lane groups and the waves, with the sink.
//  * Pass 2 per tile: S^T and dP^T = V.dO^T in the MFMA C layout (a lane
//    holds one head and 4 gathered rows), ds and p in registers; then
//      dq^T  += KV^T dS^T on v_mfma_f32_16x16x16_bf16: the C layout of dS^T
//               is its B-fragment, KV^T comes from the row-major tile through
//               the transposing LDS read (ds_read_b64_tr_b16); the 36 dq^T
//               tiles stay in AGPRs for the whole token;
//      dkv   = [scale dS | P] [q ; dO] on v_mfma_f32_16x16x32_bf16 with the
//               16 heads of dS and the 16 heads of P as the 32-deep k
//               dimension: A from a small LDS transpose of dS and P, B read
//               transposed from q and dO in LDS; the blocks are added to the
//               gathered rows of dkv with fp32 atomics (rows repeat across
//               tokens: the scatter of the pages' backward), two column
//               tiles at a time rearranged by a lane swap so that each
//               atomic instruction covers whole 128-byte lines.
//  * dq, dkv and dsink accumulate in fp32 (dq and dsink with atomics over
//    the waves and head groups); the entry point zero-fills them first.
//  * Invalid indices (-1 or outside [0, N)) gather nothing, have p = 0 and
//    add nothing.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr int kMaxKB = 4096;  // largest supported top-k

typedef short bs4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bs4 lds_bs4;

__device__ __forceinline__ bs4 tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bs4*)(p));
}

// D = A*B + C on a 16x16 fp32 tile, A/B 16x16 bf16 (4 values per lane):
// lane l holds A row l%16, k = 4(l/16)..+3; B column l%16, same k.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(const bs4& a, const bs4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int DQK, int DV>
struct BwdCfg {
  static_assert(DQK % 32 == 0 && DV % 32 == 0 && DV <= DQK, "dims");
  static constexpr int NW = 4;            // waves per workgroup
  static constexpr int THREADS = NW * kWave;
  static constexpr int HG = 16;           // heads per workgroup
  static constexpr int TR = 16;           // gathered rows per tile
  // LDS row strides (elements): odd numbers of 32-byte pairs, as in the
  // forward kernel, so that transposing reads of 4 rows x 32 bytes fill the
  // banks and 16-row 16-byte reads run at full rate
  static constexpr int RS = DQK + 16;
  static constexpr int GS = DV + 16;
  static_assert((RS * 2 / 32) % 2 == 1 && (GS * 2 / 32) % 2 == 1, "strides");
  static constexpr int KC = DQK / 32;     // 32-deep k-steps of S
  static constexpr int VC = DV / 32;      // 32-deep k-steps of dP
  static constexpr int DT = DQK / 16;     // 16-wide column tiles of dq / dkv
  static constexpr int VT = DV / 16;      // of which the first VT get the P.dO part
  static constexpr int CPR = DQK / 8;     // 16-byte chunks per kv row
  static constexpr int CPL = (TR * CPR + kWave - 1) / kWave;  // chunks per lane and tile
  static constexpr int TS = 40;           // row stride of the dS|P transpose (elements)
};

// NH = 1: one workgroup per (token, 16 heads), each wave alone on its own
// tiles.  NH = 2: one workgroup per (token, 32 heads); waves w and w + 2
// (heads 0-15 and 16-31 of the group) share each gathered tile, and each
// adds to dkv half of the columns, summed over all 32 heads: half the fp32
// atomics and half the gathers of NH = 1.
template <int DQK, int DV, int NH>
__global__ __launch_bounds__(256) void sparse_attn_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const float* __restrict__ sink, const int* __restrict__ idx, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dO, float* __restrict__ dq, float* __restrict__ dkv,
    float* __restrict__ dsink, int M, int N, int Hq, int K, float scale, float scale_log2) {
  using C = BwdCfg<DQK, DV>;
  constexpr int NW = C::NW, TR = C::TR, RS = C::RS, GS = C::GS;
  constexpr int HG = 16 * NH;       // heads per workgroup
  constexpr int NS = NW / NH;       // tile streams, NH waves each
  constexpr int CPW = C::CPL / NH;  // gather chunks per lane and wave
  constexpr int DTW = C::DT / NH;   // dkv column tiles per wave
  static_assert(NH == 1 || NH == 2, "head halves");
  static_assert(CPW * NH == C::CPL && DTW * NH == C::DT && DTW % 2 == 0, "splits");
  __shared__ __align__(16) uint16_t sKV[NS][TR * RS];
  __shared__ __align__(16) uint16_t sQ[HG * RS];
  __shared__ __align__(16) uint16_t sG[HG * GS];
  __shared__ __align__(16) uint16_t sT[NW][TR * C::TS];
  __shared__ int sIdx[kMaxKB];            // the row's indices, -1 if invalid
  __shared__ int sList[kMaxKB / TR];      // tiles holding a valid index
  __shared__ int sCnt[NW], sNvt;
  __shared__ float sM[NW][16], sL[NW][16], sDelta[HG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  // tile stream and head half (compile-time 0 for NH = 1)
  const int stream = NH == 1 ? wave : wave % NS, hl = NH == 1 ? 0 : wave / NS;
  const int hgs = Hq / HG;
  const int r = (int)(blockIdx.x / hgs);           // (b, t) row
  const int h0 = (int)(blockIdx.x % hgs) * HG;     // first head of the group
  const int hw = 16 * hl;                          // this wave's heads: h0 + hw + 0..15
  const int b = r / M;
  const int* ridx = idx + (size_t)r * K;
  const int ntiles = (K + TR - 1) / TR;  // <= THREADS (K <= kMaxKB)

  // ---- the row's indices, q and dO of the group's heads into LDS; Delta =
  // dO . o per head ------------------------------------------------------------
  {
    // invalid indices (-1 or outside [0, N)) and the padding of the last
    // tile read as -1
    for (int p = tid; p < ntiles * TR; p += C::THREADS) {
      const int v = p < K ? ridx[p] : -1;
      sIdx[p] = (v >= 0 && v < N) ? v : -1;
    }
    const uint16_t* qg = q + ((size_t)r * Hq + h0) * DQK;
    for (int u = tid; u < HG * (DQK / 8); u += C::THREADS) {
      const int hh = u / (DQK / 8), c8 = u % (DQK / 8);
      *reinterpret_cast<i32x4*>(&sQ[hh * RS + c8 * 8]) =
          *reinterpret_cast<const i32x4*>(qg + (size_t)hh * DQK + c8 * 8);
    }
    const uint16_t* gg = dO + ((size_t)r * Hq + h0) * DV;
    for (int u = tid; u < HG * (DV / 8); u += C::THREADS) {
      const int hh = u / (DV / 8), c8 = u % (DV / 8);
      *reinterpret_cast<i32x4*>(&sG[hh * GS + c8 * 8]) =
          *reinterpret_cast<const i32x4*>(gg + (size_t)hh * DV + c8 * 8);
    }
    // 16 heads per pass: wave w takes heads 4w..4w+3, 16 lanes per head
#pragma unroll
    for (int ps = 0; ps < NH; ++ps) {
      const int hh = ps * 16 + wave * 4 + g;
      const uint16_t* orow = o + ((size_t)r * Hq + h0 + hh) * DV;
      const uint16_t* grow = gg + (size_t)hh * DV;
      float acc = 0.f;
      for (int c = col; c < DV; c += 16)
        acc += __uint_as_float((uint32_t)orow[c] << 16) * __uint_as_float((uint32_t)grow[c] << 16);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
      if (col == 0) sDelta[hh] = acc;
    }
  }
  __syncthreads();
  // list of the tiles that hold a valid index, in order (one thread per tile)
  {
    bool any = false;
    if (tid < ntiles)
#pragma unroll
      for (int i = 0; i < TR; ++i) any = any || sIdx[tid * TR + i] >= 0;
    const uint64_t m = __ballot(any);
    if (lane == 0) sCnt[wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      off += w < wave ? sCnt[w] : 0;
      tot += sCnt[w];
    }
    if (any) sList[off + __popcll(m & ((1ull << lane) - 1ull))] = tid;
    if (tid == 0) sNvt = tot;
  }
  __syncthreads();
  const int nvt = sNvt;
  if (nvt == 0) return;  // uniform: no valid index, no gradient at all

  // q B-fragments (S^T = KV.Q^T): head hw + col, k-step c: columns 32c + 8g..+7
  bf16x8 qf[C::KC];
#pragma unroll
  for (int c = 0; c < C::KC; ++c)
    qf[c] = *reinterpret_cast<const bf16x8*>(&sQ[(hw + col) * RS + c * 32 + g * 8]);

  // ---- gathering: stream s takes list entries s, s + NS, ...; the rows of
  // its next tile are loaded into registers (a share per wave of the stream)
  // while it computes the current one (invalid slots load row 0 of the batch
  // entry: finite data whose p and ds are 0), so every load is unconditional
  uint16_t* kvt = sKV[stream];
  static_assert(C::CPL * kWave == TR * C::CPR, "whole chunks per lane");
  i32x4 nb[CPW];
  auto chunk = [&](int k) { return (k * NH + hl) * kWave + lane; };
  auto issue = [&](int e) {
    const int* ti = sIdx + sList[e] * TR;
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int ch = chunk(k);
      const int j = max(ti[ch / C::CPR], 0);
      nb[k] = *reinterpret_cast<const i32x4*>(kv + ((size_t)b * N + j) * DQK + (ch % C::CPR) * 8);
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int ch = chunk(k);
      *reinterpret_cast<i32x4*>(&kvt[(ch / C::CPR) * RS + (ch % C::CPR) * 8]) = nb[k];
    }
  };
  // One pass over the stream's tiles; body(act, ti, sync) runs for every
  // iteration (act: the stream has a tile in it) and calls sync() once at the
  // same place in every iteration.  NH = 1: no workgroup barriers, the wave
  // runs its own tiles.  NH = 2: every wave runs the same iteration count,
  // with barriers before a tile is stored (the stream's previous tile is no
  // longer read) and after (the tile complete).  The last iteration reloads
  // its own tile (never stored) so that the loads are unconditional.
  auto over_tiles = [&](auto&& body) {
    if constexpr (NH == 1) {
      if (stream < nvt) issue(stream);
      for (int e = stream; e < nvt; e += NS) {
        commit();
        __builtin_amdgcn_wave_barrier();
        issue(e + NS < nvt ? e + NS : e);
        body(true, sIdx + sList[e] * TR, [] { __builtin_amdgcn_wave_barrier(); });
        __builtin_amdgcn_wave_barrier();  // kvt is read until here
      }
    } else {
      const int niter = (nvt + NS - 1) / NS;
      if (stream < nvt) issue(stream);
      for (int it = 0, e = stream; it < niter; ++it, e += NS) {
        const bool act = e < nvt;  // uniform over the stream's waves
        __syncthreads();
        if (act) commit();
        __syncthreads();
        if (act) issue(e + NS < nvt ? e + NS : e);
        body(act, sIdx + sList[act ? e : 0] * TR, [] { __syncthreads(); });
      }
    }
  };
  // S^T of the current tile in the C layout: lane (col = head, g) holds rows
  // 4g + i; scores in log2 units, -inf for invalid rows
  auto scores = [&](const int* ti, float (&s2)[4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kvt[col * RS + c * 32 + g * 8]);
      acc = mfma_bf16_16x16x32(a, qf[c], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s2[i] = ti[4 * g + i] >= 0 ? acc[i] * scale_log2 : -INFINITY;
  };

  // ---- pass 1: lse per head (log2 units) ------------------------------------
  float mrun = -INFINITY, lrun = 0.f;  // per lane: its head, its rows
  over_tiles([&](bool act, const int* ti, auto&& sync) {
    if (act) {
      float s2[4];
      scores(ti, s2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (s2[i] == -INFINITY) continue;  // invalid row
        if (s2[i] > mrun) {
          lrun = lrun * fast_exp2(mrun - s2[i]);  // 0 * 0 while mrun is -inf
          mrun = s2[i];
        }
        lrun += fast_exp2(s2[i] - mrun);
      }
    }
    sync();
  });
  // combine the four lane groups of each head, then the waves of its half
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    const float mo = __shfl_xor(mrun, m, kWave), lo = __shfl_xor(lrun, m, kWave);
    const float mn = fmaxf(mrun, mo);
    lrun = (mrun == -INFINITY ? 0.f : lrun * fast_exp2(mrun - mn)) +
           (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mn));
    mrun = mn;
  }
  if (g == 0) {
    sM[wave][col] = mrun;
    sL[wave][col] = lrun;
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) mx = fmaxf(mx, sM[hl * NS + s][col]);
  const float sink2 = sink ? sink[h0 + hw + col] * kLog2eB : -INFINITY;
  // every head has a finite max: the row holds a valid index
  const float delta = sDelta[hw + col];
  float lse2, psink;
  {
    const float m2 = fmaxf(mx, sink2);
    float l = sink ? fast_exp2(sink2 - m2) : 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int w = hl * NS + s;
      l += sM[w][col] == -INFINITY ? 0.f : sL[w][col] * fast_exp2(sM[w][col] - m2);
    }
    lse2 = m2 + __log2f(l);
    psink = sink ? fast_exp2(sink2 - lse2) : 0.f;
  }
  if (stream == 0 && g == 0 && sink) unsafeAtomicAdd(dsink + h0 + hw + col, -psink * delta);

  // ---- pass 2 ----------------------------------------------------------------
  f32x4 dqa[C::DT];  // dq^T tiles: lane (col = head, g) holds columns 16t + 4g + i
#pragma unroll
  for (int t = 0; t < C::DT; ++t) dqa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* st = sT[wave];
  // transposing-read offsets: 4x16 blocks, lane (col) -> row col/4, column 4(col%4)
  const int trr = col >> 2, trc = 4 * (col & 3);
  over_tiles([&](bool act, const int* ti, auto&& sync) {
    if (act) {
      float s2[4];
      scores(ti, s2);
      // dP^T = V.dO^T
      f32x4 dpa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::VC; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kvt[col * RS + c * 32 + g * 8]);
        const bf16x8 bg =
            *reinterpret_cast<const bf16x8*>(&sG[(hw + col) * GS + c * 32 + g * 8]);
        dpa = mfma_bf16_16x16x32(a, bg, dpa);
      }
      // p and ds of rows 4g + i for this lane's head
      float p[4], ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(s2[i] - lse2);  // 0 for an invalid row
        ds[i] = p[i] * (dpa[i] - delta);
      }
      // dq^T += KV^T dS^T (k = the tile's 16 rows): B = dS^T in the C layout
      const bs4 dsb = __builtin_bit_cast(
          bs4, __builtin_convertvector(f32x4{ds[0], ds[1], ds[2], ds[3]}, bf16x4));
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        const bs4 a = tr16(&kvt[(4 * g + trr) * RS + 16 * t + trc]);
        dqa[t] = mfma_bf16_16x16x16(a, dsb, dqa[t]);
      }
      // dS and P transposed through LDS: st[j][k], k < 16: scale * ds of head
      // k, k >= 16: p of head k - 16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[(4 * g + i) * C::TS + col] = __builtin_bit_cast(uint16_t, (__bf16)(scale * ds[i]));
        st[(4 * g + i) * C::TS + 16 + col] = __builtin_bit_cast(uint16_t, (__bf16)p[i]);
      }
    }
    sync();  // the dS | P of every head half of the tile visible
    if (!act) return;
    // dkv[j, d] = sum_k A[j, k] B[k, d] over the NH head halves: A row col,
    // k = 8g..8g+7 of half hh's dS | P
    bf16x8 aT[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
      aT[hh] = *reinterpret_cast<const bf16x8*>(&sT[hh * NS + stream][col * C::TS + 8 * g]);
    // B row block k = 8g..8g+7 of half hh, column tile t: q heads (g < 2) or
    // dO heads (g >= 2), column 16t + col; two transposing reads of 4 heads
    // each (every lane reads; the dO columns past Dv are read in range and
    // replaced by zeros)
    auto dkv_tile = [&](int t) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const bool from_q = g < 2;
        const uint16_t* bp = from_q ? &sQ[(16 * hh + 8 * g + trr) * RS + 16 * t + trc]
                                    : &sG[(16 * hh + 8 * (g - 2) + trr) * GS +
                                          16 * (t < C::VT ? t : C::VT - 1) + trc];
        const int stride = from_q ? RS : GS;
        bs4 lo = tr16(bp), hi = tr16(bp + 4 * stride);
        if (!from_q && t >= C::VT) {
          lo = bs4{0, 0, 0, 0};
          hi = bs4{0, 0, 0, 0};
        }
        const bf16x8 bB = __builtin_bit_cast(bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0],
                                                            hi[1], hi[2], hi[3]});
        c = mfma_bf16_16x16x32(aT[hh], bB, c);
      }
      return c;
    };
    // This wave's column tiles, two at a time.  The C tiles of column tiles
    // t and t+1 hold, in lane (g, col), rows 4g + i at column col of each.
    // One v_permlane16_swap per i (the odd 16-lane groups of tile t exchanged
    // with the even ones of tile t+1) turns them into two sets of 2 rows x 32
    // consecutive columns: groups 0, 1 hold row 8(g/2) + i (first result) or
    // 8(g/2) + 4 + i (second), at column 16t + 16(g%2) + col.  Each atomic
    // instruction then covers two whole 128-byte lines of dkv instead of four
    // half lines.
    int jA[4], jB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      jA[i] = ti[8 * (g >> 1) + i];
      jB[i] = ti[8 * (g >> 1) + 4 + i];
    }
    float* dk = dkv + (size_t)b * N * DQK + 16 * (g & 1) + col;
    // column tiles of head half H (a compile-time index, so that every
    // column offset and the Dv test are constants)
    // (NH = 1 unrolls two pairs only: fully unrolled, its registers spill)
    constexpr int kColUnroll = NH == 1 ? 2 : DTW / 2;
    auto columns = [&](auto H) {
#pragma unroll kColUnroll
      for (int tt = 0; tt < DTW; tt += 2) {
        const int t = decltype(H)::value * DTW + tt;
        const f32x4 c0 = dkv_tile(t), c1 = dkv_tile(t + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (element values through __float_as_uint: a bit cast of a vector
          // element reads element 0 whatever the index)
          const auto sw = __builtin_amdgcn_permlane16_swap(
              __float_as_uint(c0[i]), __float_as_uint(c1[i]), false, false);
          const float va = __uint_as_float(sw[0]), vb = __uint_as_float(sw[1]);
          if (jA[i] >= 0) unsafeAtomicAdd(dk + (size_t)jA[i] * DQK + 16 * t, va);
          if (jB[i] >= 0) unsafeAtomicAdd(dk + (size_t)jB[i] * DQK + 16 * t, vb);
        }
      }
    };
    if (NH == 1 || hl == 0)
      columns(std::integral_constant<int, 0>{});
    else
      columns(std::integral_constant<int, NH - 1>{});
  });
  // dq of this wave's tiles (the streams' partial sums are added atomically)
  float* dqr = dq + ((size_t)r * Hq + h0 + hw + col) * DQK;
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dqr + 16 * t + 4 * g + i, scale * dqa[t][i]);
}

__global__ void fill_zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

hipError_t zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  const long long rows = a.B * a.M;
  const bool pair = a.Hq % 32 == 0;  // 32 heads per workgroup (NH = 2)
  const long long blocks = rows * (a.Hq / (pair ? 32 : 16));
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t err = zero(a.dq, (size_t)rows * a.Hq * DQK, stream);
  if (err == hipSuccess) err = zero(a.dkv, (size_t)a.B * a.N * DQK, stream);
  if (err == hipSuccess && a.dsink) err = zero(a.dsink, (size_t)a.Hq, stream);
  if (err != hipSuccess) return err;
  const float scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / sqrtf((float)DQK);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (pair)
    hipLaunchKernelGGL((sparse_attn_bwd_kernel<DQK, DV, 2>), dim3((unsigned)blocks),
                       dim3(BwdCfg<DQK, DV>::THREADS), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.kv, a.attn_sink, a.topk_idxs, (const uint16_t*)a.o,
                       (const uint16_t*)a.dO, a.dq, a.dkv, a.dsink, (int)a.M, (int)a.N, a.Hq,
                       a.K, scale, scale_log2);
  else
    hipLaunchKernelGGL((sparse_attn_bwd_kernel<DQK, DV, 1>), dim3((unsigned)blocks),
                       dim3(BwdCfg<DQK, DV>::THREADS), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.kv, a.attn_sink, a.topk_idxs, (const uint16_t*)a.o,
                       (const uint16_t*)a.dO, a.dq, a.dkv, a.dsink, (int)a.M, (int)a.N, a.Hq,
                       a.K, scale, scale_log2);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_supported(int Hq, int Dqk, int Dv) {
  if (Hq % 16 != 0 || Hq <= 0 || Hq > 128) return false;
  return (Dqk == 64 && Dv == 64) || (Dqk == 576 && Dv == 512);
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.Dqk == 64 && a.Dv == 64) return launch_bwd<64, 64>(a, stream);
  if (a.Dqk == 576 && a.Dv == 512) return launch_bwd<576, 512>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
