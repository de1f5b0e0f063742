// topk.hip -- exact per-row top-k on gfx950.
//
// Method (TileLang "deepseek_v32" page, "Top-k Selector"): floats become
// order-preserving unsigned keys; a histogram of the leading key bits and a
// cumulative sum locate the bin that holds the K-th largest value; only that
// bin is refined on the next bits, so the exact threshold is found without
// sorting the row.  Here the 32-bit key is resolved in up to three MSD
// rounds (11, 11, 10 bits; 12, 10, 10 for rows streamed from L2; 13, 10, 9
// for rows of up to 65536 keys held by one 1024-thread workgroup) with LDS
// histograms.
//
// Selection rule (this library's contract): the K keys of [s, e) first in
// (value descending, index ascending) order, with -0 == +0 and NaN ranked as
// -inf, written in ascending index order.  After the rounds the exact K-th
// key tau and the number of keys strictly above it are known; the emission
// pass walks the row in index order, 512 keys at a time, and uses wavefront
// ballots plus a block prefix sum to place every key > tau, and the first
// (K - #above) keys == tau, at their ascending output slot.  No atomics touch
// the output, so it is deterministic.
//
// Rows whose window has up to 8192 keys: one 256-thread workgroup per row,
// each wave holding a contiguous quarter of the row in VGPRs (digits of 11,
// 11 and 10 bits, a shared LDS histogram, wave-level scans; the rounds stop
// early once the threshold bin is wholly selected).
// The path is chosen per row from its own window, not from N: longer
// windows (only possible when N > 8192) are left to a second launch, which
// cuts them into 8192-key segments and reduces the segments' candidates, or,
// when that launch's candidate buffer would be large, gives each row one
// 512-thread workgroup that re-reads the row from L2 on each pass (digits
// 12, 10, 10).  With few rows (decode) and 8192 < N <= 65536 one 1024-thread
// workgroup per row holds the whole row in VGPRs (64 keys per lane), one
// launch; with few rows and N > 65536 every row is instead cut into
// 4096-key segments that share per-row digit histograms in global memory
// (one launch per round).  Rows with len <= K only write s..e-1 and -1
// padding.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kEPT = 16;  // register-resident keys per lane

// Order-preserving key: larger float -> larger unsigned key.  NaN -> key of
// -inf; -0 -> key of +0.
__device__ __forceinline__ uint32_t order_key(float v) {
  // -0 -> +0 (IEEE sum of opposite zeros); NaN -> -inf (maxNum returns the
  // operand that is not NaN)
  const float z = __builtin_fmaxf(v + 0.0f, -__builtin_inff());
  const uint32_t b = __float_as_uint(z);
  // negative: all bits flipped; positive: sign bit set
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// Row elements first + 64 c (c < KR) of a row of n floats into v[c], with
// 0.0 for positions >= n: buffer loads, whose range check against n does
// the bounds test (nothing is read past the row) with no per-lane address
// arithmetic; slots are grouped by 16 so that every slot's offset inside
// its group fits the instruction's immediate field.
template <int KR>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int n, int first,
                                         float (&v)[KR]) {
#pragma unroll
  for (int g = 0; g < KR; g += 16) {
    const int rem = n - g * kWave;  // elements of the row from this group on
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row) + g * kWave, (short)0, rem > 0 ? rem * 4 : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < 16 && g + j < KR; ++j)
      v[g + j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, first * 4 + j * kWave * 4, 0, 0));
  }
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value, so that per-wave loop bounds and offsets stay scalar.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Number of lanes below the calling lane whose bit is set in mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Key of element min(i, n - 1) of a row of n >= 1 floats.  Positions i >= n
// get a real key of the row: every user masks them by position.  The load is
// unconditional and always in bounds, so that a loop of these issues every
// load before waiting on the first (a load under a per-lane branch is waited
// for before the next one is issued).
__device__ __forceinline__ uint32_t key_clamped(const float* __restrict__ row, int i, int n) {
  return order_key(row[i < n ? i : n - 1]);
}

// Keys at positions >= n (loaded from a clamped position) become 0, which
// is below the key of every float (the smallest, -inf's, is 0x007FFFFF), so
// they are never selected, never equal the threshold, and fall into digit
// bin 0 of the first round, which no real key reaches: the counting and
// emission loops need no per-lane position test.  Position of keys[c]:
// first + 64 c.  The empty asm makes every load complete before the first
// test, so that the compiler cannot move the loads back under it.
template <int KR>
__device__ __forceinline__ void mask_tail(uint32_t (&keys)[KR], int first, int n) {
#pragma unroll
  for (int c = 0; c < KR; ++c) asm volatile("" : "+v"(keys[c]));
#pragma unroll
  for (int c = 0; c < KR; ++c) keys[c] = first + c * kWave < n ? keys[c] : 0u;
}

// Inclusive prefix sum over the 64 lanes (lane order) with DPP: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16 (lanes with no source add 0),
// then the last lane of each row is broadcast into the rows above it.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive prefix sum over the 512 threads of the block (thread order).
__device__ __forceinline__ int block_excl_scan(int v, int& total, int* sWave) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int x = wave_incl_scan(v);
  if (lane == 63) sWave[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    const int t = sWave[i];
    pre += i < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// One row (or, when skip_len > 0, only the rows longer than skip_len) per
// iteration of a grid-stride loop: the launch can stay small when most rows
// are left to the row kernel.
__device__ __forceinline__ void topk_stream_row(const float* __restrict__ logits,
                                                const int* __restrict__ ks,
                                                const int* __restrict__ ke,
                                                int* __restrict__ out, int N, int K,
                                                int skip_len, size_t r, uint32_t* hist,
                                                int* sWave, int (*sCnt)[kTkWaves], int* sSel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int s = clampi(ks[r], 0, N);
  const int e = clampi(ke[r], s, N);
  const int len = e - s;
  int* o = out + r * (size_t)K;
  if (skip_len > 0 && len <= skip_len) return;  // done by the row kernel

  if (len <= K) {  // short row: the whole window, then -1 padding
    for (int i = tid; i < K; i += kTkThreads) o[i] = i < len ? s + i : -1;
    return;
  }

  const float* row = logits + r * (size_t)N;
  const int nch = (len + kTkThreads - 1) / kTkThreads;
  const bool resident = nch <= kEPT;
  uint32_t keys[kEPT];
  if (resident) {
#pragma unroll
    for (int c = 0; c < kEPT; ++c) {
      const int i = s + c * kTkThreads + tid;
      keys[c] = key_clamped(row, c < nch ? i : e - 1, e);
    }
  }
  auto get = [&](int c) -> uint32_t {
    if (resident) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < kEPT; ++j) v = (j == c) ? keys[j] : v;
      return v;
    }
    const int i = s + c * kTkThreads + tid;
    return key_clamped(row, i, e);
  };

  // ---- three MSD rounds: 12 + 10 + 10 key bits ---------------------------
  uint32_t prefix = 0;
  int krem = K, above_total = 0;
#pragma unroll 1
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 20 : (round == 1 ? 10 : 0);
    const int nbins = round == 0 ? 4096 : 1024;
    const int pshift = shift + (round == 0 ? 12 : 10);  // bits above this digit
    for (int i = tid; i < nbins; i += kTkThreads) hist[i] = 0;
    __syncthreads();
    auto count = [&](int c, uint32_t u) {
      const int i = s + c * kTkThreads + tid;
      const bool match = i < e && (round == 0 || (u >> pshift) == prefix);
      if (match) atomicAdd(&hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
    };
    if (resident) {
#pragma unroll 1
      for (int c = 0; c < nch; ++c) count(c, get(c));
    } else {
      // 8 loads in flight before their keys are counted
#pragma unroll 1
      for (int c0 = 0; c0 < nch; c0 += 8) {
        uint32_t u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = c0 + j < nch ? get(c0 + j) : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + j < nch) count(c0 + j, u[j]);
      }
    }
    __syncthreads();
    // suffix counts: thread t owns bins [t*bpt, (t+1)*bpt)
    const int bpt = nbins / kTkThreads;
    int tsum = 0;
    for (int j = 0; j < bpt; ++j) tsum += (int)hist[tid * bpt + j];
    int total;
    const int pre = block_excl_scan(tsum, total, sWave);
    int above = total - pre - tsum;  // keys in bins owned by higher threads
    for (int j = bpt - 1; j >= 0; --j) {
      const int c = (int)hist[tid * bpt + j];
      if (above < krem && krem <= above + c) {
        sSel[0] = tid * bpt + j;
        sSel[1] = above;
      }
      above += c;
    }
    __syncthreads();
    const int bin = sSel[0], ab = sSel[1];
    prefix = (prefix << (round == 0 ? 12 : 10)) | (uint32_t)bin;
    krem -= ab;
    above_total += ab;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const int n_eq = K - above_total;  // keys equal to tau that are selected (>= 1)

  // ---- emission in index order -------------------------------------------
  // Wave w owns the contiguous segment [w*segw, (w+1)*segw) of the row (re-read
  // from L2): it counts its keys above tau and equal to tau, one barrier
  // exchanges the counts, then it writes its segment with ballots.
  const int segw = (len + kTkWaves * kWave - 1) / (kTkWaves * kWave) * kWave;
  const int wb = wave * segw;
  auto key_at = [&](int i) -> uint32_t { return key_clamped(row + s, i, len); };
  int gtc = 0, eqc = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < segw; c0 += 8 * kWave) {
    uint32_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = key_at(wb + c0 + j * kWave + lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = wb + c0 + j * kWave + lane;
      const bool in = c0 + j * kWave < segw && i < len;
      gtc += (int)__popcll(__ballot(in && u[j] > tau));
      eqc += (int)__popcll(__ballot(in && u[j] == tau));
    }
  }
  if (lane == 0) {
    sCnt[0][wave] = gtc;
    sCnt[1][wave] = eqc;
  }
  __syncthreads();
  int gt_base = 0, eq_base = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    gt_base += w < wave ? sCnt[0][w] : 0;
    eq_base += w < wave ? sCnt[1][w] : 0;
  }
  int eq_run = eq_base, sel_run = gt_base + min(eq_base, n_eq);
#pragma unroll 1
  for (int c0 = 0; c0 < segw; c0 += 8 * kWave) {
    uint32_t uu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uu[j] = key_at(wb + c0 + j * kWave + lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = wb + c0 + j * kWave + lane;
      const bool in = c0 + j * kWave < segw && i < len;
      const uint32_t u = uu[j];
      const bool eq = in && u == tau;
      const uint64_t meq = __ballot(eq);
      const bool sel = (in && u > tau) || (eq && eq_run + lanes_below(meq) < n_eq);
      const uint64_t msel = __ballot(sel);
      const int pos = sel_run + lanes_below(msel);
      if (sel && pos < K) o[pos] = s + i;
      sel_run += (int)__popcll(msel);
      eq_run += (int)__popcll(meq);
    }
  }
  __syncthreads();  // LDS is reused by the next row
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ logits,
                                                          const int* __restrict__ ks,
                                                          const int* __restrict__ ke,
                                                          int* __restrict__ out, int N, int K,
                                                          int skip_len, int rows) {
  __shared__ uint32_t hist[4096];
  __shared__ int sWave[kTkWaves];
  __shared__ int sCnt[2][kTkWaves];
  __shared__ int sSel[3];
  __shared__ int sRows[kTkThreads];
  __shared__ int sNum;
  if (skip_len <= 0) {
    for (int r = blockIdx.x; r < rows; r += gridDim.x)
      topk_stream_row(logits, ks, ke, out, N, K, 0, (size_t)r, hist, sWave, sCnt, sSel);
    return;
  }
  // Only rows longer than skip_len are this launch's.  Workgroup g owns rows
  // g, g + G, g + 2G, ...: each thread tests one of up to kTkThreads of them
  // at a time, the long ones are listed in LDS, and the workgroup then runs
  // them one by one.
  const long long G = gridDim.x;
  for (long long k0 = 0; k0 * G < rows; k0 += kTkThreads) {
    const long long rr = blockIdx.x + (k0 + threadIdx.x) * G;
    const int r = rr < rows ? (int)rr : rows;
    bool lng = false;
    if (r < rows) {
      const int s = clampi(ks[r], 0, N);
      lng = clampi(ke[r], s, N) - s > skip_len;
    }
    if (threadIdx.x == 0) sNum = 0;
    __syncthreads();
    if (lng) sRows[atomicAdd(&sNum, 1)] = r;  // order does not matter
    __syncthreads();
    const int n = sNum;
    for (int i = 0; i < n; ++i)
      topk_stream_row(logits, ks, ke, out, N, K, skip_len, (size_t)sRows[i], hist, sWave, sCnt,
                      sSel);
    __syncthreads();  // sRows and sNum are rewritten next
  }
}

// ---- four waves per row ----------------------------------------------------
// For rows of at most 256*KR keys: wave w holds the contiguous segment
// [w*64*KR, (w+1)*64*KR) of the row in VGPRs (lane l: keys w*64*KR + 64c +
// l), the histogram is shared in LDS, and digits are 11, 11 and 10 bits with
// three barriers per digit.  Emission: each wave counts its keys above tau
// and equal to tau, one barrier exchanges the counts, then every wave writes
// its segment in index order with ballots.  Same selection rule as above.
#ifndef DSA_TOPK_ROW_WAVES
#define DSA_TOPK_ROW_WAVES 4
#endif
constexpr int kRowWaves = DSA_TOPK_ROW_WAVES;  // waves per row (tuning knob)
constexpr int kRowThreads = kRowWaves * kWave;


// One MSD round's threshold: hist[0..nb) counts the remaining keys by digit
// (larger digit = larger key); returns the digit bin holding the krem-th
// largest of them (x), the number of keys in the bins above it (y) and the
// bin's own count (z).  Called by every thread of a workgroup of W waves;
// hist may be in LDS or in global memory; sRed holds W ints, sSel 3.
template <int W = kRowWaves>
__device__ __forceinline__ int3 threshold_bin(const uint32_t* hist, int nb, int krem, int* sRed,
                                              int* sSel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  // bins per thread; with fewer bins than threads, thread t owns bin t
  const int bpt = nb >= W * kWave ? nb / (W * kWave) : (tid < nb ? 1 : 0);
  int tsum = 0;
  for (int j = 0; j < bpt; ++j) tsum += (int)hist[tid * bpt + j];
  const int incl_w = wave_incl_scan(tsum);
  if (lane == 63) sRed[wave] = incl_w;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int t = sRed[w];
    pre += w < wave ? t : 0;
    total += t;
  }
  int above = total - (pre + incl_w);  // keys in bins of higher threads
  if (above < krem && krem <= above + tsum) {  // exactly one thread
    for (int j = bpt - 1; j >= 0; --j) {
      const int c = (int)hist[tid * bpt + j];
      if (above < krem && krem <= above + c) {
        sSel[0] = tid * bpt + j;
        sSel[1] = above;
        sSel[2] = c;
      }
      above += c;
    }
  }
  __syncthreads();
  return make_int3(sSel[0], sSel[1], sSel[2]);
}

// The same for a compile-time bin count NB, as the register-resident row
// kernels use it: each thread reads its NB / (64 W) consecutive bins once
// (16-byte reads when they come in fours, which keeps the 64 lanes of a read
// on distinct banks) and scans them from registers; with fewer bins than
// threads, thread t holds bin t.
template <int W, int NB>
__device__ __forceinline__ int3 threshold_bin_n(const uint32_t* hist, int krem, int* sRed,
                                                int* sSel) {
  constexpr int T = W * kWave, BPT = NB >= T ? NB / T : 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  uint32_t h[BPT];
  if constexpr (BPT % 4 == 0) {
#pragma unroll
    for (int q = 0; q < BPT / 4; ++q) {
      const uint4 x = reinterpret_cast<const uint4*>(hist + tid * BPT)[q];
      h[4 * q] = x.x;
      h[4 * q + 1] = x.y;
      h[4 * q + 2] = x.z;
      h[4 * q + 3] = x.w;
    }
  } else if constexpr (NB >= T) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) h[j] = hist[tid * BPT + j];
  } else {
    h[0] = tid < NB ? hist[tid] : 0u;
  }
  int tsum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) tsum += (int)h[j];
  const int incl_w = wave_incl_scan(tsum);
  if (lane == 63) sRed[wave] = incl_w;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int t = sRed[w];
    pre += w < wave ? t : 0;
    total += t;
  }
  int above = total - (pre + incl_w);  // keys in bins of higher threads
  if (above < krem && krem <= above + tsum) {  // exactly one thread
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      const int c = (int)h[j];
      if (above < krem && krem <= above + c) {
        sSel[0] = tid * BPT + j;
        sSel[1] = above;
        sSel[2] = c;
      }
      above += c;
    }
  }
  __syncthreads();
  return make_int3(sSel[0], sSel[1], sSel[2]);
}

// One wave's search for the same bin of hist[0..NB) (NB a multiple of 256):
// lane l sums its NB / 64 consecutive bins in groups of four, a wave scan
// finds the lane holding the krem-th largest key, and that lane narrows it
// to a group and then a bin.  Writes (bin, keys above it, its count) to
// sSel; the caller's barrier publishes them.  One barrier per round instead
// of two, for small bin counts (NB / 64 group sums stay in registers).
template <int NB>
__device__ __forceinline__ void threshold_wave(const uint32_t* hist, int krem, int* sSel) {
  constexpr int BPL = NB / kWave, G = BPL / 4;
  static_assert(BPL % 4 == 0, "groups of four bins");
  const int lane = threadIdx.x & 63;
  const uint4* hl = reinterpret_cast<const uint4*>(hist + lane * BPL);
  int gs[G];
  int tsum = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 x = hl[g];
    gs[g] = (int)(x.x + x.y + x.z + x.w);
    tsum += gs[g];
  }
  const int incl = wave_incl_scan(tsum);
  int above = __builtin_amdgcn_readlane(incl, 63) - incl;  // keys in higher lanes' bins
  if (above < krem && krem <= above + tsum) {  // exactly one lane
    int gsel = 0, asel = 0;
#pragma unroll
    for (int g = G - 1; g >= 0; --g) {
      if (above < krem && krem <= above + gs[g]) {
        gsel = g;
        asel = above;
      }
      above += gs[g];
    }
    const uint4 x = hl[gsel];
    const int c[4] = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (asel < krem && krem <= asel + c[j]) {
        sSel[0] = lane * BPL + 4 * gsel + j;
        sSel[1] = asel;
        sSel[2] = c[j];
      }
      asel += c[j];
    }
  }
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the wave's global loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A round's threshold after the histogram barrier: one wave for up to 2048
// bins, all waves (threshold_bin_n) for more.
template <int W, int NB>
__device__ __forceinline__ int3 threshold_step(const uint32_t* hist, int krem, int* sRed,
                                               int* sSel) {
  if constexpr (NB <= 2048) {
    if (wave_id() == 0) threshold_wave<NB>(hist, krem, sSel);
    __syncthreads();
    return make_int3(sSel[0], sSel[1], sSel[2]);
  } else {
    return threshold_bin_n<W, NB>(hist, krem, sRed, sSel);
  }
}

// Digit layout of the 32-bit key: rounds of 11, 11 and 10 bits.
__host__ __device__ constexpr int digit_bits(int round) { return round < 2 ? 11 : 10; }
// Register-resident rows: a first digit of B0 bits, then the remaining
// 32 - B0 bits in two rounds (B0 = 11: 11, 11, 10; B0 = 13: 13, 10, 9).
__host__ __device__ constexpr int rdigit_bits(int b0, int round) {
  return round == 0 ? b0 : (round == 1 ? (33 - b0) / 2 : 32 - b0 - (33 - b0) / 2);
}
__host__ __device__ constexpr int rdigit_shift(int b0, int round) {
  return round == 0 ? 32 - b0 : (round == 1 ? 32 - b0 - rdigit_bits(b0, 1) : 0);
}
__host__ __device__ constexpr int digit_shift(int round) {
  return round == 0 ? 21 : (round == 1 ? 10 : 0);
}

// Emission of a workgroup's keys (wave w holds positions w*64*KR + c*64 +
// lane, len of them; keys at positions >= len are 0, see mask_tail): every key > tau and the first n_eq keys == tau of the
// whole row go to o in ascending position order.  gt0 / eq0: keys > tau /
// == tau at positions before this workgroup's (other workgroups of the same
// row).  Writes o[pos] = first + i, or cand[i] when GATHER.
template <int KR, bool GATHER, int W = kRowWaves>
__device__ __forceinline__ void emit_selected(const uint32_t (&keys)[KR], int len, uint32_t tau,
                                              int n_eq, int gt0, int eq0, int first,
                                              const int* __restrict__ cand, int K,
                                              int* __restrict__ o, int (*sCnt)[W]) {
  constexpr int SEG = kWave * KR;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int base = wave * SEG;
  int gtc = 0, eqc = 0;
#pragma unroll
  for (int c = 0; c < KR; ++c) {
    if (base + c * kWave >= len) break;
    gtc += (int)__popcll(__builtin_amdgcn_ballot_w64(keys[c] > tau));
    eqc += (int)__popcll(__builtin_amdgcn_ballot_w64(keys[c] == tau));
  }
  if (lane == 0) {
    sCnt[0][wave] = gtc;
    sCnt[1][wave] = eqc;
  }
  __syncthreads();
  int gt_base = gt0, eq_base = eq0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    gt_base += w < wave ? sCnt[0][w] : 0;
    eq_base += w < wave ? sCnt[1][w] : 0;
  }
  // a key is selected if it is above tau, or equal to tau and among the
  // first n_eq such keys of the row; its slot is the number of selected
  // keys before it
  // The output goes through a buffer resource of K entries: its range check
  // drops any store past o[K - 1].  Keys equal to tau are rare (with
  // distinct values, one per row), so their test runs only in slots that
  // hold one.
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(o, (short)0, K * 4, 0x00020000);
  int eq_run = eq_base, sel_run = gt_base + min(eq_base, n_eq);
#pragma unroll
  for (int c = 0; c < KR; ++c) {
    if (base + c * kWave >= len) break;
    const int i = base + c * kWave + lane;
    const uint32_t u = keys[c];
    const bool eq = u == tau;
    const uint64_t meq = __builtin_amdgcn_ballot_w64(eq);
    bool sel = u > tau;
    if (meq != 0ull) sel = sel | (eq & (lanes_below(meq) + eq_run < n_eq));
    const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
    if (sel) {
      const int pos = lanes_below(msel) + sel_run;
      __builtin_amdgcn_raw_buffer_store_b32(GATHER ? cand[i] : first + i, ro, pos * 4, 0, 0);
    }
    sel_run += (int)__popcll(msel);
    eq_run += (int)__popcll(meq);
  }
}

// Keys of the register-resident rows are tested against the row length only
// once per kChunk slots: the keys of positions >= len are 0, which no key of
// a real value reaches (order_key maps -inf and NaN to 0x007FFFFF), so the
// few that a chunk holds land in bin 0 of the first round, which never holds
// the threshold (len > K real keys lie above it), and are never selected.
constexpr int kChunk = 8;

// Emission when exactly the keys >= tau are selected (K of them, no tie to
// rank): a wave's selected keys go to consecutive slots after those of the
// waves before it, in position order.  Layout and GATHER as emit_selected.
template <int KR, bool GATHER, int W = kRowWaves>
__device__ __forceinline__ void emit_at_least(const uint32_t (&keys)[KR], int len, uint32_t tau,
                                              int first, const int* __restrict__ cand, int K,
                                              int* __restrict__ o, int (*sCnt)[W]) {
  constexpr int SEG = kWave * KR;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int base = wave * SEG;
  int cnt = 0;  // per lane, summed over the wave below
#pragma unroll
  for (int c = 0; c < KR; ++c) {
    if (c % kChunk == 0 && base + c * kWave >= len) break;
    cnt += keys[c] >= tau ? 1 : 0;
  }
  cnt = wave_incl_scan(cnt);
  if (lane == 63) sCnt[0][wave] = cnt;
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) run += w < wave ? sCnt[0][w] : 0;
  run = __builtin_amdgcn_readfirstlane(run);  // wave-uniform: keep it scalar
  // stores through a buffer resource of K entries (its range check drops
  // any slot past o[K - 1])
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(o, (short)0, K * 4, 0x00020000);
#pragma unroll
  for (int c = 0; c < KR; ++c) {
    if (c % kChunk == 0 && base + c * kWave >= len) break;
    const int i = base + c * kWave + lane;
    const bool sel = keys[c] >= tau;
    const uint64_t m = __builtin_amdgcn_ballot_w64(sel);
    if (sel) {
      // slot run + (selected lanes below): the wave's part goes in soffset
      const int below = lanes_below(m);
      __builtin_amdgcn_raw_buffer_store_b32(GATHER ? cand[i] : first + i, ro, below * 4, run * 4,
                                            0);
    }
    run += (int)__popcll(m);
  }
}

// Writes to o[0..K) the positions (first + i, or cand[i] when GATHER) of the
// K largest of len > K keys src[i] (or src[cand[i]]), i < len, in ascending
// order of i.  Keys at most 64*W*KR.  Workgroup of W waves; the LDS arrays
// are the caller's.
template <int KR, bool GATHER, int W = kRowWaves, int B0 = 11>
__device__ __forceinline__ void row_select(const float* __restrict__ src,
                                           const int* __restrict__ cand, int len, int first,
                                           int K, int* __restrict__ o, uint32_t* hist, int* sRed,
                                           int* sSel, int (*sCnt)[W]) {
  constexpr int SEG = kWave * KR;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int base = wave * SEG;
  uint32_t keys[KR];
  if constexpr (GATHER) {
#pragma unroll
    for (int c = 0; c < KR; ++c) {
      const int i = base + c * kWave + lane;
      keys[c] = (uint32_t)cand[i < len ? i : len - 1];  // candidate positions first
    }
#pragma unroll
    for (int c = 0; c < KR; ++c)
      keys[c] = order_key(src[(int)keys[c]]);  // an in-row position for every lane
  } else {
    float v[KR];
    load_row<KR>(src, len, base + lane, v);
#pragma unroll
    for (int c = 0; c < KR; ++c) keys[c] = order_key(v[c]);
  }
  // both digit histograms are cleared while the loads are in flight
  {
    constexpr int nh = (1 << B0) + (1 << rdigit_bits(B0, 1));
    for (int i = 4 * tid; i < nh; i += 4 * W * kWave)
      *reinterpret_cast<uint4*>(hist + i) = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
  }
  // only the wave that holds the row's end has slots past it (later waves
  // skip all their slots)
  if (base < len && len < base + SEG) mask_tail<KR>(keys, base + lane, len);

  // After a round whose threshold bin holds exactly the keys still needed,
  // every key of that bin is selected, so the keys >= its smallest key (the
  // remaining digits zero) are exactly the K: the later rounds are skipped
  // (uniformly: the decision comes from LDS) and every key equal to that
  // bound is taken.
  uint32_t prefix = 0;
  int krem = K, above_total = 0, low_bits = 0, last_z = 0;
  uint32_t one = 1u;  // the atomics' operand, kept in one register
  asm volatile("" : "+v"(one));
#pragma unroll
  for (int round = 0; round < 3; ++round) {
    const int bits = rdigit_bits(B0, round), shift = rdigit_shift(B0, round);
    // rounds 0 and 2 count into h0, round 1 into h1 (both cleared up front;
    // h0 again during round 1)
    uint32_t* h = round == 1 ? hist + (1 << B0) : hist;
    if (low_bits == 0) {
      const int nb = 1 << bits;
      if (round == 1) {
        constexpr int nb2 = 1 << rdigit_bits(B0, 2);
        for (int i = tid; i < nb2; i += W * kWave) hist[i] = 0u;
      }
#pragma unroll
      for (int c = 0; c < KR; ++c) {
        // wave-uniform: the rest of the segment is empty
        if (c % kChunk == 0 && base + c * kWave >= len) break;
        const uint32_t u = keys[c];
        if (round == 0) {
          atomicAdd(&h[u >> shift], one);
        } else if (shift != 0) {
          // the keys under the prefix are those whose digit offset
          // (u >> shift) - (prefix << bits) is below nb; as a byte offset,
          // which cannot wrap into [0, 4 nb) while u >> shift < 2^29
          const uint32_t a = (__builtin_amdgcn_ubfe(u, shift, 32 - shift) << 2) -
                             (prefix << (bits + 2));
          if (a < (uint32_t)(4 * nb))
            atomicAdd(reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(h) + a), one);
        } else {
          const uint32_t d = u - (prefix << bits);
          if (d < (uint32_t)nb) atomicAdd(&h[d], one);
        }
      }
      __syncthreads();
      int3 sel;
      constexpr int nb0 = 1 << rdigit_bits(B0, 0), nb1 = 1 << rdigit_bits(B0, 1),
                    nb2 = 1 << rdigit_bits(B0, 2);
      if (round == 0) {
        sel = threshold_step<W, nb0>(h, krem, sRed, sSel);
      } else if (round == 1) {
        sel = threshold_step<W, nb1>(h, krem, sRed, sSel);
      } else {
        sel = threshold_step<W, nb2>(h, krem, sRed, sSel);
      }
      prefix = (prefix << bits) | (uint32_t)sel.x;
      krem -= sel.y;
      above_total += sel.y;
      last_z = sel.z;
      if (sel.z == krem) low_bits = shift;
    }
  }
  const uint32_t tau = prefix << low_bits;
  // all keys >= tau are selected after an early stop, or when the keys equal
  // to the full 32-bit tau are exactly the ones still needed
  if (low_bits || last_z == krem) {
    emit_at_least<KR, GATHER, W>(keys, len, tau, first, cand, K, o, sCnt);
  } else {
    const int n_eq = K - above_total;
    emit_selected<KR, GATHER, W>(keys, len, tau, n_eq, 0, 0, first, cand, K, o, sCnt);
  }
}

#define DSA_TOPK_LDS                                  \
  __shared__ __align__(16) uint32_t hist[4096];       \
  __shared__ int sRed[kRowWaves];                     \
  __shared__ int sSel[3];                             \
  __shared__ int sCnt[2][kRowWaves];

// W waves per row (W = kRowWaves: many rows; W = 16: the wide layout for
// few rows of up to 65536 keys, one 1024-thread workgroup per row and CU,
// which replaces several launches over row segments with one).
template <int KR, int W = kRowWaves, int B0 = 11>
__global__ __launch_bounds__(W * kWave) void topk_row_kernel(const float* __restrict__ logits,
                                                             const int* __restrict__ ks,
                                                             const int* __restrict__ ke,
                                                             int* __restrict__ out, int N, int K) {
  __shared__ __align__(16) uint32_t hist[(1 << B0) + (1 << rdigit_bits(B0, 1))];
  __shared__ int sRed[W];
  __shared__ int sSel[3];
  __shared__ int sCnt[2][W];
  const int tid = threadIdx.x;
  const size_t r = blockIdx.x;
  const int s = clampi(ks[r], 0, N);
  const int e = clampi(ke[r], s, N);
  const int len = e - s;
  int* o = out + r * (size_t)K;
  if (len <= K) {
    for (int i = tid; i < K; i += W * kWave) o[i] = i < len ? s + i : -1;
    return;
  }
  if (len > W * kWave * KR) return;  // a long row: the long-row kernels take it
  row_select<KR, false, W, B0>(logits + r * (size_t)N + s, nullptr, len, s, K, o, hist, sRed, sSel,
                               sCnt);
}

constexpr int kWideWaves = 16, kWideKR = 64;
// First-digit width of the register-resident row kernels (tuning knobs)
#ifndef DSA_TOPK_B0_ROW
#define DSA_TOPK_B0_ROW 11
#endif
#ifndef DSA_TOPK_B0_WIDE
#define DSA_TOPK_B0_WIDE 13
#endif
constexpr int kWideKeys = kWideWaves * kWave * kWideKR;  // 65536

// ---- long rows in two levels ----------------------------------------------
// Level 1: the row is cut into segments of kSegKeys keys and each segment's
// own top-K (or the whole segment if it is shorter) is written, in ascending
// index order, to K candidate slots per segment.  A key among the K first of
// the row in (value descending, index ascending) order has fewer than K keys
// ranked above it in the whole row, hence in its segment: the candidates
// hold the row's selection.  Level 2 selects the K first of the candidates
// (ranked by their logits, read back by index), whose storage order is the
// index order.
constexpr int kSegKeys = kRowThreads * 32;

__global__ __launch_bounds__(kRowThreads) void topk_seg_kernel(const float* __restrict__ logits,
                                                               const int* __restrict__ ks,
                                                               const int* __restrict__ ke,
                                                               int* __restrict__ cand, int N, int K,
                                                               int nseg, int skip_len) {
  DSA_TOPK_LDS
  const int tid = threadIdx.x;
  const size_t r = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x % nseg);
  const int s = clampi(ks[r], 0, N);
  const int e = clampi(ke[r], s, N);
  // level 2 writes rows of at most K keys directly; rows of at most
  // skip_len keys are the row kernel's
  if (e - s <= K || e - s <= skip_len) return;
  const int s0 = s + seg * kSegKeys;
  const int len = min(e - s0, kSegKeys);
  if (len <= 0) return;
  int* o = cand + (r * nseg + seg) * (size_t)K;
  if (len <= K) {
    for (int i = tid; i < len; i += kRowThreads) o[i] = s0 + i;
    return;
  }
  row_select<32, false>(logits + r * (size_t)N + s0, nullptr, len, s0, K, o, hist, sRed, sSel, sCnt);
}

template <int KR>
__global__ __launch_bounds__(kRowThreads) void topk_merge_kernel(const float* __restrict__ logits,
                                                                 const int* __restrict__ ks,
                                                                 const int* __restrict__ ke,
                                                                 const int* __restrict__ cand,
                                                                 int* __restrict__ out, int N, int K,
                                                                 int nseg, int skip_len) {
  DSA_TOPK_LDS
  const int tid = threadIdx.x;
  const size_t r = blockIdx.x;
  const int s = clampi(ks[r], 0, N);
  const int e = clampi(ke[r], s, N);
  const int len = e - s;
  int* o = out + r * (size_t)K;
  if (skip_len > 0 && len <= skip_len) return;  // done by the row kernel
  if (len <= K) {
    for (int i = tid; i < K; i += kRowThreads) o[i] = i < len ? s + i : -1;
    return;
  }
  // candidates: K per full segment, min(K, rest) for the last, contiguous
  const int ns = (len + kSegKeys - 1) / kSegKeys;
  const int n = (ns - 1) * K + min(K, len - (ns - 1) * kSegKeys);
  const int* c = cand + r * nseg * (size_t)K;
  if (n <= K) {  // a single segment of more than K keys: already selected
    for (int i = tid; i < K; i += kRowThreads) o[i] = c[i];
    return;
  }
  row_select<KR, true>(logits + r * (size_t)N, c, n, 0, K, o, hist, sRed, sSel, sCnt);
}

// ---- few long rows: several workgroups per row -----------------------------
// With few rows (decode) one workgroup per row leaves most CUs idle.  Each
// row is cut into segments of kSplitKeys keys, one workgroup each, and the
// three digit rounds run as separate launches: every workgroup adds its
// segment's LDS histogram of the round's digit (keys matching the prefix of
// the earlier rounds) into the row's global histogram, and each workgroup of
// a later launch derives the earlier rounds' threshold digits from the
// row's completed histograms (the launch boundary orders them; a fence per
// workgroup would write back the XCD's whole L2).  The last round also
// keeps, per segment, its keys above the 22-bit prefix and the suffix sums
// of its own last-digit histogram, from which the emission launch reads
// each earlier segment's keys > tau and == tau with two loads: every segment
// writes its selected keys at the offset they give, in ascending order with
// ties to the lower index, and no atomics touch the output.
constexpr int kSplitKR = 16;
constexpr int kSplitKeys = kRowThreads * kSplitKR;
// per row: 3 x 2048 histogram words; per segment: 1024 suffix sums and the
// count above the 22-bit prefix (kSplitSegWords, padded)
constexpr int kSplitRowWords = 3 * 2048;
constexpr int kSplitSegWords = 1028;

__global__ __launch_bounds__(kRowThreads) void topk_split_zero_kernel(uint32_t* __restrict__ ws) {
  uint32_t* h = ws + blockIdx.x * (size_t)kSplitRowWords;
  for (int i = threadIdx.x; i < kSplitRowWords; i += kRowThreads) h[i] = 0u;
}

// Segment of workgroup blockIdx.x (row r, segment seg): the keys in VGPRs in
// the wave-contiguous layout of emit_selected.  Returns the number of keys
// of the segment (<= 0: none), or -1 when the row has at most K keys.
__device__ __forceinline__ int split_load(const float* __restrict__ logits,
                                          const int* __restrict__ ks, const int* __restrict__ ke,
                                          int N, int K, int nseg, size_t& r, int& s0,
                                          uint32_t (&keys)[kSplitKR]) {
  r = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x % nseg);
  const int s = clampi(ks[r], 0, N);
  const int e = clampi(ke[r], s, N);
  if (e - s <= K) return -1;
  s0 = s + seg * kSplitKeys;
  const int n = min(e - s0, kSplitKeys);
  if (n <= 0) return 0;
  const float* src = logits + r * (size_t)N + s0;
  const int base = wave_id() * (kWave * kSplitKR) + (threadIdx.x & 63);
  float v[kSplitKR];
  load_row<kSplitKR>(src, n, base, v);
#pragma unroll
  for (int c = 0; c < kSplitKR; ++c) keys[c] = order_key(v[c]);
  mask_tail<kSplitKR>(keys, base, n);
  return n;
}

// Thresholds of rounds 0..nr-1 from the row's histograms h: the key prefix
// they fix and the number of keys above it.
__device__ __forceinline__ void split_prefix(const uint32_t* h, int nr, int K, uint32_t& prefix,
                                             int& above, int* sRed, int* sSel) {
  prefix = 0;
  above = 0;
  for (int q = 0; q < nr; ++q) {
    const int3 sel = threshold_bin(h + q * 2048, 1 << digit_bits(q), K - above, sRed, sSel);
    prefix = (prefix << digit_bits(q)) | (uint32_t)sel.x;
    above += sel.y;
  }
}

// Round ROUND: the segment's histogram of the digit over the keys that match
// the prefix fixed by the earlier rounds, added into the row's histogram.
template <int ROUND>
__global__ __launch_bounds__(kRowThreads) void topk_split_round_kernel(
    const float* __restrict__ logits, const int* __restrict__ ks, const int* __restrict__ ke,
    uint32_t* __restrict__ ws, int N, int K, int nseg) {
  __shared__ uint32_t lh[2048];
  __shared__ int sRed[kRowWaves];
  __shared__ int sSel[3];
  constexpr int bits = digit_bits(ROUND), shift = digit_shift(ROUND), nb = 1 << bits;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  size_t r;
  int s0;
  uint32_t keys[kSplitKR];
  const int n = split_load(logits, ks, ke, N, K, nseg, r, s0, keys);
  if (n <= 0) return;  // workgroup-uniform
  uint32_t* row = ws + r * kSplitRowWords;
  uint32_t* h = row + ROUND * 2048;
  uint32_t prefix;
  int above;
  split_prefix(row, ROUND, K, prefix, above, sRed, sSel);
  for (int i = tid; i < nb; i += kRowThreads) lh[i] = 0u;
  __syncthreads();
  const int base = wave * (kWave * kSplitKR) + lane;
  int gt = 0;  // keys above the prefix (last round)
#pragma unroll
  for (int c = 0; c < kSplitKR; ++c) {
    if (wave * (kWave * kSplitKR) + c * kWave >= n) break;  // wave-uniform
    const uint32_t u = keys[c];
    const bool v = base + c * kWave < n;
    if (v && (ROUND == 0 || (u >> (shift + bits)) == prefix))
      atomicAdd(&lh[(u >> shift) & (uint32_t)(nb - 1)], 1u);
    if (ROUND == 2) gt += (int)__popcll(__ballot(v && (u >> (shift + bits)) > prefix));
  }
  __syncthreads();
  int tsum = 0;
  constexpr int bpt = nb / kRowThreads;
  uint32_t hv[bpt];
#pragma unroll
  for (int j = 0; j < bpt; ++j) {
    hv[j] = lh[tid * bpt + j];
    tsum += (int)hv[j];
    if (hv[j]) atomicAdd(&h[tid * bpt + j], hv[j]);
  }
  if constexpr (ROUND == 2) {
    // this segment's suffix sums of the last-digit histogram, and its keys
    // above the 22-bit prefix
    const int incl_w = wave_incl_scan(tsum);
    if (lane == 63) sRed[wave] = incl_w;
    __syncthreads();
    int pre = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      const int x = sRed[w];
      pre += w < wave ? x : 0;
      total += x;
    }
    uint32_t* sg = ws + (size_t)gridDim.x / nseg * kSplitRowWords +
                   (size_t)blockIdx.x * kSplitSegWords;
    int suf = total - (pre + incl_w - tsum);
#pragma unroll
    for (int j = 0; j < bpt; ++j) {
      sg[tid * bpt + j] = (uint32_t)suf;
      suf -= (int)hv[j];
    }
    if (lane == 0) sSel[0] = 0;
    __syncthreads();
    if (lane == 0) atomicAdd(&sSel[0], gt);
    __syncthreads();
    if (tid == 0) sg[1024] = (uint32_t)sSel[0];
  }
}

// Emission (and the whole output of rows of at most K keys, by segment 0).
__global__ __launch_bounds__(kRowThreads) void topk_split_emit_kernel(
    const float* __restrict__ logits, const int* __restrict__ ks, const int* __restrict__ ke,
    const uint32_t* __restrict__ ws, int* __restrict__ out, int N, int K, int nseg) {
  __shared__ int sRed[kRowWaves];
  __shared__ int sSel[3];
  __shared__ int sCnt[2][kRowWaves];
  size_t r;
  int s0;
  uint32_t keys[kSplitKR];
  const int n = split_load(logits, ks, ke, N, K, nseg, r, s0, keys);
  const int seg = (int)(blockIdx.x % nseg);
  int* o = out + r * (size_t)K;
  if (n < 0) {  // at most K keys: the window, then -1 padding
    if (seg == 0) {
      const int s = clampi(ks[r], 0, N);
      const int len = clampi(ke[r], s, N) - s;
      for (int i = threadIdx.x; i < K; i += kRowThreads) o[i] = i < len ? s + i : -1;
    }
    return;
  }
  if (n == 0) return;
  uint32_t tau;
  int above;
  split_prefix(ws + r * kSplitRowWords, 3, K, tau, above, sRed, sSel);
  const int d = (int)(tau & 1023u);
  const uint32_t* sg = ws + (size_t)gridDim.x / nseg * kSplitRowWords +
                       (size_t)(r * nseg) * kSplitSegWords;
  int gt0 = 0, eq0 = 0;
  for (int q = 0; q < seg; ++q) {
    const uint32_t* x = sg + (size_t)q * kSplitSegWords;
    const int a1 = d < 1023 ? (int)x[d + 1] : 0;
    gt0 += (int)x[1024] + a1;
    eq0 += (int)x[d] - a1;
  }
  emit_selected<kSplitKR, false>(keys, n, tau, K - above, gt0, eq0, s0, nullptr, K, o, sCnt);
}

// Path of a call, chosen on the host from the sizes only (the windows are in
// device memory): the bytes of scratch it needs.
struct TopkPlan {
  enum Path { kRows, kWide, kSplit, kTwoLevel } path;
  int nseg;      // segments per row (split / two-level)
  size_t bytes;  // scratch
};

TopkPlan topk_plan(const TopkArgs& a) {
  const long long rows = a.B * a.M;
  // Few rows (decode) of up to 65536 keys: one wide workgroup per row.
  if (a.N > 8192 && a.N <= kWideKeys && rows < 256) return {TopkPlan::kWide, 1, 0};
  // Few rows (decode) with windows that may pass 8192 keys: several
  // workgroups per row, every row (see the split kernels).
  const long long split_nseg = (a.N + kSplitKeys - 1) / kSplitKeys;
  if (a.N > kRowThreads * (8192 / kRowThreads) && rows < 256 &&
      rows * split_nseg * kRowThreads <= 0xffffffffLL)
    return {TopkPlan::kSplit, (int)split_nseg,
            ((size_t)rows * kSplitRowWords + (size_t)rows * split_nseg * kSplitSegWords) *
                sizeof(uint32_t)};
  // Many rows, N > 8192: rows longer than 8192 keys in two levels through a
  // candidate buffer (sized for every row: the host does not know which rows
  // are long) while a row's candidates fit one workgroup's registers and the
  // buffer stays at most 256 MiB; else one streaming workgroup per long row.
  const int nseg = (int)((a.N + kSegKeys - 1) / kSegKeys);
  const long long ncand = (long long)nseg * a.K;
  const size_t cand_bytes = (size_t)rows * ncand * sizeof(int);
  if (a.N > kSegKeys && a.K <= kSegKeys && ncand <= kRowThreads * 64 &&
      rows * nseg <= 0x7fffffffLL && cand_bytes <= ((size_t)256 << 20))
    return {TopkPlan::kTwoLevel, nseg, cand_bytes};
  return {TopkPlan::kRows, nseg, 0};
}

}  // namespace

size_t topk_workspace_bytes(const TopkArgs& a) { return topk_plan(a).bytes; }

hipError_t launch_topk(const TopkArgs& a, Workspace ws, hipStream_t stream) {
  const long long rows = a.B * a.M;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr int kShort = kRowThreads * (8192 / kRowThreads);  // register-resident rows
  // Rows of up to 4096 keys: kRowWaves waves per row, keys in VGPRs.
  if (a.N <= kRowThreads * (4096 / kRowThreads)) {
    hipLaunchKernelGGL((topk_row_kernel<4096 / kRowThreads, kRowWaves, DSA_TOPK_B0_ROW>), dim3((unsigned)rows),
                       dim3(kRowThreads), 0, stream, a.logits, a.ks, a.ke, a.topk_idxs, (int)a.N,
                       (int)a.K);
    return hipGetLastError();
  }
  TopkPlan plan = topk_plan(a);
  if (plan.bytes > 0 && (ws.ptr == nullptr || ws.bytes < plan.bytes)) plan.path = TopkPlan::kRows;
  if (plan.path == TopkPlan::kWide) {
    hipLaunchKernelGGL((topk_row_kernel<kWideKR, kWideWaves, DSA_TOPK_B0_WIDE>), dim3((unsigned)rows),
                       dim3(kWideWaves * kWave), 0, stream, a.logits, a.ks, a.ke, a.topk_idxs,
                       (int)a.N, (int)a.K);
    return hipGetLastError();
  }
  if (plan.path == TopkPlan::kSplit) {
    uint32_t* w = static_cast<uint32_t*>(ws.ptr);
    const int nseg = plan.nseg;
    const dim3 grid((unsigned)(rows * nseg)), block(kRowThreads);
    hipLaunchKernelGGL(topk_split_zero_kernel, dim3((unsigned)rows), block, 0, stream, w);
    hipLaunchKernelGGL(topk_split_round_kernel<0>, grid, block, 0, stream, a.logits, a.ks, a.ke,
                       w, (int)a.N, (int)a.K, nseg);
    hipLaunchKernelGGL(topk_split_round_kernel<1>, grid, block, 0, stream, a.logits, a.ks, a.ke,
                       w, (int)a.N, (int)a.K, nseg);
    hipLaunchKernelGGL(topk_split_round_kernel<2>, grid, block, 0, stream, a.logits, a.ks, a.ke,
                       w, (int)a.N, (int)a.K, nseg);
    hipLaunchKernelGGL(topk_split_emit_kernel, grid, block, 0, stream, a.logits, a.ks, a.ke, w,
                       a.topk_idxs, (int)a.N, (int)a.K, nseg);
    return hipGetLastError();
  }
  // With few rows and two levels, the two-level kernels take every row, as
  // one more launch would cost more than the short rows gain.
  const bool two_level = plan.path == TopkPlan::kTwoLevel;
  const bool rows_first = !(two_level && rows < 256);
  const int skip_len = rows_first ? kShort : 0;
  hipError_t err = hipSuccess;
  if (rows_first) {
    hipLaunchKernelGGL((topk_row_kernel<8192 / kRowThreads, kRowWaves, DSA_TOPK_B0_ROW>), dim3((unsigned)rows),
                       dim3(kRowThreads), 0, stream, a.logits, a.ks, a.ke, a.topk_idxs, (int)a.N,
                       (int)a.K);
    err = hipGetLastError();
    if (err != hipSuccess || a.N <= kShort) return err;
  }
  if (two_level) {
    int* cand = static_cast<int*>(ws.ptr);
    const int nseg = plan.nseg;
    const long long ncand = (long long)nseg * a.K;
    hipLaunchKernelGGL(topk_seg_kernel, dim3((unsigned)(rows * nseg)), dim3(kRowThreads), 0,
                       stream, a.logits, a.ks, a.ke, cand, (int)a.N, (int)a.K, nseg, skip_len);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ncand <= kRowThreads * 16)
      hipLaunchKernelGGL(topk_merge_kernel<16>, dim3((unsigned)rows), dim3(kRowThreads), 0,
                         stream, a.logits, a.ks, a.ke, cand, a.topk_idxs, (int)a.N, (int)a.K,
                         nseg, skip_len);
    else if (ncand <= kRowThreads * 32)
      hipLaunchKernelGGL(topk_merge_kernel<32>, dim3((unsigned)rows), dim3(kRowThreads), 0,
                         stream, a.logits, a.ks, a.ke, cand, a.topk_idxs, (int)a.N, (int)a.K,
                         nseg, skip_len);
    else
      hipLaunchKernelGGL(topk_merge_kernel<64>, dim3((unsigned)rows), dim3(kRowThreads), 0,
                         stream, a.logits, a.ks, a.ke, cand, a.topk_idxs, (int)a.N, (int)a.K,
                         nseg, skip_len);
    return hipGetLastError();
  }
  // Rows longer than 8192 keys (all rows when the row kernel did not run):
  // one streaming workgroup per row, in a grid-stride loop over the rows so
  // that a launch in which most rows are short stays small.
  const long long sblocks = rows < 4LL * device_cus() ? rows : 4LL * device_cus();
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)sblocks), dim3(kTkThreads), 0, stream, a.logits,
                     a.ks, a.ke, a.topk_idxs, (int)a.N, (int)a.K, skip_len, (int)rows);
  return hipGetLastError();
}

}  // namespace dsa
