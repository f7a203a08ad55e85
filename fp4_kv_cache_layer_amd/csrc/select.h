// Segment-level exact Top-K selection shared by the Top-K / pool kernels and the fused
// scoring kernel (see topk.hip for the method).
#pragma once

#include "device.h"

namespace csa2 {


constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkEpt = 32;
constexpr int kTkSeg = kTkThreads * kTkEpt;

enum TkMode { kFromScores = 0, kFromBlockMax = 1, kFromKeys = 2 };

struct TkArgs {
  const float* scores;
  int64_t scores_stride;
  const int64_t* n_vis;
  int64_t max_vis;
  const int32_t* cand_blocks;    // pool slot map (kFromScores) or nullptr
  const int32_t* n_cand_blocks;
  int block;
  int max_cand_blocks;
  const uint64_t* keys_in;       // kFromKeys: [n_q, keys_in_per_q]
  int64_t keys_in_per_q;
  uint64_t* keys_out;            // non-final: [n_q, gridDim.x, k]
  int32_t* idx_out;              // final: [n_q, k]
  int32_t* count_out;            // final: [n_q]
  int k;
  int64_t n_slots;               // candidate slots per query at this level
  int vis_div;                   // kFromScores without a slot map: candidates are the first
                                 // ceil(n_vis / vis_div) scores (0 or 1: n_vis; block size
                                 // when the scores are block maxima)
};

__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t pos) {
  return ((uint64_t)ord_f32(s) << 32) | (uint64_t)(0xffffffffu - pos);
}
__device__ __forceinline__ int32_t key_pos(uint64_t k) { return (int32_t)(0xffffffffu - (uint32_t)k); }


// max / min over the wave with DPP row operations and four readlanes (no LDS traffic)
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false));  // row rotate 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false));  // row rotate 8
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}
__device__ __forceinline__ uint32_t dpp_min_u32(uint32_t v) { return ~dpp_max_u32(~v); }

// inclusive prefix sum over the wave with DPP: row shifts 1, 2, 4, 8 (zero fill) give each
// 16-lane row its own scan, then row broadcasts of lanes 15 and 31 carry the row totals
__device__ __forceinline__ uint32_t dpp_prefix_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr 1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr 2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr 4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr 8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast 15 -> rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast 31 -> rows 2, 3
  return v;
}


// A lower bound of the high word of a block's K-th largest key from one thread's largest
// (h1) and second largest (h2) high word of its keys (0 when it holds fewer than one or two
// keys): if every one of kThreads threads holds a key whose high word is at least b, at
// least kThreads keys are >= (b << 32), so the minimum of h1 over the block bounds the K-th
// largest key's high word from below when kThreads >= K, and the minimum of h2 does when
// 2 * kThreads >= K.  Returns this thread's share of that minimum (0: no bound).
__device__ __forceinline__ uint32_t prune_bound(uint32_t h1, uint32_t h2, int K, int threads) {
  return K <= threads ? h1 : (K <= 2 * threads ? h2 : 0u);
}

// Selects the K largest of the kEpt*kThreads keys held by a kThreads-thread workgroup (key[i]
// of thread t is candidate i*kThreads + t of the block; 0 = no candidate) and writes them
// in candidate order: non-final levels write the keys to keys_out[0 .. K), zero padded;
// the final level writes positions to idx_out[0 .. K), -1 padded, and *count_out (either
// may point to LDS).  `hist` is 2 * (kThreads / 64) * 256 * kTkCopies words of 16-byte
// aligned LDS; the caller may have used them for anything before the call (the first write
// to them follows the call's first barrier).  Each wave counts into kTkCopies interleaved
// copies of its 256 bins (word bin*kTkCopies + lane%kTkCopies), so lanes that hit the same
// bin land on different LDS banks: the digits of a segment's best keys bunch into few bins,
// and same-address atomics would serialise.  With more than four waves the selection also
// needs `scratch`: (kThreads / 256) * 256 + kWaves * kEpt words of LDS apart from `hist`
// (the two-stage histogram sums and the compaction counts); up to four waves it uses small
// static arrays of its own.
constexpr int kTkCopies = 4;
constexpr int kTkHistWords = 2 * kTkWaves * 256 * kTkCopies;

//
// Returns the selection's threshold key T (the same in every thread): the K selected keys
// are exactly the keys >= T (T = 0 when at most K keys are present, all of them kept), and
// any key < T ranks below all K of them.  kCopies (1 or kTkCopies) sets the histogram
// copies per wave: `hist` then holds 2 * (kThreads / 64) * 256 * kCopies words.
// kThreadMajor: key[i] of thread t is candidate t*kEpt + i instead (each thread holds a run
// of consecutive candidates), and the output follows that candidate order.
template <int kThreads, int kEpt, bool kFinal, int kCopies = kTkCopies, bool kThreadMajor = false>
__device__ __forceinline__ uint64_t select_block(uint64_t (&key)[kEpt], int K, uint32_t* hist,
                                                 uint64_t* __restrict__ keys_out, int32_t* __restrict__ idx_out,
                                                 int32_t* __restrict__ count_out, uint32_t* scratch = nullptr) {
  static_assert(kCopies == 1 || kCopies == kTkCopies, "one or four histogram copies");
  constexpr int kWaves = kThreads / 64;
  static_assert(kEpt <= 64 && kThreads % 64 == 0, "one lane per slot in the compaction scan");
  static_assert(!kThreadMajor || kEpt <= 32, "a thread's survivors as bits of one word");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t (*cnt)[kEpt];
  if constexpr (kWaves <= 4) {
    __shared__ uint32_t cnt_s[kWaves][kEpt];
    cnt = cnt_s;
  } else {
    cnt = reinterpret_cast<uint32_t(*)[kEpt]>(scratch + (kWaves / 4) * 256);
  }
  __shared__ uint32_t red[6][kWaves];

  // ---- count (ballots), the range of the high (score) words (DPP reductions) and a lower
  // bound of the K-th largest key's high word (prune_bound) ----
  uint32_t nw = 0, hmax = 0u, hmin = ~0u, lmax = 0u, lmin = ~0u, h2 = 0u;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    nw += (uint32_t)__popcll(__ballot(key[i] != 0ull));
    const uint32_t h = (uint32_t)(key[i] >> 32), l = (uint32_t)key[i];
    h2 = key[i] ? max(h2, min(hmax, h)) : h2;
    hmax = key[i] ? max(hmax, h) : hmax;
    hmin = key[i] ? min(hmin, h) : hmin;
    lmax = key[i] ? max(lmax, l) : lmax;
    lmin = key[i] ? min(lmin, l) : lmin;
  }
  const uint32_t tb = dpp_min_u32(prune_bound(hmax, h2, K, kThreads));
  hmax = dpp_max_u32(hmax);
  hmin = dpp_min_u32(hmin);
  lmax = dpp_max_u32(lmax);
  lmin = dpp_min_u32(lmin);
  if (lane == 0) {
    red[0][wave] = nw;
    red[1][wave] = hmax;
    red[2][wave] = hmin;
    red[3][wave] = lmax;
    red[4][wave] = lmin;
    red[5][wave] = tb;
  }
  __syncthreads();
  uint32_t n = 0, tmin = ~0u;
  hmax = 0u;
  hmin = ~0u;
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    n += red[0][wv];
    hmax = max(hmax, red[1][wv]);
    hmin = min(hmin, red[2][wv]);
    tmin = min(tmin, red[5][wv]);
  }

  // ---- radix select: find (prefix, mask) such that exactly K keys have (key&mask) >= prefix ----
  uint64_t prefix = 0, mask = 0;
  if (n > (uint32_t)K) {
    // keys below the bound rank below the K-th: drop them before the first count
    if (tmin > hmin) {
#pragma unroll
      for (int i = 0; i < kEpt; ++i) key[i] = (uint32_t)(key[i] >> 32) >= tmin ? key[i] : 0ull;
      hmin = tmin;
    }
    int hb;        // highest bit where the largest and smallest key differ
    uint64_t top;  // the largest key's bits above hb
    if (hmax != hmin) {
      hb = 32 + 31 - __clz(hmax ^ hmin);
      top = (uint64_t)hmax << 32;
    } else {       // every remaining score equal: the keys differ in their position words
      lmax = 0u;     // only (whose range over all keys covers those that remain)
      lmin = ~0u;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        lmax = max(lmax, red[3][wv]);
        lmin = min(lmin, red[4][wv]);
      }
      hb = 31 - __clz(lmax ^ lmin);  // n >= 2 unique keys: lmax != lmin
      top = ((uint64_t)hmax << 32) | lmax;
    }
    mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    prefix = top & mask;
    int shift = hb - 7 > 0 ? hb - 7 : 0;
    uint32_t need = (uint32_t)K;
    for (int pass = 0;; ++pass) {
      uint32_t* h = hist + ((pass & 1) * kWaves + wave) * 256 * kCopies;
#pragma unroll
      for (int i = 0; i < kCopies; ++i)
        reinterpret_cast<uint4*>(h)[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
      uint32_t* hc = h + (lane & (kCopies - 1));
#pragma unroll
      for (int i = 0; i < kEpt; ++i)
        if (key[i] && (key[i] & mask) == prefix) atomicAdd(&hc[((uint32_t)(key[i] >> shift) & 255u) * kCopies], 1u);
      __syncthreads();
      // every wave: lane l owns bins 4l..4l+3 of the histogram summed over waves and copies
      uint32_t hs[4] = {0u, 0u, 0u, 0u};
      if constexpr (kWaves <= 4) {
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
          const uint4* hw = reinterpret_cast<const uint4*>(hist + ((pass & 1) * kWaves + wv) * 256 * kCopies);
          if constexpr (kCopies == 1) {
            const uint4 c = hw[lane];
            hs[0] += c.x;
            hs[1] += c.y;
            hs[2] += c.z;
            hs[3] += c.w;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint4 c = hw[4 * lane + j];
              hs[j] += c.x + c.y + c.z + c.w;
            }
          }
        }
      } else {
        // More waves: every wave reading every histogram would cost LDS reads that grow
        // with the square of the wave count, so first thread t sums bin t % 256 over the
        // four waves of group t / 256 (one thread per group and bin), then every wave adds
        // the groups' sums.
        static_assert(kWaves % 4 == 0, "waves in groups of four");
        constexpr int kGroups = kWaves / 4;
        uint32_t (*part)[256] = reinterpret_cast<uint32_t(*)[256]>(scratch);
        {
          const int b = tid & 255, g = tid >> 8;
          uint32_t sum = 0u;
#pragma unroll
          for (int wv = 4 * g; wv < 4 * g + 4; ++wv) {
            if constexpr (kCopies == 1) {
              sum += hist[((pass & 1) * kWaves + wv) * 256 + b];
            } else {
              const uint4 c = reinterpret_cast<const uint4*>(hist + ((pass & 1) * kWaves + wv) * 256 * kCopies)[b];
              sum += c.x + c.y + c.z + c.w;
            }
          }
          part[g][b] = sum;
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const uint4 c = reinterpret_cast<const uint4*>(part[g])[lane];
          hs[0] += c.x;
          hs[1] += c.y;
          hs[2] += c.z;
          hs[3] += c.w;
        }
      }
      const uint32_t tot = hs[0] + hs[1] + hs[2] + hs[3];
      const uint32_t pre = dpp_prefix_sum(tot);
      const uint32_t incl = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + tot;  // bins >= 4*lane
      const uint32_t above_lane = incl - tot;
      // the boundary digit is the largest d with (count of digits >= d) >= need
      uint32_t d = 0, above = 0, inbin = 0;
      const bool mine = above_lane < need && incl >= need;
      if (mine) {
        uint32_t acc = above_lane;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (acc + hs[j] >= need) {
            d = 4 * lane + j;
            above = acc;
            inbin = hs[j];
            break;
          }
          acc += hs[j];
        }
      }
      const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
      d = __builtin_amdgcn_readlane(d, owner);
      above = __builtin_amdgcn_readlane(above, owner);
      inbin = __builtin_amdgcn_readlane(inbin, owner);
      need -= above;
      prefix |= (uint64_t)d << shift;
      mask |= 255ull << shift;
      if (inbin == need || shift == 0) break;
      shift = shift - 8 > 0 ? shift - 8 : 0;
    }
  }

  if constexpr (kThreadMajor) {
    // ---- stable compaction in candidate order (thread-major): each thread's survivors
    // after those of the threads before it (a DPP prefix sum in the wave, the waves' totals
    // through LDS), written one after another ----
    uint32_t takes = 0u;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) takes |= (key[i] && (key[i] & mask) >= prefix) ? 1u << i : 0u;
    const uint32_t mine = (uint32_t)__builtin_popcount(takes);
    const uint32_t incl = dpp_prefix_sum(mine);
    if (lane == 63) cnt[wave][0] = incl;
    __syncthreads();
    uint32_t slot = incl - mine, total = 0u;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const uint32_t c = cnt[wv][0];
      total += c;
      slot += wv < wave ? c : 0u;
    }
    const uint32_t nsel = total < (uint32_t)K ? total : (uint32_t)K;
    if constexpr (!kFinal) {
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        if ((takes >> i) & 1u) {
          if (slot < (uint32_t)K) keys_out[slot] = key[i];
          ++slot;
        }
      }
      for (int i = (int)nsel + tid; i < K; i += kThreads) keys_out[i] = 0ull;
    } else {
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        if ((takes >> i) & 1u) {
          if (slot < (uint32_t)K) idx_out[slot] = key_pos(key[i]);
          ++slot;
        }
      }
      for (int i = (int)nsel + tid; i < K; i += kThreads) idx_out[i] = -1;
      if (tid == 0) *count_out = (int32_t)nsel;
    }
    return prefix;
  }

  // ---- stable compaction in candidate order (i-major, then thread) ----
  // survivors of slot i in wave w: one ballot; cnt[w][i] = their number
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    const uint64_t m = __ballot(key[i] && (key[i] & mask) >= prefix);
    if (lane == 0) cnt[wave][i] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // lane i < 32: off = (survivors of slots < i, all waves) + (survivors of slot i, waves < w)
  uint32_t tot_i = 0, before_w = 0;
  if (lane < kEpt) {
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const uint32_t c = cnt[wv][lane];
      tot_i += c;
      before_w += wv < wave ? c : 0u;
    }
  }
  const uint32_t excl = dpp_prefix_sum(tot_i);   // inclusive over slots (lanes 0..31; the rest hold 0)
  const uint32_t total = __builtin_amdgcn_readlane(excl, kEpt - 1);
  const uint32_t off = excl - tot_i + before_w;
  const uint32_t nsel = total < (uint32_t)K ? total : (uint32_t)K;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  if (!kFinal) {
    uint64_t* out = keys_out;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
      const bool take = key[i] && (key[i] & mask) >= prefix;
      const uint64_t m = __ballot(take);
      const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
      if (take && slot < (uint32_t)K) out[slot] = key[i];
    }
    for (int i = (int)nsel + tid; i < K; i += kThreads) out[i] = 0ull;
    return prefix;
  }
  int32_t* out = idx_out;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    const bool take = key[i] && (key[i] & mask) >= prefix;
    const uint64_t m = __ballot(take);
    const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
    if (take && slot < (uint32_t)K) out[slot] = key_pos(key[i]);
  }
  for (int i = (int)nsel + tid; i < K; i += kThreads) out[i] = -1;
  if (tid == 0) *count_out = (int32_t)nsel;
  return prefix;
}


// The same exact selection by one wave alone (no barrier: a wave's LDS accesses execute in
// order), for lists that a single wave owns: key[i] of lane l is candidate i*64 + l; the K
// largest are written to out[0 .. K) in candidate order (out may alias the LDS the keys were
// read from: every key is in registers before the first write).  `hist` is 256 words of LDS
// private to the wave.  Returns the threshold T: the kept keys are exactly those >= T (0 when
// at most K keys are present; then nothing is written).
template <int kEpt>
__device__ __forceinline__ uint64_t select_wave(uint64_t (&key)[kEpt], int K, uint32_t* hist, uint64_t* out) {
  const int lane = threadIdx.x & 63;
  uint32_t n = 0, hmax = 0u, hmin = ~0u, lmax = 0u, lmin = ~0u;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    n += (uint32_t)__popcll(__ballot(key[i] != 0ull));
    const uint32_t h = (uint32_t)(key[i] >> 32), l = (uint32_t)key[i];
    hmax = key[i] ? max(hmax, h) : hmax;
    hmin = key[i] ? min(hmin, h) : hmin;
    lmax = key[i] ? max(lmax, l) : lmax;
    lmin = key[i] ? min(lmin, l) : lmin;
  }
  if (n <= (uint32_t)K) return 0ull;
  hmax = dpp_max_u32(hmax);
  hmin = dpp_min_u32(hmin);
  int hb;
  uint64_t top;
  if (hmax != hmin) {
    hb = 32 + 31 - __clz(hmax ^ hmin);
    top = (uint64_t)hmax << 32;
  } else {   // every score equal: the keys differ in their position words only
    lmax = dpp_max_u32(lmax);
    lmin = dpp_min_u32(lmin);
    hb = 31 - __clz(lmax ^ lmin);
    top = ((uint64_t)hmax << 32) | lmax;
  }
  uint64_t mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = top & mask;
  int shift = hb - 7 > 0 ? hb - 7 : 0;
  uint32_t need = (uint32_t)K;
  for (;;) {
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kEpt; ++i)
      if (key[i] && (key[i] & mask) == prefix) atomicAdd(&hist[(uint32_t)(key[i] >> shift) & 255u], 1u);
    const uint4 c = reinterpret_cast<const uint4*>(hist)[lane];   // bins 4l .. 4l+3
    const uint32_t hs[4] = {c.x, c.y, c.z, c.w};
    const uint32_t tot = hs[0] + hs[1] + hs[2] + hs[3];
    const uint32_t pre = dpp_prefix_sum(tot);
    const uint32_t incl = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + tot;  // bins >= 4*lane
    const uint32_t above_lane = incl - tot;
    uint32_t d = 0, above = 0, inbin = 0;
    const bool mine = above_lane < need && incl >= need;
    if (mine) {
      uint32_t acc = above_lane;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (acc + hs[j] >= need) {
          d = 4 * lane + j;
          above = acc;
          inbin = hs[j];
          break;
        }
        acc += hs[j];
      }
    }
    const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
    d = __builtin_amdgcn_readlane(d, owner);
    above = __builtin_amdgcn_readlane(above, owner);
    inbin = __builtin_amdgcn_readlane(inbin, owner);
    need -= above;
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    if (inbin == need || shift == 0) break;
    shift = shift - 8 > 0 ? shift - 8 : 0;
  }
  // stable compaction in candidate order: the kept keys are those >= prefix
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < kEpt; ++i) {
    const bool take = key[i] && key[i] >= prefix;
    const uint64_t m = __ballot(take);
    if (take) out[base + (uint32_t)__popcll(m & lt_mask)] = key[i];
    base += (uint32_t)__popcll(m);
  }
  return prefix;
}

// The 256-thread, 32-keys-per-thread segment of the Top-K levels: segment seg of query q
// writes keys_out[(q*n_seg + seg)*K ..] (non-final) or idx_out[q*K ..] and count_out[q].
template <bool kFinal>
__device__ __forceinline__ void select_segment(uint64_t (&key)[kTkEpt], int q, int seg, int n_seg, int K,
                                               uint32_t* hist, uint64_t* __restrict__ keys_out,
                                               int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out) {
  select_block<kTkThreads, kTkEpt, kFinal>(
      key, K, hist, kFinal ? nullptr : keys_out + ((int64_t)q * n_seg + seg) * K,
      kFinal ? idx_out + (int64_t)q * K : nullptr, kFinal ? count_out + q : nullptr);
}

// number of segments per level, level 0 first; the last entry is 1
inline int plan_levels(int64_t n0, int k, int64_t* segs, int max_levels) {
  int L = 0;
  int64_t cur = (n0 + kTkSeg - 1) / kTkSeg;
  if (cur < 1) cur = 1;
  segs[L++] = cur;
  while (cur > 1 && L < max_levels) {
    cur = (cur * k + kTkSeg - 1) / kTkSeg;
    segs[L++] = cur;
  }
  return L;
}

inline size_t ws_bytes(int n_q, int64_t n0, int k) {
  int64_t segs[16];
  int L = plan_levels(n0, k, segs, 16);
  if (L == 1) return 0;
  int64_t s1 = L > 2 ? segs[1] : 0;
  return (size_t)8 * (size_t)k * (size_t)n_q * (size_t)(segs[0] + s1) + 256;
}

int select_levels_after0(const int64_t* segs, int L, TkArgs base, int n_q, uint64_t* bufA, uint64_t* bufB,
                         hipStream_t st);

// One level of each of two selection chains in one launch of the 1,024-thread level kernel
// (segments of kTkSeg candidates): chain a reads keys, chain b keys or (b_from_scores, its
// first level) a score array without a slot map; segs 0 leaves a chain out.
int launch_wide2(const TkArgs& a, int segs_a, bool final_a, const TkArgs& b, int segs_b, bool final_b,
                 bool b_from_scores, int n_q, hipStream_t st);

// The Top-K levels over a score array (the csa2_topk path; `base` as csa2_topk fills it);
// `workspace` holds ws_bytes(n_q, n0, base.k) bytes.  Returns a csa2 status.
int select_from_scores(TkArgs base, int n_q, int64_t n0, void* workspace, size_t workspace_bytes, hipStream_t st);

}  // namespace csa2
