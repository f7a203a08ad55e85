// csa2_topk and csa2_build_pool: exact Top-K selection per query
// ([W] "CSA2：跨层复用，能借就不自己算" (Top-512), "分层稀疏索引器" and Figure 5 (pool of
// at most 2,048 blocks of 8 positions ranked by their max indexer score)).
//
// Ranking is by (score descending, position ascending).  Each candidate becomes one
// 64-bit key: the order-preserving image of the fp32 score in the high word and the
// complemented position in the low word, so keys are unique and "larger key" is exactly
// "ranked earlier".  Selecting the K largest keys is then an exact radix select.
//
// Work split: a query's candidates are cut into segments of 8,192, one 256-thread
// workgroup each with 32 keys per thread held in registers.  A workgroup finds its
// segment's K largest keys with a most-significant-digit radix select: it starts at the
// highest bit where the segment's largest and smallest keys differ and walks down 8 bits
// per pass, stopping as soon as the boundary bin is taken whole (usually after 3 passes).
// Each wave counts into its own 256-bin LDS histogram (two sets, alternating per pass),
// then every wave scans the sum of the four itself, so a pass costs one barrier and no
// wave waits on another's serial work.  The global Top-K lies inside the union of the
// segments' Top-K sets, so the survivors (n_seg * K keys) go through the same kernel again
// until one segment is left.  Survivors are compacted stably, in candidate order, with
// ballots and one prefix sum (no atomics): candidates enter every level in ascending
// position order, so the last level's output is already ascending and no sort is needed,
// and the result is deterministic.  Scores are read from HBM once; later levels read K
// keys per segment.
#include "select.h"

namespace csa2 {

template <int kMode, bool kFinal>
__global__ __launch_bounds__(kTkThreads) void k_topk(TkArgs a) {
  const int q = blockIdx.y;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int K = a.k;

  int64_t nv = a.n_vis[q];
  if (kMode == kFromScores && a.vis_div > 1) nv = nv > 0 ? (nv + a.vis_div - 1) / a.vis_div : 0;
  nv = nv < 0 ? 0 : (nv > a.max_vis ? a.max_vis : nv);
  const int64_t c0 = (int64_t)seg * kTkSeg;

  // ---- load this segment's candidates as keys (0 = no candidate); candidate c0 + i*256 + tid ----
  // Every load is unconditional, to a clamped in-bounds address, and absent candidates are
  // masked afterwards without a branch: a load under a per-lane condition compiles to a
  // branch around it and a wait for it, which turns the 32 loads of a thread into 32
  // memory round trips one after another.
  uint64_t key[kTkEpt];
  if (kMode == kFromScores && a.cand_blocks == nullptr) {
    const int lim = (int)(nv - c0 < kTkSeg ? (nv - c0 > 0 ? nv - c0 : 0) : kTkSeg);
    if (lim > 0) {  // uniform
      const float* sp = a.scores + q * a.scores_stride + c0;
      float v[kTkEpt];
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) {
        const int o = i * kTkThreads + tid;
        v[i] = sp[o < lim ? o : lim - 1];
      }
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) {
        const int o = i * kTkThreads + tid;
        key[i] = make_key(v[i], (uint32_t)(c0 + o)) & (0ull - (uint64_t)(o < lim));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) key[i] = 0ull;
    }
  } else if (kMode == kFromScores) {
    int64_t nc = a.n_cand_blocks[q];
    nc = nc < 0 ? 0 : (nc > a.max_cand_blocks ? a.max_cand_blocks : nc);
    // slots holding a candidate; at most 2^20 blocks of at most 64 slots, so 32 bits suffice
    const int64_t nslot = nc * a.block;
    if (c0 < nslot) {  // uniform
      const float* sp = a.scores + q * a.scores_stride;
      const int32_t* cb = a.cand_blocks + (int64_t)q * a.max_cand_blocks;
      const uint32_t blk = (uint32_t)a.block;
      const uint32_t last = (uint32_t)(nslot - 1);
      int32_t bv[kTkEpt];
      float v[kTkEpt];
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) {
        uint32_t c = (uint32_t)c0 + (uint32_t)(i * kTkThreads + tid);
        c = c < last ? c : last;
        bv[i] = cb[c / blk];
        v[i] = sp[c];
      }
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) {
        const int64_t c = c0 + i * kTkThreads + tid;
        const int64_t pos = (int64_t)bv[i] * blk + (uint32_t)c % blk;
        const bool ok = c < nslot && bv[i] >= 0 && pos < nv;
        key[i] = make_key(v[i], (uint32_t)pos) & (0ull - (uint64_t)ok);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) key[i] = 0ull;
    }
  } else if (kMode == kFromBlockMax) {
    const int64_t nblk = (nv + a.block - 1) / a.block;
    if (c0 < nblk) {  // uniform; then nv >= 1
      const float* sp = a.scores + q * a.scores_stride;
      float m[kTkEpt];
      // position j of every block, clamped to the last visible position: that position lies
      // in the last block, so a clamped read repeats one of that block's own scores
      // (offsets fit 32 bits: nv <= 2^31 - 1 and a block is at most 64 positions)
      const uint32_t blk = (uint32_t)a.block, lastb = (uint32_t)(nblk - 1), lastp = (uint32_t)(nv - 1);
      for (uint32_t j = 0; j < blk; ++j) {
        float x[kTkEpt];
#pragma unroll
        for (int i = 0; i < kTkEpt; ++i) {
          uint32_t c = (uint32_t)c0 + (uint32_t)(i * kTkThreads + tid);
          c = c < lastb ? c : lastb;
          uint32_t p = c * blk + j;
          p = p < lastp ? p : lastp;
          x[i] = sp[p];
        }
#pragma unroll
        for (int i = 0; i < kTkEpt; ++i) m[i] = j == 0 ? x[i] : fmaxf(m[i], x[i]);
      }
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) {
        const int64_t c = c0 + i * kTkThreads + tid;
        key[i] = make_key(m[i], (uint32_t)c) & (0ull - (uint64_t)(c < nblk));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i) key[i] = 0ull;
    }
  } else {
    const uint64_t* kp = a.keys_in + q * a.keys_in_per_q + c0;
    const int lim = (int)(a.keys_in_per_q - c0 < kTkSeg ? a.keys_in_per_q - c0 : kTkSeg);
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      const int o = i * kTkThreads + tid;
      key[i] = o < lim ? kp[o] : 0ull;
    }
  }

  __shared__ __attribute__((aligned(16))) uint32_t hist[kTkHistWords];
  select_segment<kFinal>(key, q, seg, gridDim.x, K, hist, a.keys_out, a.idx_out, a.count_out);
}

// ---- the wide level: one segment of at most 8,192 candidates, 1,024 threads x 8 keys ----
// Same selection and output as select_segment (exact radix select on the 64-bit keys, then a
// stable compaction in candidate order), laid out for 16 waves so that the serial parts of
// a workgroup are short: the count comes from ballots, the range of the keys from DPP
// reductions of their high words, each wave counts into its own 256-bin histogram and the
// sixteen are summed in two stages.  It serves the levels after the first (candidates are
// the previous level's surviving keys) and the first level over a score array without a
// slot map (the pool's block maxima).  kFinal: the query's Top-K positions; otherwise the
// segment's best K keys for the next level.
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinEpt = kTkSeg / kFinThreads;   // 8

struct WideLds {
  uint32_t hist[kFinWaves][256];
  uint32_t part[4][256];
  uint32_t red[4][kFinWaves];
  uint32_t cnt[kFinWaves][kFinEpt];
};

template <int kMode, bool kFinal>
__device__ __forceinline__ void wide_level(const TkArgs& a, int q, int seg, int n_seg, WideLds& L) {
  static_assert(kMode == kFromKeys || kMode == kFromScores, "keys, or a score array without a slot map");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.k;
  const int64_t c0 = (int64_t)seg * kTkSeg;

  // ---- keys: candidate c0 + i*1024 + tid; unconditional clamped loads, masked after ----
  uint64_t key[kFinEpt];
  if constexpr (kMode == kFromKeys) {
    const int64_t left = a.keys_in_per_q - c0;
    const int lim = (int)(left < kTkSeg ? (left > 0 ? left : 0) : kTkSeg);
    if (lim > 0) {  // uniform
      const uint64_t* kp = a.keys_in + q * a.keys_in_per_q + c0;
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) {
        const int o = i * kFinThreads + tid;
        key[i] = kp[o < lim ? o : lim - 1] & (0ull - (uint64_t)(o < lim));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) key[i] = 0ull;
    }
  } else {
    int64_t nv = a.n_vis[q];
    if (a.vis_div > 1) nv = nv > 0 ? (nv + a.vis_div - 1) / a.vis_div : 0;
    nv = nv < 0 ? 0 : (nv > a.max_vis ? a.max_vis : nv);
    const int lim = (int)(nv - c0 < kTkSeg ? (nv - c0 > 0 ? nv - c0 : 0) : kTkSeg);
    if (lim > 0) {  // uniform
      const float* sp = a.scores + q * a.scores_stride + c0;
      float v[kFinEpt];
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) {
        const int o = i * kFinThreads + tid;
        v[i] = sp[o < lim ? o : lim - 1];
      }
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) {
        const int o = i * kFinThreads + tid;
        key[i] = make_key(v[i], (uint32_t)(c0 + o)) & (0ull - (uint64_t)(o < lim));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) key[i] = 0ull;
    }
  }

  // ---- count, the range of the high (score) words and a lower bound of the K-th largest
  // key's high word (prune_bound) ----
  uint32_t nw = 0, hmax = 0u, hmin = ~0u, h2 = 0u;
#pragma unroll
  for (int i = 0; i < kFinEpt; ++i) {
    nw += (uint32_t)__popcll(__ballot(key[i] != 0ull));
    const uint32_t h = (uint32_t)(key[i] >> 32);
    h2 = key[i] ? max(h2, min(hmax, h)) : h2;
    hmax = key[i] ? max(hmax, h) : hmax;
    hmin = key[i] ? min(hmin, h) : hmin;
  }
  const uint32_t tb = dpp_min_u32(prune_bound(hmax, h2, K, kFinThreads));
  hmax = dpp_max_u32(hmax);
  hmin = dpp_min_u32(hmin);
  if (lane == 0) {
    L.red[0][wave] = nw;
    L.red[1][wave] = hmax;
    L.red[2][wave] = hmin;
    L.red[3][wave] = tb;
  }
  __syncthreads();
  uint32_t n = 0, tmin = ~0u;
  hmax = 0u;
  hmin = ~0u;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    n += L.red[0][w];
    hmax = max(hmax, L.red[1][w]);
    hmin = min(hmin, L.red[2][w]);
    tmin = min(tmin, L.red[3][w]);
  }

  // ---- radix select: (prefix, mask) such that exactly K keys have (key & mask) >= prefix ----
  uint64_t prefix = 0, mask = 0;
  if (n > (uint32_t)K) {
    // keys below the bound rank below the K-th: drop them before the first count
    if (tmin > hmin) {
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) key[i] = (uint32_t)(key[i] >> 32) >= tmin ? key[i] : 0ull;
      hmin = tmin;
    }
    int hb;        // highest bit where the largest and smallest key differ
    uint64_t top;  // the largest key's bits above hb
    if (hmax != hmin) {
      hb = 32 + 31 - __clz(hmax ^ hmin);
      top = (uint64_t)hmax << 32;
    } else {       // every remaining score equal: the keys differ in their position words only
      uint32_t lmax = 0u, lmin = ~0u;
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i) {
        lmax = key[i] ? max(lmax, (uint32_t)key[i]) : lmax;
        lmin = key[i] ? min(lmin, (uint32_t)key[i]) : lmin;
      }
      lmax = dpp_max_u32(lmax);
      lmin = dpp_min_u32(lmin);
      __syncthreads();  // red[] was read above
      if (lane == 0) {
        L.red[1][wave] = lmax;
        L.red[2][wave] = lmin;
      }
      __syncthreads();
      lmax = 0u;
      lmin = ~0u;
#pragma unroll
      for (int w = 0; w < kFinWaves; ++w) {
        lmax = max(lmax, L.red[1][w]);
        lmin = min(lmin, L.red[2][w]);
      }
      hb = 31 - __clz(lmax ^ lmin);  // n >= 2 unique keys: lmax != lmin
      top = ((uint64_t)hmax << 32) | lmax;
    }
    mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    prefix = top & mask;
    int shift = hb - 7 > 0 ? hb - 7 : 0;
    uint32_t need = (uint32_t)K;
    for (;;) {
      reinterpret_cast<uint4*>(L.hist[wave])[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int i = 0; i < kFinEpt; ++i)
        if (key[i] && (key[i] & mask) == prefix) atomicAdd(&L.hist[wave][(uint32_t)(key[i] >> shift) & 255u], 1u);
      __syncthreads();
      {  // stage 1: thread t sums bin t % 256 over waves 4*(t / 256) .. +3
        const int b = tid & 255, g4 = tid >> 8;
        L.part[g4][b] = L.hist[4 * g4][b] + L.hist[4 * g4 + 1][b] + L.hist[4 * g4 + 2][b] + L.hist[4 * g4 + 3][b];
      }
      __syncthreads();
      // stage 2, in every wave: lane l owns bins 4l..4l+3
      uint32_t hs[4];
      {
        const uint4 p0 = reinterpret_cast<const uint4*>(L.part[0])[lane];
        const uint4 p1 = reinterpret_cast<const uint4*>(L.part[1])[lane];
        const uint4 p2 = reinterpret_cast<const uint4*>(L.part[2])[lane];
        const uint4 p3 = reinterpret_cast<const uint4*>(L.part[3])[lane];
        hs[0] = p0.x + p1.x + p2.x + p3.x;
        hs[1] = p0.y + p1.y + p2.y + p3.y;
        hs[2] = p0.z + p1.z + p2.z + p3.z;
        hs[3] = p0.w + p1.w + p2.w + p3.w;
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

  // ---- stable compaction in candidate order (i-major, then thread) ----
#pragma unroll
  for (int i = 0; i < kFinEpt; ++i) {
    const uint64_t m = __ballot(key[i] && (key[i] & mask) >= prefix);
    if (lane == 0) L.cnt[wave][i] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // lane i < 8: off = (survivors of slots < i, all waves) + (survivors of slot i, waves < w)
  uint32_t tot_i = 0, before_w = 0;
  if (lane < kFinEpt) {
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) {
      const uint32_t c = L.cnt[w][lane];
      tot_i += c;
      before_w += w < wave ? c : 0u;
    }
  }
  const uint32_t excl = dpp_prefix_sum(tot_i);   // lanes 0..7 (row 0): inclusive over slots
  const uint32_t total = __builtin_amdgcn_readlane(excl, kFinEpt - 1);
  const uint32_t off = excl - tot_i + before_w;
  const uint32_t nsel = total < (uint32_t)K ? total : (uint32_t)K;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if constexpr (kFinal) {
    int32_t* out = a.idx_out + (int64_t)q * K;
#pragma unroll
    for (int i = 0; i < kFinEpt; ++i) {
      const bool take = key[i] && (key[i] & mask) >= prefix;
      const uint64_t m = __ballot(take);
      const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
      if (take && slot < (uint32_t)K) out[slot] = key_pos(key[i]);
    }
    for (int i = (int)nsel + tid; i < K; i += kFinThreads) out[i] = -1;
    if (tid == 0) a.count_out[q] = (int32_t)nsel;
  } else {
    uint64_t* out = a.keys_out + ((int64_t)q * n_seg + seg) * K;
#pragma unroll
    for (int i = 0; i < kFinEpt; ++i) {
      const bool take = key[i] && (key[i] & mask) >= prefix;
      const uint64_t m = __ballot(take);
      const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
      if (take && slot < (uint32_t)K) out[slot] = key[i];
    }
    for (int i = (int)nsel + tid; i < K; i += kFinThreads) out[i] = 0ull;
  }
}

// the last level of one query (at most 8,192 survivor keys): its Top-K positions
__global__ __launch_bounds__(kFinThreads) void k_topk_final(TkArgs a) {
  __shared__ __attribute__((aligned(16))) WideLds L;
  wide_level<kFromKeys, true>(a, blockIdx.y, 0, 1, L);
}

// Two independent wide levels in one launch: segments [0, segs_a) of task a, then
// [segs_a, segs_a + segs_b) of task b (each workgroup runs one task's segment; both tasks
// cover every query, grid y).  Two selection chains then share their launches.
template <int kModeA, bool kFinalA, int kModeB, bool kFinalB>
__global__ __launch_bounds__(kFinThreads) void k_topk_wide2(TkArgs a, int segs_a, TkArgs b, int segs_b) {
  __shared__ __attribute__((aligned(16))) WideLds L;
  const int x = blockIdx.x, q = blockIdx.y;
  if (x < segs_a) wide_level<kModeA, kFinalA>(a, q, x, segs_a, L);
  else if (x - segs_a < segs_b) wide_level<kModeB, kFinalB>(b, q, x - segs_a, segs_b, L);
}

// Launches one wide level of each of two chains (a: keys; b: keys or the first level over a
// score array); segs 0 leaves a chain out.  Returns a csa2 status.
int launch_wide2(const TkArgs& a, int segs_a, bool final_a, const TkArgs& b, int segs_b, bool final_b,
                 bool b_from_scores, int n_q, hipStream_t st) {
  const dim3 grid((unsigned)(segs_a + segs_b), (unsigned)n_q), blk(kFinThreads);
#define CSA2_WIDE2(FA, MB, FB) hipLaunchKernelGGL((k_topk_wide2<kFromKeys, FA, MB, FB>), grid, blk, 0, st, a, segs_a, b, segs_b)
  if (b_from_scores) {
    if (final_a) { if (final_b) CSA2_WIDE2(true, kFromScores, true); else CSA2_WIDE2(true, kFromScores, false); }
    else { if (final_b) CSA2_WIDE2(false, kFromScores, true); else CSA2_WIDE2(false, kFromScores, false); }
  } else {
    if (final_a) { if (final_b) CSA2_WIDE2(true, kFromKeys, true); else CSA2_WIDE2(true, kFromKeys, false); }
    else { if (final_b) CSA2_WIDE2(false, kFromKeys, true); else CSA2_WIDE2(false, kFromKeys, false); }
  }
#undef CSA2_WIDE2
  return csa2_check_launch();
}

// Launch the key-merging levels 1..L-1 (level 0 has written bufA); returns a csa2 status.
int select_levels_after0(const int64_t* segs, int L, TkArgs base, int n_q, uint64_t* bufA, uint64_t* bufB,
                         hipStream_t st) {
  for (int l = 1; l < L; ++l) {
    TkArgs a = base;
    const bool final = (l == L - 1);
    a.keys_in = (l % 2 == 1) ? bufA : bufB;
    a.keys_in_per_q = segs[l - 1] * base.k;
    a.keys_out = (l % 2 == 0) ? bufA : bufB;
    const int rc = launch_wide2(a, (int)segs[l], final, TkArgs{}, 0, false, false, n_q, st);
    if (rc != CSA2_OK) return rc;
  }
  return CSA2_OK;
}

static int run_select(int mode0, TkArgs base, int n_q, int64_t n0, void* workspace, size_t workspace_bytes,
                      hipStream_t st) {
  int64_t segs[16];
  const int L = plan_levels(n0, base.k, segs, 16);
  if (L >= 16) return CSA2_ERR_SHAPE;
  const size_t need = ws_bytes(n_q, n0, base.k);
  if (need > workspace_bytes || (need && !workspace)) return CSA2_ERR_WORKSPACE;
  uint64_t* bufA = (uint64_t*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  uint64_t* bufB = bufA + (size_t)base.k * n_q * segs[0];
  TkArgs a = base;
  a.keys_out = bufA;
  dim3 grid((unsigned)segs[0], (unsigned)n_q), blk(kTkThreads);
  if (mode0 == kFromScores) {
    if (L == 1) hipLaunchKernelGGL((k_topk<kFromScores, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_topk<kFromScores, false>), grid, blk, 0, st, a);
  } else {
    if (L == 1) hipLaunchKernelGGL((k_topk<kFromBlockMax, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_topk<kFromBlockMax, false>), grid, blk, 0, st, a);
  }
  const int rc = csa2_check_launch();
  if (rc != CSA2_OK) return rc;
  return select_levels_after0(segs, L, base, n_q, bufA, bufB, st);
}

int select_from_scores(TkArgs base, int n_q, int64_t n0, void* workspace, size_t workspace_bytes, hipStream_t st) {
  return run_select(kFromScores, base, n_q, n0 < 1 ? 1 : n0, workspace, workspace_bytes, st);
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_topk_workspace_bytes(int n_q, int64_t n_slots, int k) {
  if (n_q <= 0 || n_slots <= 0 || k < 1 || k > CSA2_MAX_TOPK) return 0;
  return ws_bytes(n_q, n_slots, k);
}

extern "C" int csa2_topk(const float* scores, int64_t scores_stride, int n_q, const int64_t* n_vis, int64_t max_vis,
                         const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block, int max_cand_blocks,
                         int k, int32_t* idx_out, int32_t* count_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (!scores || !n_vis || !idx_out || !count_out) return CSA2_ERR_NULL;
  if (n_q < 0 || n_q > 65535 || k < 1 || k > CSA2_MAX_TOPK || max_vis < 0 || max_vis > 0x7fffffffLL)
    return CSA2_ERR_SHAPE;
  int64_t n0;
  if (cand_blocks) {
    if (!n_cand_blocks) return CSA2_ERR_NULL;
    if (block < 1 || block > 64 || max_cand_blocks < 1 || max_cand_blocks > (1 << 20)) return CSA2_ERR_SHAPE;
    n0 = (int64_t)max_cand_blocks * block;
  } else {
    n0 = max_vis;
  }
  if (scores_stride < n0) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  TkArgs a = {};
  a.scores = scores;
  a.scores_stride = scores_stride;
  a.n_vis = n_vis;
  a.max_vis = max_vis;
  a.cand_blocks = cand_blocks;
  a.n_cand_blocks = n_cand_blocks;
  a.block = block;
  a.max_cand_blocks = max_cand_blocks;
  a.idx_out = idx_out;
  a.count_out = count_out;
  a.k = k;
  a.n_slots = n0;
  return run_select(kFromScores, a, n_q, n0 < 1 ? 1 : n0, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" size_t csa2_pool_workspace_bytes(int n_q, int64_t max_vis, int block, int max_blocks) {
  if (n_q <= 0 || max_vis <= 0 || block < 1 || max_blocks < 1 || max_blocks > CSA2_MAX_TOPK) return 0;
  return ws_bytes(n_q, (max_vis + block - 1) / block, max_blocks);
}

extern "C" int csa2_build_pool(const float* scores, int64_t scores_stride, int n_q, const int64_t* n_vis,
                               int64_t max_vis, int block, int max_blocks, int32_t* blocks_out, int32_t* count_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (!scores || !n_vis || !blocks_out || !count_out) return CSA2_ERR_NULL;
  if (n_q < 0 || n_q > 65535 || block < 1 || block > 64 || max_blocks < 1 || max_blocks > CSA2_MAX_TOPK ||
      max_vis < 0 || max_vis > 0x7fffffffLL || scores_stride < max_vis)
    return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  int64_t nblk = (max_vis + block - 1) / block;
  TkArgs a = {};
  a.scores = scores;
  a.scores_stride = scores_stride;
  a.n_vis = n_vis;
  a.max_vis = max_vis;
  a.block = block;
  a.idx_out = blocks_out;
  a.count_out = count_out;
  a.k = max_blocks;
  a.n_slots = nblk;
  return run_select(kFromBlockMax, a, n_q, nblk < 1 ? 1 : nblk, workspace, workspace_bytes, (hipStream_t)stream);
}
