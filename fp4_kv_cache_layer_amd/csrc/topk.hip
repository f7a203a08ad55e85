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
};

__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t pos) {
  return ((uint64_t)ord_f32(s) << 32) | (uint64_t)(0xffffffffu - pos);
}
__device__ __forceinline__ int32_t key_pos(uint64_t k) { return (int32_t)(0xffffffffu - (uint32_t)k); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// wave-wide inclusive suffix sum (lane l gets the sum over lanes >= l)
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v, int lane) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint32_t o = __shfl_down(v, m);
    v += (lane + m < 64) ? o : 0u;
  }
  return v;
}

template <int kMode, bool kFinal>
__global__ __launch_bounds__(kTkThreads) void k_topk(TkArgs a) {
  const int q = blockIdx.y;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.k;

  __shared__ uint32_t hist[2][kTkWaves][256];
  __shared__ uint32_t cnt[kTkWaves][kTkEpt];
  __shared__ uint64_t red_hi[kTkWaves], red_lo[kTkWaves];
  __shared__ uint32_t red_n[kTkWaves];

  int64_t nv = a.n_vis[q];
  nv = nv < 0 ? 0 : (nv > a.max_vis ? a.max_vis : nv);
  const int64_t c0 = (int64_t)seg * kTkSeg;

  // ---- load this segment's candidates as keys (0 = no candidate); candidate c0 + i*256 + tid ----
  uint64_t key[kTkEpt];
  if (kMode == kFromScores && a.cand_blocks == nullptr) {
    const float* sp = a.scores + q * a.scores_stride + c0;
    const int lim = (int)(nv - c0 < kTkSeg ? (nv - c0 > 0 ? nv - c0 : 0) : kTkSeg);
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      const int o = i * kTkThreads + tid;
      key[i] = o < lim ? make_key(sp[o], (uint32_t)(c0 + o)) : 0ull;
    }
  } else if (kMode == kFromScores) {
    int64_t nc = a.n_cand_blocks[q];
    nc = nc < 0 ? 0 : (nc > a.max_cand_blocks ? a.max_cand_blocks : nc);
    const float* sp = a.scores + q * a.scores_stride;
    const int32_t* cb = a.cand_blocks + (int64_t)q * a.max_cand_blocks;
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      const int64_t c = c0 + i * kTkThreads + tid;
      uint64_t kk = 0;
      if (c < nc * a.block) {
        const int32_t b = cb[c / a.block];
        const int64_t pos = (int64_t)b * a.block + c % a.block;
        if (b >= 0 && pos < nv) kk = make_key(sp[c], (uint32_t)pos);
      }
      key[i] = kk;
    }
  } else if (kMode == kFromBlockMax) {
    const int64_t nblk = (nv + a.block - 1) / a.block;
    const float* sp = a.scores + q * a.scores_stride;
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      const int64_t c = c0 + i * kTkThreads + tid;
      uint64_t kk = 0;
      if (c < nblk) {
        const float* s = sp + c * a.block;
        int64_t nin = nv - c * a.block;
        nin = nin < a.block ? nin : a.block;
        float m = s[0];
        for (int j = 1; j < nin; ++j) m = fmaxf(m, s[j]);
        kk = make_key(m, (uint32_t)c);
      }
      key[i] = kk;
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

  // ---- count, max and min of the valid keys ----
  uint32_t n = 0;
  uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
  for (int i = 0; i < kTkEpt; ++i) {
    if (key[i]) {
      ++n;
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    n += __shfl_xor(n, m);
    uint64_t o = shfl_xor_u64(kmax, m);
    kmax = o > kmax ? o : kmax;
    o = shfl_xor_u64(kmin, m);
    kmin = o < kmin ? o : kmin;
  }
  if (lane == 0) {
    red_n[wave] = n;
    red_hi[wave] = kmax;
    red_lo[wave] = kmin;
  }
  __syncthreads();
  n = 0;
  kmax = 0;
  kmin = ~0ull;
#pragma unroll
  for (int wv = 0; wv < kTkWaves; ++wv) {
    n += red_n[wv];
    kmax = red_hi[wv] > kmax ? red_hi[wv] : kmax;
    kmin = red_lo[wv] < kmin ? red_lo[wv] : kmin;
  }

  // ---- radix select: find (prefix, mask) such that exactly K keys have (key&mask) >= prefix ----
  uint64_t prefix = 0, mask = 0;
  if (n > (uint32_t)K) {
    const int hb = 63 - __clzll(kmax ^ kmin);  // n >= 2 unique keys -> kmax != kmin
    mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    prefix = kmax & mask;
    int shift = hb - 7 > 0 ? hb - 7 : 0;
    uint32_t need = (uint32_t)K;
    for (int pass = 0;; ++pass) {
      uint32_t* h = hist[pass & 1][wave];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[lane + 64 * i] = 0;
#pragma unroll
      for (int i = 0; i < kTkEpt; ++i)
        if (key[i] && (key[i] & mask) == prefix) atomicAdd(&h[(uint32_t)(key[i] >> shift) & 255u], 1u);
      __syncthreads();
      // every wave: lane l owns bins 4l..4l+3 of the summed histogram
      uint32_t hs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t v = 0;
#pragma unroll
        for (int wv = 0; wv < kTkWaves; ++wv) v += hist[pass & 1][wv][4 * lane + j];
        hs[j] = v;
      }
      const uint32_t tot = hs[0] + hs[1] + hs[2] + hs[3];
      const uint32_t incl = wave_suffix_sum(tot, lane);
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
  // survivors of slot i in wave w: one ballot; cnt[w][i] = their number
#pragma unroll
  for (int i = 0; i < kTkEpt; ++i) {
    const uint64_t m = __ballot(key[i] && (key[i] & mask) >= prefix);
    if (lane == 0) cnt[wave][i] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // lane i < 32: off = (survivors of slots < i, all waves) + (survivors of slot i, waves < w)
  uint32_t tot_i = 0, before_w = 0;
  if (lane < kTkEpt) {
#pragma unroll
    for (int wv = 0; wv < kTkWaves; ++wv) {
      const uint32_t c = cnt[wv][lane];
      tot_i += c;
      before_w += wv < wave ? c : 0u;
    }
  }
  uint32_t excl = tot_i;  // exclusive prefix over lanes 0..31
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    const uint32_t o = __shfl_up(excl, m);
    excl += (lane >= m) ? o : 0u;
  }
  const uint32_t total = __builtin_amdgcn_readlane(excl, kTkEpt - 1);
  const uint32_t off = excl - tot_i + before_w;
  const uint32_t nsel = total < (uint32_t)K ? total : (uint32_t)K;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  if (!kFinal) {
    uint64_t* out = a.keys_out + ((int64_t)q * gridDim.x + seg) * K;
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      const bool take = key[i] && (key[i] & mask) >= prefix;
      const uint64_t m = __ballot(take);
      const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
      if (take && slot < (uint32_t)K) out[slot] = key[i];
    }
    for (int i = (int)nsel + tid; i < K; i += kTkThreads) out[i] = 0ull;
    return;
  }
  int32_t* out = a.idx_out + (int64_t)q * K;
#pragma unroll
  for (int i = 0; i < kTkEpt; ++i) {
    const bool take = key[i] && (key[i] & mask) >= prefix;
    const uint64_t m = __ballot(take);
    const uint32_t slot = __builtin_amdgcn_readlane(off, i) + (uint32_t)__popcll(m & lt_mask);
    if (take && slot < (uint32_t)K) out[slot] = key_pos(key[i]);
  }
  for (int i = (int)nsel + tid; i < K; i += kTkThreads) out[i] = -1;
  if (tid == 0) a.count_out[q] = (int32_t)nsel;
}

// number of segments per level, level 0 first; the last entry is 1
static int plan_levels(int64_t n0, int k, int64_t* segs, int max_levels) {
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

static size_t ws_bytes(int n_q, int64_t n0, int k) {
  int64_t segs[16];
  int L = plan_levels(n0, k, segs, 16);
  if (L == 1) return 0;
  int64_t s1 = L > 2 ? segs[1] : 0;
  return (size_t)8 * (size_t)k * (size_t)n_q * (size_t)(segs[0] + s1) + 256;
}

static int run_select(int mode0, TkArgs base, int n_q, int64_t n0, void* workspace, size_t workspace_bytes,
                      hipStream_t st) {
  int64_t segs[16];
  int L = plan_levels(n0, base.k, segs, 16);
  if (L >= 16) return CSA2_ERR_SHAPE;
  size_t need = ws_bytes(n_q, n0, base.k);
  if (need > workspace_bytes || (need && !workspace)) return CSA2_ERR_WORKSPACE;
  uintptr_t w0 = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
  uint64_t* bufA = (uint64_t*)w0;
  uint64_t* bufB = bufA + (size_t)base.k * n_q * segs[0];
  for (int l = 0; l < L; ++l) {
    TkArgs a = base;
    bool final = (l == L - 1);
    a.keys_out = (l % 2 == 0) ? bufA : bufB;
    if (l > 0) {
      a.keys_in = (l % 2 == 1) ? bufA : bufB;
      a.keys_in_per_q = segs[l - 1] * base.k;
    }
    dim3 grid((unsigned)segs[l], (unsigned)n_q), blk(kTkThreads);
    int mode = l == 0 ? mode0 : kFromKeys;
    if (mode == kFromScores) {
      if (final) hipLaunchKernelGGL((k_topk<kFromScores, true>), grid, blk, 0, st, a);
      else hipLaunchKernelGGL((k_topk<kFromScores, false>), grid, blk, 0, st, a);
    } else if (mode == kFromBlockMax) {
      if (final) hipLaunchKernelGGL((k_topk<kFromBlockMax, true>), grid, blk, 0, st, a);
      else hipLaunchKernelGGL((k_topk<kFromBlockMax, false>), grid, blk, 0, st, a);
    } else {
      if (final) hipLaunchKernelGGL((k_topk<kFromKeys, true>), grid, blk, 0, st, a);
      else hipLaunchKernelGGL((k_topk<kFromKeys, false>), grid, blk, 0, st, a);
    }
    int rc = csa2_check_launch();
    if (rc != CSA2_OK) return rc;
  }
  return CSA2_OK;
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
