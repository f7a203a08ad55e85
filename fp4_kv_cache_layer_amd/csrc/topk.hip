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

  __shared__ __attribute__((aligned(16))) uint32_t hist[kTkHistWords];
  select_segment<kFinal>(key, q, seg, gridDim.x, K, hist, a.keys_out, a.idx_out, a.count_out);
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
    dim3 grid((unsigned)segs[l], (unsigned)n_q), blk(kTkThreads);
    if (final) hipLaunchKernelGGL((k_topk<kFromKeys, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_topk<kFromKeys, false>), grid, blk, 0, st, a);
    const int rc = csa2_check_launch();
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
