// csa2_index_score: FP4 indexer scores, one query per stream over its sequence's
// indexer-K cache ([W] "CSA2：跨层复用，能借就不自己算", "分层稀疏索引器",
// "FP4 与 SWA Bounded Replay").
//
//   score(q, j) = sum_h w[q,h] * max(0, Q[q,h,:] . K[j,:])     (MXFP4 Q and K, d = 128)
//
// Design (decode): the cache is streamed once, 68 B per entry (64 B of E2M1 codes + 4
// E8M0 scales), and each 16-entry tile is one gfx950 scaled-FP4 MFMA
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with A = the query's indexer Q (16 head rows, padded
// with zero rows when H_I < 16) and B = 16 cache entries.  The MX block of 32 elements and
// its E8M0 scale map one-to-one onto what one lane feeds the instruction, so the FP4
// products and their scaling happen inside the matrix core, exactly.  A lane loads one
// 16-byte chunk per entry (lane l: entry l%16, K-block l/16), so a wave's four loads
// cover 16 entries x 64 B = 1 KB contiguously.  The output rows are the heads; each lane
// weights and ReLUs its 4 heads, and a 3-shuffle reduce-scatter over the 4 lane groups
// leaves lane l with the score of entry l of the 64-entry step, stored coalesced.
//
// Per entry the work is 2*16*128 = 4096 FLOP on 68 B: ~60 FLOP/B, which fp32 vector ALUs
// cannot sustain at HBM speed (~480 TFLOP/s needed at 8 TB/s), but which is ~5% of the
// FP4 matrix-core rate.  The kernel is HBM-bound by design.
#include "device.h"

namespace csa2 {

constexpr int kScoreThreads = 256;   // 4 waves
constexpr int kScoreStep = 64;       // entries per wave step (4 MFMA tiles)
constexpr int kScoreChunk = 4096;    // entries per workgroup

template <bool kPool>
__global__ __launch_bounds__(kScoreThreads) void k_score_decode(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, const float* __restrict__ w,
    int n_heads, const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, int64_t seq_cap,
    int n_seq, const int32_t* __restrict__ q_seq, const int64_t* __restrict__ n_vis,
    const int32_t* __restrict__ cand_blocks, const int32_t* __restrict__ n_cand_blocks, int block,
    int max_cand_blocks, float* __restrict__ scores, int64_t scores_stride, int64_t n_slots, int chunks) {
  const int q = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;   // A row (head) / B column (entry within tile)
  const int kb = lane >> 4;    // K-block of 32 elements

  const int seq = q_seq[q];
  if (seq < 0 || seq >= n_seq) return;
  int64_t nv = n_vis[q];
  nv = nv < 0 ? 0 : (nv > seq_cap ? seq_cap : nv);
  int64_t n_valid;  // slots that may hold a real candidate
  if (kPool) {
    int64_t nc = n_cand_blocks[q];
    nc = nc < 0 ? 0 : (nc > max_cand_blocks ? max_cand_blocks : nc);
    n_valid = nc * block;
  } else {
    n_valid = nv;
  }
  const int64_t chunk_lo = (int64_t)chunk * kScoreChunk;
  const int64_t write_hi = kPool ? n_slots : n_valid;  // pool mode also writes -inf pads
  if (chunk_lo >= write_hi) return;

  // ---- A operand: the query's indexer Q, row = head, 32 FP4 values per lane ----
  v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
  int a_scale = 127;
  if (row < n_heads) {
    const uint4 qa = *reinterpret_cast<const uint4*>(q_codes + ((int64_t)q * n_heads + row) * 64 + kb * 16);
    a[0] = (int)qa.x; a[1] = (int)qa.y; a[2] = (int)qa.z; a[3] = (int)qa.w;
    a_scale = q_scales[((int64_t)q * n_heads + row) * 4 + kb];
  }
  // weights of the 4 output rows (heads 4*kb .. 4*kb+3) this lane accumulates
  float wv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int h = 4 * kb + r;
    wv[r] = h < n_heads ? w[(int64_t)q * n_heads + h] : 0.0f;
  }

  const int64_t seq_base = (int64_t)seq * seq_cap;
  const int32_t* cb = kPool ? cand_blocks + (int64_t)q * max_cand_blocks : nullptr;
  float* out = scores + (int64_t)q * scores_stride;

  int64_t hi = chunk_lo + kScoreChunk;
  hi = hi < write_hi ? hi : write_hi;
  for (int64_t base = chunk_lo + wave * kScoreStep; base < hi; base += 4 * kScoreStep) {
    uint4 bc[4];
    int bs[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      int64_t slot = base + 16 * t + row;
      int64_t pos = slot;
      bool valid = slot < n_valid;
      if (kPool && valid) {
        int32_t b = cb[slot / block];
        pos = (int64_t)b * block + slot % block;
        valid = b >= 0 && pos < nv;
      }
      if (valid) {
        bc[t] = *reinterpret_cast<const uint4*>(k_codes + (seq_base + pos) * 64 + kb * 16);
        bs[t] = k_scales[(seq_base + pos) * 4 + kb];
      } else {
        bc[t] = make_uint4(0u, 0u, 0u, 0u);
        bs[t] = 127;
      }
    }
    float part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v8i b = {(int)bc[t].x, (int)bc[t].y, (int)bc[t].z, (int)bc[t].w, 0, 0, 0, 0};
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      // formats 4/4 = E2M1 for both operands; scales are E8M0, byte 0 of each lane's VGPR
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, a_scale, 0, bs[t]);
      float p = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) p += wv[r] * fmaxf(acc[r], 0.0f);
      part[t] = p;
    }
    // reduce-scatter over the 4 lane groups: lane group g ends with tile g's full sum
    const bool b1 = (kb & 2) != 0, b0 = (kb & 1) != 0;
    float s0 = b1 ? part[0] : part[2];
    float s1 = b1 ? part[1] : part[3];
    float r0 = __shfl_xor(s0, 32);
    float r1 = __shfl_xor(s1, 32);
    float k0 = (b1 ? part[2] : part[0]) + r0;
    float k1 = (b1 ? part[3] : part[1]) + r1;
    float send = b0 ? k0 : k1;
    float recv = __shfl_xor(send, 16);
    float sc = (b0 ? k1 : k0) + recv;
    // lane l now holds entry base + l (tile kb, column row)
    int64_t slot = base + lane;
    if (slot < hi) {
      bool v;
      if (kPool) {
        v = slot < n_valid;
        if (v) {
          int32_t b = cb[slot / block];
          int64_t pos = (int64_t)b * block + slot % block;
          v = b >= 0 && pos < nv;
        }
        out[slot] = v ? sc : -__builtin_inff();
      } else {
        out[slot] = sc;  // slot < hi <= n_valid
      }
    }
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_index_score(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                int n_heads, int dim, const uint8_t* k_codes, const uint8_t* k_scales,
                                int64_t seq_cap, int n_seq, const int32_t* q_seq, const int64_t* n_vis,
                                const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block,
                                int max_cand_blocks, float* scores, int64_t scores_stride, void* stream) {
  if (!q_codes || !q_scales || !w || !k_codes || !k_scales || !q_seq || !n_vis || !scores) return CSA2_ERR_NULL;
  if (n_q < 0 || n_heads < 1 || n_heads > CSA2_MAX_INDEX_HEADS || dim != CSA2_INDEX_DIM || seq_cap < 0 ||
      n_seq < 1)
    return CSA2_ERR_SHAPE;
  if (!aligned16(q_codes) || !aligned16(k_codes)) return CSA2_ERR_SHAPE;
  const bool pool = cand_blocks != nullptr;
  int64_t n_slots;
  if (pool) {
    if (!n_cand_blocks) return CSA2_ERR_NULL;
    if (block < 1 || block > 64 || max_cand_blocks < 1 || max_cand_blocks > (1 << 20)) return CSA2_ERR_SHAPE;
    n_slots = (int64_t)max_cand_blocks * block;
  } else {
    n_slots = seq_cap;
  }
  if (scores_stride < n_slots) return CSA2_ERR_SHAPE;
  if (n_q == 0 || n_slots == 0) return CSA2_OK;
  int64_t chunks = (n_slots + kScoreChunk - 1) / kScoreChunk;
  if (chunks * (int64_t)n_q > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  dim3 grid((unsigned)(chunks * n_q)), blk(kScoreThreads);
  hipStream_t st = (hipStream_t)stream;
  if (pool)
    hipLaunchKernelGGL(k_score_decode<true>, grid, blk, 0, st, q_codes, q_scales, w, n_heads, k_codes, k_scales,
                       seq_cap, n_seq, q_seq, n_vis, cand_blocks, n_cand_blocks, block, max_cand_blocks, scores,
                       scores_stride, n_slots, (int)chunks);
  else
    hipLaunchKernelGGL(k_score_decode<false>, grid, blk, 0, st, q_codes, q_scales, w, n_heads, k_codes, k_scales,
                       seq_cap, n_seq, q_seq, n_vis, cand_blocks, n_cand_blocks, block, max_cand_blocks, scores,
                       scores_stride, n_slots, (int)chunks);
  return csa2_check_launch();
}
