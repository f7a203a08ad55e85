// csa2_index_score / csa2_index_topk: FP4 indexer scores, one query per stream over its
// sequence's indexer-K cache ([W] "CSA2：跨层复用，能借就不自己算", "分层稀疏索引器",
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
// cover 16 entries x 64 B = 1 KB contiguously.  The code and scale loads are non-temporal
// (the cache is streamed once; plain cached loads of the codes slowed the 64 x 128K stream
// from 97 to 110 us) and branch-free, and the next 64-entry step is in flight while the
// current one is multiplied.  The output rows are the heads; each lane weights and ReLUs
// its 4 heads, and a 3-shuffle reduce-scatter over the 4 lane groups leaves lane l with
// the score of entry l of the 64-entry step.
//
// Per entry the work is 2*16*128 = 4096 FLOP on 68 B: ~60 FLOP/B, which fp32 vector ALUs
// cannot sustain at HBM speed (~480 TFLOP/s needed at 8 TB/s), but which is ~5% of the
// FP4 matrix-core rate.  The kernels are HBM-bound by design.
//
// csa2_index_topk fuses the first Top-K level into the scoring pass (the selection is in
// select.h): a workgroup scores 8,192 consecutive slots, keeps its 32 scores per lane in
// registers as selection keys and writes only its K survivors.  Writing every 4-byte
// score and reading it back would add 8 B of HBM traffic per entry, and interleaving the
// score writes with the streaming reads slows the scoring pass down by about a fifth.
#include "select.h"

namespace csa2 {

constexpr int kScoreThreads = 256;   // 4 waves
constexpr int kScoreStep = 64;       // entries per wave step (4 MFMA tiles)
constexpr int kScoreChunk = 4096;    // slots per workgroup, all visible entries
constexpr int kPoolChunk = 512;      // slots per workgroup inside a pool (see launch_score)
static_assert(kScoreThreads == kTkThreads, "the fused kernel hands its registers to select_segment");

struct ScoreArgs {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  // csa2_index_score_q: the indexer Q unquantised ([n_q, n_heads, 128] f32 or bf16),
  // quantised to MXFP4 by every workgroup for itself
  const void* q_lat;
  int q_bf16;
  const float* w;
  int n_heads;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  int64_t k_ce, k_cs, k_se, k_ss;   // byte strides: code entry / sequence, scale entry / sequence
  int64_t seq_cap;
  int n_seq;
  const int32_t* q_seq;
  const int64_t* n_vis;
  const int32_t* cand_blocks;
  const int32_t* n_cand_blocks;
  int block;
  int max_cand_blocks;
  int64_t n_slots;
  // csa2_index_score
  float* scores;
  int64_t scores_stride;
  int chunks;
  int chunk_len;
  // csa2_index_topk
  int k;
  uint64_t* keys_out;
  // csa2_index_topk_pool: per-query maxima of the visible positions of each block of
  // `block` positions ([n_q, bmax_stride] f32)
  float* bmax;
  int64_t bmax_stride;
  int32_t* idx_out;
  int32_t* count_out;
  // csa2_append: each query's new main-KV / indexer-K row (app_row[q]), written by the
  // workgroup whose segment holds it (k_score_select)
  const int64_t* app_row;
  const void* app_main;
  const void* app_index;
  int app_bf16;
  uint8_t* app_kv_codes;
  uint8_t* app_kv_scales;
  int64_t app_kv_ce, app_kv_cs, app_kv_se, app_kv_ss;
};

// n consecutive latent values from p (f32, or bf16 widened by a shift) as fp32 bit patterns,
// in 16-byte loads (p 16-byte aligned)
template <int n>
__device__ __forceinline__ void load_latent_bits(const void* p, bool bf16, uint32_t (&bits)[n]) {
  if (bf16) {
    const uint4* src = static_cast<const uint4*>(p);
#pragma unroll
    for (int u = 0; u < n / 8; ++u) {
      const uint4 v = src[u];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bits[8 * u + 2 * j] = wd[j] << 16;
        bits[8 * u + 2 * j + 1] = wd[j] & 0xffff0000u;
      }
    }
  } else {
    const uint4* src = static_cast<const uint4*>(p);
#pragma unroll
    for (int u = 0; u < n / 4; ++u) {
      const uint4 v = src[u];
      bits[4 * u] = v.x;
      bits[4 * u + 1] = v.y;
      bits[4 * u + 2] = v.z;
      bits[4 * u + 3] = v.w;
    }
  }
}

// The new entry of query q at row r of sequence seq (csa2_append), by one wave: lanes 0-31
// quantise the 32 NVFP4 groups of the main-KV row, lanes 32-35 the four MXFP4 groups of the
// indexer-K row, with the quantiser's rules (nvfp4_group, mxfp4_group), and store them.
__device__ __forceinline__ void append_entry(const ScoreArgs& s, int q, int seq, int64_t r, int lane) {
  if (lane < 32 && s.app_main) {
    uint32_t bits[16];
    load_latent_bits<16>(static_cast<const uint8_t*>(s.app_main) + ((int64_t)q * 512 + 16 * lane) * (s.app_bf16 ? 2 : 4),
                         s.app_bf16, bits);
    uint32_t lo, hi;
    const int sc = nvfp4_group(bits, lo, hi);
    *reinterpret_cast<uint2*>(s.app_kv_codes + (int64_t)seq * s.app_kv_cs + r * s.app_kv_ce + 8 * lane) =
        make_uint2(lo, hi);
    s.app_kv_scales[(int64_t)seq * s.app_kv_ss + r * s.app_kv_se + lane] = (uint8_t)sc;
  } else if (lane >= 32 && lane < 36 && s.app_index) {
    const int g = lane - 32;
    uint32_t bits[32];
    load_latent_bits<32>(static_cast<const uint8_t*>(s.app_index) + ((int64_t)q * 128 + 32 * g) * (s.app_bf16 ? 2 : 4),
                         s.app_bf16, bits);
    uint32_t w[4];
    const int code = mxfp4_group(bits, w);
    uint8_t* kc = const_cast<uint8_t*>(s.k_codes) + (int64_t)seq * s.k_cs + r * s.k_ce + 16 * g;
    *reinterpret_cast<uint4*>(kc) = make_uint4(w[0], w[1], w[2], w[3]);
    const_cast<uint8_t*>(s.k_scales)[(int64_t)seq * s.k_ss + r * s.k_se + g] = (uint8_t)code;
  }
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// reduce-scatter of the four tiles' per-lane-group partial sums: lane group g ends with tile
// g's full sum, so lane l holds the score of entry l of the step.  V_PERMLANE32_SWAP of
// (tile 0, tile 2) leaves in its two results, lane by lane, the two halves of the wave that
// the lane's own half needs, so their sum is tiles 0 + 0' for the low half and 2 + 2' for
// the high one (likewise tiles 1 and 3); V_PERMLANE16_SWAP does the same across the 16-lane
// groups.  No LDS round trip; each sum adds the same two numbers as a lane exchange would.
__device__ __forceinline__ float scatter_tiles(const float (&part)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
  const float k0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float k1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ReLU on the bit pattern: a non-negative float is a non-negative int and a negative one
// (or -0) a negative int, so one integer max gives max(x, +0)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of the 64 entries of one step (four 16-entry MFMA tiles) for one query row: A =
// the row's indexer Q (16 heads x 128 channels, this lane: head `lane % 16`, channels
// 32*kb..+31), B = the tiles' indexer K.  Lane l returns the score of entry l of the step.
__device__ __forceinline__ float score_tiles(const v8i& a, int a_scale, const float (&wv)[4], int kb,
                                             const uint4 (&bc)[4], const int (&bs)[4]) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v8i b = {(int)bc[t].x, (int)bc[t].y, (int)bc[t].z, (int)bc[t].w, 0, 0, 0, 0};
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    // formats 4/4 = E2M1 for both operands; scales are E8M0, byte 0 of each lane's VGPR
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, a_scale, 0, bs[t]);
    float p = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) p += wv[r] * relu(acc[r]);
    part[t] = p;
  }
  return scatter_tiles(part);
}

// ---- NVFP4-style indexer operands (E2M1 + one E4M3 scale per 16 channels) ----
// The scaled matrix-core instruction takes power-of-two (E8M0) scales per 32 elements, so
// this format runs as fp16 MFMAs on dequantised operands.  A lane's 16 code bytes (32
// channels) become 32 fp16 values: the gfx950 converts apply only the exponent of their
// fp32 scale operand, so they run unscaled (exact E2M1 -> fp16 and E4M3 -> fp16) and the
// E4M3 scale is one packed fp16 multiply, exact because E2M1 x E4M3 has at most 5
// significant bits and |x| <= 6 * 448 (no fp16 rounding, overflow or subnormal).  Code
// bytes 0-7 take the low scale byte, 8-15 the high one.  Dword u of the codes becomes
// x[u] (byte b -> elements 2b, 2b+1), the K-slice of the u-th 16x16x32 MFMA; A and B lanes
// use the same mapping, so every step multiplies matching channels.
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void nv_dequant(const uint4& c, uint32_t sc, v8h (&x)[4]) {
  const v2h s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
  const v2h s0 = {s[0], s[0]}, s1 = {s[1], s[1]};
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const v2h su = u < 2 ? s0 : s1;
    const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[u], 1.0f, 0) * su;
    const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[u], 1.0f, 1) * su;
    const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[u], 1.0f, 2) * su;
    const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[u], 1.0f, 3) * su;
    x[u] = v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
}

// as score_tiles, for NVFP4 operands: A = the row's dequantised indexer Q, bs[t] = the two
// E4M3 scale bytes of this lane's 32 channels of tile t's entry
__device__ __forceinline__ float score_tiles_nv(const v8h (&a)[4], const float (&wv)[4], int kb,
                                                const uint4 (&bc)[4], const int (&bs)[4]) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v8h b[4];
    nv_dequant(bc[t], (uint32_t)bs[t], b);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[u], b[u], acc, 0, 0, 0);
    float p = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) p += wv[r] * relu(acc[r]);
    part[t] = p;
  }
  return scatter_tiles(part);
}

// One query's view of the cache: MFMA operands, slot -> row mapping, one scoring step.
// Slots and rows are 32-bit (seq_cap <= 2^26) and the sequence's base pointers are
// workgroup-uniform, so each load is a scalar base plus the row times the entry stride.
template <bool kPool, bool kNv, bool kQLat = false>
struct QueryScorer {
  // scale bytes per entry (and per query head row): one per 32 channels (MXFP4) or per 16
  static constexpr uint32_t kScalesPerRow = kNv ? 8u : 4u;
  v8i a;             // A operand (MXFP4): indexer Q rows (heads), 32 FP4 values per lane
  int a_scale;
  v8h an[4];         // A operand (NVFP4): the same 32 channels dequantised to fp16
  float wv[4];       // weights of the 4 output rows (heads 4*kb .. 4*kb+3) of this lane
  int nv;            // visible entries, clamped to the cache
  int n_valid;       // slots that may hold a real candidate
  const uint8_t* kc; // this sequence's indexer-K codes / scales
  const uint8_t* ks;
  const int32_t* cb;
  int blk_lim;       // nv / block: no visible position lies in a block past this one
  int row, kb;       // A row (head) / B column (entry within tile); K-block of 32

  // with_q false: everything but the A operand and the weights, which init_q then sets
  // (so that a kernel can issue its first K loads before the Q loads and their quantisation)
  __device__ __forceinline__ bool init(const ScoreArgs& s, int q, bool with_q = true) {
    const int lane = threadIdx.x & 63;
    row = lane & 15;
    kb = lane >> 4;
    const int seq = s.q_seq[q];
    if (seq < 0 || seq >= s.n_seq) return false;
    int64_t v = s.n_vis[q];
    nv = (int)(v < 0 ? 0 : (v > s.seq_cap ? s.seq_cap : v));
    if (kPool) {
      int64_t nc = s.n_cand_blocks[q];
      nc = nc < 0 ? 0 : (nc > s.max_cand_blocks ? s.max_cand_blocks : nc);
      n_valid = (int)nc * s.block;
      cb = s.cand_blocks + (int64_t)q * s.max_cand_blocks;
      blk_lim = nv / s.block;
    } else {
      n_valid = nv;
      cb = nullptr;
    }
    kc = s.k_codes + (int64_t)seq * s.k_cs;
    ks = s.k_scales + (int64_t)seq * s.k_ss;
    if (with_q) init_q(s, q);
    return true;
  }

  __device__ __forceinline__ void init_q(const ScoreArgs& s, int q) {
    a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    a_scale = 127;
#pragma unroll
    for (int u = 0; u < 4; ++u) an[u] = v8h{};
    if (row < s.n_heads) {
      const int64_t r = (int64_t)q * s.n_heads + row;
      if constexpr (kQLat) {
        // this lane's A operand is one whole MXFP4 group (head `row`, channels 32*kb ..
        // +31): quantise it here, with the same rule as csa2_quantize_kv
        uint32_t bits[32];
        load_latent_bits<32>(static_cast<const uint8_t*>(s.q_lat) + (r * 128 + kb * 32) * (s.q_bf16 ? 2 : 4), s.q_bf16,
                             bits);
        uint32_t wq[4];
        a_scale = mxfp4_group(bits, wq);
        a[0] = (int)wq[0];
        a[1] = (int)wq[1];
        a[2] = (int)wq[2];
        a[3] = (int)wq[3];
      } else {
        const uint4 qa = *reinterpret_cast<const uint4*>(s.q_codes + r * 64 + kb * 16);
        if (kNv) {
          const uint32_t qs = *reinterpret_cast<const uint16_t*>(s.q_scales + r * 8 + kb * 2);
          nv_dequant(qa, qs, an);
        } else {
          a[0] = (int)qa.x;
          a[1] = (int)qa.y;
          a[2] = (int)qa.z;
          a[3] = (int)qa.w;
          a_scale = s.q_scales[r * 4 + kb];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kb + r;
      wv[r] = h < s.n_heads ? s.w[(int64_t)q * s.n_heads + h] : 0.0f;
    }
  }

  // slot -> (row to read, valid); invalid slots read row 0 and their results are discarded,
  // so the loads need no per-lane branches.  Inside a pool the block id is loaded for every
  // slot (slot 0's for an invalid one): a load under a per-lane condition would be waited
  // for on its own, before the loads that follow it are issued.
  __device__ __forceinline__ bool slot_pos(const ScoreArgs& s, int slot, uint32_t& pos) const {
    bool valid = slot < n_valid;
    int p = slot;
    if (kPool) {
      const int32_t b = cb[(valid ? (uint32_t)slot : 0u) / (uint32_t)s.block];
      valid = valid && b >= 0 && b <= blk_lim;   // bounds b before b * block can overflow
      p = b * s.block + (int)((uint32_t)slot % (uint32_t)s.block);
      valid = valid && p < nv;
    }
    pos = valid ? (uint32_t)p : 0u;
    return valid;
  }

  __device__ __forceinline__ void load_step(const ScoreArgs& s, int base, uint4 (&bc)[4], int (&bs)[4]) const {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t pos;
      slot_pos(s, base + 16 * t + row, pos);
      const v4u v = __builtin_nontemporal_load(
          reinterpret_cast<const v4u*>(kc + ((uint64_t)pos * (uint64_t)s.k_ce + kb * 16u)));
      bc[t] = make_uint4(v.x, v.y, v.z, v.w);
      // NVFP4: the two scale bytes of this lane's 32 channels, one 16-bit load
      const uint8_t* sp = ks + (uint64_t)pos * (uint64_t)s.k_se;
      bs[t] = kNv ? (int)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sp + kb * 2u))
                  : (int)__builtin_nontemporal_load(sp + kb);
    }
  }

  // scores of the 64 entries of one step; lane l returns the score of entry l
  __device__ __forceinline__ float score_step(const uint4 (&bc)[4], const int (&bs)[4]) const {
    if (kNv) return score_tiles_nv(an, wv, kb, bc, bs);
    return score_tiles(a, a_scale, wv, kb, bc, bs);
  }
};

// ---- several query rows of one sequence over one pass of its indexer K ----
// Multi-token decode (several tokens of a sequence verified at once) and the rows of a
// prefill chunk score the same K stream: a workgroup takes a group of up to kGroupMax
// consecutive rows of one sequence and a chunk of its entries, loads each step's K tiles
// once and runs the MFMAs of every row of the group on them, so K is read once per group
// instead of once per row.  The arithmetic per (row, entry) is that of k_score_decode, so
// the scores are bit-identical to the per-row kernel's.
constexpr int kGroupMax = 8;

__global__ __launch_bounds__(kScoreThreads) void k_score_grouped(ScoreArgs s, int n_q, int group) {
  const int gi = blockIdx.y;
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15, kb = lane >> 4;
  const int r0 = gi * group;
  const int nr = n_q - r0 < group ? n_q - r0 : group;
  const int seq = s.q_seq[r0];
  if (seq < 0 || seq >= s.n_seq) return;

  // the rows' A operands, scales, head weights and visible counts; a row of another
  // sequence than the group's first row is left out (it gets no scores)
  uint4 qa[kGroupMax];
  int asc[kGroupMax];
  float wv[kGroupMax][4];
  int nvr[kGroupMax];
  int nv_max = 0;
#pragma unroll
  for (int r = 0; r < kGroupMax; ++r) {
    const int q = r0 + r;
    const bool ok = r < nr && s.q_seq[q] == seq;
    int64_t v = ok ? s.n_vis[q] : 0;
    nvr[r] = (int)(v < 0 ? 0 : (v > s.seq_cap ? s.seq_cap : v));
    nv_max = nvr[r] > nv_max ? nvr[r] : nv_max;
    qa[r] = make_uint4(0u, 0u, 0u, 0u);
    asc[r] = 127;
    if (ok && row < s.n_heads) {
      const int64_t hr = (int64_t)q * s.n_heads + row;
      qa[r] = *reinterpret_cast<const uint4*>(s.q_codes + hr * 64 + kb * 16);
      asc[r] = s.q_scales[hr * 4 + kb];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * kb + j;
      wv[r][j] = ok && h < s.n_heads ? s.w[(int64_t)q * s.n_heads + h] : 0.0f;
    }
  }
  const int chunk_lo = chunk * s.chunk_len;
  if (chunk_lo >= nv_max) return;
  const int hi = chunk_lo + s.chunk_len < nv_max ? chunk_lo + s.chunk_len : nv_max;
  const uint8_t* kc = s.k_codes + (int64_t)seq * s.k_cs;
  const uint8_t* ks = s.k_scales + (int64_t)seq * s.k_ss;
  // entries past the group's visible range read entry 0 and their results are discarded
  auto load_step = [&](int base, uint4 (&bc)[4], int (&bs)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = base + 16 * t + row;
      const uint32_t pos = e < nv_max ? (uint32_t)e : 0u;
      const v4u v = __builtin_nontemporal_load(
          reinterpret_cast<const v4u*>(kc + ((uint64_t)pos * (uint64_t)s.k_ce + kb * 16u)));
      bc[t] = make_uint4(v.x, v.y, v.z, v.w);
      bs[t] = __builtin_nontemporal_load(ks + ((uint64_t)pos * (uint64_t)s.k_se + kb));
    }
  };
  int base = chunk_lo + wave * kScoreStep;
  uint4 bc[4];
  int bs[4];
  if (base < hi) load_step(base, bc, bs);
  for (; base < hi; base += 4 * kScoreStep) {
    uint4 bcn[4];
    int bsn[4];
    const int next = base + 4 * kScoreStep;
    load_step(next < hi ? next : base, bcn, bsn);
    const int slot = base + lane;
#pragma unroll
    for (int r = 0; r < kGroupMax; ++r) {
      if (r < nr) {  // uniform
        const v8i a = {(int)qa[r].x, (int)qa[r].y, (int)qa[r].z, (int)qa[r].w, 0, 0, 0, 0};
        const float v = score_tiles(a, asc[r], wv[r], kb, bc, bs);
        if (slot < nvr[r]) s.scores[(int64_t)(r0 + r) * s.scores_stride + slot] = v;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bc[t] = bcn[t];
      bs[t] = bsn[t];
    }
  }
}

// ---- grouped rows, scored and selected in one pass: no score array ----
// The rows of a prefill chunk (or several decode tokens of one sequence) each need their own
// Top-K over the sequence's visible entries.  A workgroup takes a group of up to kGroupMax
// rows and a contiguous range of entries; each of its four waves owns kGtRowsPerWave of the
// rows and streams the whole range (the waves read the same K tiles at about the same time,
// so three of the four loads hit the L1 cache), scoring its rows on every 64-entry step.
// Per row the owning wave keeps a list of candidate keys in LDS: an entry enters only if its
// key is at or above the row's threshold, and when the list is about to overflow the wave
// selects its best K in place (select_wave, stable) and raises the threshold to the K-th key:
// keys below it can never reach the row's Top-K.  A list is written by its wave alone, in
// position order (entries are appended in order, the selection keeps the order), so no wave
// ever waits for another.  At the end of the range each row's best K, in position order, is
// what a first Top-K level writes for that range, and the last level (k_topk_final) picks the
// row's Top-K over the ranges.  Appends per row over R entries in random order: about
// K * (1 + ln(R / K)).
constexpr int kGtRowsPerWave = kGroupMax / (kScoreThreads / 64);   // 2
constexpr int kGtCap = 768;                                        // candidate keys per row in LDS

// kOff32: every entry's code and scale offsets within its sequence fit 32 bits (the host
// checks seq_cap * stride), so a load is the sequence's uniform base plus a 32-bit lane offset
// that advances by a constant per step instead of a 64-bit multiply per tile.
template <bool kOff32>
__global__ __launch_bounds__(kScoreThreads) void k_score_topk_grouped(ScoreArgs s, int n_q, int group,
                                                                      int range_len, int n_ranges) {
  const int range = blockIdx.x;    // consecutive workgroups take consecutive ranges, so one
  const int gi = blockIdx.y;       // range's workgroups share an XCD (and its L2) when n_ranges | 8
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, kb = lane >> 4;
  const int r0 = gi * group;
  const int nr = n_q - r0 < group ? n_q - r0 : group;
  const int K = s.k;
  __shared__ __attribute__((aligned(16))) uint64_t list[kGroupMax][kGtCap];          // 48 KB
  __shared__ __attribute__((aligned(16))) uint32_t hist[kScoreThreads / 64][256];   // per wave

  const int seq = s.q_seq[r0];
  const bool seq_ok = seq >= 0 && seq < s.n_seq;
  // this wave's rows: group rows wave, wave + 4 (so a group of 4 rows or fewer still spreads
  // over the waves)
  uint4 qa[kGtRowsPerWave];
  int asc[kGtRowsPerWave];
  float wv[kGtRowsPerWave][4];
  int nvr[kGtRowsPerWave];
  bool own[kGtRowsPerWave];
  int nv_max = 0;
#pragma unroll
  for (int u = 0; u < kGtRowsPerWave; ++u) {
    const int r = wave + (kScoreThreads / 64) * u;
    const int q = r0 + r;
    own[u] = r < nr;
    const bool ok = seq_ok && own[u] && s.q_seq[q] == seq;
    int64_t v = ok ? s.n_vis[q] : 0;
    nvr[u] = (int)(v < 0 ? 0 : (v > s.seq_cap ? s.seq_cap : v));
    nv_max = nvr[u] > nv_max ? nvr[u] : nv_max;
    qa[u] = make_uint4(0u, 0u, 0u, 0u);
    asc[u] = 127;
    if (ok && row < s.n_heads) {
      const int64_t hr = (int64_t)q * s.n_heads + row;
      qa[u] = *reinterpret_cast<const uint4*>(s.q_codes + hr * 64 + kb * 16);
      asc[u] = s.q_scales[hr * 4 + kb];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * kb + j;
      wv[u][j] = ok && h < s.n_heads ? s.w[(int64_t)q * s.n_heads + h] : 0.0f;
    }
  }
  const int lo = range * range_len;
  const int hi = lo + range_len < nv_max ? lo + range_len : nv_max;   // uniform over the wave
  const uint8_t* kc = s.k_codes + (int64_t)(seq_ok ? seq : 0) * s.k_cs;
  const uint8_t* ks = s.k_scales + (int64_t)(seq_ok ? seq : 0) * s.k_ss;
  // entries past hi (the next range's, or past the visible end) read entry hi - 1 and their
  // results are discarded
  const uint32_t ce = (uint32_t)s.k_ce, se = (uint32_t)s.k_se;
  const uint32_t last = hi > 0 ? (uint32_t)(hi - 1) : 0u;
  const uint32_t c_last = last * ce + kb * 16u, s_last = last * se + kb;
  uint32_t c_off[4], s_off[4];   // kOff32: offsets of the next step's entries
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t e0 = (uint32_t)(lo + 16 * t + row);
    c_off[t] = e0 * ce + kb * 16u;
    s_off[t] = e0 * se + kb;
  }
  auto load_step = [&](int base, uint4 (&bc)[4], int (&bs)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (kOff32) {
        const uint32_t co = c_off[t] < c_last ? c_off[t] : c_last;
        const uint32_t so = s_off[t] < s_last ? s_off[t] : s_last;
        const v4u v = *reinterpret_cast<const v4u*>(kc + co);
        bc[t] = make_uint4(v.x, v.y, v.z, v.w);
        bs[t] = ks[so];
        c_off[t] += 64u * ce;
        s_off[t] += 64u * se;
      } else {
        const int e = base + 16 * t + row;
        const uint32_t pos = e < hi ? (uint32_t)e : last;
        const v4u v = *reinterpret_cast<const v4u*>(kc + ((uint64_t)pos * (uint64_t)s.k_ce + kb * 16u));
        bc[t] = make_uint4(v.x, v.y, v.z, v.w);
        bs[t] = ks[(uint64_t)pos * (uint64_t)s.k_se + kb];
      }
    }
  };
  int cnt[kGtRowsPerWave];
  uint64_t thr[kGtRowsPerWave];
#pragma unroll
  for (int u = 0; u < kGtRowsPerWave; ++u) {
    cnt[u] = 0;
    thr[u] = 1ull;   // every real key (nonzero) enters until the first selection
  }
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));

  // the best K of list u, in place and in order; raises its threshold
  auto shrink = [&](int u) {
    uint64_t* l = list[wave + (kScoreThreads / 64) * u];
    uint64_t key[kGtCap / 64];
#pragma unroll
    for (int i = 0; i < kGtCap / 64; ++i) {
      const int j = i * 64 + lane;
      key[i] = j < cnt[u] ? l[j] : 0ull;
    }
    const uint64_t t = select_wave<kGtCap / 64>(key, K, hist[wave], l);
    thr[u] = t > thr[u] ? t : thr[u];
    cnt[u] = cnt[u] < K ? cnt[u] : K;
  };

  if (lo < hi) {
    uint4 bc[4];
    int bs[4];
    load_step(lo, bc, bs);
    for (int base = lo; base < hi; base += 64) {
      uint4 bcn[4];
      int bsn[4];
      load_step(base + 64 < hi ? base + 64 : base, bcn, bsn);   // past the end: entry hi - 1
      const int e = base + lane;
      // every row's matrix work first (a row whose visible range has ended is scored and
      // discarded), so one row's reductions overlap the next row's MFMAs
      float v[kGtRowsPerWave];
#pragma unroll
      for (int u = 0; u < kGtRowsPerWave; ++u) {
        const v8i a = {(int)qa[u].x, (int)qa[u].y, (int)qa[u].z, (int)qa[u].w, 0, 0, 0, 0};
        v[u] = score_tiles(a, asc[u], wv[u], kb, bc, bs);
      }
#pragma unroll
      for (int u = 0; u < kGtRowsPerWave; ++u) {
        if (nvr[u] > base) {   // uniform
          const uint64_t key = make_key(v[u], (uint32_t)e);
          const bool in = e < hi && e < nvr[u] && key >= thr[u];   // past hi: the next range's entry
          const uint64_t m = __ballot(in);
          if (in) list[wave + (kScoreThreads / 64) * u][cnt[u] + (int)__popcll(m & lt_mask)] = key;
          cnt[u] += (int)__popcll(m);
          if (cnt[u] > kGtCap - 64) shrink(u);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bc[t] = bcn[t];
        bs[t] = bsn[t];
      }
    }
  }
  // each row's best K of this range, in position order, zero padded
#pragma unroll
  for (int u = 0; u < kGtRowsPerWave; ++u) {
    if (!own[u]) continue;
    if (cnt[u] > K) shrink(u);
    const uint64_t* l = list[wave + (kScoreThreads / 64) * u];
    uint64_t* o = s.keys_out + ((int64_t)(r0 + wave + (kScoreThreads / 64) * u) * n_ranges + range) * K;
    for (int j = lane; j < K; j += 64) o[j] = j < cnt[u] ? l[j] : 0ull;
  }
}

template <bool kPool, bool kNv, bool kQLat = false>
__global__ __launch_bounds__(kScoreThreads) void k_score_decode(ScoreArgs s) {
  const int q = blockIdx.x / s.chunks;
  const int chunk = blockIdx.x % s.chunks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  QueryScorer<kPool, kNv, kQLat> sc;
  if (!sc.init(s, q)) return;
  const int chunk_lo = chunk * s.chunk_len;
  const int write_hi = kPool ? (int)s.n_slots : sc.n_valid;  // pool mode also writes -inf pads
  if (chunk_lo >= write_hi) return;
  float* out = s.scores + (int64_t)q * s.scores_stride;
  const int hi = chunk_lo + s.chunk_len < write_hi ? chunk_lo + s.chunk_len : write_hi;

  int base = chunk_lo + wave * kScoreStep;
  if (sc.nv <= 0) {  // nothing to read: pool slots are all -inf, no-pool chunks never get here
    for (; base < hi; base += 4 * kScoreStep)
      if (base + lane < hi) out[base + lane] = -__builtin_inff();
    return;
  }
  uint4 bc[4];
  int bs[4];
  if (base < hi) sc.load_step(s, base, bc, bs);
  for (; base < hi; base += 4 * kScoreStep) {
    // prefetch the next step while this one is computed; past the end, re-read this step
    // (an L2 hit) so that the load stays unconditional
    uint4 bcn[4];
    int bsn[4];
    const int next = base + 4 * kScoreStep;
    sc.load_step(s, next < hi ? next : base, bcn, bsn);
    const int slot = base + lane;
    uint32_t pos;
    const bool valid = sc.slot_pos(s, slot, pos);   // (its block-id load overlaps the MFMAs)
    const float v = sc.score_step(bc, bs);
    if (slot < hi) out[slot] = (kPool && !valid) ? -__builtin_inff() : v;   // without a pool, slot < hi <= n_valid
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bc[t] = bcn[t];
      bs[t] = bsn[t];
    }
  }
}

// Scores one segment of kTkSeg slots and selects its K best in the same workgroup.  Step i
// of wave w covers slots i*256 + w*64 + lane of the segment, so thread t scores candidates
// i*256 + t: the candidate order select_segment expects.  While the loads stream, each
// thread parks its 32 scores in its own column of an LDS array (stride 256 words: no bank
// conflicts, no barrier needed) instead of registers, so the loop keeps the register
// budget of the plain scoring kernel and four workgroups fit a CU; once the keys are back
// in registers the same LDS holds the selection histograms.
//
// kBlockMax: the segment also writes the maximum visible score of each of its blocks of
// s.block positions (the pool's block scores), read from the parked scores before the
// selection reuses that LDS.
template <bool kPool, bool kFinal, bool kBlockMax, bool kNv, bool kQLat = false>
__global__ __launch_bounds__(kScoreThreads) void k_score_select(ScoreArgs s) {
  static_assert(kTkSeg >= kTkHistWords, "the score array doubles as the selection histograms");
  __shared__ __attribute__((aligned(16))) float park[kTkSeg];
  const int seg = blockIdx.x;
  const int q = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint64_t key[kTkEpt];
  QueryScorer<kPool, kNv, kQLat> sc;
  const int c0 = seg * kTkSeg;
  if (!kNv && s.app_row) {   // uniform (a kernel argument): a csa2_append (MXFP4 indexer)
    const int seq = s.q_seq[q];
    const int64_t r = s.app_row[q];
    if (seq >= 0 && seq < s.n_seq && r >= 0 && r < s.seq_cap && r / kTkSeg == seg) {   // uniform
      // this segment holds the query's new row: write it, and let the stores complete
      // before any wave of the workgroup reads the indexer K
      if (wave == 0) append_entry(s, q, seq, r, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  const bool seq_ok = sc.init(s, q, false);
  // workgroup-uniform condition: every thread reaches select_segment's barriers
  if (seq_ok && sc.nv > 0 && c0 < sc.n_valid) {
    uint4 bc[4];
    int bs[4];
    sc.load_step(s, c0 + wave * kScoreStep, bc, bs);
    sc.init_q(s, q);   // the Q operand (and, unquantised, its quantisation) while those loads fly
#pragma unroll 2
    for (int i = 0; i < kTkEpt; ++i) {
      const int base = c0 + i * kTkThreads + wave * kScoreStep;
      uint4 bcn[4];
      int bsn[4];
      // the last step re-reads itself so that the prefetch stays unconditional
      sc.load_step(s, i + 1 < kTkEpt ? base + kTkThreads : base, bcn, bsn);
      park[i * kTkThreads + tid] = sc.score_step(bc, bs);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bc[t] = bcn[t];
        bs[t] = bsn[t];
      }
    }
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) {
      uint32_t pos;
      const bool valid = sc.slot_pos(s, c0 + i * kTkThreads + tid, pos);
      key[i] = valid ? make_key(park[i * kTkThreads + tid], pos) : 0ull;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTkEpt; ++i) key[i] = 0ull;
  }
  if (kBlockMax) {
    // block b of the segment is positions c0 + b*block .. +block-1: in the parked layout
    // (candidate i*256 + t at park[i*256 + t]) that is `block` consecutive words, written by
    // other threads
    __syncthreads();
    const int nb = kTkSeg / s.block;
    const int nv = seq_ok ? sc.nv : 0;
    const int64_t nb_q = ((int64_t)nv + s.block - 1) / s.block;   // blocks holding a visible entry
    for (int b = tid; b < nb; b += kTkThreads) {
      const int64_t gb = (int64_t)seg * nb + b;
      if (gb >= s.bmax_stride) break;
      float m = -__builtin_inff();
      if (gb < nb_q) {
        for (int j = 0; j < s.block; ++j) {
          const int p = c0 + b * s.block + j;
          if (p < nv) m = fmaxf(m, park[b * s.block + j]);
        }
      }
      s.bmax[(int64_t)q * s.bmax_stride + gb] = m;
    }
    __syncthreads();  // the parked scores are read before select_segment reuses the LDS
  }
  select_segment<kFinal>(key, q, seg, gridDim.x, s.k, reinterpret_cast<uint32_t*>(park), s.keys_out, s.idx_out,
                         s.count_out);
}

// CSA2_FMT_MXFP4_Q_*: an MXFP4 indexer whose Q comes unquantised
static bool q_latent(int fmt) { return fmt == CSA2_FMT_MXFP4_Q_F32 || fmt == CSA2_FMT_MXFP4_Q_BF16; }

// The indexer-K cache of a call: fmt (CSA2_FMT_MXFP4 or CSA2_FMT_NVFP4) fixes its scale row
// (4 bytes of E8M0 or 8 of E4M3 per 128 channels; NVFP4 scales are read two bytes at a time).
static int resolve_index_cache(int fmt, CacheRef& kr, int64_t seq_cap) {
  if (q_latent(fmt)) fmt = CSA2_FMT_MXFP4;
  if (fmt != CSA2_FMT_MXFP4 && fmt != CSA2_FMT_NVFP4) return CSA2_ERR_UNSUPPORTED;
  if (!kr.codes || !kr.scales) return CSA2_ERR_NULL;
  if (!aligned16(kr.codes)) return CSA2_ERR_SHAPE;
  const bool nv = fmt == CSA2_FMT_NVFP4;
  if (nv && ((uintptr_t)kr.scales & 1u)) return CSA2_ERR_SHAPE;
  return resolve_cache(kr, seq_cap, CSA2_INDEX_DIM / 2, nv ? CSA2_INDEX_DIM / 16 : CSA2_INDEX_DIM / 32, nv ? 2 : 1);
}

static int check_score_args(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q, int n_heads,
                            int dim, int fmt, CacheRef& kr, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                            const int64_t* n_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block,
                            int max_cand_blocks, int64_t* n_slots) {
  if (!q_codes || (!q_scales && !q_latent(fmt)) || !w || !q_seq || !n_vis) return CSA2_ERR_NULL;
  if (n_q < 0 || n_heads < 1 || n_heads > CSA2_MAX_INDEX_HEADS || dim != CSA2_INDEX_DIM || seq_cap < 0 ||
      seq_cap > CSA2_MAX_INDEX_ENTRIES || n_seq < 1)
    return CSA2_ERR_SHAPE;
  if (!aligned16(q_codes)) return CSA2_ERR_SHAPE;
  if (fmt == CSA2_FMT_NVFP4 && ((uintptr_t)q_scales & 1u)) return CSA2_ERR_SHAPE;
  const int rc = resolve_index_cache(fmt, kr, seq_cap);
  if (rc != CSA2_OK) return rc;
  if (cand_blocks) {
    if (!n_cand_blocks) return CSA2_ERR_NULL;
    if (block < 1 || block > 64 || max_cand_blocks < 1 || max_cand_blocks > (1 << 20)) return CSA2_ERR_SHAPE;
    *n_slots = (int64_t)max_cand_blocks * block;
  } else {
    *n_slots = seq_cap;
  }
  return CSA2_OK;
}

static ScoreArgs make_args(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_heads,
                           const CacheRef& kr, int64_t seq_cap, int n_seq, const int32_t* q_seq, const int64_t* n_vis,
                           const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block, int max_cand_blocks,
                           int64_t n_slots, int fmt = CSA2_FMT_MXFP4) {
  ScoreArgs a = {};
  if (q_latent(fmt)) {   // q_codes is the unquantised Q
    a.q_lat = q_codes;
    a.q_bf16 = fmt == CSA2_FMT_MXFP4_Q_BF16;
  } else {
    a.q_codes = q_codes;
    a.q_scales = q_scales;
  }
  a.w = w;
  a.n_heads = n_heads;
  a.k_codes = kr.codes;
  a.k_scales = kr.scales;
  a.k_ce = kr.ce;
  a.k_cs = kr.cs;
  a.k_se = kr.se;
  a.k_ss = kr.ss;
  a.seq_cap = seq_cap;
  a.n_seq = n_seq;
  a.q_seq = q_seq;
  a.n_vis = n_vis;
  a.cand_blocks = cand_blocks;
  a.n_cand_blocks = n_cand_blocks;
  a.block = block;
  a.max_cand_blocks = max_cand_blocks;
  a.n_slots = n_slots;
  return a;
}

// Writes scores[q, slot].  Inside a pool each slot's row comes from a block-id load, so a
// wave's step is two dependent memory round trips and a workgroup is latency-bound:
// pool chunks are small (2 steps per wave) to spread the pool over many workgroups.
static int launch_score(ScoreArgs a, int n_q, float* scores, int64_t scores_stride, bool nv, hipStream_t st,
                        bool q_lat = false) {
  a.chunk_len = a.cand_blocks ? kPoolChunk : kScoreChunk;
  const int64_t chunks = (a.n_slots + a.chunk_len - 1) / a.chunk_len;
  if (chunks * (int64_t)n_q > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  a.scores = scores;
  a.scores_stride = scores_stride;
  a.chunks = (int)chunks;
  dim3 grid((unsigned)(chunks * n_q)), blk(kScoreThreads);
  if (q_lat) {   // MXFP4 only
    if (a.cand_blocks) hipLaunchKernelGGL((k_score_decode<true, false, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_score_decode<false, false, true>), grid, blk, 0, st, a);
  } else if (nv) {
    if (a.cand_blocks) hipLaunchKernelGGL((k_score_decode<true, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_score_decode<false, true>), grid, blk, 0, st, a);
  } else {
    if (a.cand_blocks) hipLaunchKernelGGL((k_score_decode<true, false>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_score_decode<false, false>), grid, blk, 0, st, a);
  }
  return csa2_check_launch();
}

// A fused scoring call's csa2_append -> the ScoreArgs fields (nothing when app is null).
// Returns a csa2 status.
static int set_append(ScoreArgs& a, const csa2_append* app, int64_t seq_cap, int fmt) {
  if (!app) return CSA2_OK;
  if (fmt == CSA2_FMT_NVFP4) return CSA2_ERR_UNSUPPORTED;   // the appended indexer-K row is MXFP4
  if (!app->row) return CSA2_ERR_NULL;
  if (app->dtype != CSA2_DT_F32 && app->dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (app->main) {
    if (!app->kv_codes || !app->kv_scales) return CSA2_ERR_NULL;
    if (!aligned16(app->main) || !aligned16(app->kv_codes)) return CSA2_ERR_SHAPE;
    CacheRef kv{app->kv_codes, app->kv_scales, app->kv_codes_stride, app->kv_codes_seq_stride,
                app->kv_scales_stride, app->kv_scales_seq_stride};
    if (resolve_cache(kv, seq_cap, 256, 32, 1) != CSA2_OK) return CSA2_ERR_SHAPE;
    a.app_kv_codes = app->kv_codes;
    a.app_kv_scales = app->kv_scales;
    a.app_kv_ce = kv.ce;
    a.app_kv_cs = kv.cs;
    a.app_kv_se = kv.se;
    a.app_kv_ss = kv.ss;
  }
  if (app->index && !aligned16(app->index)) return CSA2_ERR_SHAPE;
  a.app_row = app->row;
  a.app_main = app->main;
  a.app_index = app->index;
  a.app_bf16 = app->dtype == CSA2_DT_BF16;
  return CSA2_OK;
}

// k_score_select for the indexer format of a call (NVFP4; MXFP4 with quantised or
// unquantised Q); the pool build (kBlockMax) exists for MXFP4 only
template <bool kFinal, bool kBlockMax>
static int launch_score_select(int fmt, dim3 grid, hipStream_t st, const ScoreArgs& a) {
  const dim3 blk(kScoreThreads);
  if (q_latent(fmt)) {
    hipLaunchKernelGGL((k_score_select<false, kFinal, kBlockMax, false, true>), grid, blk, 0, st, a);
  } else if (fmt == CSA2_FMT_NVFP4) {
    if constexpr (kBlockMax) return CSA2_ERR_UNSUPPORTED;
    else hipLaunchKernelGGL((k_score_select<false, kFinal, false, true>), grid, blk, 0, st, a);
  } else {
    hipLaunchKernelGGL((k_score_select<false, kFinal, kBlockMax, false>), grid, blk, 0, st, a);
  }
  return csa2_check_launch();
}

// Bytes of the csa2_index_topk workspace: the selection levels' keys; inside a pool also
// the score array (the pool is small: the round trip is cheap there and the unfused
// kernels spread a latency-bound gather over more workgroups).
static size_t index_topk_ws(int n_q, int64_t n_slots, int k, bool pool) {
  const size_t sel = ws_bytes(n_q, n_slots, k);
  if (!pool) return sel;
  return (((size_t)n_q * n_slots * sizeof(float) + 255) & ~(size_t)255) + sel + 256;
}

static size_t index_topk_pool_ws(int n_q, int64_t n_slots, int k, int block, int max_blocks, size_t* bmax_bytes,
                                 size_t* sel_bytes) {
  const int64_t nblk = (n_slots + block - 1) / block;
  *bmax_bytes = (((size_t)n_q * nblk * sizeof(float)) + 255) & ~(size_t)255;
  *sel_bytes = (ws_bytes(n_q, n_slots, k) + 255) & ~(size_t)255;
  return 256 + *bmax_bytes + *sel_bytes + ws_bytes(n_q, nblk, max_blocks) + 256;
}

// Ranges per row of csa2_index_topk_grouped: a power of two (so that, with consecutive
// workgroups on consecutive XCDs, one range's workgroups share an XCD and its L2 holds the
// range's indexer K), with all ranges' survivors within one last selection level (n_ranges *
// k <= 8,192) and ranges of at least 8,192 entries; as many as that allows while the grid is
// below 3 workgroups per CU (the LDS of the candidate lists fits three), and at least 16,384
// entries per range beyond.
static int grouped_ranges(int64_t seq_cap, int k, int64_t n_groups) {
  int n = 1;
  auto ok = [&](int m) { return m <= 16 && (int64_t)m * k <= kTkSeg && seq_cap >= (int64_t)m * 8192; };
  while (ok(2 * n) && (n_groups * n < 3 * 256 || seq_cap >= (int64_t)2 * n * 16384)) n *= 2;
  return n;
}

}  // namespace csa2

using namespace csa2;

#define CSA2_INDEX_CACHE_ARGS                                                                          \
  int fmt, const uint8_t *k_codes, int64_t k_codes_stride, int64_t k_codes_seq_stride,                 \
      const uint8_t *k_scales, int64_t k_scales_stride, int64_t k_scales_seq_stride
#define CSA2_INDEX_CACHE_REF \
  CacheRef { k_codes, k_scales, k_codes_stride, k_codes_seq_stride, k_scales_stride, k_scales_seq_stride }

extern "C" int csa2_index_score(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                int n_heads, int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq,
                                const int32_t* q_seq, const int64_t* n_vis, const int32_t* cand_blocks,
                                const int32_t* n_cand_blocks, int block, int max_cand_blocks, float* scores,
                                int64_t scores_stride, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis,
                            cand_blocks, n_cand_blocks, block, max_cand_blocks, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!scores) return CSA2_ERR_NULL;
  if (scores_stride < n_slots) return CSA2_ERR_SHAPE;
  if (n_q == 0 || n_slots == 0) return CSA2_OK;
  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, cand_blocks, n_cand_blocks,
                          block, max_cand_blocks, n_slots, fmt);
  return launch_score(a, n_q, scores, scores_stride, fmt == CSA2_FMT_NVFP4, (hipStream_t)stream, q_latent(fmt));
}

extern "C" int csa2_index_score_q(const void* q, int q_dtype, const float* w, int n_q, int n_heads, int dim,
                                  CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                  const int64_t* n_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks,
                                  int block, int max_cand_blocks, float* scores, int64_t scores_stride, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (q_dtype != CSA2_DT_F32 && q_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (fmt != CSA2_FMT_MXFP4) return CSA2_ERR_UNSUPPORTED;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  const uint8_t* qb = static_cast<const uint8_t*>(q);   // checked as the Q array: non-null, 16-byte aligned
  int64_t n_slots = 0;
  int rc = check_score_args(qb, qb, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis, cand_blocks,
                            n_cand_blocks, block, max_cand_blocks, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!scores) return CSA2_ERR_NULL;
  if (scores_stride < n_slots) return CSA2_ERR_SHAPE;
  if (n_q == 0 || n_slots == 0) return CSA2_OK;
  ScoreArgs a = make_args(nullptr, nullptr, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, cand_blocks, n_cand_blocks,
                          block, max_cand_blocks, n_slots);
  a.q_lat = q;
  a.q_bf16 = q_dtype == CSA2_DT_BF16;
  return launch_score(a, n_q, scores, scores_stride, false, (hipStream_t)stream, true);
}

extern "C" int csa2_index_score_grouped(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                        int n_heads, int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq,
                                        const int32_t* q_seq, const int64_t* n_vis, int group, float* scores,
                                        int64_t scores_stride, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (fmt != CSA2_FMT_MXFP4) return CSA2_ERR_UNSUPPORTED;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis, nullptr,
                            nullptr, 0, 0, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!scores) return CSA2_ERR_NULL;
  if (group < 1 || group > kGroupMax || scores_stride < n_slots) return CSA2_ERR_SHAPE;
  if (n_q == 0 || n_slots == 0) return CSA2_OK;
  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, nullptr, nullptr, 0, 0,
                          n_slots);
  const int64_t groups = ((int64_t)n_q + group - 1) / group;
  // chunks of 4,096 entries, halved (down to 1,024) while that leaves fewer than four
  // workgroups per CU
  int chunk_len = kScoreChunk;
  while (chunk_len > 1024 && ((n_slots + chunk_len - 1) / chunk_len) * groups < 1024) chunk_len /= 2;
  const int64_t chunks = (n_slots + chunk_len - 1) / chunk_len;
  if (chunks > 0x7fffffffLL || groups > 65535) return CSA2_ERR_SHAPE;
  a.scores = scores;
  a.scores_stride = scores_stride;
  a.chunk_len = chunk_len;
  a.chunks = (int)chunks;
  hipLaunchKernelGGL(k_score_grouped, dim3((unsigned)chunks, (unsigned)groups), dim3(kScoreThreads), 0,
                     (hipStream_t)stream, a, n_q, group);
  return csa2_check_launch();
}

extern "C" size_t csa2_index_topk_workspace_bytes(int n_q, int64_t n_slots, int k, int in_pool) {
  if (n_q <= 0 || n_slots <= 0 || k < 1 || k > CSA2_MAX_TOPK) return 0;
  return index_topk_ws(n_q, n_slots, k, in_pool != 0);
}

extern "C" int csa2_index_topk(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q, int n_heads,
                               int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                               const int64_t* n_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks,
                               int block, int max_cand_blocks, int k, int32_t* idx_out, int32_t* count_out,
                               void* workspace, size_t workspace_bytes, const csa2_append* append,
                               void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (append && cand_blocks) return CSA2_ERR_UNSUPPORTED;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis,
                            cand_blocks, n_cand_blocks, block, max_cand_blocks, &n_slots);
  if (rc != CSA2_OK) return rc;
  const bool nv = fmt == CSA2_FMT_NVFP4;
  if (!idx_out || !count_out) return CSA2_ERR_NULL;
  if (n_q > 65535 || k < 1 || k > CSA2_MAX_TOPK || n_slots > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  const int64_t n0 = n_slots < 1 ? 1 : n_slots;
  int64_t segs[16];
  const int L = plan_levels(n0, k, segs, 16);
  if (L >= 16) return CSA2_ERR_SHAPE;
  const size_t need = index_topk_ws(n_q, n0, k, cand_blocks != nullptr);
  if (need > workspace_bytes || (need && !workspace)) return CSA2_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (cand_blocks) {  // inside a pool: scores into the workspace, then the selection levels
    float* sc = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    const size_t sc_bytes = ((size_t)n_q * n0 * sizeof(float) + 255) & ~(size_t)255;
    ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, cand_blocks,
                            n_cand_blocks, block, max_cand_blocks, n_slots, fmt);
    rc = launch_score(a, n_q, sc, n0, nv, st, q_latent(fmt));
    if (rc != CSA2_OK) return rc;
    TkArgs t = {};
    t.scores = sc;
    t.scores_stride = n0;
    t.n_vis = n_vis;
    t.max_vis = seq_cap;
    t.cand_blocks = cand_blocks;
    t.n_cand_blocks = n_cand_blocks;
    t.block = block;
    t.max_cand_blocks = max_cand_blocks;
    t.idx_out = idx_out;
    t.count_out = count_out;
    t.k = k;
    t.n_slots = n0;
    uint8_t* rest = (uint8_t*)sc + sc_bytes;
    return select_from_scores(t, n_q, n0, rest, workspace_bytes - (size_t)(rest - (uint8_t*)workspace), st);
  }
  uint64_t* bufA = (uint64_t*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  uint64_t* bufB = bufA + (size_t)k * n_q * segs[0];
  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, cand_blocks, n_cand_blocks,
                          block, max_cand_blocks, n_slots, fmt);
  a.k = k;
  a.keys_out = bufA;
  a.idx_out = idx_out;
  a.count_out = count_out;
  rc = set_append(a, append, seq_cap, fmt);
  if (rc != CSA2_OK) return rc;
  const dim3 grid((unsigned)segs[0], (unsigned)n_q);
  rc = L == 1 ? launch_score_select<true, false>(fmt, grid, st, a) : launch_score_select<false, false>(fmt, grid, st, a);
  if (rc != CSA2_OK) return rc;
  TkArgs t = {};
  t.n_vis = n_vis;
  t.max_vis = seq_cap;
  t.k = k;
  t.idx_out = idx_out;
  t.count_out = count_out;
  return select_levels_after0(segs, L, t, n_q, bufA, bufB, st);
}

// ---- csa2_index_segments: the fused first level alone; the last one runs in the
// attention kernel (csa2_sparse_attn_topk) ----
extern "C" int64_t csa2_segment_keys(int64_t n_slots, int k) {
  if (n_slots < 0 || k < 1 || k > CSA2_MAX_TOPK) return 0;
  const int64_t n_seg = n_slots > 0 ? (n_slots + kTkSeg - 1) / kTkSeg : 1;
  return n_seg * k;
}

extern "C" int csa2_index_segments(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                   int n_heads, int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq,
                                   const int32_t* q_seq, const int64_t* n_vis, int k, uint64_t* cand_keys,
                                   const csa2_append* append, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis, nullptr,
                            nullptr, 8, 1, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!cand_keys) return CSA2_ERR_NULL;
  if (n_q > 65535 || k < 1 || k > CSA2_MAX_TOPK || n_slots > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  const int64_t n_seg = csa2_segment_keys(n_slots, k) / k;
  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, nullptr, nullptr, 8, 1,
                          n_slots, fmt);
  a.k = k;
  a.keys_out = cand_keys;
  rc = set_append(a, append, seq_cap, fmt);
  if (rc != CSA2_OK) return rc;
  return launch_score_select<false, false>(fmt, dim3((unsigned)n_seg, (unsigned)n_q), (hipStream_t)stream, a);
}

// ---- csa2_index_topk_grouped: grouped rows, scored and selected without a score array ----
extern "C" size_t csa2_index_topk_grouped_workspace_bytes(int n_q, int64_t seq_cap, int k, int group) {
  if (n_q <= 0 || seq_cap < 0 || k < 1 || k > CSA2_MAX_GROUPED_TOPK || group < 1 || group > kGroupMax) return 0;
  return (size_t)n_q * grouped_ranges(seq_cap, k, (n_q + group - 1) / group) * k * sizeof(uint64_t) + 256;
}

extern "C" int csa2_index_topk_grouped(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                       int n_heads, int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq,
                                       const int32_t* q_seq, const int64_t* n_vis, int group, int k,
                                       int32_t* idx_out, int32_t* count_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (fmt != CSA2_FMT_MXFP4) return CSA2_ERR_UNSUPPORTED;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis, nullptr,
                            nullptr, 8, 1, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!idx_out || !count_out) return CSA2_ERR_NULL;
  if (group < 1 || group > kGroupMax || k < 1 || k > CSA2_MAX_GROUPED_TOPK || n_q > 65535 * group)
    return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  const size_t need = csa2_index_topk_grouped_workspace_bytes(n_q, seq_cap, k, group);
  if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  const int n_groups = (n_q + group - 1) / group;
  const int n_ranges = grouped_ranges(seq_cap, k, n_groups);
  int64_t range_len = (seq_cap + n_ranges - 1) / n_ranges;
  range_len = (range_len + 63) / 64 * 64;
  if (range_len < 64) range_len = 64;
  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, nullptr, nullptr, 8, 1,
                          n_slots);
  a.k = k;
  a.keys_out = (uint64_t*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  hipStream_t st = (hipStream_t)stream;
  // 32-bit offsets within a sequence: a lane's offsets run at most 128 entries past the last
  // one before they are clamped, and must not wrap on the way
  const bool off32 = (uint64_t)(seq_cap + 128) * (uint64_t)a.k_ce + 64 <= 0xffffffffull &&
                     (uint64_t)(seq_cap + 128) * (uint64_t)a.k_se + 4 <= 0xffffffffull;
  if (off32)
    hipLaunchKernelGGL(k_score_topk_grouped<true>, dim3((unsigned)n_ranges, (unsigned)n_groups), dim3(kScoreThreads),
                       0, st, a, n_q, group, (int)range_len, n_ranges);
  else
    hipLaunchKernelGGL(k_score_topk_grouped<false>, dim3((unsigned)n_ranges, (unsigned)n_groups), dim3(kScoreThreads),
                       0, st, a, n_q, group, (int)range_len, n_ranges);
  rc = csa2_check_launch();
  if (rc != CSA2_OK) return rc;
  const int64_t segs[2] = {n_ranges, 1};
  TkArgs t = {};
  t.n_vis = n_vis;
  t.max_vis = seq_cap;
  t.k = k;
  t.idx_out = idx_out;
  t.count_out = count_out;
  return select_levels_after0(segs, 2, t, n_q, a.keys_out, nullptr, st);
}

extern "C" size_t csa2_index_topk_pool_workspace_bytes(int n_q, int64_t n_slots, int k, int block, int max_blocks) {
  if (n_q <= 0 || n_slots <= 0 || k < 1 || k > CSA2_MAX_TOPK || block < 1 || block > 64 || (block & (block - 1)) ||
      max_blocks < 1 || max_blocks > CSA2_MAX_TOPK)
    return 0;
  size_t b, t;
  return index_topk_pool_ws(n_q, n_slots, k, block, max_blocks, &b, &t);
}

extern "C" int csa2_index_topk_pool(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                                    int n_heads, int dim, CSA2_INDEX_CACHE_ARGS, int64_t seq_cap, int n_seq,
                                    const int32_t* q_seq, const int64_t* n_vis, int k, int32_t* idx_out,
                                    int32_t* count_out, int block, int max_blocks, int32_t* blocks_out,
                                    int32_t* blocks_count, void* workspace, size_t workspace_bytes,
                                    const csa2_append* append, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (fmt != CSA2_FMT_MXFP4 && !q_latent(fmt)) return CSA2_ERR_UNSUPPORTED;
  CacheRef kr = CSA2_INDEX_CACHE_REF;
  int64_t n_slots = 0;
  int rc = check_score_args(q_codes, q_scales, w, n_q, n_heads, dim, fmt, kr, seq_cap, n_seq, q_seq, n_vis, nullptr,
                            nullptr, 0, 0, &n_slots);
  if (rc != CSA2_OK) return rc;
  if (!idx_out || !count_out || !blocks_out || !blocks_count) return CSA2_ERR_NULL;
  if (n_q > 65535 || k < 1 || k > CSA2_MAX_TOPK || block < 1 || block > 64 || (block & (block - 1)) ||
      max_blocks < 1 || max_blocks > CSA2_MAX_TOPK)
    return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  const int64_t n0 = n_slots < 1 ? 1 : n_slots;
  int64_t segs[16];
  const int L = plan_levels(n0, k, segs, 16);
  if (L >= 16) return CSA2_ERR_SHAPE;
  size_t bmax_bytes, sel_bytes;
  const size_t need = index_topk_pool_ws(n_q, n0, k, block, max_blocks, &bmax_bytes, &sel_bytes);
  if (need > workspace_bytes || !workspace) return CSA2_ERR_WORKSPACE;
  uint8_t* w0 = (uint8_t*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  float* bmax = (float*)w0;
  uint64_t* bufA = (uint64_t*)(w0 + bmax_bytes);
  uint64_t* bufB = bufA + (size_t)k * n_q * segs[0];
  uint8_t* pool_ws = w0 + bmax_bytes + sel_bytes;
  const size_t pool_ws_bytes = workspace_bytes - (size_t)(pool_ws - (uint8_t*)workspace);
  const int64_t nblk = (n0 + block - 1) / block;

  ScoreArgs a = make_args(q_codes, q_scales, w, n_heads, kr, seq_cap, n_seq, q_seq, n_vis, nullptr, nullptr, block, 0,
                          n_slots, fmt);
  a.k = k;
  a.keys_out = bufA;
  a.idx_out = idx_out;
  a.count_out = count_out;
  a.bmax = bmax;
  a.bmax_stride = nblk;
  rc = set_append(a, append, seq_cap, fmt);
  if (rc != CSA2_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)segs[0], (unsigned)n_q);
  rc = L == 1 ? launch_score_select<true, true>(fmt, grid, st, a) : launch_score_select<false, true>(fmt, grid, st, a);
  if (rc != CSA2_OK) return rc;
  TkArgs t = {};
  t.n_vis = n_vis;
  t.max_vis = seq_cap;
  t.k = k;
  t.idx_out = idx_out;
  t.count_out = count_out;
  // the pool: top max_blocks blocks by block maximum (ties to the lower block id)
  TkArgs pa = {};
  pa.scores = bmax;
  pa.scores_stride = nblk;
  pa.n_vis = n_vis;
  pa.vis_div = block;
  pa.max_vis = nblk;
  pa.k = max_blocks;
  pa.idx_out = blocks_out;
  pa.count_out = blocks_count;
  pa.n_slots = nblk;
  // Two selection chains: A, the Top-k over the segment survivors (levels 1 .. L-1), and B,
  // the pool over the block maxima (levels 0 .. LB-1).  Launch j runs level j+1 of A and
  // level j of B together (they are independent), so the chains share their launches.
  int64_t segs_b[16];
  const int LB = plan_levels(nblk < 1 ? 1 : nblk, max_blocks, segs_b, 16);
  if (LB >= 16) return CSA2_ERR_SHAPE;
  if (ws_bytes(n_q, nblk < 1 ? 1 : nblk, max_blocks) > pool_ws_bytes) return CSA2_ERR_WORKSPACE;
  uint64_t* poolA = (uint64_t*)(((uintptr_t)pool_ws + 255) & ~(uintptr_t)255);
  uint64_t* poolB = poolA + (size_t)max_blocks * n_q * segs_b[0];
  const int LA = L - 1;
  for (int j = 0; j < (LA > LB ? LA : LB); ++j) {
    TkArgs ta = t, tb = pa;
    int sa = 0, sb = 0;
    bool fa = false, fb = false;
    if (j < LA) {
      const int l = j + 1;
      ta.keys_in = (l % 2 == 1) ? bufA : bufB;
      ta.keys_in_per_q = segs[l - 1] * k;
      ta.keys_out = (l % 2 == 0) ? bufA : bufB;
      sa = (int)segs[l];
      fa = l == L - 1;
    }
    if (j < LB) {
      if (j > 0) {
        tb.keys_in = (j % 2 == 1) ? poolA : poolB;
        tb.keys_in_per_q = segs_b[j - 1] * max_blocks;
      }
      tb.keys_out = (j % 2 == 0) ? poolA : poolB;
      sb = (int)segs_b[j];
      fb = j == LB - 1;
    }
    rc = launch_wide2(ta, sa, fa, tb, sb, fb, j == 0, n_q, st);
    if (rc != CSA2_OK) return rc;
  }
  return CSA2_OK;
}
