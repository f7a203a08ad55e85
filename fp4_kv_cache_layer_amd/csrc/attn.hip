// csa2_sparse_attn: attention of each query over its selected main-KV entries (FP4,
// dequantised exactly) and its sliding window (FP8) in one softmax
// ([W] "CSA2：跨层复用，能借就不自己算", "FP4 与 SWA Bounded Replay";
//  [J] "缓存压缩真的是越大越好吗").
//
// Per query the key set is at most k + window entries (640 in the decode configurations)
// of 512 channels, with V = K, against H heads: two dense H x 640 x 512 products, run on
// the fp16 matrix cores with fp32 accumulation.
//
// Exactness of the operands: every main-KV value is E2M1 x E4M3 (at most 6 significant
// bits, magnitude in [2^-10, 2688]) and every window value is E4M3, so both are exact in
// fp16.  Q (bf16) enters the products as fp16 after a power-of-two scale per head: the
// head's largest |q| is brought into [2^14, 2^15), which keeps every bf16 value within 2^32
// of that maximum exact (8 significant bits in fp16's 11, normal or subnormal) over the
// whole bf16 range, and the logits take the scale back exactly (a power of two commutes
// with the fp32 rounding of the sums).  P = exp2(logit - max) is rounded to fp16 (11
// significant bits) for the P.V product.
//
// Two decompositions share one workgroup shape, (query, 16 heads, slice of the key list) with
// 8 waves, and everything outside the tile loop.  The full-channel kernel (k_attn_fc), taken
// whenever the window is at most 128 keys (the decode configurations), makes each wave a key
// stream of its own over all 512 channels: no partial S crosses waves, Q is staged once in
// LDS, and the eight streams merge at the end (its own header comment has the details).
// The split-channel kernel (k_attn) below takes any window up to the maximum:
//
// Split-channel decomposition: 8 waves in four
// pairs.  The key list is cut into tiles of 16 keys; pair p takes every fourth tile of the
// slice (window tiles first, since their rows need no index), and the two waves of a pair
// split the 512 channels into halves.  Per tile a wave
//   * gathers its half of the 16 keys straight into registers (lane = key x 64 channels:
//     32 B of E2M1 codes + 4 B of E4M3 scales, or 64 B of window E4M3), three tiles ahead;
//   * dequantises them with the hardware FP4/FP8 -> fp16 converts and an exact packed
//     multiply by the group scale, directly in the A-operand layout of
//     V_MFMA_F32_16X16X32_F16, and forms the partial S^T = K Q^T over its 256 channels
//     (Q held in registers in the same channel order);
//   * writes the same fp16 values as its own V half-tile in LDS (row stride 528 B, double
//     buffered);
//   * adds its partner's partial S^T, exchanged through LDS with a flag handshake between
//     the two waves (the step's only synchronisation; the four key streams never wait for
//     one another inside the loop), so both waves hold the same S^T and run the same
//     online softmax;
//   * turns S^T into P^T in fp16: the accumulator layout of the QK MFMA (lane: head l%16,
//     keys 4(l/16)..+3) is exactly the B-operand layout of V_MFMA_F32_16X16X16_F16, so P
//     needs no shuffle; and accumulates O^T += V^T P^T over its 256 channels, V^T read from
//     its V half-tile through DS_READ_B64_TR_B16 (each lane receives one channel of 4 keys).
// Steps are software-pipelined: a wave posts its partial S of tile i+1, runs P.V of tile i
// while its partner finishes, then collects the partner's half and runs the softmax of tile
// i+1.  At the end the four pairs merge (O, m, l) with the
// log-sum-exp rule through LDS.  The workgroups of one query are numbered so that they land
// on the same XCD (dispatch is round-robin over the 8 XCDs) and share its L2 for the
// gathered rows.  When a batch has too few queries to fill the GPU, the key list is split
// over workgroups and a combine kernel merges the partial (O, m, l).
//
// Two pieces of neighbouring work can run in the kernel's prologue, each saving a launch:
// the last Top-K level (the index set selected from the first level's survivors or from
// the pool's slot scores; see k_attn's kSel) and, in single-token decode, the append of the
// row's own window entry (new_win).
#include <mutex>
#include <type_traits>

#include "select.h"

namespace csa2 {

constexpr int kPairs = 4;                      // key streams per workgroup
constexpr int kAttnThreads = 2 * kPairs * 64;  // 8 waves: each stream has two channel halves
constexpr int kT = 16;                         // keys per tile (one MFMA block)
constexpr int kHG = 16;                        // heads per workgroup
constexpr int kD = 512;
constexpr int kHalf = kD / 2;                  // channels per wave
constexpr int kQS = kHalf / 32;                // QK steps per wave and tile: 8
constexpr int kDT = kHalf / 16;                // 16-channel blocks of a wave's O^T: 16
constexpr int kVRow = kHalf * 2 + 16;          // bytes per V row in LDS (padding against bank conflicts)
constexpr int kVBuf = kT * kVRow;              // one wave's V half-tile: 8,448 B
constexpr int kRing = 3;                       // tiles whose raw bytes are in flight
constexpr float kLazy = 8.0f;                  // log2 headroom of the lazy softmax reference
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct AttnArgs {
  const uint16_t* q;
  int n_q, n_heads;
  const uint8_t* kv_codes;
  const uint8_t* kv_scales;
  int64_t kv_ce, kv_cs, kv_se, kv_ss;   // byte strides: code entry / sequence, scale entry / sequence
  int64_t seq_cap;
  int n_seq;
  const int32_t* q_seq;
  const int32_t* idx;
  int k;
  const uint8_t* swa;
  uint8_t* swa_w;     // the same ring, written only by the window append
  int64_t swa_re, swa_rs;   // byte strides of the ring: row, sequence
  int64_t swa_cap;
  const int64_t* swa_base;
  const int64_t* q_pos;
  const int64_t* replay_start;
  int window;
  float scale_log2;
  void* out;
  int out_dtype;
  float* lse;
  float* ws_o;
  float* ws_ml;
  int nsplit, tiles_per_split, n_tiles, main_tiles, head_groups;
  // csa2_sparse_attn_topk: the segment survivors of the first Top-K level ([n_q, cand_per_q]
  // selection keys) and the index set the selection writes for later layers
  const uint64_t* cand_keys;
  int cand_per_q;
  int32_t* idx_out;
  int32_t* count_out;
  // window append: [n_q, 512] f32 or bf16 latents of each row's own token (or nullptr)
  const void* new_win;
  int new_win_bf16;
  // csa2_sparse_attn_pool_topk: the pool's slot scores [n_q, pool_stride] and slot map
  const float* pool_scores;
  int64_t pool_stride;
  const int32_t* cand_blocks;
  const int32_t* n_cand_blocks;
  const int64_t* n_vis;
  int block, max_cand_blocks;
  // the partner-flag wait gives up after wait_limit polls; it then stores a nonzero code
  // into the library's status word (pinned host memory; nullptr before csa2_init)
  int wait_limit;
  uint32_t* status;
};

// Reductions over the lanes l, l^16, l^32, l^48 (the four lane groups of one MFMA column) in
// the VALU, without an LDS round trip.  V_PERMLANE16_SWAP of a register with itself returns
// the even 16-lane rows in its first result and the odd ones in its second, each row next to
// its neighbour, so combining the two results pairs every lane with lane l^16;
// V_PERMLANE32_SWAP does the same for the two halves of the wave (l^32).  The sum adds
// (l + l^16) + (l^32 + l^48) in that grouping at every lane.
__device__ __forceinline__ float lanes4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lanes4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint32_t lanes4_umax(uint32_t x) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] > a[1] ? a[0] : a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] > b[1] ? b[0] : b[1];
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// bf16 bits times 2^-shift -> fp16 (exact for the values the header comment names)
__device__ __forceinline__ _Float16 bf16_to_f16(uint32_t b, int shift) {
  return (_Float16)ldexpf(__uint_as_float(b << 16), -shift);
}

// Exponent shift that brings a head's largest |q| (given as bf16 magnitude bits) into
// [2^14, 2^15): q * 2^-shift then fits fp16 with its top bits in the normal range.  An
// all-zero head keeps shift 0; a subnormal maximum counts as 2^-127.
__device__ __forceinline__ int q_shift(uint32_t max_bits) {
  const int e = (int)(max_bits >> 7);
  return max_bits == 0 ? 0 : (e == 0 ? -127 : e - 127) - 14;
}

// 8 E2M1 values of one code dword (channel 2i in the low nibble of byte i) times a group
// scale given as an fp16 pair, as 8 fp16; exact (E2M1 x E4M3 has at most 6 significant
// bits and lies inside the fp16 range)
__device__ __forceinline__ v8h fp4x8_to_f16(uint32_t codes, v2h ss) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E4M3 values (two dwords) as 8 fp16; exact
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// raw bytes of one gather slot (one key, 64 channels of the wave's half): main = 32 B of
// codes (r[0..1]) and 4 scale bytes (sc); window = 64 B of E4M3 (r[0..3])
struct GatherSlot {
  uint4 r[4];
  uint32_t sc;
  uint32_t ok;
  uint32_t is_new;   // the window key of the row's own token, appended by this call
};

// The per-query arrays come as restrict-qualified arguments of their own: nothing this
// kernel writes can alias them, so their uniform loads go through the scalar cache.
//
// kSel != 0: the index list is not given but selected here, in every workgroup of the
// query: from the survivors of the first Top-K level (kSel 1, csa2_index_segments, 16
// consecutive keys per thread) or from the scores of the pool's slots (kSel 2, at most 2,048
// blocks x 8 = 16,384 slots, 32 consecutive slots per thread), with the same exact radix
// select as the Top-K levels (select.h; its thread-major compaction keeps the candidate
// order), its histograms and scratch in the LDS of the V buffers (unused until the first
// tile), straight into the staged index list.  Workgroup (head group 0, split 0) of
// the query also writes the list and its count out for the layers that reuse it.
constexpr int kSelMax = kAttnThreads * 16;      // 8,192 survivor keys per query at most
constexpr int kPoolMax = kAttnThreads * 32;     // 16,384 pool slots per query at most
constexpr int kSelHistWords = 2 * (kAttnThreads / 64) * 256 * kTkCopies;
static_assert((kSelHistWords + 2 * 256 + 8 * 32) * 4 <= 2 * kPairs * 2 * kVBuf, "selection LDS");

template <int kSel>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn(AttnArgs a, const int32_t* __restrict__ q_seq,
                                                           const int64_t* __restrict__ q_pos,
                                                           const int64_t* __restrict__ replay_start,
                                                           const int64_t* __restrict__ swa_base) {
  // ---- which (query, head group, split) this workgroup is; same query -> same XCD ----
  const int G = a.head_groups * a.nsplit;
  const int L = blockIdx.x;
  const int xcd = L & 7, jj = L >> 3;
  const int q = 8 * (jj / G) + xcd;
  if (q >= a.n_q) return;
  const int rem = jj % G;
  const int hg = rem % a.head_groups;
  const int split = rem / a.head_groups;

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform over the wave; saying so keeps tile-level decisions scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (kPairs - 1), half = wave / kPairs;  // key stream, channel half
  const int partner = wave ^ kPairs;                           // the other half of the stream
  // MFMA lane roles: col = key row of K / head column of Q^T and S^T, grp = lane group
  const int col = lane & 15, grp = lane >> 4;

  // LDS: two V half-tiles per wave, two partial-S exchange slots per wave and the staged
  // index list; after the loop the first 128 KB hold the partial outputs of the merge
  constexpr int kVBytes = 2 * kPairs * 2 * kVBuf;               // 135,168
  constexpr int kSxBytes = 2 * kPairs * 2 * 64 * 16;            // 16,384
  constexpr int kLdsBytes = kVBytes + kSxBytes + CSA2_MAX_TOPK * 4;   // 159,744
  static_assert(2 * kPairs * kDT * 64 * 16 <= kLdsBytes, "merge area");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ float s_ml[kPairs][kHG][2];
  __shared__ uint32_t s_flag[2 * kPairs];   // per wave: number of partial-S slots written
  uint8_t* vbuf = lds + wave * 2 * kVBuf;                       // [buffer][16 rows][kVRow]
  float4* sx = reinterpret_cast<float4*>(lds + kVBytes);        // [wave][slot][lane]
  int32_t* s_idx = reinterpret_cast<int32_t*>(lds + kVBytes + kSxBytes);

  // ---- this split's tiles: main tiles [tile_lo, main_hi), window tiles after them ----
  const int tile_lo = split * a.tiles_per_split;
  const int tile_hi = tile_lo + a.tiles_per_split < a.n_tiles ? tile_lo + a.tiles_per_split : a.n_tiles;
  const int main_hi = a.main_tiles < tile_hi ? a.main_tiles : tile_hi;
  const int n_main = main_hi > tile_lo ? main_hi - tile_lo : 0;

  // ---- this pair's tiles: window tiles first (their rows need no index), then main tiles;
  // pair p takes positions p, p+4, ... of that order.  Every wave runs the same number of
  // steps (one exchange with its partner each) and masks the steps past its pair's end ----
  const int span = tile_hi - tile_lo;
  const int n_win = span - n_main;
  const int n_steps = (span + kPairs - 1) / kPairs;
  const int n_my = span > pair ? (span - pair + kPairs - 1) / kPairs : 0;
  auto my_tile = [&](int i) {
    const int j = pair + kPairs * (i < n_my ? i : (n_my > 0 ? n_my - 1 : 0));
    return j < n_win ? tile_lo + n_main + j : tile_lo + (j - n_win);
  };

  // ---- the query's sequence and positions head the memory queue (scalar loads), then this
  // split's slice of the index list (it does not depend on them), then Q ----
  const int seq = q_seq[q];
  const int64_t t = q_pos[q], s = replay_start[q];
  constexpr bool kSelect = kSel != 0;
  constexpr int kEpt = kSel == 2 ? 32 : 16;
  constexpr int kIdxPer = CSA2_MAX_TOPK / kAttnThreads;
  const int n_keys = n_main * kT;
  int32_t iv[kIdxPer];
  uint64_t key[kEpt];
  if constexpr (kSel == 1) {
    // survivors tid*16 .. tid*16+15 of the query (cand_per_q >= 1): runs of 16 B loads where
    // the wave's whole range is inside the list (uniform), clamped single loads otherwise
    const uint64_t* kp = a.cand_keys + (int64_t)q * a.cand_per_q;
    const int lim = a.cand_per_q;
    const int c0 = tid * kEpt;
    if ((wave + 1) * 64 * kEpt <= lim) {
      typedef uint64_t u64x2 __attribute__((ext_vector_type(2), aligned(8)));
#pragma unroll
      for (int i = 0; i < kEpt; i += 2) {
        const u64x2 v = *reinterpret_cast<const u64x2*>(kp + c0 + i);
        key[i] = v.x;
        key[i + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        const int o = c0 + i;
        key[i] = kp[o < lim ? o : lim - 1] & (0ull - (uint64_t)(o < lim));
      }
    }
  } else if constexpr (kSel == 2) {
    // pool slot c = tid*32 + i: block cand_blocks[q][c / block], position block id * block
    // + c % block; a candidate if c lies in the query's first n_cand_blocks blocks, the block
    // id is valid and the position visible (as the first Top-K level inside a pool).  The
    // loads are clamped to the row (max_cand_blocks * block slots, all inside the arrays),
    // not to the query's slot count, so they go out without waiting for n_cand_blocks; the
    // scores come in 16 B loads where the wave's whole range is inside the row (uniform),
    // and the slot's block and offset advance by one slot per step (one division).
    const uint32_t blk = (uint32_t)a.block;
    const uint32_t row_slots = (uint32_t)a.max_cand_blocks * blk;   // <= 16,384
    const float* sp = a.pool_scores + (int64_t)q * a.pool_stride;
    const int32_t* cb = a.cand_blocks + (int64_t)q * a.max_cand_blocks;
    const uint32_t c0 = (uint32_t)tid * kEpt;
    const uint32_t last_blk = (uint32_t)a.max_cand_blocks - 1u;
    int nc = a.n_cand_blocks[q];
    nc = nc < 0 ? 0 : (nc > a.max_cand_blocks ? a.max_cand_blocks : nc);
    int64_t nv = a.n_vis[q];
    nv = nv < 0 ? 0 : (nv > a.seq_cap ? a.seq_cap : nv);
    const uint32_t nslot = (uint32_t)nc * blk;   // <= 16,384
    // Each path issues all of its loads (block ids, then scores) and builds the keys itself:
    // only finished keys meet after the branch, so no load is waited for before the rest are
    // issued.  kBlk8: the pool's 8-position blocks, a thread's 32 slots being blocks c0/8 ..
    // c0/8 + 3 (four loads, one per 8 slots); otherwise each slot's block id is loaded, its
    // block and offset advanced by one slot per step.
    auto build = [&](auto blk8) {
      constexpr bool kBlk8 = decltype(blk8)::value;
      int32_t bv[kEpt];
      uint32_t so[kEpt];
      float v[kEpt];
      if constexpr (kBlk8) {
        int32_t b4[kEpt / 8];
#pragma unroll
        for (int j = 0; j < kEpt / 8; ++j) {
          const uint32_t bj = c0 / 8u + (uint32_t)j;
          b4[j] = cb[bj < last_blk ? bj : last_blk];
        }
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          bv[i] = b4[i / 8];
          so[i] = (uint32_t)(i % 8);
        }
      } else {
        uint32_t b = c0 / blk, o = c0 % blk;
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          bv[i] = cb[b < last_blk ? b : last_blk];
          so[i] = o;
          const bool carry = o + 1u == blk;
          o = carry ? 0u : o + 1u;
          b += carry ? 1u : 0u;
        }
      }
      if ((uint32_t)(wave + 1) * 64u * kEpt <= row_slots) {   // uniform: 16 B score loads
        typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));
#pragma unroll
        for (int i = 0; i < kEpt; i += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(sp + c0 + i);
          v[i] = x.x;
          v[i + 1] = x.y;
          v[i + 2] = x.z;
          v[i + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          const uint32_t c = c0 + (uint32_t)i;
          v[i] = sp[c < row_slots ? c : row_slots - 1u];
        }
      }
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        const uint32_t c = c0 + (uint32_t)i;
        const int64_t pos = (int64_t)bv[i] * blk + so[i];
        const bool ok = c < nslot && bv[i] >= 0 && pos < nv;
        key[i] = make_key(v[i], (uint32_t)pos) & (0ull - (uint64_t)ok);
      }
    };
    if (blk == 8u) build(std::true_type{});   // uniform
    else build(std::false_type{});
  }
  // A given index list: this thread's slice of it (staged in LDS below), and this lane's keys
  // of its first three tiles, read straight from it so that their gathers need neither the
  // staged list nor the prologue's barrier (a slot past k gets -1).  All of
  // these loads are unconditional, from clamped in-bounds addresses (q_seq stands in for an
  // absent list when k == 0), and branch-free: a load inside a branch would be waited for
  // at the branch's end, one memory round trip after another.
  int32_t idx0[3] = {-1, -1, -1};
  if constexpr (!kSelect) {
    const bool have = a.k > 0;
    const int32_t* ib = have ? a.idx + (int64_t)q * a.k : q_seq;
    const int klast = have ? a.k - 1 : 0;
#pragma unroll
    for (int r = 0; r < kIdxPer; ++r) {
      int i = tid + r * kAttnThreads;
      i = i < n_keys ? i : (n_keys > 0 ? n_keys - 1 : 0);
      const int slot = tile_lo * kT + i;
      iv[r] = ib[slot < klast ? slot : klast];
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int tile = my_tile(i);
      const int slot = tile * kT + col;
      const int32_t v = ib[slot < klast ? slot : klast];
      idx0[i] = slot < a.k ? v : -1;   // (load_slot ignores it for a window tile)
    }
  }

  // ---- Q of head (hg*16 + col): step st of this wave holds channels
  //      256*half + 64*grp + 8*st .. +7 (the same channel order as the K operand) ----
  uint4 qraw[kQS];
  {
    const uint16_t* qp = a.q + ((int64_t)q * a.n_heads + hg * kHG + col) * kD + kHalf * half + 64 * grp;
#pragma unroll
    for (int st = 0; st < kQS; ++st) qraw[st] = *reinterpret_cast<const uint4*>(qp + 8 * st);
  }

  // Window append: thread c quantises channel c of the row's new window latent (the
  // quantiser's exact E4M3 rounding); the bytes are staged in LDS for this workgroup's own
  // window tiles, and workgroup (head group 0, split 0) writes them to the ring.  The latent
  // is loaded here and converted just before the prologue's barrier: a wait for it here
  // would wait for every load issued before it and hold back the per-query scalars below.
  static_assert(kAttnThreads == kD, "one thread per channel of the appended window entry");
  __shared__ __attribute__((aligned(16))) uint8_t s_new[kD];
  // One unconditional 32-bit load (branch-free, see above): an f32 element, or the word
  // holding this bf16 element (Q stands in when there is no latent)
  uint32_t new_bits;
  {
    const int64_t e = (int64_t)q * kD + tid;
    const uint32_t* nwp = reinterpret_cast<const uint32_t*>(a.new_win ? a.new_win : (const void*)a.q);
    const uint32_t w = nwp[a.new_win_bf16 || !a.new_win ? e >> 1 : e];
    new_bits = a.new_win_bf16 ? ((tid & 1) ? (w & 0xffff0000u) : (w << 16)) : w;
  }
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int64_t lo = s > t - a.window + 1 ? s : t - a.window + 1;
  const int64_t n_swa = seq_ok && t >= lo ? t - lo + 1 : 0;
  const int64_t swa_b = seq_ok ? swa_base[seq] : 0;
  // ring row of the first window key; later keys wrap at most once (window <= swa_cap).
  // The offset from the ring base nearly always fits 32 bits: then a 32-bit remainder
  const int64_t rel = lo - swa_b;
  const uint32_t swa_cap32 = (uint32_t)a.swa_cap;
  int64_t r_lo;
  if (rel >= 0 && rel <= 0xffffffffLL) {
    r_lo = (uint32_t)rel % swa_cap32;
  } else {
    r_lo = rel % a.swa_cap;
    r_lo = r_lo < 0 ? r_lo + a.swa_cap : r_lo;
  }
  const uint32_t win_row0 = (uint32_t)r_lo;
  const uint8_t* kvc = a.kv_codes + (int64_t)(seq_ok ? seq : 0) * a.kv_cs;
  const uint8_t* kvs = a.kv_scales + (int64_t)(seq_ok ? seq : 0) * a.kv_ss;
  const uint8_t* swq = a.swa + (int64_t)(seq_ok ? seq : 0) * a.swa_rs;
  // Every gather load is unconditional, to an in-bounds address (an absent key reads row 0
  // and is flagged), so no branch sits around the loads of the ring.  Lane (col, grp)
  // fetches key col of the tile, channels 256*half + 64*grp .. +63.
  auto load_slot = [&](int tile, bool real, GatherSlot& g, const int32_t* direct = nullptr) {
    const bool is_main = tile < a.main_tiles;  // wave-uniform
    int si = (tile - tile_lo) * kT + col;
    si = si < 0 ? 0 : (si >= n_main * kT ? (n_main > 0 ? n_main * kT - 1 : 0) : si);
    // with kSelect s_idx holds the whole list (k entries, -1 padded), and a main tile's
    // slots from k on (the last tile when k is not a multiple of 16) are empty; otherwise
    // s_idx is this split's slice, or the key comes from `direct` (read from the list)
    const int slot = tile_lo * kT + si;
    const int32_t pv = direct ? *direct : s_idx[kSelect ? (slot < a.k ? slot : a.k - 1) : si];
    const int32_t p = (kSelect && slot >= a.k) ? -1 : pv;
    const bool ok_main = real && is_main && seq_ok && p >= 0 && p < a.seq_cap;
    const uint32_t pm = ok_main ? (uint32_t)p : 0u;
    const int j = (tile - a.main_tiles) * kT + col;
    const bool ok_win = real && !is_main && seq_ok && j >= 0 && j < n_swa;
    g.is_new = a.new_win != nullptr && ok_win && j == n_swa - 1;   // window key j is token lo + j
    uint32_t row = win_row0 + (uint32_t)j;
    row = ok_win ? (row >= swa_cap32 ? row - swa_cap32 : row) : 0u;
    // rows and positions are 32-bit (seq_cap <= 2^24, swa_cap <= 2^23), byte offsets 64-bit
    const uint4* c = is_main
        ? reinterpret_cast<const uint4*>(kvc + ((uint64_t)pm * (uint64_t)a.kv_ce + 128 * half + 32 * grp))
        : reinterpret_cast<const uint4*>(swq + ((uint64_t)row * (uint64_t)a.swa_re + kHalf * half + 64 * grp));
    const uint4* c2 = is_main ? c : c + 2;  // main needs 32 B: the second pair re-reads them
    g.r[0] = c[0];
    g.r[1] = c[1];
    g.r[2] = c2[0];
    g.r[3] = c2[1];
    g.sc = *reinterpret_cast<const uint32_t*>(kvs + ((uint64_t)pm * (uint64_t)a.kv_se + 16 * half + 4 * grp));
    g.ok = is_main ? ok_main : ok_win;
  };

  // With a given index list the first three gathers of every key stream go out here, their
  // keys read directly (idx0).  When the list is selected in this kernel, the first two
  // tiles of every key stream are window tiles when the slice holds at least 2 * kPairs of
  // them (always without a key split); their rows need no index, so their gathers go out
  // before the selection.  Either way the ring slots are filled in the order g0, g1, g2.
  const bool early = n_win >= 2 * kPairs;   // uniform over the workgroup
  GatherSlot g0, g1, g2;
  if constexpr (!kSelect) {   // the given list: all three gathers now (keys read directly)
    load_slot(my_tile(0), 0 < n_my, g0, &idx0[0]);
    load_slot(my_tile(1), 1 < n_my, g1, &idx0[1]);
    load_slot(my_tile(2), 2 < n_my, g2, &idx0[2]);
  } else if (early) {
    load_slot(my_tile(0), 0 < n_my, g0);
    load_slot(my_tile(1), 1 < n_my, g1);
  }

  if constexpr (kSelect) {
    // the whole index list, s_idx[0 .. k), ascending; the tiles index it from tile_lo * 16
    __shared__ int32_t s_count;
    uint32_t* hist = reinterpret_cast<uint32_t*>(lds);
    select_block<kAttnThreads, kEpt, true, kTkCopies, true>(key, a.k, hist, nullptr, s_idx, &s_count,
                                                            hist + kSelHistWords);
    __syncthreads();
    if (hg == 0 && split == 0) {
      for (int i = tid; i < a.k; i += kAttnThreads) a.idx_out[(int64_t)q * a.k + i] = s_idx[i];
      if (tid == 0) a.count_out[q] = s_count;
    }
  } else if (n_keys > 0) {
#pragma unroll
    for (int r = 0; r < kIdxPer; ++r) {
      const int i = tid + r * kAttnThreads;
      if (i < n_keys) s_idx[i] = tile_lo * kT + i < a.k ? iv[r] : -1;
    }
  }
  // the largest |q| of head col over this wave's 256 channels (bf16 magnitude bits; the
  // order of finite bf16 magnitudes is that of their bit patterns), then over both halves
  // through LDS at the prologue's barrier
  __shared__ uint32_t s_qmax[2][kHG];
  {
    uint32_t qm = 0;
#pragma unroll
    for (int st = 0; st < kQS; ++st) {
      const uint32_t w4[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w4[i] & 0x7fffu, hi = (w4[i] >> 16) & 0x7fffu;
        qm = lo > qm ? lo : qm;
        qm = hi > qm ? hi : qm;
      }
    }
    qm = lanes4_umax(qm);
    if (pair == 0 && grp == 0) s_qmax[half][col] = qm;
  }
  if (a.new_win) {  // uniform: the window append (see above)
    const uint32_t new_code = fp8_code_bits(new_bits);
    s_new[tid] = (uint8_t)new_code;
    if (hg == 0 && split == 0 && seq_ok && t >= 0) {
      // ring row of token t: the window keys [lo, t] are consecutive rows from win_row0
      int64_t rt = (t - swa_b) % a.swa_cap;
      rt = rt < 0 ? rt + a.swa_cap : rt;
      a.swa_w[(int64_t)seq * a.swa_rs + rt * a.swa_re + tid] = (uint8_t)new_code;
    }
  }
  if (lane == 0) s_flag[wave] = 0u;
  __syncthreads();  // s_idx, s_flag, s_qmax, s_new
  if (kSelect && !early) {
    load_slot(my_tile(0), 0 < n_my, g0);
    load_slot(my_tile(1), 1 < n_my, g1);
  }

  // Q as the fp16 B operand, scaled by 2^-shift per head; the logits of head col take
  // 2^shift back in qsl (log2-domain scale of this lane's head)
  v8h qf[kQS];
  const uint32_t qmax_bits = s_qmax[0][col] > s_qmax[1][col] ? s_qmax[0][col] : s_qmax[1][col];
  const int qsh = q_shift(qmax_bits);
  const float qsl = ldexpf(a.scale_log2, qsh);

  // Dequantise the slot (the wave's 256 channels of 16 keys), write them as this wave's
  // V half-tile and form the partial S^T = K Q^T over those channels.  The format is
  // uniform over the wave (a tile holds main entries only or window keys only), so the only
  // branch is a scalar one; an absent key's raw bytes are zeroed (E2M1 / E4M3 zero is +0,
  // a zero scale zeroes a main key) instead of branching per lane.  Returns the partial S^T
  // (lane: head col, keys 4*grp..+3); *valid receives bit k for each present key k.
  auto qk_tile = [&](const GatherSlot& g, bool is_main, uint8_t* vb, uint32_t* valid) -> v4f {
    const uint32_t keep = 0u - g.ok;
    uint8_t* dst = vb + col * kVRow + 128 * grp;
    v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    if (is_main) {
      const uint32_t cw[8] = {g.r[0].x, g.r[0].y, g.r[0].z, g.r[0].w, g.r[1].x, g.r[1].y, g.r[1].z, g.r[1].w};
      const uint32_t sc = g.sc & keep;
      // the four E4M3 group scales to fp16 with the hardware convert (exact)
      const v2h s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
      const v2h s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);
      const v2h ss[4] = {__builtin_shufflevector(s01, s01, 0, 0), __builtin_shufflevector(s01, s01, 1, 1),
                         __builtin_shufflevector(s23, s23, 0, 0), __builtin_shufflevector(s23, s23, 1, 1)};
#pragma unroll
      for (int st = 0; st < kQS; st += 2) {
        const v8h k0 = fp4x8_to_f16(cw[st], ss[st >> 1]);
        const v8h k1 = fp4x8_to_f16(cw[st + 1], ss[st >> 1]);
        *reinterpret_cast<v8h*>(dst + 16 * st) = k0;
        *reinterpret_cast<v8h*>(dst + 16 * (st + 1)) = k1;
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[st], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[st + 1], sb, 0, 0, 0);
      }
    } else {
      uint32_t w[16] = {g.r[0].x, g.r[0].y, g.r[0].z, g.r[0].w, g.r[1].x, g.r[1].y, g.r[1].z, g.r[1].w,
                        g.r[2].x, g.r[2].y, g.r[2].z, g.r[2].w, g.r[3].x, g.r[3].y, g.r[3].z, g.r[3].w};
      if (a.new_win) {  // uniform: the row's own token comes from the LDS copy, not the ring
        const uint4* sn = reinterpret_cast<const uint4*>(s_new + kHalf * half + 64 * grp);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 n = sn[u];
          w[4 * u] = g.is_new ? n.x : w[4 * u];
          w[4 * u + 1] = g.is_new ? n.y : w[4 * u + 1];
          w[4 * u + 2] = g.is_new ? n.z : w[4 * u + 2];
          w[4 * u + 3] = g.is_new ? n.w : w[4 * u + 3];
        }
      }
#pragma unroll
      for (int st = 0; st < kQS; st += 2) {
        const v8h k0 = fp8x8_to_f16(w[2 * st] & keep, w[2 * st + 1] & keep);
        const v8h k1 = fp8x8_to_f16(w[2 * st + 2] & keep, w[2 * st + 3] & keep);
        *reinterpret_cast<v8h*>(dst + 16 * st) = k0;
        *reinterpret_cast<v8h*>(dst + 16 * (st + 1)) = k1;
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[st], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[st + 1], sb, 0, 0, 0);
      }
    }
    *valid = (uint32_t)__ballot(g.ok != 0) & 0xffffu;  // lanes 0..15 hold keys 0..15
    return sa + sb;
  };

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v4f o[kDT];
#pragma unroll
  for (int i = 0; i < kDT; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // online softmax over one tile's full S^T (lane: head col, keys 4*grp + r); returns P^T
  // in fp16, which is exactly the B operand of V_MFMA_F32_16X16X16_F16, and in *alpha the
  // factor the accumulators must be scaled by once the previous tile's P.V is in them
  auto softmax_tile = [&](v4f sv, uint32_t valid, float* alpha_out) -> v4h {
    float x[4];
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (valid >> (4 * grp + r)) & 1u;
      x[r] = ok ? sv[r] * qsl : -__builtin_inff();
      mt = fmaxf(mt, x[r]);
    }
    mt = lanes4_max(mt);
    // Lazy rescaling: m_run is a reference, not necessarily the running maximum.  It moves
    // only when a logit exceeds it by more than 2^kLazy (or on the first key), so
    // p = 2^(x - m_run) <= 2^kLazy stays far inside fp16 and the accumulators are rescaled
    // only rarely.  The softmax is invariant to the reference.
    const bool first = m_run == -__builtin_inff();
    const bool move = first ? mt != -__builtin_inff() : mt > m_run + kLazy;
    const float m_new = move ? mt : m_run;
    const float alpha = (move && !first) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const bool none = m_new == -__builtin_inff();
    v4h pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = none ? 0.0f : __builtin_amdgcn_exp2f(x[r] - m_new);
      psum += pr;
      pb[r] = (_Float16)pr;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    *alpha_out = alpha;
    return pb;
  };
  auto rescale = [&](float alpha) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) o[dt] *= alpha;
    }
  };

  // O^T += V^T P^T over this wave's 256 channels.  A = V^T (16 channels x 16 keys): in each
  // 16-lane group (keys 4grp..4grp+3), lane 4a+b receives element b of the 8-byte reads of
  // lanes a, a+4, a+8, a+12, so lane r of the group points at channels 4*(r & 3).. of key
  // 4*grp + (r >> 2)
  auto pv_tile = [&](v4h pb, const uint8_t* vt) {
    const __attribute__((address_space(3))) uint8_t* vb =
        (const __attribute__((address_space(3))) uint8_t*)vt + (4 * grp + (col >> 2)) * kVRow + 8 * (col & 3);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const v4h av = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + 32 * dt)));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, o[dt], 0, 0, 0);
    }
  };

  // Combine this wave's partial S^T with its partner's.  Exchange number `id` goes through
  // slot id % 2: the wave writes its slot, then its flag (id + 1) (post); later it waits for
  // the partner's flag to reach id + 1 and reads the partner's slot (collect).  Between the
  // two a wave does work that does not need the partner (the previous tile's P.V).  Only the
  // two waves of a stream synchronise, so the four streams drift freely.  Both waves make
  // the same sequence of exchanges, each posting before it collects, so every wait is met; a
  // slot is rewritten two exchanges later, which the writer can only reach after the
  // partner's flag shows the read was done (a wave posts only after its last collect).  The
  // wait is bounded so that it always ends; a wait that gives up stores a nonzero code
  // into the library's status word, which the host reports at its next call (the output
  // of this call is then not to be trusted).  Both waves add in the same order up to
  // commutation, so the pair holds bit-identical S^T, softmax state and P.
  auto post = [&](v4f own, int id) {
    sx[(wave * 2 + (id & 1)) * 64 + lane] = make_float4(own[0], own[1], own[2], own[3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_store(&s_flag[wave], (uint32_t)(id + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto collect = [&](v4f own, int id) -> v4f {
    const int sl = id & 1;
    bool seen = false;
    for (int spin = 0; spin < a.wait_limit; ++spin) {
      if (__hip_atomic_load(&s_flag[partner], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= (uint32_t)(id + 1)) {
        seen = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!seen && lane == 0 && a.status)
      __hip_atomic_store(a.status, (uint32_t)CSA2_STATUS_ATTN_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const float4 o2 = sx[(partner * 2 + sl) * 64 + lane];
    return v4f{own[0] + o2.x, own[1] + o2.y, own[2] + o2.z, own[3] + o2.w};
  };

  // the V reads of tile i-1 must stay before the V writes of tile i+1 in the same buffer
  // (LDS executes one wave's accesses in order; this keeps the compiler from reordering)
  auto lds_order = [] { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); };

  // ---- software pipeline.  Step i dequantises tile i+1 into V buffer (i+1) % 2, forms its
  // partial S and posts it to its partner; P.V of tile i (buffer i % 2) then keeps the
  // matrix cores busy until the partner's half is collected (the step's one wait), and the
  // softmax of tile i+1 follows.  The raw bytes of tiles i+2 .. i+4 are in flight meanwhile:
  // ring slot (i+1) % 3 is refilled with tile i+4 as soon as tile i+1 has left it ----
  auto tile_is_main = [&](int i) { return my_tile(i) < a.main_tiles; };
  if constexpr (kSelect) load_slot(my_tile(2), 2 < n_my, g2);
#pragma unroll
  for (int st = 0; st < kQS; ++st) {
    const uint32_t w4[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
    v8h h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = bf16_to_f16(w4[i] & 0xffffu, qsh);
      h[2 * i + 1] = bf16_to_f16(w4[i] >> 16, qsh);
    }
    qf[st] = h;
  }
  uint32_t vmask;
  float alpha;
  v4f sp = qk_tile(g0, tile_is_main(0), vbuf, &vmask);
  load_slot(my_tile(3), 3 < n_my, g0);
  post(sp, 0);
  v4h pb = softmax_tile(collect(sp, 0), vmask, &alpha);

  auto step = [&](int i, GatherSlot& g) {
    const int nb = (i + 1) & 1;
    lds_order();
    sp = qk_tile(g, tile_is_main(i + 1), vbuf + nb * kVBuf, &vmask);
    load_slot(my_tile(i + 4), i + 4 < n_my, g);
    post(sp, i + 1);
    pv_tile(pb, vbuf + (nb ^ 1) * kVBuf);   // tile i, while the partner finishes tile i+1
    const v4f sv = collect(sp, i + 1);
    pb = softmax_tile(sv, vmask, &alpha);   // tile i+1
    rescale(alpha);
  };
  // Steps 0 .. n_steps-2 form S of tiles 1 .. n_steps-1; the last tile then only needs its
  // P.V (a full last step would form and exchange the S of a tile past the end).  Whole
  // rounds of the ring inside the loop and the remainder after it: a loop with exits
  // between its steps would make the compiler wait for every load in flight at its head.
  const int n_full = n_steps - 1;
  int i = 0;
  for (; i + kRing <= n_full; i += kRing) {
    step(i, g1);
    step(i + 1, g2);
    step(i + 2, g0);
  }
  if (i < n_full) step(i, g1);  // uniform over the workgroup
  if (i + 1 < n_full) step(i + 1, g2);
  if (n_steps > 0) pv_tile(pb, vbuf + (n_full & 1) * kVBuf);   // tile n_steps-1

  // ---- merge the four pairs' (O, m, l); the two waves of a pair hold the same (m, l) ----
  float l_tot = lanes4_sum(l_run);
  if (half == 0 && lane < kHG) {
    s_ml[pair][lane][0] = m_run;
    s_ml[pair][lane][1] = l_tot;
  }
  __syncthreads();  // every wave is past its loop: the V buffers and exchange slots are free
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kPairs; ++w) M = fmaxf(M, s_ml[w][col][0]);
  float Ltot = 0.0f, mine = 0.0f;
#pragma unroll
  for (int w = 0; w < kPairs; ++w) {
    const float mw = s_ml[w][col][0];
    const float sw = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
    Ltot += sw * s_ml[w][col][1];
    mine = w == pair ? sw : mine;
  }
  const int head = hg * kHG + col;
  const float inv = Ltot > 0.0f ? 1.0f / Ltot : 0.0f;
  float4* part = reinterpret_cast<float4*>(lds);   // [half][pair][16 blocks][64 lanes]: 128 KB
#pragma unroll
  for (int b = 0; b < kDT; ++b) {
    const v4f v = o[b] * mine;
    part[((half * kPairs + pair) * kDT + b) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();
  // wave w sums blocks 4*(w % 4) .. +3 of channel half w / 4 over the four pairs
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = 4 * pair + bb;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kPairs; ++w) {
      const float4 v = part[((half * kPairs + w) * kDT + b) * 64 + lane];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int ch = 256 * half + 16 * b + 4 * grp;   // channels ch..ch+3 of head col
    if (a.nsplit == 1) {
      const int64_t ob = ((int64_t)q * a.n_heads + head) * kD + ch;
      if (a.out_dtype == CSA2_DT_F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + ob) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      } else {
        uint2 pk;
        pk.x = f32_to_bf16_rne(acc.x * inv) | (f32_to_bf16_rne(acc.y * inv) << 16);
        pk.y = f32_to_bf16_rne(acc.z * inv) | (f32_to_bf16_rne(acc.w * inv) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob) = pk;
      }
    } else {
      const int64_t pb = ((int64_t)split * a.n_q + q) * a.n_heads + head;
      *reinterpret_cast<float4*>(a.ws_o + pb * kD + ch) = acc;
    }
  }
  if (wave == 0 && lane < kHG) {
    if (a.nsplit == 1) {
      if (a.lse) a.lse[(int64_t)q * a.n_heads + head] = Ltot > 0.0f ? (M + __log2f(Ltot)) * kLn2 : -__builtin_inff();
    } else {
      const int64_t pb = ((int64_t)split * a.n_q + q) * a.n_heads + head;
      a.ws_ml[pb * 2] = M;
      a.ws_ml[pb * 2 + 1] = Ltot;
    }
  }
}

// ---- the full-channel variant: each wave is a key stream of its own over all 512 channels ----
//
// One workgroup = (query, 16 heads, slice of the key list), as k_attn, but its 8 waves are 8
// key streams: stream p takes tiles p, p+8, ... of the slice (window tiles first).  A wave
// forms S^T = K Q^T over all 512 channels itself, so no partial S is exchanged and each
// stream runs its own online softmax; Q is staged once per workgroup in LDS (scaled to fp16
// by a power of two per head, as in k_attn) and each 32-channel MFMA step reads its slice.
// Lane (key col, group grp) gathers channels 128*grp .. +127 of its key: 64 B of E2M1 codes
// and 8 scale bytes, or 128 B of window E4M3.  The host takes this kernel only for a window
// of at most kStreams tiles, so only a stream's first tile can be a window tile: the
// gathers of its later tiles use main-tile slots (18 registers instead of 36), which keeps
// the kernel at two waves per SIMD without spills.  V is single-buffered per wave: in step i the
// P.V of tile i reads channel blocks m, m+8, m+16, m+24 of the V tile just before the
// dequantisation of tile i+1 overwrites exactly those blocks (LDS executes one wave's
// accesses in order), interleaved over m = 0..7 with tile i+1's QK steps 2m, 2m+1.  O^T of
// all 512 channels stays in 32 accumulator blocks; at the end the eight streams merge
// (O, m, l) with the log-sum-exp rule in two rounds through LDS.  Same arithmetic per (key,
// head, channel) as k_attn: exact fp16 keys and values, P rounded to fp16, fp32 sums.
constexpr int kStreams = 8;
constexpr int kFcRow = kD * 2 + 16;   // bytes per V / Q row in LDS (padding against bank conflicts)
constexpr int kFcVBuf = kT * kFcRow;  // one wave's V tile: 16,640 B
constexpr int kFcDT = kD / 16;        // 16-channel blocks of O^T: 32
static_assert(kStreams * 64 == kAttnThreads, "one wave per key stream");

// raw bytes of one gather slot: main = 64 B of codes (r[0..3]; r[4..7] re-read them) and 8
// scale bytes (sc0, sc1); window = 128 B of E4M3 (r[0..7])
struct FcSlot {
  uint4 r[8];
  uint32_t sc0, sc1;
  uint32_t ok;
  uint32_t is_new;
};
// a main-tile slot: 64 B of codes and 8 scale bytes (every tile of a stream after its first
// is a main tile: the window has at most kStreams tiles, and they come first)
struct FcMainSlot {
  uint4 r[4];
  uint32_t sc0, sc1;
  uint32_t ok;
};

template <int kSel>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_fc(AttnArgs a, const int32_t* __restrict__ q_seq,
                                                              const int64_t* __restrict__ q_pos,
                                                              const int64_t* __restrict__ replay_start,
                                                              const int64_t* __restrict__ swa_base) {
  // ---- which (query, head group, split) this workgroup is; same query -> same XCD ----
  const int G = a.head_groups * a.nsplit;
  const int L = blockIdx.x;
  const int xcd = L & 7, jj = L >> 3;
  const int q = 8 * (jj / G) + xcd;
  if (q >= a.n_q) return;
  const int rem = jj % G;
  const int hg = rem % a.head_groups;
  const int split = rem / a.head_groups;

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index (the key stream) is uniform over the wave; saying so keeps tile-level
  // decisions scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // MFMA lane roles: col = key row of K / head column of Q^T and S^T, grp = lane group
  const int col = lane & 15, grp = lane >> 4;

  // LDS: one V tile per wave, Q of the 16 heads, the staged index list; after the loop the
  // first 128 KB hold the partial outputs of the merge
  constexpr int kVBytes = kStreams * kFcVBuf;                       // 133,120
  constexpr int kQBytes = kHG * kFcRow;                             // 16,640
  constexpr int kLdsBytes = kVBytes + kQBytes + CSA2_MAX_TOPK * 4;  // 157,952
  static_assert(4 * kFcDT * 64 * 16 <= kVBytes, "merge area");
  static_assert((kSelHistWords + 2 * 256 + 8 * 32) * 4 <= kVBytes, "selection LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ float s_ml[kStreams][kHG][2];
  __shared__ int s_qsh[kHG];
  uint8_t* vbuf = lds + wave * kFcVBuf;                             // [16 rows][kFcRow]
  uint8_t* qst = lds + kVBytes;                                     // [16 heads][kFcRow]
  int32_t* s_idx = reinterpret_cast<int32_t*>(lds + kVBytes + kQBytes);

  // ---- this split's tiles: main tiles [tile_lo, main_hi), window tiles after them ----
  const int tile_lo = split * a.tiles_per_split;
  const int tile_hi = tile_lo + a.tiles_per_split < a.n_tiles ? tile_lo + a.tiles_per_split : a.n_tiles;
  const int main_hi = a.main_tiles < tile_hi ? a.main_tiles : tile_hi;
  const int n_main = main_hi > tile_lo ? main_hi - tile_lo : 0;

  // ---- this stream's tiles: window tiles first (their rows need no index), then main
  // tiles; stream p takes positions p, p+8, ... of that order.  The streams never wait for
  // one another inside the loop, so each runs its own number of steps ----
  const int span = tile_hi - tile_lo;
  const int n_win = span - n_main;
  const int n_my = span > wave ? (span - wave + kStreams - 1) / kStreams : 0;
  auto my_tile = [&](int i) {
    const int j = wave + kStreams * (i < n_my ? i : (n_my > 0 ? n_my - 1 : 0));
    return j < n_win ? tile_lo + n_main + j : tile_lo + (j - n_win);
  };

  // ---- the query's sequence and positions head the memory queue (scalar loads), then this
  // split's slice of the index list (it does not depend on them), then Q ----
  const int seq = q_seq[q];
  const int64_t t = q_pos[q], s = replay_start[q];
  constexpr bool kSelect = kSel != 0;
  constexpr int kEpt = kSel == 2 ? 32 : 16;
  constexpr int kIdxPer = CSA2_MAX_TOPK / kAttnThreads;
  const int n_keys = n_main * kT;
  int32_t iv[kIdxPer];
  uint64_t key[kEpt];
  if constexpr (kSel == 1) {
    // survivors tid*16 .. tid*16+15 of the query (cand_per_q >= 1): runs of 16 B loads where
    // the wave's whole range is inside the list (uniform), clamped single loads otherwise
    const uint64_t* kp = a.cand_keys + (int64_t)q * a.cand_per_q;
    const int lim = a.cand_per_q;
    const int c0 = tid * kEpt;
    if ((wave + 1) * 64 * kEpt <= lim) {
      typedef uint64_t u64x2 __attribute__((ext_vector_type(2), aligned(8)));
#pragma unroll
      for (int i = 0; i < kEpt; i += 2) {
        const u64x2 v = *reinterpret_cast<const u64x2*>(kp + c0 + i);
        key[i] = v.x;
        key[i + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        const int o = c0 + i;
        key[i] = kp[o < lim ? o : lim - 1] & (0ull - (uint64_t)(o < lim));
      }
    }
  } else if constexpr (kSel == 2) {
    // pool slot c = tid*32 + i: block cand_blocks[q][c / block], position block id * block
    // + c % block; a candidate if c lies in the query's first n_cand_blocks blocks, the block
    // id is valid and the position visible (as the first Top-K level inside a pool).  The
    // loads are clamped to the row (max_cand_blocks * block slots, all inside the arrays),
    // not to the query's slot count, so they go out without waiting for n_cand_blocks; the
    // scores come in 16 B loads where the wave's whole range is inside the row (uniform),
    // and the slot's block and offset advance by one slot per step (one division).
    const uint32_t blk = (uint32_t)a.block;
    const uint32_t row_slots = (uint32_t)a.max_cand_blocks * blk;   // <= 16,384
    const float* sp = a.pool_scores + (int64_t)q * a.pool_stride;
    const int32_t* cb = a.cand_blocks + (int64_t)q * a.max_cand_blocks;
    const uint32_t c0 = (uint32_t)tid * kEpt;
    const uint32_t last_blk = (uint32_t)a.max_cand_blocks - 1u;
    int nc = a.n_cand_blocks[q];
    nc = nc < 0 ? 0 : (nc > a.max_cand_blocks ? a.max_cand_blocks : nc);
    int64_t nv = a.n_vis[q];
    nv = nv < 0 ? 0 : (nv > a.seq_cap ? a.seq_cap : nv);
    const uint32_t nslot = (uint32_t)nc * blk;   // <= 16,384
    // Each path issues all of its loads (block ids, then scores) and builds the keys itself:
    // only finished keys meet after the branch, so no load is waited for before the rest are
    // issued.  kBlk8: the pool's 8-position blocks, a thread's 32 slots being blocks c0/8 ..
    // c0/8 + 3 (four loads, one per 8 slots); otherwise each slot's block id is loaded, its
    // block and offset advanced by one slot per step.
    auto build = [&](auto blk8) {
      constexpr bool kBlk8 = decltype(blk8)::value;
      int32_t bv[kEpt];
      uint32_t so[kEpt];
      float v[kEpt];
      if constexpr (kBlk8) {
        int32_t b4[kEpt / 8];
#pragma unroll
        for (int j = 0; j < kEpt / 8; ++j) {
          const uint32_t bj = c0 / 8u + (uint32_t)j;
          b4[j] = cb[bj < last_blk ? bj : last_blk];
        }
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          bv[i] = b4[i / 8];
          so[i] = (uint32_t)(i % 8);
        }
      } else {
        uint32_t b = c0 / blk, o = c0 % blk;
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          bv[i] = cb[b < last_blk ? b : last_blk];
          so[i] = o;
          const bool carry = o + 1u == blk;
          o = carry ? 0u : o + 1u;
          b += carry ? 1u : 0u;
        }
      }
      if ((uint32_t)(wave + 1) * 64u * kEpt <= row_slots) {   // uniform: 16 B score loads
        typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));
#pragma unroll
        for (int i = 0; i < kEpt; i += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(sp + c0 + i);
          v[i] = x.x;
          v[i + 1] = x.y;
          v[i + 2] = x.z;
          v[i + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kEpt; ++i) {
          const uint32_t c = c0 + (uint32_t)i;
          v[i] = sp[c < row_slots ? c : row_slots - 1u];
        }
      }
#pragma unroll
      for (int i = 0; i < kEpt; ++i) {
        const uint32_t c = c0 + (uint32_t)i;
        const int64_t pos = (int64_t)bv[i] * blk + so[i];
        const bool ok = c < nslot && bv[i] >= 0 && pos < nv;
        key[i] = make_key(v[i], (uint32_t)pos) & (0ull - (uint64_t)ok);
      }
    };
    if (blk == 8u) build(std::true_type{});   // uniform
    else build(std::false_type{});
  }
  // A given index list: this thread's slice of it (staged in LDS below), and this lane's keys
  // of its first three tiles, read straight from it so that their gathers need neither the
  // staged list nor the prologue's barrier (a slot past k gets -1).  All of
  // these loads are unconditional, from clamped in-bounds addresses (q_seq stands in for an
  // absent list when k == 0), and branch-free: a load inside a branch would be waited for
  // at the branch's end, one memory round trip after another.
  int32_t idx0[3] = {-1, -1, -1};
  if constexpr (!kSelect) {
    const bool have = a.k > 0;
    const int32_t* ib = have ? a.idx + (int64_t)q * a.k : q_seq;
    const int klast = have ? a.k - 1 : 0;
#pragma unroll
    for (int r = 0; r < kIdxPer; ++r) {
      int i = tid + r * kAttnThreads;
      i = i < n_keys ? i : (n_keys > 0 ? n_keys - 1 : 0);
      const int slot = tile_lo * kT + i;
      iv[r] = ib[slot < klast ? slot : klast];
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int tile = my_tile(i);
      const int slot = tile * kT + col;
      const int32_t v = ib[slot < klast ? slot : klast];
      idx0[i] = slot < a.k ? v : -1;   // (load_slot ignores it for a window tile)
    }
  }

  // ---- Q of the 16 heads, once for the workgroup: thread t loads head t / 32, channels
  //      16 * (t % 32) .. +15 (scaled and staged in LDS before the prologue's barrier) ----
  const int qh = tid >> 5, qc = (tid & 31) * 16;
  uint4 qr[2];
  {
    const uint16_t* qp = a.q + ((int64_t)q * a.n_heads + hg * kHG + qh) * kD + qc;
    qr[0] = reinterpret_cast<const uint4*>(qp)[0];
    qr[1] = reinterpret_cast<const uint4*>(qp)[1];
  }

  // Window append: thread c quantises channel c of the row's new window latent (the
  // quantiser's exact E4M3 rounding); the bytes are staged in LDS for this workgroup's own
  // window tiles, and workgroup (head group 0, split 0) writes them to the ring.  The latent
  // is loaded here and converted just before the prologue's barrier: a wait for it here
  // would wait for every load issued before it and hold back the per-query scalars below.
  static_assert(kAttnThreads == kD, "one thread per channel of the appended window entry");
  __shared__ __attribute__((aligned(16))) uint8_t s_new[kD];
  // One unconditional 32-bit load (branch-free, see above): an f32 element, or the word
  // holding this bf16 element (Q stands in when there is no latent)
  uint32_t new_bits;
  {
    const int64_t e = (int64_t)q * kD + tid;
    const uint32_t* nwp = reinterpret_cast<const uint32_t*>(a.new_win ? a.new_win : (const void*)a.q);
    const uint32_t w = nwp[a.new_win_bf16 || !a.new_win ? e >> 1 : e];
    new_bits = a.new_win_bf16 ? ((tid & 1) ? (w & 0xffff0000u) : (w << 16)) : w;
  }
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int64_t lo = s > t - a.window + 1 ? s : t - a.window + 1;
  const int64_t n_swa = seq_ok && t >= lo ? t - lo + 1 : 0;
  const int64_t swa_b = seq_ok ? swa_base[seq] : 0;
  // ring row of the first window key; later keys wrap at most once (window <= swa_cap).
  // The offset from the ring base nearly always fits 32 bits: then a 32-bit remainder
  const int64_t rel = lo - swa_b;
  const uint32_t swa_cap32 = (uint32_t)a.swa_cap;
  int64_t r_lo;
  if (rel >= 0 && rel <= 0xffffffffLL) {
    r_lo = (uint32_t)rel % swa_cap32;
  } else {
    r_lo = rel % a.swa_cap;
    r_lo = r_lo < 0 ? r_lo + a.swa_cap : r_lo;
  }
  const uint32_t win_row0 = (uint32_t)r_lo;
  const uint8_t* kvc = a.kv_codes + (int64_t)(seq_ok ? seq : 0) * a.kv_cs;
  const uint8_t* kvs = a.kv_scales + (int64_t)(seq_ok ? seq : 0) * a.kv_ss;
  const uint8_t* swq = a.swa + (int64_t)(seq_ok ? seq : 0) * a.swa_rs;
  // Every gather load is unconditional, to an in-bounds address (an absent key reads row 0
  // and is flagged), so no branch sits around the loads of the ring.  Lane (col, grp)
  // fetches key col of the tile, channels 128*grp .. +127.
  auto load_slot = [&](int tile, bool real, FcSlot& g, const int32_t* direct = nullptr) {
    const bool is_main = tile < a.main_tiles;  // wave-uniform
    int si = (tile - tile_lo) * kT + col;
    si = si < 0 ? 0 : (si >= n_main * kT ? (n_main > 0 ? n_main * kT - 1 : 0) : si);
    const int slot = tile_lo * kT + si;
    const int32_t pv = direct ? *direct : s_idx[kSelect ? (slot < a.k ? slot : a.k - 1) : si];
    const int32_t p = (kSelect && slot >= a.k) ? -1 : pv;
    const bool ok_main = real && is_main && seq_ok && p >= 0 && p < a.seq_cap;
    const uint32_t pm = ok_main ? (uint32_t)p : 0u;
    const int j = (tile - a.main_tiles) * kT + col;
    const bool ok_win = real && !is_main && seq_ok && j >= 0 && j < n_swa;
    g.is_new = a.new_win != nullptr && ok_win && j == n_swa - 1;   // window key j is token lo + j
    uint32_t row = win_row0 + (uint32_t)j;
    row = ok_win ? (row >= swa_cap32 ? row - swa_cap32 : row) : 0u;
    const uint4* c = is_main
        ? reinterpret_cast<const uint4*>(kvc + ((uint64_t)pm * (uint64_t)a.kv_ce + 64 * grp))
        : reinterpret_cast<const uint4*>(swq + ((uint64_t)row * (uint64_t)a.swa_re + 128 * grp));
    const uint4* c2 = is_main ? c : c + 4;  // main needs 64 B: the second four re-read them
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      g.r[u] = c[u];
      g.r[4 + u] = c2[u];
    }
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(kvs + ((uint64_t)pm * (uint64_t)a.kv_se + 8 * grp));
    g.sc0 = sp[0];
    g.sc1 = sp[1];
    g.ok = is_main ? ok_main : ok_win;
  };

  // the main-tile gather of a stream's later tiles (always main tiles)
  auto load_main = [&](int tile, bool real, FcMainSlot& g, const int32_t* direct = nullptr) {
    int si = (tile - tile_lo) * kT + col;
    si = si < 0 ? 0 : (si >= n_main * kT ? (n_main > 0 ? n_main * kT - 1 : 0) : si);
    const int slot = tile_lo * kT + si;
    const int32_t pv = direct ? *direct : s_idx[kSelect ? (slot < a.k ? slot : a.k - 1) : si];
    const int32_t p = (kSelect && slot >= a.k) ? -1 : pv;
    const bool ok_main = real && tile < a.main_tiles && seq_ok && p >= 0 && p < a.seq_cap;
    const uint32_t pm = ok_main ? (uint32_t)p : 0u;
    const uint4* c = reinterpret_cast<const uint4*>(kvc + ((uint64_t)pm * (uint64_t)a.kv_ce + 64 * grp));
#pragma unroll
    for (int u = 0; u < 4; ++u) g.r[u] = c[u];
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(kvs + ((uint64_t)pm * (uint64_t)a.kv_se + 8 * grp));
    g.sc0 = sp[0];
    g.sc1 = sp[1];
    g.ok = ok_main;
  };

  // With a given index list the first three gathers of every key stream go out here, their
  // keys read directly (idx0).  When the list is selected in this kernel, the first tile of
  // every stream is a window tile when the slice holds at least kStreams of them (always
  // without a key split); its rows need no index, so its gather goes out before the
  // selection.  Slot g0 holds the first tile (main or window); the main slots gA, gB ring
  // through the later ones.
  const bool early = n_win >= kStreams;   // uniform over the workgroup
  FcSlot g0;
  FcMainSlot gA, gB;
  if constexpr (!kSelect) {   // the given list: all three gathers now (keys read directly)
    load_slot(my_tile(0), 0 < n_my, g0, &idx0[0]);
    load_main(my_tile(1), 1 < n_my, gA, &idx0[1]);
    load_main(my_tile(2), 2 < n_my, gB, &idx0[2]);
  } else if (early) {
    load_slot(my_tile(0), 0 < n_my, g0);
  }

  if constexpr (kSelect) {
    // the whole index list, s_idx[0 .. k), ascending; the tiles index it from tile_lo * 16
    __shared__ int32_t s_count;
    uint32_t* hist = reinterpret_cast<uint32_t*>(lds);
    select_block<kAttnThreads, kEpt, true, kTkCopies, true>(key, a.k, hist, nullptr, s_idx, &s_count,
                                                            hist + kSelHistWords);
    __syncthreads();
    if (hg == 0 && split == 0) {
      for (int i = tid; i < a.k; i += kAttnThreads) a.idx_out[(int64_t)q * a.k + i] = s_idx[i];
      if (tid == 0) a.count_out[q] = s_count;
    }
  } else if (n_keys > 0) {
#pragma unroll
    for (int r = 0; r < kIdxPer; ++r) {
      const int i = tid + r * kAttnThreads;
      if (i < n_keys) s_idx[i] = tile_lo * kT + i < a.k ? iv[r] : -1;
    }
  }
  // Q scaled per head: the largest |q| of head qh over its 512 channels (bf16 magnitude bits;
  // the order of finite bf16 magnitudes is that of their bit patterns), over the 32 threads
  // of the head, gives the power-of-two shift of k_attn; the scaled fp16 Q goes to LDS
  {
    const uint32_t w8[8] = {qr[0].x, qr[0].y, qr[0].z, qr[0].w, qr[1].x, qr[1].y, qr[1].z, qr[1].w};
    uint32_t qm = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo16 = w8[i] & 0x7fffu, hi16 = (w8[i] >> 16) & 0x7fffu;
      qm = lo16 > qm ? lo16 : qm;
      qm = hi16 > qm ? hi16 : qm;
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_xor((int)qm, o);
      qm = v > qm ? v : qm;
    }
    const int sh = q_shift(qm);
    v8h h0, h1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h0[2 * i] = bf16_to_f16(w8[i] & 0xffffu, sh);
      h0[2 * i + 1] = bf16_to_f16(w8[i] >> 16, sh);
      h1[2 * i] = bf16_to_f16(w8[4 + i] & 0xffffu, sh);
      h1[2 * i + 1] = bf16_to_f16(w8[4 + i] >> 16, sh);
    }
    *reinterpret_cast<v8h*>(qst + qh * kFcRow + qc * 2) = h0;
    *reinterpret_cast<v8h*>(qst + qh * kFcRow + qc * 2 + 16) = h1;
    if ((tid & 31) == 0) s_qsh[qh] = sh;
  }
  if (a.new_win) {  // uniform: the window append (see above)
    const uint32_t new_code = fp8_code_bits(new_bits);
    s_new[tid] = (uint8_t)new_code;
    if (hg == 0 && split == 0 && seq_ok && t >= 0) {
      // ring row of token t: the window keys [lo, t] are consecutive rows from win_row0
      int64_t rt = (t - swa_b) % a.swa_cap;
      rt = rt < 0 ? rt + a.swa_cap : rt;
      a.swa_w[(int64_t)seq * a.swa_rs + rt * a.swa_re + tid] = (uint8_t)new_code;
    }
  }
  __syncthreads();  // s_idx, Q, s_qsh, s_new
  if (kSelect && !early) load_slot(my_tile(0), 0 < n_my, g0);
  if constexpr (kSelect) {
    load_main(my_tile(1), 1 < n_my, gA);
    load_main(my_tile(2), 2 < n_my, gB);
  }

  const float qsl = ldexpf(a.scale_log2, s_qsh[col]);   // log2-domain scale of head col
  const uint8_t* qrow = qst + col * kFcRow + 256 * grp;   // head col, channels 128*grp ..
  uint8_t* vrow = vbuf + col * kFcRow + 256 * grp;        // key col, channels 128*grp ..
  // P.V reads: A = V^T (16 channels x 16 keys) through DS_READ_B64_TR_B16: in each 16-lane
  // group (keys 4grp..4grp+3), lane 4a+b receives element b of the 8-byte reads of lanes a,
  // a+4, a+8, a+12, so lane r of the group points at channels 4*(r & 3).. of key
  // 4*grp + (r >> 2); block b adds 32 b bytes
  const __attribute__((address_space(3))) uint8_t* vtr =
      (const __attribute__((address_space(3))) uint8_t*)vbuf + (4 * grp + (col >> 2)) * kFcRow + 8 * (col & 3);

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v4f o[kFcDT];
#pragma unroll
  for (int i = 0; i < kFcDT; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // the V reads of tile i must stay before the V writes of tile i+1 (LDS executes one wave's
  // accesses in order; this keeps the compiler from reordering them)
  auto lds_order = [] { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); };

  // One tile's QK over all 512 channels (16 steps of 32: lane group grp supplies channels
  // 128*grp + 8*j .. +7 in step j, for K and Q alike), its V written in place, and, when
  // with_pv, the P.V of the previous tile from the same buffer, block by block just before
  // it is overwritten.  Returns S^T (lane: head col, keys 4*grp..+3); *valid receives bit k
  // for each present key k.
  auto tile_step = [&](const auto& g, bool is_main, bool with_pv, v4h pb_prev, uint32_t* valid) -> v4f {
    constexpr bool kFirst = std::is_same<std::decay_t<decltype(g)>, FcSlot>::value;
    const uint32_t keep = 0u - g.ok;
    v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    auto word = [&](int d) -> uint32_t {   // raw dword d of the lane's slot
      const uint4 v = g.r[d >> 2];
      return (d & 3) == 0 ? v.x : ((d & 3) == 1 ? v.y : ((d & 3) == 2 ? v.z : v.w));
    };
    v2h ss[8];
    {  // the eight E4M3 group scales to fp16 (exact); an absent key's scale is 0
      const uint32_t s0 = g.sc0 & keep, s1 = g.sc1 & keep;
      const v2h a01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, false);
      const v2h a23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, true);
      const v2h b01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, false);
      const v2h b23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, true);
      ss[0] = __builtin_shufflevector(a01, a01, 0, 0);
      ss[1] = __builtin_shufflevector(a01, a01, 1, 1);
      ss[2] = __builtin_shufflevector(a23, a23, 0, 0);
      ss[3] = __builtin_shufflevector(a23, a23, 1, 1);
      ss[4] = __builtin_shufflevector(b01, b01, 0, 0);
      ss[5] = __builtin_shufflevector(b01, b01, 1, 1);
      ss[6] = __builtin_shufflevector(b23, b23, 0, 0);
      ss[7] = __builtin_shufflevector(b23, b23, 1, 1);
    }
    // Q of the next two QK steps is read one iteration ahead, so its LDS latency is not
    // waited for just before the MFMA that takes it
    v8h qa0 = *reinterpret_cast<const v8h*>(qrow);
    v8h qa1 = *reinterpret_cast<const v8h*>(qrow + 16);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const v8h qc0 = qa0, qc1 = qa1;
      if (m < 7) {
        qa0 = *reinterpret_cast<const v8h*>(qrow + 16 * (2 * m + 2));
        qa1 = *reinterpret_cast<const v8h*>(qrow + 16 * (2 * m + 3));
      }
      if (with_pv) {   // uniform: blocks m, m+8, m+16, m+24 of the previous tile
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int b = m + 8 * gq;
          const v4h av = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vtr + 32 * b)));
          o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb_prev, o[b], 0, 0, 0);
        }
        lds_order();
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * m + h;
        v8h k;
        if constexpr (kFirst) {
          if (is_main) {
            k = fp4x8_to_f16(word(j), ss[j >> 1]);
          } else {
            uint32_t d0 = word(2 * j), d1 = word(2 * j + 1);
            if (a.new_win) {  // uniform: the row's own token comes from the LDS copy, not the ring
              const uint2 n = *reinterpret_cast<const uint2*>(s_new + 128 * grp + 8 * j);
              d0 = g.is_new ? n.x : d0;
              d1 = g.is_new ? n.y : d1;
            }
            k = fp8x8_to_f16(d0 & keep, d1 & keep);
          }
        } else {
          k = fp4x8_to_f16(word(j), ss[j >> 1]);
        }
        *reinterpret_cast<v8h*>(vrow + 16 * j) = k;
        if (h == 0) sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qc0, sa, 0, 0, 0);
        else sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qc1, sb, 0, 0, 0);
      }
    }
    *valid = (uint32_t)__ballot(g.ok != 0) & 0xffffu;  // lanes 0..15 hold keys 0..15
    return sa + sb;
  };

  // online softmax over one tile's S^T (lane: head col, keys 4*grp + r), with k_attn's lazy
  // reference; returns P^T in fp16 and in *alpha the factor for the accumulators
  auto softmax_tile = [&](v4f sv, uint32_t valid, float* alpha_out) -> v4h {
    float x[4];
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (valid >> (4 * grp + r)) & 1u;
      x[r] = ok ? sv[r] * qsl : -__builtin_inff();
      mt = fmaxf(mt, x[r]);
    }
    mt = lanes4_max(mt);
    const bool first = m_run == -__builtin_inff();
    const bool move = first ? mt != -__builtin_inff() : mt > m_run + kLazy;
    const float m_new = move ? mt : m_run;
    const float alpha = (move && !first) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const bool none = m_new == -__builtin_inff();
    v4h pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = none ? 0.0f : __builtin_amdgcn_exp2f(x[r] - m_new);
      psum += pr;
      pb[r] = (_Float16)pr;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    *alpha_out = alpha;
    return pb;
  };
  auto rescale = [&](float alpha) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kFcDT; ++dt) o[dt] *= alpha;
    }
  };

  // ---- software pipeline.  Step i forms S of tile i+1 (main slot gA or gB) with the P.V of
  // tile i interleaved, refills that slot with tile i+3, then runs the softmax of tile i+1.
  // Each load has two steps to arrive ----
  auto tile_is_main = [&](int i) { return my_tile(i) < a.main_tiles; };
  uint32_t vmask = 0u;
  float alpha = 1.0f;
  v4h pb = {};
  if (n_my > 0) {   // uniform over the wave
    const v4f sp = tile_step(g0, tile_is_main(0), false, pb, &vmask);
    pb = softmax_tile(sp, vmask, &alpha);
  }
  auto step = [&](int i, FcMainSlot& g) {
    lds_order();
    const v4f sp = tile_step(g, true, true, pb, &vmask);   // tile i+1, the P.V of tile i inside
    load_main(my_tile(i + 3), i + 3 < n_my, g);
    pb = softmax_tile(sp, vmask, &alpha);   // tile i+1
    rescale(alpha);
  };
  // Steps 0 .. n_my-2 form S of tiles 1 .. n_my-1; then the last tile's P.V.  Whole rounds
  // of the ring inside the loop and the remainder after it.
  const int n_full = n_my - 1;
  int i = 0;
  for (; i + 2 <= n_full; i += 2) {
    step(i, gA);
    step(i + 1, gB);
  }
  if (i < n_full) step(i, gA);   // uniform over the wave
  if (n_my > 0) {
    lds_order();
#pragma unroll
    for (int b = 0; b < kFcDT; ++b) {
      const v4h av = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vtr + 32 * b)));
      o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, o[b], 0, 0, 0);
    }
  }

  // ---- merge the eight streams' (O, m, l) ----
  const float l_tot = lanes4_sum(l_run);
  if (lane < kHG) {
    s_ml[wave][lane][0] = m_run;
    s_ml[wave][lane][1] = l_tot;
  }
  __syncthreads();  // every wave is past its loop: the V buffers are free
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kStreams; ++w) M = fmaxf(M, s_ml[w][col][0]);
  float Ltot = 0.0f, mine = 0.0f;
#pragma unroll
  for (int w = 0; w < kStreams; ++w) {
    const float mw = s_ml[w][col][0];
    const float sw = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
    Ltot += sw * s_ml[w][col][1];
    mine = w == wave ? sw : mine;
  }
  const int head = hg * kHG + col;
  const float inv = Ltot > 0.0f ? 1.0f / Ltot : 0.0f;
  float4* part = reinterpret_cast<float4*>(lds);   // [4 slots][32 blocks][64 lanes]: 128 KB
  // round 1: streams 4..7 store their weighted O^T in slot wave - 4; streams 0..3 add it
  if (wave >= 4) {
#pragma unroll
    for (int b = 0; b < kFcDT; ++b) {
      const v4f v = o[b] * mine;
      part[((wave - 4) * kFcDT + b) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int b = 0; b < kFcDT; ++b) {
      const float4 p4 = part[(wave * kFcDT + b) * 64 + lane];
      const v4f v = o[b] * mine + v4f{p4.x, p4.y, p4.z, p4.w};
      part[(wave * kFcDT + b) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  __syncthreads();
  // round 2: wave w sums blocks 4w .. 4w+3 over the four slots
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int b = 4 * wave + bb;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const float4 v = part[(sl * kFcDT + b) * 64 + lane];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int ch = 16 * b + 4 * grp;   // channels ch..ch+3 of head col
    if (a.nsplit == 1) {
      const int64_t ob = ((int64_t)q * a.n_heads + head) * kD + ch;
      if (a.out_dtype == CSA2_DT_F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + ob) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      } else {
        uint2 pk;
        pk.x = f32_to_bf16_rne(acc.x * inv) | (f32_to_bf16_rne(acc.y * inv) << 16);
        pk.y = f32_to_bf16_rne(acc.z * inv) | (f32_to_bf16_rne(acc.w * inv) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob) = pk;
      }
    } else {
      const int64_t pbx = ((int64_t)split * a.n_q + q) * a.n_heads + head;
      *reinterpret_cast<float4*>(a.ws_o + pbx * kD + ch) = acc;
    }
  }
  if (wave == 0 && lane < kHG) {
    if (a.nsplit == 1) {
      if (a.lse) a.lse[(int64_t)q * a.n_heads + head] = Ltot > 0.0f ? (M + __log2f(Ltot)) * kLn2 : -__builtin_inff();
    } else {
      const int64_t pbx = ((int64_t)split * a.n_q + q) * a.n_heads + head;
      a.ws_ml[pbx * 2] = M;
      a.ws_ml[pbx * 2 + 1] = Ltot;
    }
  }
}


// merge the per-split (O, m, l) of one (query, head): 128 threads x 4 channels.  The first
// eight splits' partial outputs are loaded first (they do not depend on (m, l)), while
// thread sp < nsplit reads split sp's (m, l) into LDS, so up to eight splits cost one memory
// round trip; further splits are read eight at a time.  Every load is unconditional (clamped
// split index) and the weights past the last split are zero.  (Merging inside the attention
// kernel, in the last split's workgroup to finish, was measured much slower: the agent-scope
// release that publishes the partial results writes back the L2.)
constexpr int kCombThreads = 128;   // also the most splits a merge takes

__global__ __launch_bounds__(kCombThreads) void k_attn_combine(AttnArgs a) {
  const int qh = blockIdx.x;  // q * n_heads + h
  const int tid = threadIdx.x;
  const int ns = a.nsplit;
  const int64_t stride = (int64_t)a.n_q * a.n_heads;
  __shared__ float s_m[kCombThreads], s_l[kCombThreads];
  auto load8 = [&](int sp0, float4 (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = sp0 + u < ns ? sp0 + u : ns - 1;
      v[u] = *reinterpret_cast<const float4*>(a.ws_o + (sp * stride + qh) * kD + tid * 4);
    }
  };
  float4 v[8];
  load8(0, v);
  {
    const int sp = tid < ns ? tid : ns - 1;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (sp * stride + qh) * 2);
    if (tid < ns) {
      s_m[tid] = ml.x;
      s_l[tid] = ml.y;
    }
  }
  __syncthreads();
  float M = -__builtin_inff();
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, s_m[sp]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp0 = 0; sp0 < ns && M != -__builtin_inff(); sp0 += 8) {
    if (sp0 > 0) load8(sp0, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = sp0 + u < ns ? sp0 + u : ns - 1;
      const float m = s_m[sp];
      const float wgt = (sp0 + u < ns && m != -__builtin_inff()) ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
      L += wgt * s_l[sp];
      acc.x += wgt * v[u].x;
      acc.y += wgt * v[u].y;
      acc.z += wgt * v[u].z;
      acc.w += wgt * v[u].w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t ob = (int64_t)qh * kD + tid * 4;
  if (a.out_dtype == CSA2_DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + ob) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 pk;
    pk.x = f32_to_bf16_rne(acc.x * inv) | (f32_to_bf16_rne(acc.y * inv) << 16);
    pk.y = f32_to_bf16_rne(acc.z * inv) | (f32_to_bf16_rne(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob) = pk;
  }
  if (a.lse && tid == 0) a.lse[qh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

// ---- many query rows: one workgroup per row, every head ----
//
// With thousands of rows (a prefill chunk, an encoder group) the grid is full without
// cutting a row's heads into 16-head workgroups, so a row's keys can be dequantised once
// for all of its heads instead of once per head group.  One workgroup = one row and 64
// heads, 4 waves of 16 heads each.  Per tile of 32 keys all 256 threads gather the raw
// bytes (thread = key x 64 channels, two tiles ahead) and dequantise them once into an
// fp16 tile in LDS (three buffers, one barrier per tile); every wave then forms S^T =
// K Q^T for its 16 heads over all 512 channels (K read from the tile, Q in registers),
// runs the online softmax of its own heads (no exchange between waves: a wave holds whole
// heads) and accumulates O^T += V^T P^T on V_MFMA_F32_16X16X32_F16 over the 32 keys, V^T
// read from the same tile through DS_READ_B64_TR_B16.  The 32 keys of a P.V product are
// taken in the order in which the two 16-key S^T blocks leave them in the lanes (keys
// 4g..4g+3 and 16+4g..16+4g+3 for lane group g), and the V^T reads follow that order, so P
// needs no shuffle.  Step i forms S of tile i and P.V of tile i-1 (independent matrix
// work) beside the dequantisation of tile i+1 and the softmax of tile i.  Rows are dealt
// to the XCDs in contiguous ranges, so neighbouring rows, whose windows overlap, share an
// L2.  The arithmetic per (row, head) is that of k_attn: exact fp16 keys and values, Q
// scaled by a power of two per head, P rounded to fp16, fp32 accumulation.
constexpr int kRWaves = 4;                  // waves per workgroup, 16 heads each
constexpr int kRThreads = kRWaves * 64;
constexpr int kRHeads = kRWaves * kHG;      // heads per row
constexpr int kRT = 32;                     // keys per tile
// A key row of the fp16 tile (1,024 B) starts at r * kRRow + rpad(r): the per-row offsets
// put the 16 rows of a K-operand read (16 B per lane) in 16 different bank slots, the 8 rows
// of a transposed V read (32 B per 4 lanes) in 8 different 32-byte spans, and the rows of
// one dequantisation store in different slots, so none of the three conflicts
constexpr int kRRow = kD * 2 + 256;         // row pitch: the data plus room for the offset
constexpr int kRBuf = kRT * kRRow;          // 40,960 B
__device__ __forceinline__ int rpad(int r) { return 32 * (r & 7) + 16 * ((r >> 3) & 1); }
constexpr int kRBufs = 3;
constexpr int kRSteps = kD / 32;            // QK steps per tile and 16-key block: 16
constexpr int kRDT = kD / 16;               // 16-channel blocks of O^T: 32
constexpr int kRIdxPer = CSA2_MAX_TOPK / kRThreads;
static_assert(kRT * 8 == kRThreads, "one thread per (key, 64 channels) of a tile");

__global__ __launch_bounds__(kRThreads, 1) void k_attn_rows(AttnArgs a, const int32_t* __restrict__ q_seq,
                                                            const int64_t* __restrict__ q_pos,
                                                            const int64_t* __restrict__ replay_start,
                                                            const int64_t* __restrict__ swa_base) {
  const int rows_per_xcd = (a.n_q + 7) >> 3;
  const int q = (blockIdx.x & 7) * rows_per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= rows_per_xcd || q >= a.n_q) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;    // MFMA roles: key row / head column, lane group
  const int kk = tid & 31, ck = tid >> 5;         // gather role: key of the tile, 64-channel chunk

  __shared__ __attribute__((aligned(16))) uint8_t tiles[kRBufs * kRBuf];
  __shared__ int32_t s_idx[CSA2_MAX_TOPK];
  __shared__ uint32_t s_mask[kRBufs];             // bit k: key k of the tile is present

  const int seq = q_seq[q];
  const int64_t t = q_pos[q], s = replay_start[q];
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int n_mt = (a.k + kRT - 1) / kRT;                 // main tiles
  const int n_wt = (a.window + kRT - 1) / kRT;            // window tiles (processed first)
  const int n_tiles = n_mt + n_wt;

  // the row's index list (unconditional clamped loads), then Q
  int32_t iv[kRIdxPer];
  const int n_slots = n_mt * kRT;
  if (a.k > 0) {  // uniform
#pragma unroll
    for (int r = 0; r < kRIdxPer; ++r) {
      const int i = tid + r * kRThreads;
      iv[r] = a.idx[(int64_t)q * a.k + (i < a.k ? i : a.k - 1)];
    }
  }
  const int head = wave * kHG + col;
  uint4 qraw[kRSteps];   // step st: channels 32*st + 8*grp .. +7 of the lane's head
  {
    const uint16_t* qp = a.q + ((int64_t)q * a.n_heads + head) * kD + 8 * grp;
#pragma unroll
    for (int st = 0; st < kRSteps; ++st) qraw[st] = *reinterpret_cast<const uint4*>(qp + 32 * st);
  }

  const int64_t lo = s > t - a.window + 1 ? s : t - a.window + 1;
  const int64_t n_swa = seq_ok && t >= lo ? t - lo + 1 : 0;
  const int64_t swa_b = seq_ok ? swa_base[seq] : 0;
  const int64_t rel = lo - swa_b;
  const uint32_t swa_cap32 = (uint32_t)a.swa_cap;
  int64_t r_lo;
  if (rel >= 0 && rel <= 0xffffffffLL) {
    r_lo = (uint32_t)rel % swa_cap32;
  } else {
    r_lo = rel % a.swa_cap;
    r_lo = r_lo < 0 ? r_lo + a.swa_cap : r_lo;
  }
  const uint32_t win_row0 = (uint32_t)r_lo;
  const uint8_t* kvc = a.kv_codes + (int64_t)(seq_ok ? seq : 0) * a.kv_cs;
  const uint8_t* kvs = a.kv_scales + (int64_t)(seq_ok ? seq : 0) * a.kv_ss;
  const uint8_t* swq = a.swa + (int64_t)(seq_ok ? seq : 0) * a.swa_rs;

  // Tile i < n_wt holds window keys 32i .. 32i+31, tile n_wt + m the list's slots 32m ..
  // 32m+31.  Every load is unconditional, to an in-bounds address (an absent key reads
  // row 0 and is flagged).  Tiles past the end load row 0 of both caches, flagged absent.
  auto load_slot = [&](int i, GatherSlot& g) {
    const bool is_win = i < n_wt;   // uniform
    const int slot = (i - n_wt) * kRT + kk;
    const int sc = slot < 0 ? 0 : (slot < n_slots ? slot : (n_slots > 0 ? n_slots - 1 : 0));
    const int32_t p = (!is_win && i < n_tiles && slot < a.k && n_slots > 0) ? s_idx[sc] : -1;
    const bool ok_main = !is_win && seq_ok && p >= 0 && p < a.seq_cap;
    const uint32_t pm = ok_main ? (uint32_t)p : 0u;
    const int j = i * kRT + kk;
    const bool ok_win = is_win && seq_ok && j < n_swa;
    uint32_t row = win_row0 + (uint32_t)j;
    row = ok_win ? (row >= swa_cap32 ? row - swa_cap32 : row) : 0u;
    const uint4* c = !is_win
        ? reinterpret_cast<const uint4*>(kvc + ((uint64_t)pm * (uint64_t)a.kv_ce + 32 * ck))
        : reinterpret_cast<const uint4*>(swq + ((uint64_t)row * (uint64_t)a.swa_re + 64 * ck));
    const uint4* c2 = !is_win ? c : c + 2;
    g.r[0] = c[0];
    g.r[1] = c[1];
    g.r[2] = c2[0];
    g.r[3] = c2[1];
    g.sc = *reinterpret_cast<const uint32_t*>(kvs + ((uint64_t)pm * (uint64_t)a.kv_se + 4 * ck));
    g.ok = is_win ? ok_win : ok_main;
  };

  // dequantise this thread's 64 channels of its key into the tile (absent keys: zeros)
  // and record which keys are present
  auto dequant = [&](int i, const GatherSlot& g, int buf) {
    const uint32_t keep = 0u - g.ok;
    uint8_t* dst = tiles + buf * kRBuf + kk * kRRow + rpad(kk) + 128 * ck;
    if (i >= n_wt) {   // uniform: main entries
      const uint32_t cw[8] = {g.r[0].x, g.r[0].y, g.r[0].z, g.r[0].w, g.r[1].x, g.r[1].y, g.r[1].z, g.r[1].w};
      const uint32_t sc = g.sc & keep;
      const v2h s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
      const v2h s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);
      const v2h ss[4] = {__builtin_shufflevector(s01, s01, 0, 0), __builtin_shufflevector(s01, s01, 1, 1),
                         __builtin_shufflevector(s23, s23, 0, 0), __builtin_shufflevector(s23, s23, 1, 1)};
#pragma unroll
      for (int d = 0; d < 8; ++d) *reinterpret_cast<v8h*>(dst + 16 * d) = fp4x8_to_f16(cw[d], ss[d >> 1]);
    } else {
      const uint32_t w[16] = {g.r[0].x, g.r[0].y, g.r[0].z, g.r[0].w, g.r[1].x, g.r[1].y, g.r[1].z, g.r[1].w,
                              g.r[2].x, g.r[2].y, g.r[2].z, g.r[2].w, g.r[3].x, g.r[3].y, g.r[3].z, g.r[3].w};
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<v8h*>(dst + 16 * d) = fp8x8_to_f16(w[2 * d] & keep, w[2 * d + 1] & keep);
    }
    // lane k < 32 of every wave holds key k: wave 0 writes the tile's presence mask
    const uint32_t m32 = (uint32_t)__ballot(g.ok != 0);
    if (tid == 0) s_mask[buf] = m32;
  };

  const bool early = n_wt >= 2;   // the first two tiles are window tiles: no index needed
  GatherSlot g0, g1;
  if (early) {
    load_slot(0, g0);
    load_slot(1, g1);
  }
  if (a.k > 0) {
#pragma unroll
    for (int r = 0; r < kRIdxPer; ++r) {
      const int i = tid + r * kRThreads;
      if (i < n_slots) s_idx[i] = i < a.k ? iv[r] : -1;
    }
  }
  // the head's largest |q| over its 512 channels (bf16 magnitude bits), over the 4 lanes of
  // the head
  uint32_t qm = 0;
#pragma unroll
  for (int st = 0; st < kRSteps; ++st) {
    const uint32_t w4[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t l16 = w4[i] & 0x7fffu, h16 = (w4[i] >> 16) & 0x7fffu;
      qm = l16 > qm ? l16 : qm;
      qm = h16 > qm ? h16 : qm;
    }
  }
  {
    qm = lanes4_umax(qm);
  }
  const int qsh = q_shift(qm);
  const float qsl = ldexpf(a.scale_log2, qsh);
  v8h qf[kRSteps];
#pragma unroll
  for (int st = 0; st < kRSteps; ++st) {
    const uint32_t w4[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
    v8h h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = bf16_to_f16(w4[i] & 0xffffu, qsh);
      h[2 * i + 1] = bf16_to_f16(w4[i] >> 16, qsh);
    }
    qf[st] = h;
  }
  __syncthreads();   // s_idx
  if (!early) {
    load_slot(0, g0);
    load_slot(1, g1);
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v4f o[kRDT];
#pragma unroll
  for (int i = 0; i < kRDT; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // S^T of tile buf for this wave's heads: two 16-key blocks, each over the 512 channels
  // (K rows read from the tile: lane = key col, channels 32*st + 8*grp .. +7)
  auto qk = [&](int buf, v4f* s2) {
    const uint8_t* tb = tiles + buf * kRBuf + col * kRRow + rpad(col) + 16 * grp;
    v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
#pragma unroll
    for (int st = 0; st < kRSteps; st += 2) {
      const v8h k00 = *reinterpret_cast<const v8h*>(tb + 64 * st);
      const v8h k01 = *reinterpret_cast<const v8h*>(tb + 64 * (st + 1));
      const v8h k10 = *reinterpret_cast<const v8h*>(tb + 16 * kRRow + 64 * st);
      const v8h k11 = *reinterpret_cast<const v8h*>(tb + 16 * kRRow + 64 * (st + 1));
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k00, qf[st], a0, 0, 0, 0);
      b0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k10, qf[st], b0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k01, qf[st + 1], a1, 0, 0, 0);
      b1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k11, qf[st + 1], b1, 0, 0, 0);
    }
    s2[0] = a0 + a1;
    s2[1] = b0 + b1;
  };

  // online softmax of one tile (lane: head col; keys 4*grp + r and 16 + 4*grp + r) with the
  // lazy reference of k_attn; returns P^T in fp16 in the K order of the P.V product
  auto softmax = [&](const v4f* s2, uint32_t valid, float* alpha_out) -> v8h {
    float x[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = (r < 4 ? 0 : 16) + 4 * grp + (r & 3);
      const bool ok = (valid >> key) & 1u;
      x[r] = ok ? s2[r >> 2][r & 3] * qsl : -__builtin_inff();
      mt = fmaxf(mt, x[r]);
    }
    mt = lanes4_max(mt);
    const bool first = m_run == -__builtin_inff();
    const bool move = first ? mt != -__builtin_inff() : mt > m_run + kLazy;
    const float m_new = move ? mt : m_run;
    const float alpha = (move && !first) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const bool none = m_new == -__builtin_inff();
    v8h pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float pr = none ? 0.0f : __builtin_amdgcn_exp2f(x[r] - m_new);
      psum += pr;
      pb[r] = (_Float16)pr;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    *alpha_out = alpha;
    return pb;
  };

  // O^T += V^T P^T over the 32 keys of tile buf: A = V^T (16 channels x 32 keys in the K
  // order above), two transposed reads of 4 keys each per lane
  auto pv = [&](v8h pb, int buf) {
    const __attribute__((address_space(3))) uint8_t* vb =
        (const __attribute__((address_space(3))) uint8_t*)(tiles + buf * kRBuf) + (4 * grp + (col >> 2)) * kRRow +
        rpad(4 * grp + (col >> 2)) +
        8 * (col & 3);
#pragma unroll
    for (int dt = 0; dt < kRDT; ++dt) {
      const v4h lo4 = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + 32 * dt)));
      const v4h hi4 =
          __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + 16 * kRRow + 32 * dt)));
      const v8h av = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, o[dt], 0, 0, 0);
    }
  };

  // ---- pipeline.  Tile i lives in buffer i % 3 and its raw bytes in slot g(i % 2).  Step i
  // (after a barrier) dequantises tile i+1, refills its slot with tile i+3, then forms S of
  // tile i, P.V of tile i-1 and the softmax of tile i.  The barrier of step i orders the
  // dequantisation of tile i (step i-1) before the S of tile i, and the P.V of tile i-2
  // (step i-1) before the dequantisation of tile i+1 into the same buffer ----
  dequant(0, g0, 0);
  load_slot(2, g0);
  __syncthreads();
  dequant(1, g1, 1);
  load_slot(3, g1);
  v4f s2[2];
  float alpha;
  qk(0, s2);
  v8h pb = softmax(s2, s_mask[0], &alpha);
  auto step = [&](int i, GatherSlot& g) {   // 1 <= i < n_tiles; g holds tile i+1
    __syncthreads();
    dequant(i + 1, g, (i + 1) % kRBufs);   // past the last tile: absent keys, never read
    load_slot(i + 3, g);
    qk(i % kRBufs, s2);
    pv(pb, (i - 1) % kRBufs);
    pb = softmax(s2, s_mask[i % kRBufs], &alpha);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kRDT; ++dt) o[dt] *= alpha;
    }
  };
  // whole rounds of the two slots inside the loop, the remainder after it
  int i = 1;
  for (; i + 1 < n_tiles; i += 2) {
    step(i, g0);
    step(i + 1, g1);
  }
  if (i < n_tiles) step(i, g0);   // uniform
  pv(pb, (n_tiles - 1) % kRBufs);

  // ---- output: lane (head col, grp) holds channels 16*dt + 4*grp .. +3 of its head ----
  float l_tot = lanes4_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int64_t ob = ((int64_t)q * a.n_heads + head) * kD + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < kRDT; ++dt) {
    const v4f v = o[dt] * inv;
    if (a.out_dtype == CSA2_DT_F32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + ob + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      uint2 pk;
      pk.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      pk.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob + 16 * dt) = pk;
    }
  }
  if (grp == 0 && a.lse) a.lse[(int64_t)q * a.n_heads + head] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}

struct AttnPlan {
  int head_groups, n_tiles, main_tiles, tiles_per_split, nsplit;
  bool full_channel;   // k_attn_fc: a window of at most one tile per key stream (128 keys)
  int64_t grid;
};

// One workgroup per CU (its eight waves, two per SIMD, and its 160 KB of LDS): split the
// key list only while the (query, head group) pairs are too few, keeping at least one tile
// per key stream in every split (8 streams in the full-channel kernel, 4 in the
// split-channel one).  The split-channel kernel splits up to 256 workgroups (every CU); the
// full-channel kernel up to 128: its streams are independent, so a longer key slice costs
// little, while each split repeats the prologue (a selection in the Top-K modes) and adds a
// combine launch (at 32 queries x 64 heads one slice per pair beats two by ~2 us a call;
// at 8 queries four or five slices beat one or two).
static AttnPlan plan(int n_q, int n_heads, int k, int window) {
  AttnPlan p;
  p.head_groups = n_heads / kHG;
  p.main_tiles = (k + kT - 1) / kT;
  p.n_tiles = p.main_tiles + (window + kT - 1) / kT;
  const int64_t base = (int64_t)n_q * p.head_groups;
  p.full_channel = p.n_tiles - p.main_tiles <= kStreams;
  const int fill = p.full_channel ? 128 : 256;
  int want = (int)((fill + base - 1) / (base > 0 ? base : 1));
  const int streams = p.full_channel ? kStreams : kPairs;
  const int max_split = (p.n_tiles + streams - 1) / streams;
  want = want < 1 ? 1 : (want > max_split ? max_split : want);
  p.tiles_per_split = (p.n_tiles + want - 1) / want;
  p.nsplit = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  const int64_t q_pad = ((int64_t)n_q + 7) / 8 * 8;
  p.grid = q_pad * p.head_groups * p.nsplit;
  return p;
}

// The row kernel serves batches of many rows with an index list given and 64 heads, where
// one workgroup per row fills the GPU several times over (at least 4 rows per CU).
constexpr int kRowsMinQ = 1024;
static bool use_rows_kernel(int n_q, int n_heads, int sel_mode, bool new_win) {
  return sel_mode == 0 && !new_win && n_heads == kRHeads && n_q >= kRowsMinQ;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attn_workspace_bytes(int n_q, int n_heads, int dim, int k, int window) {
  if (n_q <= 0 || n_heads < kHG || n_heads % kHG || dim != kD || k < 0 || window < 1) return 0;
  AttnPlan p = plan(n_q, n_heads, k, window);
  if (p.nsplit == 1) return 0;
  return (size_t)p.nsplit * n_q * n_heads * (kD + 2) * sizeof(float) + 256;
}

// Where the index set comes from: a given list (mode 0), the first Top-K level's survivors
// (mode 1) or the pool's slot scores (mode 2); the last two select inside the kernel.
struct AttnSel {
  int mode;
  const uint64_t* cand_keys;
  int cand_per_q;
  const float* pool_scores;
  int64_t pool_stride;
  const int32_t* cand_blocks;
  const int32_t* n_cand_blocks;
  const int64_t* n_vis;
  int block, max_cand_blocks;
};

static int sparse_attn(const void* q, int n_q, int n_heads, int dim, CacheRef kv,
                       int64_t seq_cap, int n_seq, const int32_t* q_seq, const int32_t* idx, const AttnSel& sel,
                       int32_t* idx_out, int32_t* count_out, int k, uint8_t* swa, int64_t swa_re, int64_t swa_rs, int64_t swa_cap,
                       const int64_t* swa_base, const int64_t* q_pos, const int64_t* replay_start,
                       const void* new_win, int new_win_dtype, int window, float sm_scale, void* out, int out_dtype,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = csa2_take_device_status()) return rc;
  if (!q || !kv.codes || !kv.scales || !q_seq || !swa || !swa_base || !q_pos || !replay_start || !out)
    return CSA2_ERR_NULL;
  const bool select = sel.mode != 0;
  if (!select && k > 0 && !idx) return CSA2_ERR_NULL;
  if (n_q < 0 || n_heads < kHG || n_heads > 256 || n_heads % kHG || dim != kD || seq_cap < 0 ||
      seq_cap > CSA2_MAX_ATTN_ENTRIES || n_seq < 1 || k < 0 || k > CSA2_MAX_TOPK || window < 1 ||
      window > CSA2_MAX_WINDOW || swa_cap < window || swa_cap > CSA2_MAX_WINDOW_ROWS)
    return CSA2_ERR_SHAPE;
  if (sel.mode == 1 && (k < 1 || sel.cand_per_q < 1 || sel.cand_per_q > kSelMax)) return CSA2_ERR_SHAPE;
  if (sel.mode == 2 && (k < 1 || sel.block < 1 || sel.block > 64 || sel.max_cand_blocks < 1 ||
                        (int64_t)sel.max_cand_blocks * sel.block > kPoolMax ||
                        sel.pool_stride < (int64_t)sel.max_cand_blocks * sel.block))
    return CSA2_ERR_SHAPE;
  if (out_dtype != CSA2_DT_F32 && out_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (new_win && new_win_dtype != CSA2_DT_F32 && new_win_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if ((uintptr_t)new_win & 3) return CSA2_ERR_SHAPE;   // read in 32-bit words
  if (!aligned16(q) || !aligned16(kv.codes) || !aligned16(swa) || !aligned16(out) || ((uintptr_t)kv.scales & 3))
    return CSA2_ERR_SHAPE;
  // the main-KV cache (D/2 code bytes, D/16 scale bytes per entry; 4-byte scale loads) and
  // the window ring (D bytes per row, 16-byte loads)
  if (resolve_cache(kv, seq_cap, kD / 2, kD / 16, 4) != CSA2_OK) return CSA2_ERR_SHAPE;
  if (swa_re == 0) swa_re = kD;
  if (swa_rs == 0) swa_rs = swa_cap * swa_re;
  if (swa_re < kD || swa_rs < 0 || swa_re % 16 || swa_rs % 16) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  AttnPlan p = plan(n_q, n_heads, k, window);
  if (p.grid > 0x7fffffffLL || p.nsplit > kCombThreads) return CSA2_ERR_SHAPE;
  AttnArgs a = {};
  a.q = (const uint16_t*)q;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.kv_codes = kv.codes;
  a.kv_scales = kv.scales;
  a.kv_ce = kv.ce;
  a.kv_cs = kv.cs;
  a.kv_se = kv.se;
  a.kv_ss = kv.ss;
  a.seq_cap = seq_cap;
  a.n_seq = n_seq;
  a.q_seq = q_seq;
  a.idx = idx;
  a.k = k;
  a.swa = swa;
  a.swa_w = swa;
  a.swa_re = swa_re;
  a.swa_rs = swa_rs;
  a.swa_cap = swa_cap;
  a.swa_base = swa_base;
  a.q_pos = q_pos;
  a.replay_start = replay_start;
  a.window = window;
  a.scale_log2 = sm_scale * kLog2e;
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = lse;
  a.nsplit = p.nsplit;
  a.tiles_per_split = p.tiles_per_split;
  a.n_tiles = p.n_tiles;
  a.main_tiles = p.main_tiles;
  a.head_groups = p.head_groups;
  a.cand_keys = sel.cand_keys;
  a.cand_per_q = sel.cand_per_q;
  a.pool_scores = sel.pool_scores;
  a.pool_stride = sel.pool_stride;
  a.cand_blocks = sel.cand_blocks;
  a.n_cand_blocks = sel.n_cand_blocks;
  a.n_vis = sel.n_vis;
  a.block = sel.block;
  a.max_cand_blocks = sel.max_cand_blocks;
  a.idx_out = idx_out;
  a.count_out = count_out;
  a.new_win = new_win;
  a.new_win_bf16 = new_win_dtype == CSA2_DT_BF16;
  a.wait_limit = csa2_wait_limit();
  a.status = csa2_status_word();
  if (p.nsplit > 1) {
    size_t need = csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window);
    if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    uintptr_t w0 = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
    a.ws_o = (float*)w0;
    a.ws_ml = a.ws_o + (size_t)p.nsplit * n_q * n_heads * kD;
  }
  hipStream_t st = (hipStream_t)stream;
  if (use_rows_kernel(n_q, n_heads, sel.mode, new_win != nullptr)) {
    const int64_t grid = 8 * (((int64_t)n_q + 7) / 8);
    hipLaunchKernelGGL(k_attn_rows, dim3((unsigned)grid), dim3(kRThreads), 0, st, a, a.q_seq, a.q_pos,
                       a.replay_start, a.swa_base);
    return csa2_check_launch();
  }
  // The full-channel kernel takes a window of at most one tile per key stream (128 keys);
  // a wider window goes to the split-channel kernel, whose streams take any mix of tiles
  const bool full_channel = p.full_channel;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)p.grid), dim3(kAttnThreads), 0, st, a, a.q_seq, a.q_pos,
                       a.replay_start, a.swa_base);
  };
  if (sel.mode == 2) full_channel ? go(k_attn_fc<2>) : go(k_attn<2>);
  else if (sel.mode == 1) full_channel ? go(k_attn_fc<1>) : go(k_attn<1>);
  else full_channel ? go(k_attn_fc<0>) : go(k_attn<0>);
  int rc = csa2_check_launch();
  if (rc != CSA2_OK || p.nsplit == 1) return rc;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(n_q * n_heads)), dim3(kCombThreads), 0, st, a);
  return csa2_check_launch();
}

extern "C" int csa2_sparse_attn(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes, int64_t kv_codes_stride, int64_t kv_codes_seq_stride, const uint8_t* kv_scales, int64_t kv_scales_stride, int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                const int32_t* idx, int k, uint8_t* swa, int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap, const int64_t* swa_base,
                                const int64_t* q_pos, const int64_t* replay_start, const void* new_win,
                                int new_win_dtype, int window, float sm_scale, void* out, int out_dtype, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  AttnSel sel = {};
  return sparse_attn(q, n_q, n_heads, dim,
                     CacheRef{kv_codes, kv_scales, kv_codes_stride, kv_codes_seq_stride, kv_scales_stride,
                              kv_scales_seq_stride}, seq_cap, n_seq, q_seq, idx, sel, nullptr, nullptr, k,
                     swa, swa_row_stride, swa_seq_stride, swa_cap, swa_base, q_pos, replay_start, new_win, new_win_dtype, window, sm_scale, out,
                     out_dtype, lse, workspace, workspace_bytes, stream);
}

// ---- the no-allocation variant: the split partials live in a static device array ----
// Each GPU the library runs on holds its own copy of `scratch` (at its own address) until the
// process ends.  Host code never passes the array's name to a kernel (on the host it is only
// a stand-in symbol): the device address comes from hipGetSymbolAddress, once per device,
// with that device current, and is kept per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices] = {};
static std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (nullptr and a recorded HIP error if the
// runtime cannot give it).  Called by csa2_init and, for a device csa2_init never saw, by the
// entry point's first call there.
void* csa2_attn_scratch(int* rc_out) {
  int dev = 0;
  int rc = csa2_record_hip_error(hipGetDevice(&dev));
  if (rc == CSA2_OK && (dev < 0 || dev >= kMaxDevices)) rc = CSA2_ERR_UNSUPPORTED;
  if (rc != CSA2_OK) {
    *rc_out = rc;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    rc = csa2_record_hip_error(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (rc == CSA2_OK) g_scratch_ptr[dev] = p;
  }
  *rc_out = rc;
  return g_scratch_ptr[dev];
}

extern "C" size_t csa2_sparse_attn_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int csa2_sparse_attn_noalloc(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes, int64_t kv_codes_stride, int64_t kv_codes_seq_stride, const uint8_t* kv_scales, int64_t kv_scales_stride, int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                        const int32_t* idx, int k, uint8_t* swa, int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap,
                                        const int64_t* swa_base, const int64_t* q_pos, const int64_t* replay_start,
                                        const void* new_win, int new_win_dtype, int window, float sm_scale,
                                        void* out, int out_dtype, float* lse, void* stream) {
  const size_t need = csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window);
  if (need > kScratchBytes) return CSA2_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    int rc = CSA2_OK;
    ws = csa2_attn_scratch(&rc);
    if (!ws) return rc != CSA2_OK ? rc : CSA2_ERR_HIP;
  }
  AttnSel sel = {};
  return sparse_attn(q, n_q, n_heads, dim,
                     CacheRef{kv_codes, kv_scales, kv_codes_stride, kv_codes_seq_stride, kv_scales_stride,
                              kv_scales_seq_stride}, seq_cap, n_seq, q_seq, idx, sel, nullptr, nullptr, k,
                     swa, swa_row_stride, swa_seq_stride, swa_cap, swa_base, q_pos, replay_start, new_win, new_win_dtype, window, sm_scale, out,
                     out_dtype, lse, ws, need > 0 ? kScratchBytes : 0, stream);
}

extern "C" int csa2_sparse_attn_topk(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes, int64_t kv_codes_stride, int64_t kv_codes_seq_stride, const uint8_t* kv_scales, int64_t kv_scales_stride, int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                     const uint64_t* cand_keys, int cand_per_q, int k, int32_t* idx_out,
                                     int32_t* count_out, uint8_t* swa, int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap, const int64_t* swa_base,
                                     const int64_t* q_pos, const int64_t* replay_start, const void* new_win,
                                     int new_win_dtype, int window, float sm_scale, void* out, int out_dtype,
                                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cand_keys || !idx_out || !count_out) return CSA2_ERR_NULL;
  AttnSel sel = {};
  sel.mode = 1;
  sel.cand_keys = cand_keys;
  sel.cand_per_q = cand_per_q;
  return sparse_attn(q, n_q, n_heads, dim,
                     CacheRef{kv_codes, kv_scales, kv_codes_stride, kv_codes_seq_stride, kv_scales_stride,
                              kv_scales_seq_stride}, seq_cap, n_seq, q_seq, nullptr, sel, idx_out,
                     count_out, k, swa, swa_row_stride, swa_seq_stride, swa_cap, swa_base, q_pos, replay_start, new_win, new_win_dtype, window,
                     sm_scale, out, out_dtype, lse, workspace, workspace_bytes, stream);
}

extern "C" int csa2_sparse_attn_pool_topk(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes, int64_t kv_codes_stride, int64_t kv_codes_seq_stride, const uint8_t* kv_scales, int64_t kv_scales_stride, int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                          const float* scores, int64_t scores_stride, const int64_t* n_vis,
                                          const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block,
                                          int max_cand_blocks, int k, int32_t* idx_out, int32_t* count_out,
                                          uint8_t* swa, int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap, const int64_t* swa_base,
                                          const int64_t* q_pos, const int64_t* replay_start, const void* new_win,
                                          int new_win_dtype, int window, float sm_scale, void* out, int out_dtype,
                                          float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !n_vis || !cand_blocks || !n_cand_blocks || !idx_out || !count_out) return CSA2_ERR_NULL;
  AttnSel sel = {};
  sel.mode = 2;
  sel.pool_scores = scores;
  sel.pool_stride = scores_stride;
  sel.cand_blocks = cand_blocks;
  sel.n_cand_blocks = n_cand_blocks;
  sel.n_vis = n_vis;
  sel.block = block;
  sel.max_cand_blocks = max_cand_blocks;
  return sparse_attn(q, n_q, n_heads, dim,
                     CacheRef{kv_codes, kv_scales, kv_codes_stride, kv_codes_seq_stride, kv_scales_stride,
                              kv_scales_seq_stride}, seq_cap, n_seq, q_seq, nullptr, sel, idx_out,
                     count_out, k, swa, swa_row_stride, swa_seq_stride, swa_cap, swa_base, q_pos, replay_start, new_win, new_win_dtype, window,
                     sm_scale, out, out_dtype, lse, workspace, workspace_bytes, stream);
}
