// csa2_sparse_attn: attention of each query over its selected main-KV entries (FP4,
// dequantised exactly) and its sliding window (FP8) in one softmax
// ([W] "CSA2：跨层复用，能借就不自己算", "FP4 与 SWA Bounded Replay";
//  [J] "缓存压缩真的是越大越好吗").
//
// Per query the key set is at most k + window entries (640 in the decode configurations)
// of 512 channels, with V = K, against H heads: two dense H x 640 x 512 products, run on
// the fp16 matrix cores (V_MFMA_F32_16X16X32_F16) with fp32 accumulation.
//
// Exactness of the operands: every main-KV value is E2M1 x E4M3 (at most 6 significant
// bits, magnitude in [2^-10, 2688]) and every window value is E4M3, so both are exact in
// fp16.  Q (bf16) is converted to fp16, which is exact for |q| in [2^-14, 65504); smaller
// magnitudes round to fp16 subnormals (absolute error below 2^-25).  P = exp2(logit - max)
// is rounded to fp16 (11 significant bits) for the P.V product.
//
// Decomposition: one workgroup = (query, 16 heads, slice of the key list), 4 waves.  The
// workgroups of one query are numbered so that they land on the same XCD (dispatch is
// round-robin over the 8 XCDs) and share its L2 for the gathered rows.  The key list is the
// k main slots rounded up to whole tiles of 32, then the window keys, so every tile is
// all-main or all-window.  Per tile:
//   * gather: thread (key, 64-channel block) issues 3 wide loads (32 B of E2M1 codes + 4 B
//     of E4M3 scales, or 64 B of window E4M3), dequantises with the hardware FP4/FP8 -> fp16
//     converts (then an exact packed fp16 multiply by the group scale) and writes 128 B of
//     the tile's K rows, [key][channel] fp16, into LDS (row stride 1,072 B: conflict-free for
//     both reads below).
//   * S^T = K Q^T: wave w takes the tile's 16 keys (w & 1) and channel half (w >> 1): 8 MFMAs
//     with K read from LDS and Q in registers; the two channel halves meet in a small LDS
//     buffer.
//   * every wave forms P for the 16 heads x 32 keys (identical online-softmax statistics in
//     all 4 waves) and accumulates O^T for its 128 channels.  The V^T operand of P.V comes
//     from the same K rows through DS_READ_B64_TR_B16, which hands each lane one channel of
//     4 keys: no transposed copy is stored.
// LDS is double buffered, so each tile costs one barrier; the raw bytes of tile i+1 and the
// index of tile i+2 are in flight while tile i is processed.  When a batch has too few
// queries to fill the GPU, the key list is split over workgroups and a combine kernel merges
// the partial (O, m, l) with the log-sum-exp rule.
#include "device.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kT = 32;                    // keys per tile
constexpr int kHG = 16;                   // heads per workgroup
constexpr int kD = 512;
constexpr int kKRow = kD * 2 + 48;        // bytes per K row in LDS: 1,072 (see the header)
constexpr int kKBuf = kT * kKRow;
constexpr int kSRow = 20;                 // floats per key row of the logit exchange
constexpr int kSBuf = 2 * kT * kSRow;     // floats: 2 channel halves x 32 keys
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
  int64_t seq_cap;
  int n_seq;
  const int32_t* q_seq;
  const int32_t* idx;
  int k;
  const uint8_t* swa;
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
};

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// bf16 bits -> fp16 (see the header comment for the range)
__device__ __forceinline__ _Float16 bf16_to_f16(uint32_t b) { return (_Float16)__uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t h2_bits(v2h v) { return *reinterpret_cast<uint32_t*>(&v); }

// 8 E2M1 values of one code dword (channel 2i in the low nibble of byte i) times an E4M3
// scale, as 4 packed fp16 pairs; exact
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t codes, uint32_t scale_code) {
  const _Float16 s = (_Float16)e4m3_val(scale_code);
  const v2h ss = {s, s};
  return make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss));
}

// 8 E4M3 values (two dwords) as 4 packed fp16 pairs; exact
__device__ __forceinline__ uint4 fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  return make_uint4(h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
                    h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true)));
}

__global__ __launch_bounds__(kAttnThreads, 2) void k_attn(AttnArgs a) {
  // ---- which (query, head group, split) this workgroup is; same query -> same XCD ----
  const int G = a.head_groups * a.nsplit;
  const int L = blockIdx.x;
  const int xcd = L & 7, jj = L >> 3;
  const int q = 8 * (jj / G) + xcd;
  if (q >= a.n_q) return;
  const int rem = jj % G;
  const int hg = rem % a.head_groups;
  const int split = rem / a.head_groups;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int gk = tid & 31, cb = tid >> 5;       // gather role: key of the tile, 64-channel block
  const int rt = wave & 1, dh = wave >> 1;      // QK role: key half of the tile, channel half

  __shared__ __attribute__((aligned(16))) uint8_t kl[2][kKBuf];
  __shared__ float sx[2][kSBuf];
  __shared__ int s_valid[2][kT];

  const int seq = a.q_seq[q];
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int64_t t = a.q_pos[q], s = a.replay_start[q];
  const int64_t lo = s > t - a.window + 1 ? s : t - a.window + 1;
  const int64_t n_swa = seq_ok && t >= lo ? t - lo + 1 : 0;
  const int64_t swa_b = seq_ok ? a.swa_base[seq] : 0;
  const uint8_t* kvc = a.kv_codes + (int64_t)(seq_ok ? seq : 0) * a.seq_cap * (kD / 2);
  const uint8_t* kvs = a.kv_scales + (int64_t)(seq_ok ? seq : 0) * a.seq_cap * (kD / 16);
  const uint8_t* swq = a.swa + (int64_t)(seq_ok ? seq : 0) * a.swa_cap * kD;
  const int32_t* idxq = a.idx + (int64_t)q * a.k;

  // ---- Q of head (hg*16 + col) as the fp16 B operand, 8 steps of 8 channels ----
  // step (e, s4): channels 256*dh + 128*e + 32*g + 8*s4 .. +7 (same order as the K operand)
  v8h qf[8];
  {
    const uint16_t* qp = a.q + ((int64_t)q * a.n_heads + hg * kHG + col) * kD + 256 * dh + 32 * g;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const uint4 v = *reinterpret_cast<const uint4*>(qp + 128 * e + 8 * s4);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        v8h h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[2 * i] = bf16_to_f16(w4[i] & 0xffffu);
          h[2 * i + 1] = bf16_to_f16(w4[i] >> 16);
        }
        qf[4 * e + s4] = h;
      }
  }

  // position of this thread's gather key in a main tile (-1: none)
  auto load_idx = [&](int tile) -> int32_t {
    const int slot = tile * kT + gk;
    return (seq_ok && tile < a.main_tiles && slot < a.k) ? idxq[slot] : -1;
  };
  // raw bytes of the gather key's 64 channels: main = 2 x 16 B codes + 4 scale bytes,
  // window = 4 x 16 B of E4M3; r[4] = 0 marks "no key"
  auto load_raw = [&](int tile, int32_t p, uint4 r[4], uint32_t& kind) {
    kind = 0;
    r[0] = r[1] = r[2] = r[3] = make_uint4(0u, 0u, 0u, 0u);
    if (tile < a.main_tiles) {
      if (p >= 0 && p < a.seq_cap) {
        const uint4* c = reinterpret_cast<const uint4*>(kvc + (int64_t)p * (kD / 2) + cb * 32);
        r[0] = c[0];
        r[1] = c[1];
        r[2].x = *reinterpret_cast<const uint32_t*>(kvs + (int64_t)p * (kD / 16) + cb * 4);
        kind = 1;
      }
    } else {
      const int64_t j = (int64_t)(tile - a.main_tiles) * kT + gk;
      if (seq_ok && j < n_swa) {
        int64_t row = (lo + j - swa_b) % a.swa_cap;
        row = row < 0 ? row + a.swa_cap : row;
        const uint4* c = reinterpret_cast<const uint4*>(swq + row * kD + cb * 64);
        r[0] = c[0];
        r[1] = c[1];
        r[2] = c[2];
        r[3] = c[3];
        kind = 2;
      }
    }
  };

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v4f o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int tile_lo = split * a.tiles_per_split;
  int tile_hi = tile_lo + a.tiles_per_split;
  tile_hi = tile_hi < a.n_tiles ? tile_hi : a.n_tiles;

  uint4 raw[4], raw_n[4];
  uint32_t kind = 0, kind_n = 0;
  int32_t p_next = -1;
  if (tile_lo < tile_hi) {
    load_raw(tile_lo, load_idx(tile_lo), raw, kind);
    if (tile_lo + 1 < tile_hi) p_next = load_idx(tile_lo + 1);
  }

  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    const int buf = (tile - tile_lo) & 1;
    int32_t p_after = -1;
    if (tile + 1 < tile_hi) load_raw(tile + 1, p_next, raw_n, kind_n);
    if (tile + 2 < tile_hi) p_after = load_idx(tile + 2);

    // ---- gather: dequantise 64 channels of one key into the K tile ----
    {
      uint4 h[8];
      if (kind == 1) {
        const uint32_t cw[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = fp4x8_to_f16(cw[i], (raw[2].x >> (8 * (i >> 1))) & 255u);
      } else {
        // window bytes (or zeros for an empty slot: E4M3 0x00 is +0)
        const uint32_t bw[16] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w,
                                 raw[2].x, raw[2].y, raw[2].z, raw[2].w, raw[3].x, raw[3].y, raw[3].z, raw[3].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = fp8x8_to_f16(bw[2 * i], bw[2 * i + 1]);
      }
      uint4* dst = reinterpret_cast<uint4*>(&kl[buf][gk * kKRow + cb * 128]);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = h[i];
      if (cb == 0) s_valid[buf][gk] = kind != 0;
    }
    __syncthreads();

    // ---- QK role: partial S^T over one channel half ----
    {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* kr = &kl[buf][(16 * rt + col) * kKRow + (256 * dh + 32 * g) * 2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const v8h av = *reinterpret_cast<const v8h*>(kr + (128 * e + 8 * s4) * 2);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qf[4 * e + s4], acc, 0, 0, 0);
        }
      // lane holds S^T[key 16*rt + 4*g + r][head col] for this channel half
      float* sp = &sx[buf][(dh * kT + 16 * rt + 4 * g) * kSRow + col];
#pragma unroll
      for (int r = 0; r < 4; ++r) sp[r * kSRow] = acc[r];
    }
    __syncthreads();

    // ---- softmax over the tile's 32 keys for head col (all waves, same statistics) ----
    float x[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int key = 8 * g + e8;
      const float sv = sx[buf][key * kSRow + col] + sx[buf][(kT + key) * kSRow + col];
      const float xv = s_valid[buf][key] ? sv * a.scale_log2 : -__builtin_inff();
      x[e8] = xv;
      mt = fmaxf(mt, xv);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool none = m_new == -__builtin_inff();
    const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    v8h pb;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const float p = none ? 0.0f : __builtin_amdgcn_exp2f(x[e8] - m_new);
      psum += p;
      pb[e8] = (_Float16)p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }

    // ---- O^T += V^T P^T for this wave's 128 channels; V^T via transposing LDS reads ----
    // lane (c, g) needs V[keys 8g..8g+7][channel c]; in its 16-lane group, lane 4a+b gets
    // element b of the 8-byte chunks of lanes a, a+4, a+8, a+12, so lane r of the group points
    // at channels 4*(r & 3).. of key (r >> 2).
    {
      const int kq = col >> 2, cq = col & 3;
      const __attribute__((address_space(3))) uint8_t* kb =
          (const __attribute__((address_space(3))) uint8_t*)&kl[buf][0];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int ch = 128 * wave + 16 * dt + 4 * cq;
        // whole-vector casts: building the operand element by element from the i16 lanes
        // was observed to lose the upper dword of each read in this compiler
        const v4h h0 = __builtin_bit_cast(
            v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kb + (8 * g + kq) * kKRow + ch * 2)));
        const v4h h1 = __builtin_bit_cast(
            v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(kb + (8 * g + 4 + kq) * kKRow + ch * 2)));
        const v8h av = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, o[dt], 0, 0, 0);
      }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = raw_n[i];
    kind = kind_n;
    p_next = p_after;
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = l_tot + __shfl_xor(l_tot, 32);
  const int head = hg * kHG + col;
  const int ch0 = 128 * wave + 4 * g;

  if (a.nsplit == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t ob = ((int64_t)q * a.n_heads + head) * kD + ch0;
    if (a.out_dtype == CSA2_DT_F32) {
      float* out = reinterpret_cast<float*>(a.out) + ob;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(out + 16 * dt) =
            make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ob;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 pk;
        pk.x = f32_to_bf16_rne(o[dt][0] * inv) | (f32_to_bf16_rne(o[dt][1] * inv) << 16);
        pk.y = f32_to_bf16_rne(o[dt][2] * inv) | (f32_to_bf16_rne(o[dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + 16 * dt) = pk;
      }
    }
    if (a.lse && wave == 0 && g == 0)
      a.lse[(int64_t)q * a.n_heads + head] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
  } else {
    const int64_t pbase = ((int64_t)split * a.n_q + q) * a.n_heads + head;
    float* wo = a.ws_o + pbase * kD + ch0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(wo + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (wave == 0 && g == 0) {
      a.ws_ml[pbase * 2] = m_run;
      a.ws_ml[pbase * 2 + 1] = l_tot;
    }
  }
}

// merge the per-split (O, m, l) of one (query, head): 128 threads x 4 channels
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int qh = blockIdx.x;  // q * n_heads + h
  const int tid = threadIdx.x;
  const int64_t stride = (int64_t)a.n_q * a.n_heads;
  float M = -__builtin_inff();
  for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, a.ws_ml[(sp * stride + qh) * 2]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -__builtin_inff()) {
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const int64_t pb = sp * stride + qh;
      const float m = a.ws_ml[pb * 2];
      const float wgt = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      L += wgt * a.ws_ml[pb * 2 + 1];
      const float4 v = *reinterpret_cast<const float4*>(a.ws_o + pb * kD + tid * 4);
      acc.x += wgt * v.x;
      acc.y += wgt * v.y;
      acc.z += wgt * v.z;
      acc.w += wgt * v.w;
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

struct AttnPlan {
  int head_groups, n_tiles, main_tiles, tiles_per_split, nsplit;
  int64_t grid;
};

// Split the key list only when (query, head group) pairs alone cannot fill the 256 CUs.
static AttnPlan plan(int n_q, int n_heads, int k, int window) {
  AttnPlan p;
  p.head_groups = n_heads / kHG;
  p.main_tiles = (k + kT - 1) / kT;
  p.n_tiles = p.main_tiles + (window + kT - 1) / kT;
  const int64_t base = (int64_t)n_q * p.head_groups;
  int want = (int)((256 + base - 1) / (base > 0 ? base : 1));
  want = want < 1 ? 1 : (want > p.n_tiles ? p.n_tiles : want);
  p.tiles_per_split = (p.n_tiles + want - 1) / want;
  p.nsplit = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  const int64_t q_pad = ((int64_t)n_q + 7) / 8 * 8;
  p.grid = q_pad * p.head_groups * p.nsplit;
  return p;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attn_workspace_bytes(int n_q, int n_heads, int dim, int k, int window) {
  if (n_q <= 0 || n_heads < kHG || n_heads % kHG || dim != kD || k < 0 || window < 1) return 0;
  AttnPlan p = plan(n_q, n_heads, k, window);
  if (p.nsplit == 1) return 0;
  return (size_t)p.nsplit * n_q * n_heads * (kD + 2) * sizeof(float) + 256;
}

extern "C" int csa2_sparse_attn(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes,
                                const uint8_t* kv_scales, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                                const int32_t* idx, int k, const uint8_t* swa, int64_t swa_cap,
                                const int64_t* swa_base, const int64_t* q_pos, const int64_t* replay_start,
                                int window, float sm_scale, void* out, int out_dtype, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!q || !kv_codes || !kv_scales || !q_seq || !swa || !swa_base || !q_pos || !replay_start || !out)
    return CSA2_ERR_NULL;
  if (k > 0 && !idx) return CSA2_ERR_NULL;
  if (n_q < 0 || n_heads < kHG || n_heads > 256 || n_heads % kHG || dim != kD || seq_cap < 0 || n_seq < 1 ||
      k < 0 || k > CSA2_MAX_TOPK || window < 1 || window > CSA2_MAX_WINDOW || swa_cap < window)
    return CSA2_ERR_SHAPE;
  if (out_dtype != CSA2_DT_F32 && out_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv_codes) || !aligned16(swa) || !aligned16(out)) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  AttnPlan p = plan(n_q, n_heads, k, window);
  if (p.grid > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  AttnArgs a = {};
  a.q = (const uint16_t*)q;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.kv_codes = kv_codes;
  a.kv_scales = kv_scales;
  a.seq_cap = seq_cap;
  a.n_seq = n_seq;
  a.q_seq = q_seq;
  a.idx = idx;
  a.k = k;
  a.swa = swa;
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
  if (p.nsplit > 1) {
    size_t need = csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window);
    if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    uintptr_t w0 = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
    a.ws_o = (float*)w0;
    a.ws_ml = a.ws_o + (size_t)p.nsplit * n_q * n_heads * kD;
  }
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(k_attn, dim3((unsigned)p.grid), dim3(kAttnThreads), 0, st, a);
  int rc = csa2_check_launch();
  if (rc != CSA2_OK || p.nsplit == 1) return rc;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(n_q * n_heads)), dim3(128), 0, st, a);
  return csa2_check_launch();
}
