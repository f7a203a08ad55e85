// csa2_sparse_attn: attention of each query over its selected main-KV entries (FP4,
// dequantised exactly) and its sliding window (FP8) in one softmax
// ([W] "CSA2：跨层复用，能借就不自己算", "FP4 与 SWA Bounded Replay";
//  [J] "缓存压缩真的是越大越好吗").
//
// Per query the key set is at most k + window = 640 entries of 512 channels with V = K,
// contracted against 64 heads: two dense 64 x 640 x 512 products, the only dense
// contractions of the step, so they run on matrix cores.
//
// Workgroup = (query, group of 64 heads, slice of the key list); 4 waves, 16 heads each.
// Keys are processed in tiles of 32:
//   gather:  the 256 threads fetch the 32 entries (main KV: 4 code bytes + 1 E4M3 scale
//            per 8 channels; window: 8 E4M3 bytes) and dequantise them exactly, writing
//            K as bf16 rows [key][channel] and V^T as fp16 rows [channel][key] into LDS
//            (E2M1 x E4M3 has <= 6 significant bits and lies in [2^-10, 2688], so both
//            encodings are exact).
//   S^T = K Q^T  with V_MFMA_F32_16X16X32_BF16 (Q held in registers as the B operand);
//            each lane ends with 8 logits of one head, so the online-softmax statistics
//            of a head live in the 4 lanes that share its column.
//   O^T += V^T P^T with V_MFMA_F32_16X16X32_F16; P is rounded to fp16 (11 significant
//            bits), the key order inside the MFMA's K dimension is permuted identically
//            on both operands so P never leaves registers.
// When a query's keys are split over several workgroups, each writes (O, m, l) and a
// small combine kernel merges them with the log-sum-exp rule.
#include "device.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kTile = 32;
constexpr int kD = 512;
constexpr int kKRow = kD * 2 + 16;       // bytes per K row in LDS (bf16 + 16 B pad)
constexpr int kVRow = kTile * 2 + 8;     // bytes per V^T row in LDS (fp16 + 8 B pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
  int nsplit, tiles_per_split, n_tiles, head_groups;
};

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(kAttnThreads) void k_attn(AttnArgs a) {
  const int q = blockIdx.x / a.head_groups;
  const int hg = blockIdx.x % a.head_groups;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int head = hg * 64 + wave * 16 + col;
  const bool active = hg * 64 + wave * 16 < a.n_heads;  // n_heads % 16 == 0

  __shared__ __attribute__((aligned(16))) uint8_t klds[kTile * kKRow];
  __shared__ __attribute__((aligned(16))) uint8_t vlds[kD * kVRow];
  __shared__ int s_valid[kTile];

  const int seq = a.q_seq[q];
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  const int64_t t = a.q_pos[q], s = a.replay_start[q];
  const int64_t lo = s > t - a.window + 1 ? s : t - a.window + 1;
  const int64_t n_swa = seq_ok && t >= lo ? t - lo + 1 : 0;
  const int64_t swa_b = seq_ok ? a.swa_base[seq] : 0;

  // Q of this lane's head as the B operand: 16 steps of 8 channels (32*s + 8*g ..)
  v8bf qreg[16];
  if (active) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)q * a.n_heads + head) * kD);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      uint4 v = qp[st * 4 + g];
      qreg[st] = *reinterpret_cast<v8bf*>(&v);
    }
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v4f o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int tile_lo = split * a.tiles_per_split;
  int tile_hi = tile_lo + a.tiles_per_split;
  tile_hi = tile_hi < a.n_tiles ? tile_hi : a.n_tiles;

  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    // ---- gather + exact dequant of 32 keys into LDS ----
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = tid + kAttnThreads * it;
      const int dc = item & 63;   // 8-channel chunk
      const int kg = item >> 6;   // group of 4 keys
      float v[4][8];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int slot = tile * kTile + kg * 4 + kk;
        bool valid = false;
        if (seq_ok && slot < a.k) {
          const int32_t p = a.idx[(int64_t)q * a.k + slot];
          if (p >= 0 && p < a.seq_cap) {
            valid = true;
            const int64_t row = (int64_t)seq * a.seq_cap + p;
            const uint32_t c = *reinterpret_cast<const uint32_t*>(a.kv_codes + row * (kD / 2) + dc * 4);
            const float sc = e4m3_val(a.kv_scales[row * (kD / 16) + (dc >> 1)]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[kk][i] = e2m1_val((c >> (4 * i)) & 15u) * sc;
          }
        } else if (slot >= a.k && slot - a.k < n_swa) {
          valid = true;
          const int64_t p = lo + (slot - a.k);
          int64_t r = (p - swa_b) % a.swa_cap;
          r = r < 0 ? r + a.swa_cap : r;
          const uint2 c = *reinterpret_cast<const uint2*>(a.swa + ((int64_t)seq * a.swa_cap + r) * kD + dc * 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[kk][i] = e4m3_val((c.x >> (8 * i)) & 255u);
            v[kk][4 + i] = e4m3_val((c.y >> (8 * i)) & 255u);
          }
        }
        if (!valid) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[kk][i] = 0.0f;
        }
        if (dc == 0) s_valid[kg * 4 + kk] = valid;
        // K row (bf16, 8 channels)
        uint4 kb;
        kb.x = exact_bf16_bits(v[kk][0]) | ((uint32_t)exact_bf16_bits(v[kk][1]) << 16);
        kb.y = exact_bf16_bits(v[kk][2]) | ((uint32_t)exact_bf16_bits(v[kk][3]) << 16);
        kb.z = exact_bf16_bits(v[kk][4]) | ((uint32_t)exact_bf16_bits(v[kk][5]) << 16);
        kb.w = exact_bf16_bits(v[kk][6]) | ((uint32_t)exact_bf16_bits(v[kk][7]) << 16);
        *reinterpret_cast<uint4*>(klds + (kg * 4 + kk) * kKRow + dc * 16) = kb;
      }
      // V^T rows (fp16, 4 keys per channel)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v4h hv = {(_Float16)v[0][i], (_Float16)v[1][i], (_Float16)v[2][i], (_Float16)v[3][i]};
        *reinterpret_cast<v4h*>(vlds + (dc * 8 + i) * kVRow + kg * 8) = hv;
      }
    }
    __syncthreads();

    if (active) {
      // ---- S^T = K Q^T: lane holds keys rt*16 + 4g + r of head `col` ----
      v4f st[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const uint8_t* kr = klds + (rt * 16 + col) * kKRow + g * 16;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
          v8bf av = *reinterpret_cast<const v8bf*>(kr + s2 * 64);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s2], acc, 0, 0, 0);
        }
        st[rt] = acc;
      }
      float x[8];
      float mt = -__builtin_inff();
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = rt * 16 + 4 * g + r;
          float xv = s_valid[key] ? st[rt][r] * a.scale_log2 : -__builtin_inff();
          x[rt * 4 + r] = xv;
          mt = fmaxf(mt, xv);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const bool none = m_new == -__builtin_inff();
      const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
      _Float16 ph[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p = none ? 0.0f : __builtin_amdgcn_exp2f(x[i] - m_new);
        psum += p;
        ph[i] = (_Float16)p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      v8h pb = {ph[0], ph[1], ph[2], ph[3], ph[4], ph[5], ph[6], ph[7]};
      // ---- O^T += V^T P^T over 32 channel tiles ----
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const uint8_t* vr = vlds + (dt * 16 + col) * kVRow;
        v4h lo4 = *reinterpret_cast<const v4h*>(vr + g * 8);
        v4h hi4 = *reinterpret_cast<const v4h*>(vr + 32 + g * 8);
        v8h av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        v4f acc = o[dt] * alpha;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!active) return;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = l_tot + __shfl_xor(l_tot, 32);

  if (a.nsplit == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t ob = ((int64_t)q * a.n_heads + head) * kD;
    if (a.out_dtype == CSA2_DT_F32) {
      float* out = reinterpret_cast<float*>(a.out) + ob;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt)
        *reinterpret_cast<float4*>(out + dt * 16 + 4 * g) =
            make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ob;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        uint2 pk;
        pk.x = f32_to_bf16_rne(o[dt][0] * inv) | (f32_to_bf16_rne(o[dt][1] * inv) << 16);
        pk.y = f32_to_bf16_rne(o[dt][2] * inv) | (f32_to_bf16_rne(o[dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + dt * 16 + 4 * g) = pk;
      }
    }
    if (a.lse && g == 0)
      a.lse[(int64_t)q * a.n_heads + head] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
  } else {
    const int64_t pb = ((int64_t)split * a.n_q + q) * a.n_heads + head;
    float* wo = a.ws_o + pb * kD;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<float4*>(wo + dt * 16 + 4 * g) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
      a.ws_ml[pb * 2] = m_run;
      a.ws_ml[pb * 2 + 1] = l_tot;
    }
  }
}

// merge the per-split (O, m, l) of one (query, head): 128 threads x 4 channels
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a) {
  const int qh = blockIdx.x;  // q * n_heads + h
  const int tid = threadIdx.x;
  float M = -__builtin_inff();
  for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, a.ws_ml[((int64_t)sp * a.n_q * a.n_heads + qh) * 2]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -__builtin_inff()) {
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const int64_t pb = (int64_t)sp * a.n_q * a.n_heads + qh;
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
  int head_groups, n_tiles, tiles_per_split, nsplit;
};

static AttnPlan plan(int n_q, int n_heads, int k, int window) {
  AttnPlan p;
  p.head_groups = (n_heads + 63) / 64;
  p.n_tiles = (k + window + kTile - 1) / kTile;
  if (p.n_tiles < 1) p.n_tiles = 1;
  int64_t wgs = (int64_t)n_q * p.head_groups;
  int want = (int)((512 + wgs - 1) / (wgs > 0 ? wgs : 1));
  want = want < 1 ? 1 : (want > p.n_tiles ? p.n_tiles : want);
  p.tiles_per_split = (p.n_tiles + want - 1) / want;
  p.nsplit = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attn_workspace_bytes(int n_q, int n_heads, int dim, int k, int window) {
  if (n_q <= 0 || n_heads <= 0 || dim != kD || k < 0 || window < 1) return 0;
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
  if (n_q < 0 || n_heads < 16 || n_heads > 256 || n_heads % 16 || dim != kD || seq_cap < 0 || n_seq < 1 || k < 0 ||
      k > CSA2_MAX_TOPK || window < 1 || window > CSA2_MAX_WINDOW || swa_cap < window)
    return CSA2_ERR_SHAPE;
  if (out_dtype != CSA2_DT_F32 && out_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv_codes) || !aligned16(swa) || !aligned16(out)) return CSA2_ERR_SHAPE;
  if (n_q == 0) return CSA2_OK;
  AttnPlan p = plan(n_q, n_heads, k, window);
  if ((int64_t)n_q * p.head_groups > 0x7fffffffLL) return CSA2_ERR_SHAPE;
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
  a.head_groups = p.head_groups;
  if (p.nsplit > 1) {
    size_t need = csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window);
    if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    uintptr_t w0 = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
    a.ws_o = (float*)w0;
    a.ws_ml = a.ws_o + (size_t)p.nsplit * n_q * n_heads * kD;
  }
  hipStream_t st = (hipStream_t)stream;
  dim3 grid((unsigned)(n_q * p.head_groups), (unsigned)p.nsplit);
  hipLaunchKernelGGL(k_attn, grid, dim3(kAttnThreads), 0, st, a);
  int rc = csa2_check_launch();
  if (rc != CSA2_OK || p.nsplit == 1) return rc;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(n_q * n_heads)), dim3(128), 0, st, a);
  return csa2_check_launch();
}
