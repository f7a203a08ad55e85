// csa2_quantize_kv: quantise post-RoPE rows to NVFP4 / MXFP4 / FP8 and scatter them
// into a cache ([W] "FP4 与 SWA Bounded Replay"; [L] 4.3 and 5; OCP MX v1.0).
//
// Every code is the exact round-to-nearest, ties-to-even, of the real value.  E2M1 codes
// compare x against the exact midpoints between neighbouring codes times the scale; FP8
// codes round the fp32 bit pattern directly; the NVFP4 scale code (nearest to amax/6)
// starts from the fp32 quotient and is settled by exact midpoint tests.  All midpoints
// and their products with the scale carry at most 7 significant bits, so every comparison
// is exact in fp32 and the codes are bit-exact.
//
// One thread quantises one scale group (16 / 32 channels) or, for FP8, 8 channels.
// Consecutive threads take consecutive groups of a row, so a wave reads a contiguous
// stretch of the source.  This runs once per new cache row (one row per sequence per
// decode step), so it is far from any roofline; it is written for exactness first.
#include "device.h"

namespace csa2 {

// An empty asm that takes a group's results as inputs: the arithmetic (and the loads it
// depends on) must then run before the destination check that follows, instead of being
// moved behind it, where the loads would only be issued once the destination row has
// arrived.
__device__ __forceinline__ void keep_before_branch(uint32_t a, uint32_t b, uint32_t c) {
  asm volatile("" ::"v"(a), "v"(b), "v"(c));
}

template <typename T>
__device__ __forceinline__ uint32_t load_bits(const T* p, int64_t i);

template <>
__device__ __forceinline__ uint32_t load_bits<float>(const float* p, int64_t i) {
  return __float_as_uint(p[i]);
}
template <>
__device__ __forceinline__ uint32_t load_bits<uint16_t>(const uint16_t* p, int64_t i) {
  return (uint32_t)p[i] << 16;
}

// ---- NVFP4: one thread per 16-channel group ----
template <bool kMap, typename T>
__device__ __forceinline__ void quant_group_nvfp4(const T* __restrict__ src, int64_t rows, int dim,
                                                  const int64_t* __restrict__ dst_row, int64_t dst_rows,
                                                  uint8_t* __restrict__ codes, int64_t cst,
                                                  uint8_t* __restrict__ scales, int64_t sst, int64_t gid) {
  const int gpr = dim / 16;
  if (gid >= rows * gpr) return;
  int64_t r = gid / gpr;
  int g = (int)(gid % gpr);
  // the destination row is loaded together with the source values and checked only at the
  // stores, so that both loads are one memory round trip
  const int64_t d = kMap ? dst_row[r] : r;
  uint32_t bits[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) bits[i] = load_bits(src, r * dim + g * 16 + i);
  uint32_t lo, hi;
  const int sc = nvfp4_group(bits, lo, hi);
  keep_before_branch(lo, hi, (uint32_t)sc);
  if (d < 0 || d >= dst_rows) return;
  uint2* out = reinterpret_cast<uint2*>(codes + d * cst + g * 8);
  *out = make_uint2(lo, hi);
  scales[d * sst + g] = (uint8_t)sc;
}

// ---- MXFP4: one thread per 32-channel group ----
template <bool kMap, typename T>
__device__ __forceinline__ void quant_group_mxfp4(const T* __restrict__ src, int64_t rows, int dim,
                                                  const int64_t* __restrict__ dst_row, int64_t dst_rows,
                                                  uint8_t* __restrict__ codes, int64_t cst,
                                                  uint8_t* __restrict__ scales, int64_t sst, int64_t gid) {
  const int gpr = dim / 32;
  if (gid >= rows * gpr) return;
  int64_t r = gid / gpr;
  int g = (int)(gid % gpr);
  const int64_t d = kMap ? dst_row[r] : r;   // checked at the stores (see above)
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) bits[i] = load_bits(src, r * dim + g * 32 + i);
  uint32_t w[4];
  const int code = mxfp4_group(bits, w);
  keep_before_branch(w[0] ^ w[1], w[2] ^ w[3], (uint32_t)code);
  if (d < 0 || d >= dst_rows) return;
  uint4* out = reinterpret_cast<uint4*>(codes + d * cst + g * 16);
  *out = make_uint4(w[0], w[1], w[2], w[3]);
  scales[d * sst + g] = (uint8_t)code;
}

// ---- FP8 (E4M3, unscaled): one thread per 8 channels ----
template <bool kMap, typename T>
__device__ __forceinline__ void quant_group_fp8(const T* __restrict__ src, int64_t rows, int dim,
                                                const int64_t* __restrict__ dst_row, int64_t dst_rows,
                                                uint8_t* __restrict__ codes, int64_t cst, int64_t gid) {
  const int gpr = dim / 8;
  if (gid >= rows * gpr) return;
  int64_t r = gid / gpr;
  int g = (int)(gid % gpr);
  const int64_t d = kMap ? dst_row[r] : r;   // checked at the store (see above)
  uint32_t bits[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) bits[i] = load_bits(src, r * dim + g * 8 + i);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = bits[i];
    const uint32_t c = fp8_code_bits(b);
    if (i < 4) lo |= c << (8 * i);
    else hi |= c << (8 * (i - 4));
  }
  keep_before_branch(lo, hi, 0u);
  if (d < 0 || d >= dst_rows) return;
  *reinterpret_cast<uint2*>(codes + d * cst + g * 8) = make_uint2(lo, hi);
}

// one job of a (multi-)quantise launch
struct QuantJob {
  const void* src;
  int64_t rows;
  const int64_t* dst_row;
  int64_t dst_rows;
  uint8_t* codes;
  uint8_t* scales;
  int64_t codes_stride, scales_stride;   // bytes between destination rows
  int dim, fmt, bf16;
  int64_t block0;   // first workgroup of this job
};

struct QuantJobs {
  QuantJob job[CSA2_MAX_QUANT_JOBS];
  int n;
};

template <bool kMap>
__device__ __forceinline__ void quant_dispatch_map(const QuantJob& j, int64_t gid) {
  if (j.fmt == CSA2_FMT_NVFP4) {
    if (j.bf16)
      quant_group_nvfp4<kMap>((const uint16_t*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride,
                              j.scales, j.scales_stride, gid);
    else
      quant_group_nvfp4<kMap>((const float*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride,
                              j.scales, j.scales_stride, gid);
  } else if (j.fmt == CSA2_FMT_MXFP4) {
    if (j.bf16)
      quant_group_mxfp4<kMap>((const uint16_t*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride,
                              j.scales, j.scales_stride, gid);
    else
      quant_group_mxfp4<kMap>((const float*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride,
                              j.scales, j.scales_stride, gid);
  } else {
    if (j.bf16)
      quant_group_fp8<kMap>((const uint16_t*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride, gid);
    else
      quant_group_fp8<kMap>((const float*)j.src, j.rows, j.dim, j.dst_row, j.dst_rows, j.codes, j.codes_stride, gid);
  }
}

// (the row map is a separate instantiation: a load behind a branch on whether the map
// exists would be waited for before the source values are requested)
__device__ __forceinline__ void quant_dispatch(const QuantJob& j, int64_t gid) {
  if (j.dst_row) quant_dispatch_map<true>(j, gid);
  else quant_dispatch_map<false>(j, gid);
}

// Every job of the launch gets its own range of workgroups; a workgroup finds its job by the
// (uniform) range its index falls in.
__global__ __launch_bounds__(256) void k_quant(QuantJobs jobs) {
  int j = 0;
  for (int i = 1; i < jobs.n; ++i)
    if ((int64_t)blockIdx.x >= jobs.job[i].block0) j = i;
  const QuantJob& jb = jobs.job[j];
  quant_dispatch(jb, ((int64_t)blockIdx.x - jb.block0) * blockDim.x + threadIdx.x);
}

static int make_job(const void* src, int src_dtype, int64_t rows, int dim, int fmt, const int64_t* dst_row,
                    int64_t dst_rows, uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                    QuantJob* out, int64_t* blocks) {
  if (fmt != CSA2_FMT_NVFP4 && fmt != CSA2_FMT_MXFP4 && fmt != CSA2_FMT_FP8) return CSA2_ERR_UNSUPPORTED;
  if (src_dtype != CSA2_DT_F32 && src_dtype != CSA2_DT_BF16) return CSA2_ERR_UNSUPPORTED;
  if (rows != 0 && (!src || !codes || (fmt != CSA2_FMT_FP8 && !scales))) return CSA2_ERR_NULL;
  const int group = fmt == CSA2_FMT_NVFP4 ? 16 : (fmt == CSA2_FMT_MXFP4 ? 32 : 8);
  if (rows < 0 || dim <= 0 || dim > 8192 || dim % group || dst_rows < 0) return CSA2_ERR_SHAPE;
  if (rows != 0 && !aligned16(codes)) return CSA2_ERR_SHAPE;
  // destination rows: dense by default; an explicit stride holds the row and keeps the code
  // stores aligned (16-byte stores for MXFP4, 8-byte ones otherwise)
  const int64_t code_row = fmt == CSA2_FMT_FP8 ? dim : dim / 2, scale_row = fmt == CSA2_FMT_FP8 ? 0 : dim / group;
  if (codes_stride == 0) codes_stride = code_row;
  if (scales_stride == 0) scales_stride = scale_row;
  if (codes_stride < code_row || scales_stride < scale_row || codes_stride % (fmt == CSA2_FMT_MXFP4 ? 16 : 8))
    return CSA2_ERR_SHAPE;
  const int64_t work = rows * (dim / group);
  *blocks = (work + 255) / 256;
  if (*blocks > 0x7fffffff) return CSA2_ERR_SHAPE;
  out->src = src;
  out->rows = rows;
  out->dst_row = dst_row;
  out->dst_rows = dst_rows;
  out->codes = codes;
  out->scales = scales;
  out->codes_stride = codes_stride;
  out->scales_stride = scales_stride;
  out->dim = dim;
  out->fmt = fmt;
  out->bf16 = src_dtype == CSA2_DT_BF16;
  return CSA2_OK;
}

static int launch_jobs(QuantJobs& jobs, int64_t total_blocks, hipStream_t st) {
  if (total_blocks == 0) return CSA2_OK;
  if (total_blocks > 0x7fffffff) return CSA2_ERR_SHAPE;
  hipLaunchKernelGGL(k_quant, dim3((unsigned)total_blocks), dim3(256), 0, st, jobs);
  return csa2_check_launch();
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_quantize_kv(const void* src, int src_dtype, int64_t rows, int dim, int fmt,
                                const int64_t* dst_row, int64_t dst_rows, uint8_t* codes, int64_t codes_stride,
                                uint8_t* scales, int64_t scales_stride, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  QuantJobs jobs = {};
  int64_t blocks = 0;
  const int rc = make_job(src, src_dtype, rows, dim, fmt, dst_row, dst_rows, codes, codes_stride, scales,
                          scales_stride, &jobs.job[0], &blocks);
  if (rc != CSA2_OK) return rc;
  jobs.n = 1;
  return launch_jobs(jobs, blocks, (hipStream_t)stream);
}

extern "C" int csa2_quantize_kv_multi(const csa2_quant_job* jobs, int n_jobs, void* stream) {
  if (int rc_status = csa2_take_device_status()) return rc_status;
  if (!jobs) return CSA2_ERR_NULL;
  if (n_jobs < 0 || n_jobs > CSA2_MAX_QUANT_JOBS) return CSA2_ERR_SHAPE;
  QuantJobs kj = {};
  int64_t total = 0;
  for (int i = 0; i < n_jobs; ++i) {
    const csa2_quant_job& j = jobs[i];
    int64_t blocks = 0;
    QuantJob q;
    const int rc = make_job(j.src, j.src_dtype, j.rows, j.dim, j.fmt, j.dst_row, j.dst_rows, j.codes,
                            j.codes_stride, j.scales, j.scales_stride, &q, &blocks);
    if (rc != CSA2_OK) return rc;
    if (blocks == 0) continue;
    q.block0 = total;
    kj.job[kj.n++] = q;
    total += blocks;
  }
  return launch_jobs(kj, total, (hipStream_t)stream);
}
