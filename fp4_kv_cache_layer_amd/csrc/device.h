// Internal device helpers shared by the CSA2 HIP kernels (gfx950 only).
//
// FP4/FP8 encodings follow the OCP MX v1.0 (E2M1, E8M0) and OCP FP8 (E4M3, no
// infinities) definitions: E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; E4M3 bias 7
// with subnormals m*2^-9 and max 448; E8M0 = 2^(c-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// vector loads/stores assume 16-byte aligned bases
__host__ __device__ inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// magnitude of a finite non-negative E4M3 code (0..126), exact in fp32
__device__ __forceinline__ float e4m3_mag(int c) {
  int e = c >> 3, m = c & 7;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((uint32_t)(e + 120) << 23) | ((uint32_t)m << 20));
}

// signed value of any non-NaN E4M3 byte
__device__ __forceinline__ float e4m3_val(uint32_t c) {
  float v = e4m3_mag((int)(c & 0x7f));
  return (c & 0x80) ? -v : v;
}

// signed value of an E2M1 nibble, as fp32 bits (exact)
__device__ __forceinline__ float e2m1_val(uint32_t c) {
  uint32_t m = c & 7;
  uint32_t bits = m >= 2 ? (((m >> 1) + 126u) << 23) | ((m & 1u) << 22) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// E4M3 magnitude code (0..126) nearest to a >= 0 (finite), ties to the even code,
// saturating at 448 (code 126).  Normal range (a >= 2^-6): the fp32 significand is rounded
// to 3 bits, ties to even, on the bit pattern (a carry out of the significand is the next
// binade, as it should be) and the exponent is rebiased from 127 to 7.  Subnormal range:
// the code is a * 2^9 rounded to an integer, ties to even (a * 2^9 is exact); 8 is the
// smallest normal code, so a carry there is also right.
// Both ranges are computed and one is selected, so that the code has no branch (a branch
// here would sit between the loads of a group's values and make them wait one by one).
// Used by the quantiser and by the attention kernel's window append, so both write the
// same bytes.
__device__ __forceinline__ int fp8_mag_code(float a) {
  const int sub = (int)__builtin_rintf(fminf(a, 0x1p-6f) * 512.0f);
  const uint32_t b = __float_as_uint(a);
  int c = (int)((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120 << 3);
  c = c > 126 ? 126 : c;
  return a < 0x1p-6f ? sub : c;
}

// E4M3 byte of a finite fp32 value given as bits (unscaled: nearest code, ties to even,
// saturating at +-448; the sign is kept, so -0 and small negatives give 0x80)
__device__ __forceinline__ uint32_t fp8_code_bits(uint32_t b) {
  return (uint32_t)fp8_mag_code(__uint_as_float(b & 0x7fffffffu)) | ((b >> 24) & 0x80u);
}

// fp32 holding a value exactly representable in bf16 -> bf16 bits (truncation is exact)
__device__ __forceinline__ uint16_t exact_bf16_bits(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }

// E2M1 magnitude code of a/s (a >= 0, s > 0), ties to even, saturating at 6.
// Midpoints between the E2M1 magnitudes: .25 .75 1.25 1.75 2.5 3.5 5.
__device__ __forceinline__ uint32_t e2m1_code(float a, float s) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const float t = s * mids[i];
    // code >= i+1 iff a > t, or a == t and i+1 is even
    c += (a > t) || (a == t && (i & 1));
  }
  return c;
}

// "a/6 rounds to an E4M3 code >= c" for c >= 1: a/6 lies above the midpoint of codes c-1
// and c, or on it with c even.  6 * midpoint = 3 * (v(c-1) + v(c)) is exact in fp32.
__device__ __forceinline__ bool scale_at_least(float a, int c) {
  const float t = 3.0f * (e4m3_mag(c - 1) + e4m3_mag(c));
  return a > t || (a == t && !(c & 1));
}

// E4M3 code nearest to the exact quotient a/6 (a >= 0), ties to even, saturating at 448.
// The correctly rounded fp32 quotient lands on the right code or, when a/6 sits within
// an fp32 ulp of a midpoint, on its neighbour; the exact midpoint tests settle which.
__device__ __forceinline__ int nvfp4_scale_code(float a) {
  int c = fp8_mag_code(a / 6.0f);
  if (c < 126 && scale_at_least(a, c + 1)) ++c;
  else if (c > 0 && !scale_at_least(a, c)) --c;
  return c;
}

// One NVFP4 group: 16 finite fp32 values (as bits; bf16 inputs widened by a shift) -> E4M3
// scale code (returned; nearest to amax/6) and 16 E2M1 codes of x / scale packed as two
// words, channel 2i in the low nibble of byte i (lo: channels 0-7, hi: 8-15).
__device__ __forceinline__ int nvfp4_group(const uint32_t (&bits)[16], uint32_t& lo, uint32_t& hi) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t ab = bits[i] & 0x7fffffffu;  // |x|; integer order == float order for x >= 0
    amax_bits = ab > amax_bits ? ab : amax_bits;
  }
  const int sc = nvfp4_scale_code(__uint_as_float(amax_bits));
  const float s = e4m3_mag(sc);
  lo = hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t mag = s > 0.0f ? e2m1_code(__uint_as_float(bits[i] & 0x7fffffffu), s) : 0u;
    const uint32_t c = mag | ((bits[i] >> 28) & 8u);
    if (i < 8) lo |= c << (4 * i);
    else hi |= c << (4 * (i - 8));
  }
  return sc;
}

// One MXFP4 group: 32 finite fp32 values (as bits; bf16 inputs widened by a shift) ->
// E8M0 scale code (returned) and 32 E2M1 codes packed as four words, channel 2i in the low
// nibble of byte i.  E = floor(log2 amax) - 2 clamped to [-127, 127] (an all-zero group or
// a subnormal amax gives -127).  The codes come from the hardware down-convert with scale
// 2^E (V_CVT_SCALEF32_PK_FP4_F32: x / 2^E rounded to the nearest E2M1 value, ties to the
// even code, saturating at 6, sign kept, -0 included), which gives the same code as
// comparing |x| with the E2M1 midpoints times 2^E (e2m1_code) on every code boundary, the
// floats next to each, the saturation range and scales from 2^-127 to 2^125 (measured on
// this GPU).
__device__ __forceinline__ int mxfp4_group(const uint32_t (&bits)[32], uint32_t (&w)[4]) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t ab = bits[i] & 0x7fffffffu;
    amax_bits = ab > amax_bits ? ab : amax_bits;
  }
  const int e_field = (int)(amax_bits >> 23);
  int E = e_field - 127 - 2;
  E = (amax_bits == 0 || e_field == 0 || E < -127) ? -127 : E;
  const int code = amax_bits == 0 ? 0 : E + 127;
  const float s = ldexpf(1.0f, code - 127);
  w[0] = w[1] = w[2] = w[3] = 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {   // channels 2j (low nibble) and 2j+1 (high nibble) -> byte j
    const uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(bits[2 * j]),
                                                                __uint_as_float(bits[2 * j + 1]), s, 0) & 0xffu;
    w[j >> 2] |= b << (8 * (j & 3));
  }
  return code;
}

// A cache's addressing (see the header's cache layouts): entry e of sequence b has its
// codes at codes + b*cs + e*ce and its scales at scales + b*ss + e*se (bytes).
struct CacheRef {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t ce, cs, se, ss;
};

// Fills the dense default for every stride given as 0 and checks the rest: entry strides at
// least the row size, every stride non-negative, code strides multiples of 16 (16-byte code
// loads), scale strides multiples of scale_align.  Returns a csa2 status.
inline int resolve_cache(CacheRef& c, int64_t seq_cap, int64_t code_row, int64_t scale_row, int scale_align) {
  if (c.ce == 0) c.ce = code_row;
  if (c.se == 0) c.se = scale_row;
  if (c.cs == 0) c.cs = seq_cap * c.ce;
  if (c.ss == 0) c.ss = seq_cap * c.se;
  if (c.ce < code_row || c.se < scale_row || c.cs < 0 || c.ss < 0) return CSA2_ERR_SHAPE;
  if (c.ce % 16 || c.cs % 16 || c.se % scale_align || c.ss % scale_align) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

}  // namespace csa2

// Launch-error bookkeeping used by every entry point (defined in abi.hip).
int csa2_record_hip_error(hipError_t e);
int csa2_check_launch();
// The device status word (device-visible address, nullptr before csa2_init), the bound of
// the attention kernel's partner wait, and the check every compute entry point makes first:
// CSA2_ERR_DEVICE (and the text in csa2_last_error) if a kernel stored a status code.
uint32_t* csa2_status_word();
int csa2_wait_limit();
int csa2_take_device_status();
// Device address of the no-allocation attention entry point's static scratch on the current
// device (looked up once per device; nullptr with *rc set on failure).
void* csa2_attn_scratch(int* rc);
