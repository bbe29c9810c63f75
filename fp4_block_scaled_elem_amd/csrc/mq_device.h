// mq_device.h - device-side helpers shared by the NVFP4 kernels (gfx950).
//
// NVFP4 as used by the prefill path of "Mix-Quant: Quantized Prefilling,
// Precise Decoding for Agentic LLMs" (gist.science English explainer,
// Technical Summary s.2, Hybrid Precision Strategy): a scale per 16-element
// group plus a tensor-level scale, elements rounded to nearest.  Formats:
// E2M1 elements, OCP E4M3 ("fn") group scales, binary32 tensor scale
// s_t = amax / 2688.  Every floating-point result here is the correctly
// rounded binary32 result of the operation it stands for (the library is
// built with -ffp-contract=off and with correctly rounded division), so
// results are bit-reproducible; where a cheaper instruction sequence gives
// that same result, the comment beside it says why.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kGroup = 16;          // elements per local (E4M3) scale
constexpr float kTensorDiv = 2688.0f;  // 6 (E2M1 max) * 448 (E4M3 max)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte streaming load (data read once: do not keep it in the caches).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// max over the two bf16 magnitudes of a word, as a 15-bit integer.  For
// non-negative finite floats the bit pattern orders like the value.
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

// max over the bf16 magnitudes of n words (packed 16-bit maxima, one
// instruction per word, then one across the two halves).
template <int N>
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t* w) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
  const uint32_t lo = m[0], hi = m[1];
  return lo > hi ? lo : hi;
}

// Nearest E4M3 byte to rho >= 0, ties to even, saturating at 448 (0x7E),
// subnormals (multiples of 2^-9) kept; NaN -> 0x7E.  This is the hardware
// fp32 -> fp8 conversion (OCP E4M3 on gfx950) of min(rho, 448) (minNum: a
// NaN rho gives 448).  tests/test_gpu_codecs.py runs this function on every
// non-negative binary32 pattern (finite, +inf and NaN) and compares it with
// the oracle's E4M3 rounding.
__device__ __forceinline__ uint32_t e4m3_from_f32(float rho) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(rho, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// Exact binary32 value of an E4M3 byte (0x00..0x7E).
__device__ __forceinline__ float e4m3_to_f32(uint32_t s) {
  uint32_t e = s >> 3, m = s & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// E2M1 magnitude index of |y|: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
// even index, saturating; NaN -> 0.  Each comparison is one threshold, '>'
// where the tie goes down to an even index and '>=' where it goes up.
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
  float t = __builtin_fabsf(y);
  return (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) +
         (uint32_t)(t >= 1.75f) + (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) +
         (uint32_t)(t > 5.0f);
}

// Tensor scale from the absolute maximum's bit pattern.
__device__ __forceinline__ float tensor_scale_from_amax(uint32_t amax_bits) {
  float a = __uint_as_float(amax_bits);
  return a > 0.0f ? a / kTensorDiv : 1.0f;
}

// Codes of 8 bf16 values (4 words, element 2i in the low half of word i)
// under the reciprocal scale e: byte i = code(2i) | code(2i+1) << 4.
// The hardware fp32->fp4 conversion (scale 1: no extra power of two) rounds
// y = x*e to the nearest E2M1 value with ties to the even code, saturates at
// 6 and keeps the sign of y; that equals e2m1_mag(y) | signbit(x) << 3 for
// every non-NaN binary32 y (tests/test_gpu_codecs.py runs this function on
// all of them and compares with the oracle's E2M1 rounding).  y is NaN only
// for x = +-0 with e = +inf (a group scale whose
// reciprocal overflows); those elements get the sign-only code, as
// e2m1_mag(NaN) = 0 prescribes.  That fix-up is compiled in only with OVF,
// which callers select when the tensor scale is small enough for some
// reciprocal to overflow (GroupScaleTab::ovf).
template <bool OVF>
__device__ __forceinline__ uint32_t encode8(const uint32_t w[4], float e) {
  uint32_t c = w[0];  // any value: the four conversions overwrite all four bytes
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[0]) * e, bf16_hi(w[0]) * e, 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[1]) * e, bf16_hi(w[1]) * e, 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[2]) * e, bf16_hi(w[2]) * e, 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[3]) * e, bf16_hi(w[3]) * e, 1.0f, 3);
  if (OVF && e > 3.0e38f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((w[i] & 0x7FFFu) == 0) c = (c & ~(0xFu << (8 * i))) | (((w[i] >> 15) & 1u) << (8 * i + 3));
      if ((w[i] & 0x7FFF0000u) == 0) c = (c & ~(0xF0u << (8 * i))) | ((w[i] >> 31) << (8 * i + 7));
    }
  }
  return c;
}

// 1 / (value(S) * s_t) for one E4M3 byte S, 0 when that product is 0: the
// reciprocal group scale, tabulated per workgroup for the tensor scale s_t.
__device__ __forceinline__ float group_recip(uint32_t S, float s_t) {
  const float d = e4m3_to_f32(S) * s_t;
  return d > 0.0f ? 1.0f / d : 0.0f;
}

// Per-tensor constants of the group-scale computation: inv = RN64(1 / s_t),
// the table recip[S] = group_recip(S, s_t) for S = 0..127 (entry 127, not an
// E4M3 finite value, is never selected for a valid s_t; it is filled so that
// every index is defined), and ovf: whether some entry lies in the range
// where encode8 needs its fix-up (an OR over the table: with a subnormal s_t
// the smallest scales give d = 0 and a zero entry while larger ones still
// overflow).  Every thread of the block (kBlock threads, a compile-time
// constant: blockDim would be a memory load) must call this; it ends with a
// barrier, after which the table is complete.
struct GroupScaleTab {
  double inv;
  const float* recip;  // LDS
  bool ovf;
};
template <int kBlock>
__device__ __forceinline__ GroupScaleTab group_scale_tab(float s_t, float* recip_lds) {
  int big = 0;
  for (int i = threadIdx.x; i < 128; i += kBlock) {
    const float r = group_recip((uint32_t)i, s_t);
    recip_lds[i] = r;
    big |= r > 3.0e38f;
  }
  // uniform by construction; readfirstlane lets the compiler branch on it
  // with a scalar test
  const bool ovf = __builtin_amdgcn_readfirstlane(__syncthreads_or(big)) != 0;
  return GroupScaleTab{1.0 / (double)s_t, recip_lds, ovf};
}

// Group scale of a group whose absolute maximum has the bf16 magnitude bits
// am: returns the E4M3 byte S of rho = (a / 6) / s_t (both divisions
// correctly rounded binary32) and sets e = 1 / (value(S) * s_t).
// The divisions are exact-rounding products: for binary32 x and y != 0,
// rounding the binary64 product x * RN64(1/y) to binary32 gives RN32(x / y),
// since a binary32 quotient that is not representable lies at least about
// 2^-48 of its size from every binary32 rounding midpoint, well beyond the
// product's 2^-52 error, and the quotient is a midpoint only when y is a
// power of two, where the product is exact.
__device__ __forceinline__ uint32_t group_scale(uint32_t am, const GroupScaleTab& tab, float& e) {
  const float a = __uint_as_float(am << 16);
  const float q = (float)((double)a * (1.0 / 6.0));
  const float rho = (float)((double)q * tab.inv);
  const uint32_t S = e4m3_from_f32(rho);
  e = tab.recip[S & 0x7Fu];  // S <= 0x7E for a finite positive s_t
  return S;
}

// Quantize one group of 16 bf16 values (8 words).  Writes 8 code bytes (two
// words, even element in the low nibble) and returns the E4M3 scale byte.
template <bool OVF>
__device__ __forceinline__ uint32_t quantize_group16(const uint32_t w[8], const GroupScaleTab& tab,
                                                     uint32_t& codes_lo, uint32_t& codes_hi) {
  float e;
  const uint32_t S = group_scale(bf16_absmax_bits<8>(w), tab, e);
  codes_lo = encode8<OVF>(w, e);
  codes_hi = encode8<OVF>(w + 4, e);
  return S;
}

// A compile-time bool passed to generic lambdas, which then instantiate one
// copy of their body per value.
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// 8 E2M1 codes (one dword) times the group scale -> 8 exact binary16 values.
// The hardware conversion yields the E2M1 values themselves (its scale
// operand only applies a power of two, so it is left at 1); one packed
// binary16 multiply per pair applies the E4M3 group scale exactly.  With
// sigma_pair below, checked for every (scale byte, code) pair against the
// oracle's decoded values in tests/test_gpu_codecs.py.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, _Float16 sigma) {
  const half2_t s = {sigma, sigma};
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// Two E4M3 scale bytes of a dword (bytes 0,1, or 2,3 with HIGH) as a
// binary16 pair, in one hardware fp8 -> f16 conversion (its scale operand at
// 1 = 2^0).  Every E4M3 value, normal or subnormal, is a normal binary16
// value, so the conversion is exact.
template <bool HIGH>
__device__ __forceinline__ half2_t sigma_pair(uint32_t scale_dword) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_dword, 1.0f, HIGH);
}

}  // namespace mq
