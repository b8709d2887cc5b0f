// Device helpers for OCP microscaling (MX) formats on gfx950.
//
// Formats (mxfp6-sm120 page, "Execution model": E4M3 activations and E3M2
// weights with a UE8M0 scale per 32 K values; TokenSpeed SiTU page,
// "Supported contract": MXFP4 E2M1 weights).  Field widths and biases are the
// OCP MX v1.0 ones: E2M1 bias 1, E3M2 bias 3, E4M3 bias 7 (no infinities,
// S.1111.111 is NaN), E8M0 = 2**(c-127).
//
// Encoding is done on the integer bits of fp32 values so that the result is
// exactly "nearest element value, ties to the even code, saturate to the
// largest finite value" for every finite input.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mx.h"

namespace moe_mx {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Element format parameters: exponent bits, mantissa bits, bias, largest
// finite magnitude code, emax (exponent of the largest finite value) and the
// format operand code of the gfx950 scaled MFMA (0 = E4M3, 3 = E3M2, 4 = E2M1).
template <int FMT> struct Fmt;
template <> struct Fmt<1> { static constexpr int EB = 2, MB = 1, BIAS = 1, MAXC = 7,   EMAX = 2, BITS = 4, MFMA = 4; };
template <> struct Fmt<2> { static constexpr int EB = 3, MB = 2, BIAS = 3, MAXC = 31,  EMAX = 4, BITS = 6, MFMA = 3; };
template <> struct Fmt<3> { static constexpr int EB = 4, MB = 3, BIAS = 7, MAXC = 126, EMAX = 8, BITS = 8, MFMA = 0; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round half to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 code -> fp32 2**(c-127); code 0 is the fp32 subnormal 2**-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return c ? __uint_as_float(c << 23) : __uint_as_float(0x00400000u);
}

// Shared exponent of a block from the bits of its largest magnitude:
// clamp(floor(log2 amax) - emax, -127, 127); zero and fp32-subnormal maxima
// give -127 (their floor(log2) is below -126, and emax >= 2).
template <int FMT>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  int E = (int)(amax_bits >> 23);
  if (E == 0) return -127;
  int s = E - 127 - Fmt<FMT>::EMAX;
  return s < -127 ? -127 : s;  // E <= 254 keeps s <= 127 - emax
}

// 2**-s as an exact fp32 (|s| <= 127 and s <= 125 in use, so always normal).
__device__ __forceinline__ float exp2_neg(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }

// Nearest element code of q (already divided by the block scale).
template <int FMT>
__device__ __forceinline__ uint32_t encode(float q) {
  using F = Fmt<FMT>;
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 31) << (F::EB + F::MB);
  const uint32_t mag = u & 0x7fffffffu;
  const int E = (int)(mag >> 23);
  if (E == 0) return sign;  // |q| < 2**-126: far below half of the smallest subnormal
  const int e = E - 127;
  const uint32_t sig = (mag & 0x7fffffu) | 0x800000u;  // 1.m * 2**23
  constexpr int emin = 1 - F::BIAS;
  const int shift = 23 - F::MB + (e < emin ? emin - e : 0);
  if (shift > 25) return sign;  // below a quarter of the smallest subnormal
  uint32_t kept = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  kept += (rem > half || (rem == half && (kept & 1u))) ? 1u : 0u;
  uint32_t code = (e < emin) ? kept : ((uint32_t)(e + F::BIAS) << F::MB) + kept - (1u << F::MB);
  code = code > (uint32_t)F::MAXC ? (uint32_t)F::MAXC : code;
  return code | sign;
}

// E4M3 codes (bytes 0 and 1) of two values already divided by their block
// scale, by the hardware conversion: nearest, ties to even, signed zeros kept,
// the same as encode<3>; the conversion turns magnitudes past 448 into NaN
// instead of saturating, hence the clamp first.  The scale operand 1.0 leaves
// the values as they are.
typedef short v2s16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  const v2s16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s16){0, 0}, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

// SiLU(g) * u in fp32.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Gated activations of FC1's two halves (b12x page, "What's in here", MoE:
// SiLU, ReLU2 and SwiGLU-OAI), in fp32; `fn` is a moe_act_fn_t value and is
// uniform across a launch.
//   SiLU        SiLU(g) * u
//   ReLU2       max(g, 0)^2 * u
//   SwiGLU-OAI  (clamp(u, -7, 7) + 1) * g' * sigmoid(1.702 g'), g' = min(g, 7)
constexpr float kOaiLimit = 7.0f;
constexpr float kOaiAlpha = 1.702f;
__device__ __forceinline__ float gated_act(int fn, float g, float u) {
  if (fn == MOE_FN_RELU2) {
    const float r = fmaxf(g, 0.0f);
    return r * r * u;
  }
  if (fn == MOE_FN_SWIGLU_OAI) {
    const float gc = fminf(g, kOaiLimit);
    const float uc = fminf(fmaxf(u, -kOaiLimit), kOaiLimit);
    return (uc + 1.0f) * (gc / (1.0f + expf(-kOaiAlpha * gc)));
  }
  return silu_mul(g, u);
}

// SiLU(g) * u with the hardware exp2 and reciprocal (about 2 ulp in fp32;
// the result is then rounded to E4M3, 3 mantissa bits).
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504f)) * u;
}
// the gated activation, fixed per instantiation (a run-time choice in this
// epilogue made the compiler spill registers in the step loop): SiLU as
// above, the other forms as in every other kernel
template <int ACT>
__device__ __forceinline__ float act_mul(float g, float u) {
  return ACT == MOE_FN_SILU ? silu_mul_fast(g, u) : gated_act(ACT, g, u);
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xf, 0xf, true));  // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, true));  // row_ror 8
  return v;
}

}  // namespace moe_mx
