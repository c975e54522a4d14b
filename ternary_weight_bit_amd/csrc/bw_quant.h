// 4-bit activation codes shared by the standalone quantizer and the fused
// quantize + GEMV kernel, so both produce the same bytes.  INT4 values can also
// be stored as e2m3 (fp6) fields, the operand of the f8f6f4 matrix instruction.
//
// BitNet a4.8 abstract: 4-bit activations (INT4/FP4) at the inputs of attention
// and FFN; toshoseti review «Метод»: FP4 as the wider-range alternative.
// Per token: a' = max(max|x|, 1e-5); INT4: t = fl(x * fl(7/a')), code =
// clamp(rne(t), -8, 7); e2m1: t = fl(x * fl(6/a')), nearest of
// {0,.5,1,1.5,2,3,4,6} with ties to the even code, saturating, sign of t.
#pragma once

#include "bw_device.h"

namespace bw {

// INT4 code clamp(rne(t), -8, 7) as a 4-bit field, for |t| <= 7.5 (always the
// case for an absmax scale: |x * fl(7/a')| <= 7 (1 + 2^-24)): adding 1.5 * 2^23
// rounds t to an integer with ties to even, and the low 4 bits of the sum are
// that integer in two's complement; the clamp can never act.
__device__ __forceinline__ uint32_t int4_code_absmax(float t) {
  return __float_as_uint(t + 12582912.0f) & 0xFu;
}

// FMT 0 = INT4: the code of one element given inv = fl(qmax / a').
template <int FMT>
__device__ __forceinline__ uint32_t act4_code(float x, float inv) {
  static_assert(FMT == 0, "e2m1 codes come in words (act4_word), e2m3 fields in streams (e2m3_input)");
  return int4_code_absmax(mul_rn(x, inv));
}

// INT4 values stored as 6-bit e2m3 fields (bit 5 the sign, clear for 0; bits
// 4..0 the magnitude |q|, which e2m3 reads as |q| / 8) come from the f32 -> fp6
// conversion of t / 8: q / 8 lies on e2m3's subnormal grid (step 1/8), so
// nearest with ties to even gives the field of rne(t).  rne(|t|) is 0 exactly
// when |t| <= 0.5, i.e. for bit patterns of t up to that of -0.5 (0xBF000000)
// read as unsigned among the negatives; such a t is passed as |t| so that its
// zero field has the sign clear.
__device__ __forceinline__ float e2m3_input(float t) {
  return __float_as_uint(t) > 0xBF000000u ? t : fabsf(t);
}

// Eight 4-bit codes as one word, element i in nibble i: FMT 0 = INT4, 1 =
// e2m1.  e2m1 is the nearest of {0,.5,1,1.5,2,3,4,6} to t = fl(x * inv), at
// a midpoint the neighbour with the even code, saturating at 6, with the sign
// bit of t (zeros included); the f32 -> fp4 conversion instruction (scale 1)
// rounds exactly so, two elements per instruction into one byte of the word.
template <int FMT>
__device__ __forceinline__ uint32_t act4_word(const float (&x)[8], float inv) {
  static_assert(FMT == 0 || FMT == 1, "4-bit codes");
  uint32_t w = 0;
  if constexpr (FMT == 1) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, mul_rn(x[0], inv), mul_rn(x[1], inv), 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, mul_rn(x[2], inv), mul_rn(x[3], inv), 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, mul_rn(x[4], inv), mul_rn(x[5], inv), 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, mul_rn(x[6], inv), mul_rn(x[7], inv), 1.0f, 3);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= act4_code<0>(x[i], inv) << (4 * i);
  }
  return w;
}

template <int FMT>
constexpr float act4_qmax() {
  return FMT == 1 ? 6.0f : 7.0f;
}

}  // namespace bw
