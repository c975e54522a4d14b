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

// e2m1 code of t: nearest of {0,.5,1,1.5,2,3,4,6}; at a midpoint the
// neighbour with the even code wins; saturates at 6; sign bit from t.
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float m = fabsf(t);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) +
               (m > 5.0f);
  return c | ((__float_as_uint(t) >> 31) << 3);
}

// The INT4 value rne(t) of int4_code_absmax as a 6-bit e2m3 field: bit 5 the
// sign (clear for 0), bits 4..0 the magnitude (e2m3 reads them as |q| / 8).
// rne(|t|) is 0 exactly when |t| <= 0.5, so the sign bit belongs to t < -0.5,
// i.e. to the bit patterns above that of -0.5 (0xBF000000) read as unsigned.
__device__ __forceinline__ uint32_t e2m3_field_absmax(float t) {
  const uint32_t mag = __float_as_uint(fabsf(t) + 12582912.0f) & 0xFu;
  return mag | (__float_as_uint(t) > 0xBF000000u ? 32u : 0u);
}

// FMT 0 = INT4, 1 = e2m1, 2 = INT4 as an e2m3 field: the code of one element
// given inv = fl(qmax / a').
template <int FMT>
__device__ __forceinline__ uint32_t act4_code(float x, float inv) {
  const float t = mul_rn(x, inv);
  return FMT == 0 ? int4_code_absmax(t) : FMT == 1 ? e2m1_code(t) : e2m3_field_absmax(t);
}

template <int FMT>
constexpr float act4_qmax() {
  return FMT == 1 ? 6.0f : 7.0f;
}

}  // namespace bw
