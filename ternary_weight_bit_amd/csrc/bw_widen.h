// Operand widening for the BitLinear contractions (gfx950 MFMA operands).
//
// The order of k inside one matrix instruction is free as long as the two
// operands agree; the packed weight layout puts each ternary code in the slot
// that lines up with the widened activation byte or nibble of the same k:
//   * INT4 codes -> int8 bytes of 16*q (nibble moved to the high half);
//   * ternary codes -> int8 bytes of 64*t (code moved to bits 7..6:
//     00 -> 0, 01 -> 64, 11 -> -64);
//   * INT8 codes are used as they are;
//   * e2m1 codes are used as they are; ternary codes become e2m1 +-2.0 (the
//     code moved to bits 3..2 of a nibble: sign and high exponent bit), and the
//     MFMA's block scale for the weight operand is 2^-1, so the products are
//     exactly v * t.
//   * INT4 values stored as e2m3 (fp6) fields are used as they are against the
//     same e2m1 weights: a field holds sign and |q| as a 5-bit magnitude, which
//     e2m3 reads as |q| / 8 (the subnormal and first normal binade are evenly
//     spaced by 1/8); the activation operand's block scale 2^3 restores q, so
//     the products are exactly q * t and the fp32 sums are exact integers.
#pragma once

#include "bw_device.h"

namespace bw {

constexpr uint32_t kHiNib = 0xF0F0F0F0u;
constexpr uint32_t kTopBits = 0xC0C0C0C0u;

enum { MODE_INT4 = 0, MODE_FP4 = 1, MODE_INT8 = 2, MODE_E2M3 = 3 };

// Right shift that turns an int8-MFMA accumulator back into sum q*t:
// INT4 operands carry 16*q and 64*t (x1024), INT8 operands carry q and 64*t (x64).
template <int MODE>
constexpr int acc_shift() {
  return MODE == MODE_INT4 ? 10 : 6;
}

// 16 INT4 codes (two words, even k in the low nibble) -> int8 operand of 16*q;
// byte p = 4d + b holds k offset (d >= 2 ? 8 : 0) + 2b + (d & 1).
__device__ __forceinline__ v4i widen_int4(uint32_t x0, uint32_t x1) {
  v4i r;
  r[0] = static_cast<int>((x0 << 4) & kHiNib);
  r[1] = static_cast<int>(x0 & kHiNib);
  r[2] = static_cast<int>((x1 << 4) & kHiNib);
  r[3] = static_cast<int>(x1 & kHiNib);
  return r;
}

// Ternary word in A4 slot order -> int8 operand of 64*t matching widen_int4.
__device__ __forceinline__ v4i widen_w_a4(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>((w << 6) & kTopBits);
  r[1] = static_cast<int>((w << 2) & kTopBits);
  r[2] = static_cast<int>((w << 4) & kTopBits);
  r[3] = static_cast<int>(w & kTopBits);
  return r;
}

// Ternary word in A8 slot order -> int8 operand of 64*t, byte p holding k offset p.
__device__ __forceinline__ v4i widen_w_a8(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>((w << 6) & kTopBits);
  r[1] = static_cast<int>((w << 4) & kTopBits);
  r[2] = static_cast<int>((w << 2) & kTopBits);
  r[3] = static_cast<int>(w & kTopBits);
  return r;
}

// Ternary word in A4 slot order -> two words of e2m1 nibbles: `lo` holds k
// offsets 0..7, `hi` 8..15 (nibble j of each = offset j of its half).  The
// code already sits in two bits of a nibble; moved to bits 3..2 it reads as
// e2m1: 01 (+1) -> 0b0100 (+2.0), 11 (-1) -> 0b1100 (-2.0), 00 -> 0.
// The weight operand's MFMA scale kE2m1WeightScale halves it back.
constexpr int kE2m1WeightScale = 126;  // E8M0 block scale 2^(126 - 127)
__device__ __forceinline__ void widen_w_e2m1(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = (w << 2) & 0xCCCCCCCCu;
  hi = w & 0xCCCCCCCCu;
}

__device__ __forceinline__ v4i as_v4i(uint4 x) {
  v4i r;
  r[0] = static_cast<int>(x.x);
  r[1] = static_cast<int>(x.y);
  r[2] = static_cast<int>(x.z);
  r[3] = static_cast<int>(x.w);
  return r;
}

// e2m1 operand (32 codes, 4 words) for the scaled f8f6f4 MFMA; upper words unused.
__device__ __forceinline__ v8i fp4_operand(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v8i r;
  r[0] = static_cast<int>(a);
  r[1] = static_cast<int>(b);
  r[2] = static_cast<int>(c);
  r[3] = static_cast<int>(d);
  r[4] = 0;
  r[5] = 0;
  r[6] = 0;
  r[7] = 0;
  return r;
}

// e2m3 operand: 32 fields of 6 bits (value j at bits 6j..6j+5 of the six
// words), given as the first 16 and the last 8 bytes; upper words unused.
constexpr int kE2m3ActScale = 130;  // E8M0 block scale 2^(130 - 127): field |q| / 8 -> q
__device__ __forceinline__ v8i fp6_operand(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t e,
                                           uint32_t f) {
  const v8i r = {static_cast<int>(a), static_cast<int>(b), static_cast<int>(c), static_cast<int>(d),
                 static_cast<int>(e), static_cast<int>(f), 0, 0};
  return r;
}

// Ternary words w0 (k 0..15) and w1 (k 16..31) -> e2m1 operand for 32 k.
__device__ __forceinline__ v8i fp4_weights(uint32_t w0, uint32_t w1) {
  uint32_t a, b, c, d;
  widen_w_e2m1(w0, a, b);
  widen_w_e2m1(w1, c, d);
  return fp4_operand(a, b, c, d);
}

// Epilogue value y = fl(fl(acc * sx) * beta).
__device__ __forceinline__ float dequant(float acc, float sx, float beta) {
  return mul_rn(mul_rn(acc, sx), beta);
}

}  // namespace bw
