// W1.58A4 / W1.58A8 BitLinear contractions for gfx950.
//
// BitNet a4.8 abstract: ternary-weight layers consume 4-bit activations
// (INT4/FP4 kernels) at the attention/FFN inputs and 8-bit codes of the
// sparsified intermediate states.
//
//   acc[m][n] = sum_k v(code[m][k]) * t[n][k],   y = fl(fl(acc * sx[m]) * beta[n])
//
// Operands are widened in registers right before the matrix instruction:
//   * INT4 codes -> int8 bytes holding 16*q (nibble moved to the high half of
//     its byte: one AND, or one shift and one AND, per 4 codes);
//   * ternary 2-bit codes -> int8 bytes holding 64*t (code moved to bits 7..6
//     of its byte; 00 -> 0, 01 -> 64, 11 -> -64);
//   * INT8 codes are used as they are;
//   * e2m1 codes are used as they are; ternary codes become e2m1 +-1.0
//     (0b0010 / 0b1010) with two shifts, two ANDs and an OR per 8 codes.
// v_mfma_i32_32x32x32_i8 accumulates 1024*acc (INT4) or 64*acc (INT8) exactly
// in int32; v_mfma_scale_f32_32x32x64_f8f6f4 (block scales 2^0) accumulates the
// e2m1 x ternary sums exactly in fp32 (multiples of 1/2 far below 2^24).
//
// The order of k inside a matrix instruction is free as long as both operands
// agree; the packed weight layout (role-specific slot order) is chosen so each
// widened weight byte lines up with the widened activation byte of the same k.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;

constexpr uint32_t kHiNib = 0xF0F0F0F0u;
constexpr uint32_t kTopBits = 0xC0C0C0C0u;

enum { MODE_INT4 = 0, MODE_FP4 = 1, MODE_INT8 = 2 };

// 16 INT4 codes (two words, even k in low nibbles) -> int8 operand of 16*q,
// byte p = 4d + b holding k offset (d >= 2 ? 8 : 0) + 2b + (d & 1).
__device__ __forceinline__ v4i widen_int4(uint32_t x0, uint32_t x1) {
  v4i r;
  r[0] = static_cast<int>((x0 << 4) & kHiNib);
  r[1] = static_cast<int>(x0 & kHiNib);
  r[2] = static_cast<int>((x1 << 4) & kHiNib);
  r[3] = static_cast<int>(x1 & kHiNib);
  return r;
}

// Ternary word, A4 slot order -> int8 operand of 64*t matching widen_int4.
__device__ __forceinline__ v4i widen_w_a4(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>((w << 6) & kTopBits);
  r[1] = static_cast<int>((w << 2) & kTopBits);
  r[2] = static_cast<int>((w << 4) & kTopBits);
  r[3] = static_cast<int>(w & kTopBits);
  return r;
}

// Ternary word, A8 slot order -> int8 operand of 64*t, byte p holding k offset p.
__device__ __forceinline__ v4i widen_w_a8(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>((w << 6) & kTopBits);
  r[1] = static_cast<int>((w << 4) & kTopBits);
  r[2] = static_cast<int>((w << 2) & kTopBits);
  r[3] = static_cast<int>(w & kTopBits);
  return r;
}

// Ternary word, A4 slot order -> two words of e2m1 nibbles: the first holds k
// offsets 0..7, the second 8..15 (nibble j = offset j of its half).
__device__ __forceinline__ void widen_w_e2m1(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = ((w << 1) & 0x22222222u) | ((w << 2) & 0x88888888u);
  hi = ((w >> 1) & 0x22222222u) | (w & 0x88888888u);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_bitlinear(
    const uint8_t* __restrict__ A, const float* __restrict__ sx, int64_t M, int64_t K,
    const uint8_t* __restrict__ Wp, const float* __restrict__ beta, int64_t N,
    float* __restrict__ y, void* __restrict__ acc_dbg) {
  constexpr int ABYTES = (MODE == MODE_INT8) ? 64 : 32;  // bytes of one row per BK
  constexpr int ACHUNKS = BM * ABYTES / 16 / kThreads;   // 16-byte A loads per thread
  __shared__ __attribute__((aligned(16))) uint8_t As[BM * ABYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int li = lane & 31;
  const int lh = lane >> 5;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t nk = K / BK;
  const int64_t a_row_bytes = (MODE == MODE_INT8) ? K : (K >> 1);
  const int64_t kblocks = K / 64;

  uint4 ra[ACHUNKS];
  uint4 rb;
  auto gload = [&](int64_t kb) {
#pragma unroll
    for (int c = 0; c < ACHUNKS; ++c) {
      const int q = tid + c * kThreads;
      const int row = q / (ABYTES / 16);
      const int part = q % (ABYTES / 16);
      const int64_t gm = m0 + row;
      if (gm < M) {
        ra[c] = *reinterpret_cast<const uint4*>(A + gm * a_row_bytes + kb * ABYTES + part * 16);
      } else {
        ra[c] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BN) {
      const int64_t gn = n0 + tid;
      if (gn < N) {
        const int64_t off = ((gn >> 4) * kblocks + kb) * 256 + (gn & 15) * 16;
        rb = *reinterpret_cast<const uint4*>(Wp + off);
      } else {
        rb = make_uint4(0, 0, 0, 0);
      }
    }
  };

  using acc_t = typename std::conditional<MODE == MODE_FP4, v16f, v16i>::type;
  acc_t acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0;

  gload(0);
  for (int64_t kb = 0; kb < nk; ++kb) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < ACHUNKS; ++c) {
      const int q = tid + c * kThreads;
      *reinterpret_cast<uint4*>(As + q * 16) = ra[c];
    }
    if (tid < BN) *reinterpret_cast<uint4*>(Bs + tid * 16) = rb;
    __syncthreads();
    if (kb + 1 < nk) gload(kb + 1);

    uint2 wq[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int col = wn * 64 + c * 32 + li;
      wq[c] = *reinterpret_cast<const uint2*>(Bs + col * 16 + 8 * lh);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = wm * 64 + r * 32 + li;
      if constexpr (MODE == MODE_INT4) {
        const uint4 x = *reinterpret_cast<const uint4*>(As + row * 32 + 16 * lh);
        const v4i a0 = widen_int4(x.x, x.y);
        const v4i a1 = widen_int4(x.z, x.w);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[r][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, widen_w_a4(wq[c].x), acc[r][c], 0, 0, 0);
          acc[r][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, widen_w_a4(wq[c].y), acc[r][c], 0, 0, 0);
        }
      } else if constexpr (MODE == MODE_INT8) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(As + row * 64 + 32 * lh);
        const uint4 x1 = *reinterpret_cast<const uint4*>(As + row * 64 + 32 * lh + 16);
        v4i a0, a1;
        a0[0] = x0.x; a0[1] = x0.y; a0[2] = x0.z; a0[3] = x0.w;
        a1[0] = x1.x; a1[1] = x1.y; a1[2] = x1.z; a1[3] = x1.w;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[r][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, widen_w_a8(wq[c].x), acc[r][c], 0, 0, 0);
          acc[r][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, widen_w_a8(wq[c].y), acc[r][c], 0, 0, 0);
        }
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(As + row * 32 + 16 * lh);
        v8i a;
        a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
        a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint32_t b0, b1, b2, b3;
          widen_w_e2m1(wq[c].x, b0, b1);
          widen_w_e2m1(wq[c].y, b2, b3);
          v8i b;
          b[0] = b0; b[1] = b1; b[2] = b2; b[3] = b3;
          b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
          acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[r][c], 4, 4, 0, 127,
                                                                      0, 127);
        }
      }
    }
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32) and rows
  // 8*(e/4) + 4*(lane/32) + (e%4) for its 16 elements e.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t gn = n0 + wn * 64 + c * 32 + li;
      if (gn >= N) continue;
      const float bn = beta[gn];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t gm = m0 + wm * 64 + r * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (gm >= M) continue;
        float accf;
        if constexpr (MODE == MODE_FP4) {
          accf = acc[r][c][e];
          if (acc_dbg) static_cast<float*>(acc_dbg)[gm * N + gn] = accf;
        } else {
          const int shift = (MODE == MODE_INT4) ? 10 : 6;
          const int32_t a = acc[r][c][e] >> shift;
          if (acc_dbg) static_cast<int32_t*>(acc_dbg)[gm * N + gn] = a;
          accf = static_cast<float>(a);
        }
        y[gm * N + gn] = mul_rn(mul_rn(accf, sx[gm]), bn);
      }
    }
  }
}

}  // namespace

hipError_t launch_bitlinear(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                            const uint8_t* w_packed, const float* beta, int64_t N, float* y,
                            void* acc_dbg, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  const dim3 block(kThreads);
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  switch (mode) {
    case MODE_INT4:
      hipLaunchKernelGGL(k_bitlinear<MODE_INT4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg);
      break;
    case MODE_FP4:
      hipLaunchKernelGGL(k_bitlinear<MODE_FP4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg);
      break;
    default:
      hipLaunchKernelGGL(k_bitlinear<MODE_INT8>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg);
      break;
  }
  return hipGetLastError();
}

}  // namespace bw
