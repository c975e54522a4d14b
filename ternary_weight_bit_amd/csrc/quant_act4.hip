// Per-token 4-bit activation quantizer (INT4 absmax or e2m1 FP4) for gfx950.
//
// BitNet a4.8 abstract: 4-bit activations at the inputs of attention and FFN
// (INT4/FP4 kernels).  toshoseti review «Метод»: the q/k/v/gate/up inputs are
// the 4-bit group; FP4 is the wider-range alternative to INT4.
//
// One wave per token row, four rows per workgroup: the row maximum is a
// wave-level reduction (no workgroup barrier).  Each lane owns 8-element
// chunks c = lane + 64*i; rows of up to 64*8*kMaxChunks elements stay in
// registers, loaded with unconditional (clamped-address) loads so all of them
// are in flight before the first use; longer rows are streamed twice (the
// second read hits L2).  The absmax is exact and order-free.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kMaxChunks = 8;  // 8-element chunks per lane held in registers (K <= 4096)

// INT4 code of t = fl(x * inv): clamp(rne(t), -8, 7) as a 4-bit field.
__device__ __forceinline__ uint32_t int4_code(float t) {
  const float q = fminf(fmaxf(__builtin_rintf(t), -8.0f), 7.0f);
  return static_cast<uint32_t>(static_cast<int>(q)) & 0xFu;
}

// e2m1 code of t: nearest of {0,.5,1,1.5,2,3,4,6}; at a midpoint the
// neighbour with the even code wins; saturates at 6; sign bit from t.
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float m = fabsf(t);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) +
               (m > 5.0f);
  return c | ((__float_as_uint(t) >> 31) << 3);
}

template <int FMT>
__device__ __forceinline__ uint32_t encode8(const float (&v)[8], float inv) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = mul_rn(v[i], inv);
    const uint32_t c = (FMT == 0) ? int4_code(t) : e2m1_code(t);
    w |= c << (4 * i);
  }
  return w;
}

template <bool BF16, int FMT, bool RESIDENT>
__global__ __launch_bounds__(kThreads) void k_quantize_act4(const void* __restrict__ x, int64_t M, int64_t K,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave leaves together
  const int64_t nchunk = K >> 3;
  const int64_t row = m * K;
  uint32_t* __restrict__ out = reinterpret_cast<uint32_t*>(codes + m * (K >> 1));

  float amax = 0.0f;
  float v[kMaxChunks][8];
  if constexpr (RESIDENT) {
    // unconditional loads (chunks past the row re-read chunk 0), so every load
    // is in flight before the first use
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int64_t ch = lane + c * kWave;
      load8<BF16>(x, row + (ch < nchunk ? ch : 0) * 8, v[c]);
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int64_t ch = lane + c * kWave;
      const bool in_row = ch < nchunk;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, in_row ? fabsf(v[c][i]) : 0.0f);
    }
  } else {
    for (int64_t ch = lane; ch < nchunk; ch += kWave) {
      float t[8];
      load8<BF16>(x, row + ch * 8, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
  }
  amax = wave_max(amax);
  const float a = fmaxf(amax, 1e-5f);
  const float qmax = (FMT == 0) ? 7.0f : 6.0f;
  const float inv = div_rn(qmax, a);

  if constexpr (RESIDENT) {
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int64_t ch = lane + c * kWave;
      if (ch < nchunk) out[ch] = encode8<FMT>(v[c], inv);
    }
  } else {
    for (int64_t ch = lane; ch < nchunk; ch += kWave) {
      float t[8];
      load8<BF16>(x, row + ch * 8, t);
      out[ch] = encode8<FMT>(t, inv);
    }
  }
  if (lane == 0) scales[m] = div_rn(a, qmax);
}

template <bool BF16, int FMT>
hipError_t launch_t(const void* x, int64_t M, int64_t K, uint8_t* codes, float* scales, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  if (K <= static_cast<int64_t>(kWave) * 8 * kMaxChunks) {
    hipLaunchKernelGGL((k_quantize_act4<BF16, FMT, true>), grid, block, 0, s, x, M, K, codes, scales);
  } else {
    hipLaunchKernelGGL((k_quantize_act4<BF16, FMT, false>), grid, block, 0, s, x, M, K, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_act4(const void* x, bool bf16, int64_t M, int64_t K, int fmt,
                                uint8_t* codes, float* scales, hipStream_t s) {
  if (bf16) {
    return fmt == 0 ? launch_t<true, 0>(x, M, K, codes, scales, s)
                    : launch_t<true, 1>(x, M, K, codes, scales, s);
  }
  return fmt == 0 ? launch_t<false, 0>(x, M, K, codes, scales, s)
                  : launch_t<false, 1>(x, M, K, codes, scales, s);
}

}  // namespace bw
