// Per-token 4-bit activation quantizer (INT4 absmax or e2m1 FP4) for gfx950.
//
// BitNet a4.8 abstract: 4-bit activations at the inputs of attention and FFN
// (INT4/FP4 kernels).  toshoseti review «Метод»: the q/k/v/gate/up inputs are
// the 4-bit group; FP4 is the wider-range alternative to INT4.
//
// Rows of up to 8192 elements: one workgroup (256 threads) per token row; each
// thread holds CPT chunks of 8 elements (chunk t + 256*c), loaded with
// unconditional (clamped-address) loads so all are in flight before the first
// use; the row maximum is a DPP wave maximum plus one LDS exchange.  Longer
// rows: one wave per row, four rows per workgroup, streamed twice (the second
// read hits L2).  The absmax is exact and order-free.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;

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

// One wave per row (rows longer than 8192): the row is read twice, once for
// the maximum and once to encode (the second read hits L2).
template <bool BF16, int FMT>
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
  for (int64_t ch = lane; ch < nchunk; ch += kWave) {
    float t[8];
    load8<BF16>(x, row + ch * 8, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
  }
  amax = wave_max(amax);
  const float a = fmaxf(amax, 1e-5f);
  const float qmax = (FMT == 0) ? 7.0f : 6.0f;
  const float inv = div_rn(qmax, a);
  for (int64_t ch = lane; ch < nchunk; ch += kWave) {
    float t[8];
    load8<BF16>(x, row + ch * 8, t);
    out[ch] = encode8<FMT>(t, inv);
  }
  if (lane == 0) scales[m] = div_rn(a, qmax);
}

// One workgroup per row, CPT chunks of 8 elements per thread (K <= 2048 * CPT).
template <bool BF16, int FMT, int CPT>
__global__ __launch_bounds__(kThreads) void k_quantize_act4_row(const void* __restrict__ x, int64_t K,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  __shared__ uint32_t wmax[kThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int64_t nchunk = K >> 3;
  const int64_t row = m * K;
  float v[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t ch = tid + c * kThreads;
    load8<BF16>(x, row + (ch < nchunk ? ch : 0) * 8, v[c]);
  }
  uint32_t amax = 0;  // |x| bits: non-negative floats order as integers
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const bool in_row = tid + c * kThreads < nchunk;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, in_row ? (__float_as_uint(v[c][i]) & 0x7FFFFFFFu) : 0u);
  }
  amax = static_cast<uint32_t>(lane_value(static_cast<int>(wave_incl_umax(amax)), kWave - 1));
  if ((tid & (kWave - 1)) == 0) wmax[tid / kWave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float a = fmaxf(__uint_as_float(amax), 1e-5f);
  const float qmax = (FMT == 0) ? 7.0f : 6.0f;
  const float inv = div_rn(qmax, a);
  uint32_t* __restrict__ out = reinterpret_cast<uint32_t*>(codes + m * (K >> 1));
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t ch = tid + c * kThreads;
    if (ch < nchunk) out[ch] = encode8<FMT>(v[c], inv);
  }
  if (tid == 0) scales[m] = div_rn(a, qmax);
}

template <bool BF16, int FMT>
hipError_t launch_t(const void* x, int64_t M, int64_t K, uint8_t* codes, float* scales, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  const dim3 rgrid(static_cast<unsigned>(M));
  if (K <= 2048) {
    hipLaunchKernelGGL((k_quantize_act4_row<BF16, FMT, 1>), rgrid, block, 0, s, x, K, codes, scales);
  } else if (K <= 4096) {
    hipLaunchKernelGGL((k_quantize_act4_row<BF16, FMT, 2>), rgrid, block, 0, s, x, K, codes, scales);
  } else if (K <= 8192) {
    hipLaunchKernelGGL((k_quantize_act4_row<BF16, FMT, 4>), rgrid, block, 0, s, x, K, codes, scales);
  } else {
    hipLaunchKernelGGL((k_quantize_act4<BF16, FMT>), grid, block, 0, s, x, M, K, codes, scales);
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
