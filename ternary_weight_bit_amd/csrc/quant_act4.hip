// Per-token 4-bit activation quantizer (INT4 absmax or e2m1 FP4) for gfx950;
// INT4 values are stored as nibbles or as e2m3 fields.
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
#include "bw_quant.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;

// Eight codes as one word (even k in the low nibble).  inv = fl(qmax / a') with
// a' >= max|v|, so act4_code's INT4 rounding add applies (no clamp needed).
template <int FMT>
__device__ __forceinline__ uint32_t encode8(const float (&v)[8], float inv) {
  return act4_word<FMT>(v, inv);
}

// e2m3 fields of the INT4 values of up to four chunks (v[C0 + k], k < 4, of
// the CPT a thread holds) by one conversion of 32 values.  The conversion
// writes field j (bits 6j .. 6j+5 of its 192-bit output) from its first
// operand's element j / 2 when j is even and from its second operand's when j
// is odd, so value j of the 32 goes there; chunk k then takes bits 48k .. 48k
// + 47, returned as lo = its bits 0..31 and hi = its bits 32..47.
template <int CPT, int C0>
__device__ __forceinline__ void encode_e2m3(const float (&v)[CPT][8], float inv, uint32_t (&lo)[CPT],
                                            uint32_t (&hi)[CPT]) {
  constexpr int n = CPT - C0 < 4 ? CPT - C0 : 4;
  v16f a, b;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int k = (j >> 3) % n;  // slots past the chunks repeat one (their fields are not used)
    const float t = e2m3_input(mul_rn(v[C0 + k][j & 7], inv));
    if (j & 1) b[j >> 1] = t;
    else a[j >> 1] = t;
  }
  const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 8.0f);
#pragma unroll
  for (int k = 0; k < n; ++k) {
    const uint32_t w0 = r[3 * (k >> 1)], w1 = r[3 * (k >> 1) + 1], w2 = r[3 * (k >> 1) + 2];
    lo[C0 + k] = (k & 1) ? ((w1 >> 16) | (w2 << 16)) : w0;
    hi[C0 + k] = (k & 1) ? (w2 >> 16) : (w1 & 0xFFFFu);
  }
}

// Row bytes of K values: two codes per byte, or e2m3 fields (3 bytes per 4).
template <int FMT>
__device__ __forceinline__ int64_t code_row_bytes(int64_t K) {
  return FMT == 2 ? (K >> 2) * 3 : (K >> 1);
}

// Store the codes of chunk ch (values 8ch .. 8ch+7) of a row.  Nibbles: one
// word.  e2m3 fields (given as the chunk's 48 bits lo | hi << 32): 64 values
// form a group of 48 bytes, the 24-byte bit streams of values 0..31 (S0) and
// 32..63 (S1) stored as S0[0:16], S1[0:16], S0[16:24], S1[16:24]; chunk j of a
// half covers bytes 6j .. 6j+5 of its stream.  The even lane of each lane pair
// (chunks 2p, 2p+1 of a half) writes their 12 bytes; every lane of the wave
// must call the e2m3 store (a lane exchange).
template <int FMT>
__device__ __forceinline__ void store_chunk(uint8_t* __restrict__ row, int64_t ch, bool valid,
                                            const float (&v)[8], float inv) {
  static_assert(FMT != 2, "e2m3 fields: store_e2m3");
  if (valid) reinterpret_cast<uint32_t*>(row)[ch] = encode8<FMT>(v, inv);
}

__device__ __forceinline__ void store_e2m3(uint8_t* __restrict__ row, int64_t ch, bool valid, uint32_t lo,
                                           uint32_t hi) {
  // the other lane of the pair (DPP quad_perm 1,0,3,2: a VALU move, no LDS)
  const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(lo), 0xB1, 0xF, 0xF, false));
  const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(hi), 0xB1, 0xF, 0xF, false));
  if (valid && (ch & 1) == 0) {
    const uint32_t d0 = lo, d1 = hi | (plo << 16), d2 = (plo >> 16) | (phi << 16);
    uint8_t* g = row + 48 * (ch >> 3) + 16 * ((ch >> 2) & 1);  // this half's first 16 bytes
    if ((ch & 2) == 0) {  // stream bytes 0..11
      *reinterpret_cast<uint3*>(g) = make_uint3(d0, d1, d2);
    } else {              // stream bytes 12..23: the last word of the first 16, then the last 8
      reinterpret_cast<uint32_t*>(g)[3] = d0;
      *reinterpret_cast<uint2*>(row + 48 * (ch >> 3) + 32 + 8 * ((ch >> 2) & 1)) = make_uint2(d1, d2);
    }
  }
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
  uint8_t* __restrict__ out = codes + m * code_row_bytes<FMT>(K);
  float amax = 0.0f;
  for (int64_t ch = lane; ch < nchunk; ch += kWave) {
    float t[8];
    load8<BF16>(x, row + ch * 8, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
  }
  amax = wave_max(amax);
  const float a = fmaxf(amax, 1e-5f);
  const float qmax = act4_qmax<FMT>();
  const float inv = div_rn(qmax, a);
  // nchunk is a multiple of 8: the lanes of a pair leave the loop together
  for (int64_t ch = lane; ch < nchunk; ch += kWave) {
    float t[1][8];
    load8<BF16>(x, row + ch * 8, t[0]);
    if constexpr (FMT == 2) {
      uint32_t lo[1], hi[1];
      encode_e2m3<1, 0>(t, inv, lo, hi);
      store_e2m3(out, ch, true, lo[0], hi[0]);
    } else {
      store_chunk<FMT>(out, ch, true, t[0], inv);
    }
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
  uint32_t amax = 0;  // |x| bits: non-negative floats order as integers
  if constexpr (BF16) {
    // raw bf16 words: the row maximum on packed 16-bit magnitudes (one masked
    // max per two elements), widened once at the end
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 m2 = {0, 0};
    uint4 w[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int64_t ch = tid + c * kThreads;
      w[c] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row + (ch < nchunk ? ch : 0) * 8);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const uint32_t keep = (tid + c * kThreads < nchunk) ? 0x7FFF7FFFu : 0u;
      const uint32_t ws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, ws[j] & keep));
        v[c][2 * j] = bf16_lo(ws[j]);
        v[c][2 * j + 1] = bf16_hi(ws[j]);
      }
    }
    amax = static_cast<uint32_t>(m2.x > m2.y ? m2.x : m2.y) << 16;
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int64_t ch = tid + c * kThreads;
      load8<BF16>(x, row + (ch < nchunk ? ch : 0) * 8, v[c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const bool in_row = tid + c * kThreads < nchunk;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = max(amax, in_row ? (__float_as_uint(v[c][i]) & 0x7FFFFFFFu) : 0u);
    }
  }
  amax = static_cast<uint32_t>(lane_value(static_cast<int>(wave_incl_umax(amax)), kWave - 1));
  if ((tid & (kWave - 1)) == 0) wmax[tid / kWave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float a = fmaxf(__uint_as_float(amax), 1e-5f);
  const float qmax = act4_qmax<FMT>();
  const float inv = div_rn(qmax, a);
  uint8_t* __restrict__ out = codes + m * code_row_bytes<FMT>(K);
  if constexpr (FMT == 2) {
    uint32_t lo[CPT], hi[CPT];
    encode_e2m3<CPT, 0>(v, inv, lo, hi);
    if constexpr (CPT > 4) encode_e2m3<CPT, 4>(v, inv, lo, hi);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int64_t ch = tid + c * kThreads;
      store_e2m3(out, ch, ch < nchunk, lo[c], hi[c]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int64_t ch = tid + c * kThreads;
      store_chunk<FMT>(out, ch, ch < nchunk, v[c], inv);
    }
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
           : fmt == 1 ? launch_t<true, 1>(x, M, K, codes, scales, s)
                      : launch_t<true, 2>(x, M, K, codes, scales, s);
  }
  return fmt == 0 ? launch_t<false, 0>(x, M, K, codes, scales, s)
         : fmt == 1 ? launch_t<false, 1>(x, M, K, codes, scales, s)
                    : launch_t<false, 2>(x, M, K, codes, scales, s);
}

}  // namespace bw
