// Absmean ternary weight packer for gfx950.
//
// toshoseti review, opening lines: BitNet b1.58 (whose weights BitNet a4.8
// keeps) has ternary {-1, 0, +1} weights.  The per-tensor scale is the mean
// magnitude, and t = RoundClip(w / beta', -1, 1).
//
// beta must come out bit-identical whatever the launch shape, so the sum of
// the N*K magnitudes is formed EXACTLY: every fp32 magnitude is m * 2^(e-150)
// with an integer mantissa m < 2^24 and a biased exponent e in [1, 254], so
// the kernel adds the mantissas into one uint64 bucket per exponent (integer
// addition: order-free).  A single thread then folds the 254 buckets into a
// 352-bit integer and rounds it once to fp64, which is the correctly-rounded
// sum; beta = fp32(sum / (N*K)).
//
// Launches: clear workspace -> bucket sums -> finalize beta' -> pack words.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
// workspace: uint64 bucket[256] at 0, float beta' at byte 2048.
constexpr int kBetaOffset = 2048;

__global__ void k_ws_clear(uint64_t* __restrict__ ws) {
  // 4096 bytes = 512 uint64
  ws[threadIdx.x] = 0;
  ws[threadIdx.x + 256] = 0;
}

__device__ __forceinline__ void bucket_add(unsigned long long* hist, uint32_t bits) {
  const uint32_t u = bits & 0x7FFFFFFFu;
  uint32_t e = u >> 23;
  uint32_t m = u & 0x7FFFFFu;
  if (e) {
    m |= 0x800000u;
  } else {
    e = 1;  // subnormals share the scale of exponent field 1
  }
  if (m) atomicAdd(&hist[e], static_cast<unsigned long long>(m));
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_abs_buckets(const void* __restrict__ W, int64_t total,
                                                          uint64_t* __restrict__ ws) {
  __shared__ unsigned long long hist[256];
  hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t nchunk = total >> 3;
  for (int64_t ch = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; ch < nchunk;
       ch += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v[8];
    load8<BF16>(W, ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) bucket_add(hist, __float_as_uint(v[i]));
  }
  __syncthreads();
  const unsigned long long h = hist[threadIdx.x];
  if (h) atomicAdd(reinterpret_cast<unsigned long long*>(ws) + threadIdx.x, h);
}

// Bits [lo, lo+n) of a little-endian array of 32-bit limbs (n <= 64, lo >= 0).
__device__ uint64_t limb_bits(const uint32_t* limb, int nlimb, int lo, int n) {
  uint64_t r = 0;
  for (int i = 0; i < n; ++i) {
    const int b = lo + i;
    const int L = b >> 5;
    if (L < nlimb && ((limb[L] >> (b & 31)) & 1u)) r |= (1ull << i);
  }
  return r;
}

__global__ void k_beta_finalize(uint64_t* __restrict__ ws, double count) {
  if (threadIdx.x != 0) return;
  constexpr int kL = 11;
  uint32_t limb[kL];
  for (int i = 0; i < kL; ++i) limb[i] = 0;
  // integer I = sum_e bucket[e] * 2^(e-1); the exact sum is I * 2^-149
  for (int e = 1; e <= 254; ++e) {
    const uint64_t B = ws[e];
    if (!B) continue;
    const int s = e - 1;
    const int L = s >> 5;
    const int b = s & 31;
    const uint64_t lo = B << b;
    const uint64_t hi = b ? (B >> (64 - b)) : 0ull;
    const uint32_t parts[3] = {static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                               static_cast<uint32_t>(hi)};
    uint64_t carry = 0;
    for (int i = 0; L + i < kL; ++i) {
      const uint64_t add = (i < 3 ? parts[i] : 0u);
      if (i >= 3 && carry == 0) break;
      const uint64_t t = static_cast<uint64_t>(limb[L + i]) + add + carry;
      limb[L + i] = static_cast<uint32_t>(t);
      carry = t >> 32;
    }
  }
  int top = -1;
  for (int i = kL - 1; i >= 0; --i) {
    if (limb[i]) {
      top = 32 * i + (31 - __builtin_clz(limb[i]));
      break;
    }
  }
  double sum = 0.0;
  if (top >= 0) {
    if (top < 53) {
      sum = ldexp(static_cast<double>(limb_bits(limb, kL, 0, top + 1)), -149);
    } else {
      uint64_t mant = limb_bits(limb, kL, top - 52, 53);
      const bool round_bit = limb_bits(limb, kL, top - 53, 1) != 0;
      bool sticky = false;
      for (int b = 0; b < top - 53 && !sticky; ++b) sticky = limb_bits(limb, kL, b, 1) != 0;
      int exp = top - 52;
      if (round_bit && (sticky || (mant & 1ull))) {
        mant += 1;
        if (mant == (1ull << 53)) {
          mant >>= 1;
          exp += 1;
        }
      }
      sum = ldexp(static_cast<double>(mant), exp - 149);
    }
  }
  const float beta = static_cast<float>(sum / count);
  reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + kBetaOffset)[0] = fmaxf(beta, 1e-5f);
}

// Slot (0..15) that holds input offset `off` inside a packed word.
template <int ROLE>
__device__ __forceinline__ int slot_of_offset(int off) {
  if constexpr (ROLE == 0) {
    return off < 8 ? 2 * off : 2 * (off - 8) + 1;
  } else {
    return 4 * (off & 3) + (off >> 2);
  }
}

template <bool BF16, int ROLE>
__global__ __launch_bounds__(kThreads) void k_pack_words(const void* __restrict__ W, int64_t N,
                                                         int64_t K, const uint64_t* __restrict__ ws,
                                                         uint32_t* __restrict__ packed,
                                                         float* __restrict__ beta) {
  const float bp =
      reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ws) + kBetaOffset)[0];
  const int64_t nwords = N * K / 16;
  const int64_t kblocks = K / 64;
  for (int64_t w = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; w < nwords;
       w += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t tile = w >> 6;
    const int c = static_cast<int>((w >> 2) & 15);
    const int j = static_cast<int>(w & 3);
    const int64_t nb = tile / kblocks;
    const int64_t kb = tile - nb * kblocks;
    const int64_t n = nb * 16 + c;
    const int64_t k0 = kb * 64 + j * 16;
    float v[16];
    load8<BF16>(W, n * K + k0, *reinterpret_cast<float(*)[8]>(&v[0]));
    load8<BF16>(W, n * K + k0 + 8, *reinterpret_cast<float(*)[8]>(&v[8]));
    uint32_t word = 0;
#pragma unroll
    for (int off = 0; off < 16; ++off) {
      const bool keep = mul_rn(2.0f, fabsf(v[off])) > bp;
      const uint32_t code = keep ? (v[off] < 0.0f ? 3u : 1u) : 0u;
      word |= code << (2 * slot_of_offset<ROLE>(off));
    }
    packed[w] = word;
  }
  for (int64_t n = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; n < N;
       n += static_cast<int64_t>(gridDim.x) * kThreads) {
    beta[n] = bp;
  }
}

template <bool BF16, int ROLE>
hipError_t launch_t(const void* W, int64_t N, int64_t K, uint8_t* packed, float* beta, void* ws,
                    hipStream_t s) {
  uint64_t* w64 = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(k_ws_clear, dim3(1), dim3(256), 0, s, w64);
  const int64_t total = N * K;
  int64_t blocks = (total / 8 + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL((k_abs_buckets<BF16>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     s, W, total, w64);
  hipLaunchKernelGGL(k_beta_finalize, dim3(1), dim3(64), 0, s, w64, static_cast<double>(total));
  int64_t pblocks = (total / 16 + kThreads - 1) / kThreads;
  if (pblocks > 16384) pblocks = 16384;
  hipLaunchKernelGGL((k_pack_words<BF16, ROLE>), dim3(static_cast<unsigned>(pblocks)),
                     dim3(kThreads), 0, s, W, N, K, w64, reinterpret_cast<uint32_t*>(packed), beta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_ternary(const void* W, bool bf16, int64_t N, int64_t K, int role,
                               uint8_t* packed, float* beta, void* ws, hipStream_t s) {
  if (bf16) {
    return role == 0 ? launch_t<true, 0>(W, N, K, packed, beta, ws, s)
                     : launch_t<true, 1>(W, N, K, packed, beta, ws, s);
  }
  return role == 0 ? launch_t<false, 0>(W, N, K, packed, beta, ws, s)
                   : launch_t<false, 1>(W, N, K, packed, beta, ws, s);
}

}  // namespace bw
