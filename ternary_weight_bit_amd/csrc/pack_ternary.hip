// Absmean ternary weight packer for gfx950.
//
// toshoseti review, opening lines: BitNet b1.58 (whose weights BitNet a4.8
// keeps) has ternary {-1, 0, +1} weights.  The per-tensor scale is the mean
// magnitude, and t = RoundClip(w / beta', -1, 1).
//
// beta must come out bit-identical whatever the launch shape, so the sum of
// the N*K magnitudes is formed EXACTLY: every fp32 magnitude is m * 2^(e-150)
// with an integer mantissa m < 2^24 and a biased exponent e in [1, 254].
// Each thread adds m << (e - lo) into a private 128-bit integer for the
// exponents of a 41-wide window [lo, lo + 40] set by its first nonzero
// magnitude (weights of one tensor span far fewer exponents), and sends any
// other magnitude to a per-exponent uint64 bucket; at the end its 128-bit
// total goes to the buckets as four 32-bit pieces at exponents lo, lo + 32,
// ... All of it is integer addition, so the order does not matter.  One
// thread then folds the buckets into a 608-bit integer and rounds it once to
// fp64, which is the correctly-rounded sum; beta = fp32(sum / (N*K)).
//
// Launches: clear workspace -> bucket sums -> finalize beta' -> pack words
// (tile layouts for the GEMMs, or the K-major layout of the gather product).
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
// workspace: uint64 bucket[kBuckets] at 0, float beta' at byte kBetaOffset.
constexpr int kBuckets = 512;  // exponent slots: 1..254, plus the 128-bit pieces up to 254 + 96
constexpr int kBetaOffset = kBuckets * 8;
static_assert(kBetaOffset + 4 <= static_cast<int>(kPackWorkspaceBytes), "workspace too small");

__global__ void k_ws_clear(uint64_t* __restrict__ ws) {
  for (int i = threadIdx.x; i < kBuckets + 1; i += blockDim.x) ws[i] = 0;
}

constexpr int kUnroll = 4;  // 8-element chunks in flight per thread

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_abs_buckets(const void* __restrict__ W, int64_t total,
                                                          uint64_t* __restrict__ ws) {
  __shared__ unsigned long long hist[kBuckets];
  for (int i = threadIdx.x; i < kBuckets; i += kThreads) hist[i] = 0;
  __syncthreads();
  uint64_t acc_lo = 0, acc_hi = 0;  // private 128-bit sum at scale 2^(lo - 150)
  int lo = 0;                       // window base; 0 = not chosen yet
  auto add = [&](float x) {
    const uint32_t u = __float_as_uint(x) & 0x7FFFFFFFu;
    const int ef = static_cast<int>(u >> 23);
    const uint32_t m = (u & 0x7FFFFFu) | (ef ? 0x800000u : 0u);
    const int e = ef ? ef : 1;  // subnormals share the scale of exponent field 1
    if (m == 0) return;
    if (lo == 0) lo = (e > 20) ? e - 20 : 1;
    const int d = e - lo;
    if (d >= 0 && d <= 40) {
      const uint64_t v = static_cast<uint64_t>(m) << d;  // < 2^64
      acc_lo += v;
      acc_hi += (acc_lo < v) ? 1u : 0u;
    } else {
      atomicAdd(&hist[e], static_cast<unsigned long long>(m));
    }
  };
  const int64_t nchunk = total >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t ch = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x;
  for (; ch + (kUnroll - 1) * stride < nchunk; ch += kUnroll * stride) {
    float v[kUnroll][8];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) load8<BF16>(W, (ch + q * stride) * 8, v[q]);
#pragma unroll
    for (int q = 0; q < kUnroll; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) add(v[q][i]);
  }
  for (; ch < nchunk; ch += stride) {
    float v[8];
    load8<BF16>(W, ch * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) add(v[i]);
  }
  if (lo) {
    // acc * 2^(lo-150): 32-bit piece p sits at exponent lo + 32p
    const uint32_t piece[4] = {static_cast<uint32_t>(acc_lo), static_cast<uint32_t>(acc_lo >> 32),
                               static_cast<uint32_t>(acc_hi), static_cast<uint32_t>(acc_hi >> 32)};
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (piece[p]) atomicAdd(&hist[lo + 32 * p], static_cast<unsigned long long>(piece[p]));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBuckets; i += kThreads) {
    const unsigned long long h = hist[i];
    if (h) atomicAdd(reinterpret_cast<unsigned long long*>(ws) + i, h);
  }
}

__global__ __launch_bounds__(kBuckets) void k_beta_finalize(uint64_t* __restrict__ ws, double count) {
  // integer I = sum_e bucket[e] * 2^(e-1), in 32-bit limbs; the sum is I * 2^-149.
  // Bucket e (one thread each) adds its 96-bit shifted value as three 32-bit
  // parts into per-limb uint64 column sums; one thread then carries.
  constexpr int kL = 19;  // 608 bits >= 2^(kBuckets - 2) * 2^64
  __shared__ unsigned long long col[kL + 2];
  if (threadIdx.x < kL + 2) col[threadIdx.x] = 0;
  __syncthreads();
  const int e = threadIdx.x;
  if (e >= 1) {
    const uint64_t B = ws[e];
    if (B) {
      const int s = e - 1;
      const int L = s >> 5;
      const int b = s & 31;
      const uint64_t lo = B << b;
      const uint64_t hi = b ? (B >> (64 - b)) : 0ull;
      atomicAdd(&col[L], static_cast<unsigned long long>(static_cast<uint32_t>(lo)));
      atomicAdd(&col[L + 1], static_cast<unsigned long long>(static_cast<uint32_t>(lo >> 32)));
      atomicAdd(&col[L + 2], static_cast<unsigned long long>(static_cast<uint32_t>(hi)));
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t limb[kL];
  uint64_t carry = 0;
  for (int i = 0; i < kL; ++i) {
    const uint64_t t = col[i] + carry;  // column sums stay far below 2^63
    limb[i] = static_cast<uint32_t>(t);
    carry = t >> 32;
  }
  // bits [b, b + 64) of I (b >= 0)
  auto bits64 = [&](int b) -> uint64_t {
    uint64_t r = 0;
    for (int k = 0; k < 64; k += 32) {
      const int L = (b + k) >> 5, sh = (b + k) & 31;
      uint64_t w = (L < kL) ? (limb[L] >> sh) : 0u;
      if (sh && L + 1 < kL) w |= static_cast<uint64_t>(limb[L + 1]) << (32 - sh);
      r |= (w & 0xFFFFFFFFull) << k;
    }
    return r;
  };
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
      sum = ldexp(static_cast<double>(bits64(0) & ((1ull << (top + 1)) - 1)), -149);
    } else {
      // 53 bits below and including the top bit, the next bit, and a sticky OR
      uint64_t mant = (bits64(top - 52)) & ((1ull << 53) - 1);
      const bool round_bit = (bits64(top - 53) & 1ull) != 0;
      bool sticky = false;
      const int nlow = top - 53;  // bits [0, nlow) below the round bit
      for (int i = 0; i < kL && !sticky && 32 * i < nlow; ++i) {
        const int span = nlow - 32 * i;
        const uint32_t msk = span >= 32 ? 0xFFFFFFFFu : ((1u << span) - 1u);
        sticky = (limb[i] & msk) != 0;
      }
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

// K-major layout (out/down weights for the single-token gather product):
// input k owns the N/4 bytes at k*N/4; word g of that run holds outputs
// 16g + i at bits 2i, code t + 1.  Thread w covers word (g = w / K, k = w % K),
// so for each of its 16 reads consecutive threads read consecutive inputs.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_pack_kmajor(const void* __restrict__ W, int64_t N,
                                                          int64_t K, const uint64_t* __restrict__ ws,
                                                          uint32_t* __restrict__ packed,
                                                          float* __restrict__ beta) {
  const float bp =
      reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ws) + kBetaOffset)[0];
  const int64_t groups = N / 16;
  const int64_t nwords = groups * K;
  for (int64_t w = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; w < nwords;
       w += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t g = w / K;
    const int64_t k = w - g * K;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = load1<BF16>(W, (g * 16 + i) * K + k);
      const bool keep = mul_rn(2.0f, fabsf(v)) > bp;
      const uint32_t code = keep ? (v < 0.0f ? 0u : 2u) : 1u;  // t + 1
      word |= code << (2 * i);
    }
    packed[k * groups + g] = word;
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
  // about 16 chunks per thread: few end-of-thread bucket updates, loads in flight
  int64_t blocks = (total / 8 + 16 * kThreads - 1) / (16 * kThreads);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((k_abs_buckets<BF16>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     s, W, total, w64);
  hipLaunchKernelGGL(k_beta_finalize, dim3(1), dim3(kBuckets), 0, s, w64, static_cast<double>(total));
  int64_t pblocks = (total / 16 + kThreads - 1) / kThreads;
  if (pblocks > 16384) pblocks = 16384;
  if constexpr (ROLE == 2) {
    hipLaunchKernelGGL((k_pack_kmajor<BF16>), dim3(static_cast<unsigned>(pblocks)), dim3(kThreads), 0,
                       s, W, N, K, w64, reinterpret_cast<uint32_t*>(packed), beta);
  } else {
    hipLaunchKernelGGL((k_pack_words<BF16, ROLE>), dim3(static_cast<unsigned>(pblocks)),
                       dim3(kThreads), 0, s, W, N, K, w64, reinterpret_cast<uint32_t*>(packed), beta);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_ternary(const void* W, bool bf16, int64_t N, int64_t K, int role,
                               uint8_t* packed, float* beta, void* ws, hipStream_t s) {
  if (bf16) {
    if (role == 2) return launch_t<true, 2>(W, N, K, packed, beta, ws, s);
    return role == 0 ? launch_t<true, 0>(W, N, K, packed, beta, ws, s)
                     : launch_t<true, 1>(W, N, K, packed, beta, ws, s);
  }
  if (role == 2) return launch_t<false, 2>(W, N, K, packed, beta, ws, s);
  return role == 0 ? launch_t<false, 0>(W, N, K, packed, beta, ws, s)
                   : launch_t<false, 1>(W, N, K, packed, beta, ws, s);
}

}  // namespace bw
