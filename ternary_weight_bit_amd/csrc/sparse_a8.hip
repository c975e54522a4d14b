// Fused ReLU^2 gate + per-token top-k + INT8 absmax quantizer for gfx950.
//
// BitNet a4.8 abstract: intermediate states are sparsified, then quantized to
// 8 bits.  toshoseti review «Метод»: top-k at 50 % sparsity for the out
// projection input; ReLU^2 replaces swish in the FFN gate to sparsify the
// down projection input.  9pt.com article, methodology: the low-magnitude
// entries are the ones dropped.
//
// One workgroup (256 threads) per token row; thread t owns entries
// t + 256*r, kept in registers.  The k-th largest magnitude tau is found by
// bisection over the 31 magnitude bits (count of keys >= candidate, reduced
// across the block); entries equal to tau are taken lowest index first, the
// cut found from per-64-entry ballot masks.  Everything runs on the row held
// in registers: the row is read from HBM once and its codes written once.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;

template <bool BF16, bool GATED, int R>
__global__ __launch_bounds__(kThreads) void k_sparse_a8(const void* __restrict__ g,
                                                        const void* __restrict__ u, int K, int k_keep,
                                                        int8_t* __restrict__ codes,
                                                        float* __restrict__ scales,
                                                        uint32_t* __restrict__ mask) {
  __shared__ int part[2][4];
  __shared__ float red[4];
  __shared__ unsigned long long segmask[R * 4];
  __shared__ int segcnt[R * 4];
  __shared__ int cut_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * K;
  const int nr = (K + kThreads - 1) / kThreads;  // rounds actually used (K % 64 == 0)

  float h[R];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    h[r] = 0.0f;
    const int idx = tid + r * kThreads;
    if (r < nr && idx < K) {
      float v = load1<BF16>(g, row + idx);
      if constexpr (GATED) {
        const float rr = v > 0.0f ? v : 0.0f;
        v = mul_rn(mul_rn(rr, rr), load1<BF16>(u, row + idx));
      }
      h[r] = v;
      amax = fmaxf(amax, fabsf(v));
    }
  }
  amax = block_max256(amax, red);

  // tau = largest key value with count(key >= tau) >= k_keep (bisection over bits 30..0).
  uint32_t tau = 0;
  int it = 0;
  for (int b = 30; b >= 0; --b, ++it) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += ((__float_as_uint(h[r]) & 0x7FFFFFFFu) >= cand) ? 1 : 0;
    // entries beyond K hold +0.0 and never reach cand >= 1
    cnt = wave_sum(cnt);
    if (lane == 0) part[it & 1][wave] = cnt;
    __syncthreads();
    const int total = part[it & 1][0] + part[it & 1][1] + part[it & 1][2] + part[it & 1][3];
    if (total >= k_keep) tau = cand;
  }
  // count of keys strictly above tau
  int gt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) gt += ((__float_as_uint(h[r]) & 0x7FFFFFFFu) > tau) ? 1 : 0;
  gt = wave_sum(gt);
  if (lane == 0) part[it & 1][wave] = gt;
  __syncthreads();
  const int n_gt = part[it & 1][0] + part[it & 1][1] + part[it & 1][2] + part[it & 1][3];
  const int need = k_keep - n_gt;  // >= 1 entries equal to tau, lowest index first

  // per-segment (64 consecutive entries) masks of key == tau
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < nr && tid + r * kThreads < K) {
      const bool eq = (__float_as_uint(h[r]) & 0x7FFFFFFFu) == tau;
      const unsigned long long bal = __ballot(eq);
      if (lane == 0) {
        segmask[r * 4 + wave] = bal;
        segcnt[r * 4 + wave] = __popcll(bal);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane l scans segments [l*S, l*S + S) with S = ceil(nseg / 64)
    const int nseg = K / 64;
    const int per = (nseg + 63) / 64;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int sidx = lane * per + i;
      if (sidx < nseg) local += segcnt[sidx];
    }
    // exclusive prefix over lanes
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += t;
    }
    const int excl = incl - local;
    if (excl < need && need <= incl) {
      int acc = excl;
      for (int i = 0; i < per; ++i) {
        const int sidx = lane * per + i;
        if (sidx >= nseg) break;
        const int c = segcnt[sidx];
        if (acc + c >= need) {
          unsigned long long m = segmask[sidx];
          int skip = need - acc - 1;  // drop this many lowest set bits
          while (skip-- > 0) m &= m - 1;
          cut_sh = sidx * 64 + __ffsll(static_cast<long long>(m)) - 1;
          break;
        }
        acc += c;
      }
    }
  }
  __syncthreads();
  const int cut = cut_sh;

  const float a = fmaxf(amax, 1e-5f);
  const float inv = div_rn(127.0f, a);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = tid + r * kThreads;
    if (r < nr && idx < K) {
      const uint32_t key = __float_as_uint(h[r]) & 0x7FFFFFFFu;
      const bool keep = key > tau || (key == tau && idx <= cut);
      int q = 0;
      if (keep) q = static_cast<int>(fminf(fmaxf(__builtin_rintf(mul_rn(h[r], inv)), -128.0f), 127.0f));
      codes[row + idx] = static_cast<int8_t>(q);
      if (mask) {
        const unsigned long long bal = __ballot(keep);
        if (lane == 0) {
          uint32_t* mw = mask + (row >> 5) + (idx >> 5);
          mw[0] = static_cast<uint32_t>(bal);
          mw[1] = static_cast<uint32_t>(bal >> 32);
        }
      }
    }
  }
  if (tid == 0) scales[blockIdx.x] = div_rn(a, 127.0f);
}

template <bool BF16, bool GATED>
hipError_t launch_t(const void* g, const void* u, int64_t M, int64_t K, int64_t k_keep, int8_t* codes,
                    float* scales, uint32_t* mask, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  const int k = static_cast<int>(K), kk = static_cast<int>(k_keep);
  if (K <= 4096) {
    hipLaunchKernelGGL((k_sparse_a8<BF16, GATED, 16>), grid, block, 0, s, g, u, k, kk, codes, scales, mask);
  } else if (K <= 12288) {
    hipLaunchKernelGGL((k_sparse_a8<BF16, GATED, 48>), grid, block, 0, s, g, u, k, kk, codes, scales, mask);
  } else {
    hipLaunchKernelGGL((k_sparse_a8<BF16, GATED, 64>), grid, block, 0, s, g, u, k, kk, codes, scales, mask);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_a8(const void* g, const void* u, bool bf16, int64_t M, int64_t K,
                            int64_t k_keep, int8_t* codes, float* scales, uint32_t* mask,
                            hipStream_t s) {
  if (bf16) {
    return u ? launch_t<true, true>(g, u, M, K, k_keep, codes, scales, mask, s)
             : launch_t<true, false>(g, u, M, K, k_keep, codes, scales, mask, s);
  }
  return u ? launch_t<false, true>(g, u, M, K, k_keep, codes, scales, mask, s)
           : launch_t<false, false>(g, u, M, K, k_keep, codes, scales, mask, s);
}

}  // namespace bw
