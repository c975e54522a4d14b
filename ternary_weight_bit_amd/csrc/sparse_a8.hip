// Fused ReLU^2 gate + per-token top-k + INT8 absmax quantizer for gfx950.
//
// BitNet a4.8 abstract: intermediate states are sparsified, then quantized to
// 8 bits.  toshoseti review «Метод»: top-k at 50 % sparsity for the out
// projection input; ReLU^2 replaces swish in the FFN gate to sparsify the
// down projection input.  9pt.com article, methodology: the low-magnitude
// entries are the ones dropped.
//
// One workgroup (256 threads) per token row.  The row is read with 16-byte
// loads (8 consecutive entries per thread, all issued before the first use),
// h is formed and written to LDS, and read back so that thread t owns entries
// t + 256*r in registers.  The k-th largest magnitude tau is found by
// bisection over the magnitude bits below the row maximum's top bit; each
// step counts keys >= candidate with one ballot + popcount per register (a
// scalar-unit count, no cross-lane shuffles) and one workgroup barrier.  When
// a row has fewer than k nonzero magnitudes (common after ReLU^2), tau = 0 and
// no search runs.  Entries equal to tau are taken lowest index first, the
// cut found from per-64-entry ballot masks.  The row is read from HBM once
// and its codes written once.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;

// Number of this wave's keys >= cand, as a wave-uniform value: one ballot and
// one popcount per register (scalar unit), no cross-lane shuffles.
template <int R>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&key)[R], uint32_t cand) {
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(key[r] >= cand));
  return cnt;
}

template <bool BF16, bool GATED, int R>
__global__ __launch_bounds__(kThreads) void k_sparse_a8(const void* __restrict__ g,
                                                        const void* __restrict__ u, int K, int k_keep,
                                                        int8_t* __restrict__ codes,
                                                        float* __restrict__ scales,
                                                        uint32_t* __restrict__ mask) {
  __shared__ int part[2][4];
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) float hs[R * kThreads];
  __shared__ unsigned long long segmask[R * 4];
  __shared__ int segcnt[R * 4];
  __shared__ int cut_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * K;
  const int nr = (K + kThreads - 1) / kThreads;  // rounds actually used (K % 64 == 0)

  // Block-wide total of a wave-uniform count (one barrier; parity-buffered).
  int par = 0;
  auto block_total = [&](int wave_cnt) {
    if (lane == 0) part[par][wave] = wave_cnt;
    __syncthreads();
    const int t = part[par][0] + part[par][1] + part[par][2] + part[par][3];
    par ^= 1;
    return t;
  };

  // load: thread t takes 8-entry chunks t + 256*c (clamped in-bounds, masked later)
  constexpr int CPT = R / 8;  // chunks per thread
  const int nch = K >> 3;
  {
    float gv[CPT][8];
    float uv[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * kThreads;
      const int64_t e0 = row + static_cast<int64_t>(ch < nch ? ch : 0) * 8;
      load8<BF16>(g, e0, gv[c]);
      if constexpr (GATED) load8<BF16>(u, e0, uv[c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * kThreads;
      if (ch < nch) {
        float hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v = gv[c][i];
          if constexpr (GATED) {
            const float rr = v > 0.0f ? v : 0.0f;
            v = mul_rn(mul_rn(rr, rr), uv[c][i]);
          }
          hv[i] = v;
        }
        *reinterpret_cast<float4*>(&hs[ch * 8]) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        *reinterpret_cast<float4*>(&hs[ch * 8 + 4]) = make_float4(hv[4], hv[5], hv[6], hv[7]);
      }
    }
  }
  __syncthreads();

  float h[R];
  uint32_t key[R];  // |h| as ordered integer bits; entries past K hold 0
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = tid + r * kThreads;
    h[r] = (r < nr && idx < K) ? hs[idx] : 0.0f;
    amax = fmaxf(amax, fabsf(h[r]));
    key[r] = __float_as_uint(h[r]) & 0x7FFFFFFFu;
  }
  amax = block_max256(amax, red);

  // tau = the k-th largest key = largest value with count(key >= tau) >= k_keep.
  uint32_t tau = 0;
  int n_gt;
  const int nnz = block_total(wave_count_ge<R>(key, 1u));
  if (nnz < k_keep) {
    n_gt = nnz;  // fewer than k nonzeros: tau = 0, every nonzero survives, zeros fill the rest
  } else {
    const uint32_t top = __float_as_uint(amax) & 0x7FFFFFFFu;  // >= 1 here
    for (int b = 31 - __builtin_clz(top); b >= 0; --b) {
      const uint32_t cand = tau | (1u << b);
      if (block_total(wave_count_ge<R>(key, cand)) >= k_keep) tau = cand;
    }
    n_gt = block_total(wave_count_ge<R>(key, tau + 1u));
  }
  const int need = k_keep - n_gt;  // >= 1 entries equal to tau, lowest index first

  // per-segment (64 consecutive entries) masks of key == tau
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < nr && tid + r * kThreads < K) {
      const unsigned long long bal = __ballot(key[r] == tau);
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
