// 3-bit KV-cache codec with 4-bit special tokens for gfx950.
//
// toshoseti review «Эксперименты»: KV caches are quantized to 3 bits, except
// the bos/eos tokens, which are kept at 4 bits.  BitNet a4.8 abstract: the
// model supports a 3-bit KV cache.
//
// Each lane owns 8 consecutive elements of one (b, s, h) vector, so a vector
// of D elements spans D/8 lanes and a wave holds 512/D vectors per step; a
// wave runs kSteps steps at once with every load issued before the first use.
// The absmax is reduced across the vector's lanes with shuffles; four lanes
// make one group of 32 codes, and lane i of the group (codes 8i .. 8i+7)
// writes byte i of each of the group's three words: with u_j = q_j + 4,
//   W0 = u0 | u1 << 3 | (u6 & 3) << 6
//   W1 = u2 | u3 << 3 | (u6 >> 2) << 6 | (u7 & 1) << 7
//   W2 = u4 | u5 << 3 | (u7 >> 1) << 6,
// so a reader gets code+4 of four codes per 32-bit word with one shift and
// one mask for six of the eight slices.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int kSteps = 4;         // vectors per lane in flight
constexpr int64_t kMaxBlocks = int64_t{1} << 20;  // one pass over the grid for caches up to 2^20 blocks of work
// 1.5 * 2^23: adding it to |t| < 2^22 rounds t to an integer (ties to even) that
// sits, two's complement, in the low mantissa bits; OR-ing a small integer n
// into its bits gives the float 1.5 * 2^23 + n.
constexpr float kRoundMagic = 12582912.0f;
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

template <int LPV>  // lanes per vector = D / 8
__device__ __forceinline__ float vec_max(float v) {
#pragma unroll
  for (int off = LPV / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

template <bool BF16, int LPV>
__global__ __launch_bounds__(kThreads) void k_kv_pack3(const void* __restrict__ kv, int64_t nvec,
                                                       int64_t H, const int32_t* __restrict__ slot_of,
                                                       int64_t n_special, uint8_t* __restrict__ p3,
                                                       float* __restrict__ s3, uint8_t* __restrict__ p4,
                                                       float* __restrict__ s4) {
  constexpr int D = LPV * 8;
  constexpr int VPW = kWave / LPV;  // vectors per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPV;       // lane within its vector
  const int64_t waves_total = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6);
  for (int64_t base = wave_id * VPW * kSteps; base < nvec; base += waves_total * VPW * kSteps) {
    // every load of the group (values and the token's slot) is issued before
    // the first use; vectors past the end re-read the last vector
    float xs[kSteps][8];
    int32_t sl[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t v = base + u * VPW + lane / LPV;
      const int64_t vc = v < nvec ? v : nvec - 1;
      load8<BF16>(kv, vc * D + sub * 8, xs[u]);
      sl[u] = slot_of[vc / H];
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t v = base + u * VPW + lane / LPV;
      const bool active = v < nvec;
      const float (&x)[8] = xs[u];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = vec_max<LPV>(amax);
      const float a = fmaxf(amax, 1e-5f);
      const float inv3 = div_rn(3.0f, a);
      // fields u = q + 4 of this lane's 8 codes.  |x| <= a' makes
      // |x * fl(3/a')| < 3.5, so rne() lands in [-3, 3] and the clamp to
      // [-4, 3] never acts; adding 1.5 * 2^23 rounds to an integer (ties to
      // even) and leaves it, two's complement, in the low mantissa bits, so
      // (bits & 7) ^ 4 = q + 4.
      uint32_t f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (__float_as_uint(mul_rn(x[i], inv3) + kRoundMagic) & 7u) ^ 4u;
      const uint32_t pl0 = f[0] | (f[1] << 3) | ((f[6] & 3u) << 6);
      const uint32_t pl1 = f[2] | (f[3] << 3) | ((f[6] >> 2) << 6) | ((f[7] & 1u) << 7);
      const uint32_t pl2 = f[4] | (f[5] << 3) | ((f[7] >> 1) << 6);
      // group of 32 codes = 4 lanes; lane q of the group writes byte q of each
      // of the group's three words (bytes, not shuffles: cheaper here)
      if (active) {
        const int grp = sub >> 2;
        uint8_t* out = p3 + v * (3 * D / 8) + 12 * grp + (sub & 3);
        out[0] = static_cast<uint8_t>(pl0);
        out[4] = static_cast<uint8_t>(pl1);
        out[8] = static_cast<uint8_t>(pl2);
        if (sub == 0) s3[v] = div_rn(a, 3.0f);
        const int64_t bs = v / H;
        const int32_t slot = sl[u];
        if (slot >= 0 && slot < n_special) {
          const int64_t hh = v - bs * H;
          const float inv4 = div_rn(7.0f, a);
          uint32_t w = 0;  // |x * fl(7/a')| < 7.5: codes in [-7, 7], no clamp needed
#pragma unroll
          for (int i = 0; i < 8; ++i)
            w |= (__float_as_uint(mul_rn(x[i], inv4) + kRoundMagic) & 0xFu) << (4 * i);
          const int64_t sv = static_cast<int64_t>(slot) * H + hh;
          reinterpret_cast<uint32_t*>(p4 + sv * (D / 2))[sub] = w;
          if (sub == 0) s4[sv] = div_rn(a, 7.0f);
        }
      }
    }
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ void store8(void* __restrict__ out, int64_t e, const float (&v)[8]) {
  if constexpr (BF16) {
    // v_cvt_pk_bf16_f32: two fp32 -> bf16 with round-to-nearest-even
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 p = {v[2 * i], v[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float* o = static_cast<float*>(out) + e;
    *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <bool BF16, int LPV>
__global__ __launch_bounds__(kThreads) void k_kv_unpack3(const uint8_t* __restrict__ p3,
                                                         const float* __restrict__ s3,
                                                         const uint8_t* __restrict__ p4,
                                                         const float* __restrict__ s4,
                                                         const int32_t* __restrict__ slot_of,
                                                         int64_t nvec, int64_t H, int64_t n_special,
                                                         void* __restrict__ out) {
  constexpr int D = LPV * 8;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPV;
  const int64_t lanes_total = static_cast<int64_t>(gridDim.x) * kThreads;
  const int64_t gl = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nch = nvec * LPV;
  // every lane owns kSteps (vector, 8-element chunk) pairs: chunk = base + u * lanes_total
  for (int64_t base = gl; base < nch; base += lanes_total * kSteps) {
    uint32_t pw[kSteps][3];
    float sc[kSteps];
    int32_t sl[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t ch = base + u * lanes_total;
      const int64_t v = (ch < nch ? ch : nch - 1) / LPV;
      const uint32_t* gp = reinterpret_cast<const uint32_t*>(p3 + v * (3 * D / 8)) + 3 * (sub >> 2);
      pw[u][0] = gp[0];
      pw[u][1] = gp[1];
      pw[u][2] = gp[2];
      sc[u] = s3[v];
      sl[u] = slot_of[v / H];
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t ch = base + u * lanes_total;
      if (ch >= nch) continue;
      const int64_t v = ch / LPV;
      float x[8];
      const int32_t slot = sl[u];
      if (slot >= 0 && slot < n_special) {
        const int64_t bs = v / H;
        const int64_t sv = static_cast<int64_t>(slot) * H + (v - bs * H);
        const uint32_t w = reinterpret_cast<const uint32_t*>(p4 + sv * (D / 2))[sub];
        const float s4v = s4[sv];
        // (nibble ^ 8) = q + 8 in [0, 15]: q exactly as 2^23*1.5 + q + 8 - (2^23*1.5 + 8)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t c = (w >> (4 * i)) & 0xFu;
          x[i] = mul_rn(__uint_as_float(kRoundMagicBits | (c ^ 8u)) - (kRoundMagic + 8.0f), s4v);
        }
      } else {
        const int sh = 8 * (sub & 3);
        const uint32_t b0 = (pw[u][0] >> sh) & 0xFFu;
        const uint32_t b1 = (pw[u][1] >> sh) & 0xFFu;
        const uint32_t b2 = (pw[u][2] >> sh) & 0xFFu;
        // fields u = q + 4 in [0, 7], turned into the float q exactly as above
        const uint32_t f[8] = {b0 & 7u, (b0 >> 3) & 7u, b1 & 7u, (b1 >> 3) & 7u, b2 & 7u, (b2 >> 3) & 7u,
                               (b0 >> 6) | (((b1 >> 6) & 1u) << 2), (b1 >> 7) | ((b2 >> 6) << 1)};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          x[i] = mul_rn(__uint_as_float(kRoundMagicBits | f[i]) - (kRoundMagic + 4.0f), sc[u]);
      }
      store8<BF16>(out, v * D + sub * 8, x);
    }
  }
}

template <bool BF16>
hipError_t pack_t(const void* kv, int64_t nvec, int64_t H, int64_t D, const int32_t* slot_of,
                  int64_t ns, uint8_t* p3, float* s3, uint8_t* p4, float* s4, hipStream_t s) {
  const int64_t lpv = D / 8;
  const int64_t vpb = (kThreads / lpv) * kSteps;  // vectors per block per iteration
  int64_t blocks = (nvec + vpb - 1) / vpb;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  switch (lpv) {
    case 4: hipLaunchKernelGGL((k_kv_pack3<BF16, 4>), grid, block, 0, s, kv, nvec, H, slot_of, ns, p3, s3, p4, s4); break;
    case 8: hipLaunchKernelGGL((k_kv_pack3<BF16, 8>), grid, block, 0, s, kv, nvec, H, slot_of, ns, p3, s3, p4, s4); break;
    case 16: hipLaunchKernelGGL((k_kv_pack3<BF16, 16>), grid, block, 0, s, kv, nvec, H, slot_of, ns, p3, s3, p4, s4); break;
    case 32: hipLaunchKernelGGL((k_kv_pack3<BF16, 32>), grid, block, 0, s, kv, nvec, H, slot_of, ns, p3, s3, p4, s4); break;
    default: hipLaunchKernelGGL((k_kv_pack3<BF16, 64>), grid, block, 0, s, kv, nvec, H, slot_of, ns, p3, s3, p4, s4); break;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t unpack_t(const uint8_t* p3, const float* s3, const uint8_t* p4, const float* s4,
                    const int32_t* slot_of, int64_t nvec, int64_t H, int64_t D, int64_t ns, void* out,
                    hipStream_t s) {
  const int64_t lpv = D / 8;
  int64_t blocks = (nvec * lpv + kThreads * kSteps - 1) / (kThreads * kSteps);
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  switch (lpv) {
    case 4: hipLaunchKernelGGL((k_kv_unpack3<BF16, 4>), grid, block, 0, s, p3, s3, p4, s4, slot_of, nvec, H, ns, out); break;
    case 8: hipLaunchKernelGGL((k_kv_unpack3<BF16, 8>), grid, block, 0, s, p3, s3, p4, s4, slot_of, nvec, H, ns, out); break;
    case 16: hipLaunchKernelGGL((k_kv_unpack3<BF16, 16>), grid, block, 0, s, p3, s3, p4, s4, slot_of, nvec, H, ns, out); break;
    case 32: hipLaunchKernelGGL((k_kv_unpack3<BF16, 32>), grid, block, 0, s, p3, s3, p4, s4, slot_of, nvec, H, ns, out); break;
    default: hipLaunchKernelGGL((k_kv_unpack3<BF16, 64>), grid, block, 0, s, p3, s3, p4, s4, slot_of, nvec, H, ns, out); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_pack3(const void* kv, bool bf16, int64_t B, int64_t S, int64_t H, int64_t D,
                           const int32_t* slot_of, int64_t n_special, uint8_t* p3, float* s3,
                           uint8_t* p4, float* s4, hipStream_t s) {
  const int64_t nvec = B * S * H;
  return bf16 ? pack_t<true>(kv, nvec, H, D, slot_of, n_special, p3, s3, p4, s4, s)
              : pack_t<false>(kv, nvec, H, D, slot_of, n_special, p3, s3, p4, s4, s);
}

hipError_t launch_kv_unpack3(const uint8_t* p3, const float* s3, const uint8_t* p4, const float* s4,
                             const int32_t* slot_of, int64_t B, int64_t S, int64_t H, int64_t D,
                             int64_t n_special, bool out_bf16, void* out, hipStream_t s) {
  const int64_t nvec = B * S * H;
  return out_bf16 ? unpack_t<true>(p3, s3, p4, s4, slot_of, nvec, H, D, n_special, out, s)
                  : unpack_t<false>(p3, s3, p4, s4, slot_of, nvec, H, D, n_special, out, s);
}

}  // namespace bw
