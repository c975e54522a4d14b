// Single-token attention over the 3-bit KV cache, for gfx950.
//
// BitNet a4.8 abstract: the model supports a 3-bit KV cache; toshoseti
// review, «Эксперименты»: bos/eos tokens keep 4-bit codes.  The pages give no
// attention formula; this computes standard scaled dot-product attention of
// one new query per (batch, head) over all S cached positions,
//   z_s = (q . k_s) / sqrt(D),  p = softmax(z),  out = sum_s p_s v_s,
// with k_s, v_s the codec's dequantized vectors (code * scale; the side-slab
// 4-bit codes at special positions).  The codes are never expanded in HBM:
// the kernel reads 3*D/8 + 4 bytes per vector, a fifth of a bf16 cache.
//
// One workgroup (512 threads) per (batch, head); the block index runs over
// batches fastest, so with 8 batches each batch's heads share one XCD (the
// dispatcher's round robin) and its L2 (scales and plane bytes of
// neighbouring heads share cache lines).  Thread t takes 32-dim group
// g = t % G (G = D/32) of the positions s = t / G + i * (512 / G):
//   pass 1: the group's three plane words are unpacked four codes per 32-bit
//     word: ((P >> k) & 0x01010101) holds bit j of codes k, k+8, k+16, k+24
//     in its bytes, so u = b0 + 2 b1 + 4 (1 - b2) = code + 4 is built with
//     shifts and masks and converted per byte; sum q*u, minus 4 * sum q, is
//     reduced over the G lanes of a position (DPP) and scaled;
//   special positions (slot_of in [0, n_special)) are rescored from their
//     4-bit codes by one wave each, and are flagged in an LDS bitmask;
//   softmax in LDS (max, exp, sum; fp32);
//   pass 2: acc[d] += w_s * u_d with w_s = e_s * s3_s (0 at special
//     positions), minus 4 * sum w; special positions are added from their
//     4-bit codes by one wave each; lanes, waves and the special part are
//     summed and divided by sum e.
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kAttnThreads = 512;
constexpr uint32_t kBytes = 0x01010101u;

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  // sum over the G consecutive lanes that share a position (G = 2 or 4)
  v += __shfl_xor(v, 1);
  if constexpr (G == 4) v += __shfl_xor(v, 2);
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// x shifted right by n (left by -n); n is a compile-time constant
template <int n>
__device__ __forceinline__ uint32_t shift_r(uint32_t x) {
  if constexpr (n >= 0) return x >> n;
  else return x << (-n);
}

// Unpacked codes of one 32-code group: u[k] holds code+4 of codes k, k+8,
// k+16, k+24 in bytes 0..3.  Bit j of code i sits at bit i of plane j; it is
// moved to bit j of byte i / 8 by one shift of the whole plane (right by
// k - j, or left where k < j), so no bit is shifted out of the word.
template <int k>
__device__ __forceinline__ uint32_t unpack_k(uint32_t p0, uint32_t p1, uint32_t p2n) {
  uint32_t x = shift_r<k>(p0) & kBytes;
  x |= shift_r<k - 1>(p1) & (kBytes << 1);
  x |= shift_r<k - 2>(p2n) & (kBytes << 2);
  return x;
}

__device__ __forceinline__ void unpack_group(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t (&u)[8]) {
  const uint32_t p2n = ~p2;  // 4 (1 - b2): code + 4 is b0 + 2 b1 + 4 (1 - b2)
  u[0] = unpack_k<0>(p0, p1, p2n);
  u[1] = unpack_k<1>(p0, p1, p2n);
  u[2] = unpack_k<2>(p0, p1, p2n);
  u[3] = unpack_k<3>(p0, p1, p2n);
  u[4] = unpack_k<4>(p0, p1, p2n);
  u[5] = unpack_k<5>(p0, p1, p2n);
  u[6] = unpack_k<6>(p0, p1, p2n);
  u[7] = unpack_k<7>(p0, p1, p2n);
}

// byte b of x as a float (one v_cvt_f32_ubyteN)
__device__ __forceinline__ float byte_f(uint32_t x, int b) {
  return static_cast<float>((x >> (8 * b)) & 0xFFu);
}

// 4-bit two's-complement nibble n (0..15) -> value
__device__ __forceinline__ float nib_f(uint32_t byte, int hi) {
  const int n = static_cast<int>((byte >> (4 * hi)) & 0xFu);
  return static_cast<float>(n >= 8 ? n - 16 : n);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_decode3(
    const float* __restrict__ q, const uint8_t* __restrict__ kp3, const float* __restrict__ ks3,
    const uint8_t* __restrict__ kp4, const float* __restrict__ ks4, const uint8_t* __restrict__ vp3,
    const float* __restrict__ vs3, const uint8_t* __restrict__ vp4, const float* __restrict__ vs4,
    const int32_t* __restrict__ slot_of, int64_t n_special, int64_t B, int64_t S, int64_t H,
    float* __restrict__ out) {
  constexpr int G = D / 32;                 // 32-dim groups per vector
  constexpr int SL = kAttnThreads / G;      // positions in flight per pass step
  constexpr int VB = 3 * D / 8;             // plane bytes per vector
  extern __shared__ float s_z[];            // [S] scores, then exp weights
  __shared__ uint32_t s_spec[kAttnMaxS / 32];
  __shared__ float s_red[kAttnThreads / 64];
  __shared__ float s_acc[kAttnThreads / 64][D];
  __shared__ float s_fix[kAttnThreads / 64][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = tid % G;
  const int slice = tid / G;
  const int64_t b = blockIdx.x % B;
  const int64_t h = blockIdx.x / B;
  const float* __restrict__ qv = q + (b * H + h) * D;
  const int32_t* __restrict__ slots = slot_of + b * S;
  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));

  // this thread's 32 query values (group g)
  float qg[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) qg[i] = qv[32 * g + i];
  float qsum = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qsum += qg[i];

  // special-position bitmask
  const int nwords = static_cast<int>((S + 31) / 32);
  for (int w = tid; w < nwords; w += kAttnThreads) s_spec[w] = 0u;
  __syncthreads();
  for (int64_t s = tid; s < S; s += kAttnThreads) {
    const int32_t sl = slots[s];
    if (sl >= 0 && sl < n_special) atomicOr(&s_spec[s >> 5], 1u << (s & 31));
  }

  // pass 1: scores from the 3-bit codes
  for (int64_t s = slice; s < S; s += SL) {
    const int64_t vec = (b * S + s) * H + h;
    const uint32_t* __restrict__ pw = reinterpret_cast<const uint32_t*>(kp3 + vec * VB) + 3 * g;
    uint32_t u[8];
    unpack_group(pw[0], pw[1], pw[2], u);
    float dot = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int by = 0; by < 4; ++by) dot = fmaf(qg[k + 8 * by], byte_f(u[k], by), dot);
    dot = group_sum<G>(dot - 4.0f * qsum);
    if (g == 0) s_z[s] = dot * ks3[vec] * inv_sqrt_d;
  }
  __syncthreads();

  // special positions: rescore from the 4-bit codes, one wave per position
  for (int w = wave; w < nwords; w += kAttnThreads / 64) {
    uint32_t bits = s_spec[w];
    while (bits) {
      const int i = __builtin_ctz(bits);
      bits &= bits - 1;
      const int64_t s = 32 * static_cast<int64_t>(w) + i;
      const int64_t sl = slots[s];
      const uint8_t* __restrict__ p4 = kp4 + (sl * H + h) * (D / 2);
      float part = 0.0f;
      for (int d2 = lane; d2 < D / 2; d2 += 64) {
        const uint32_t byte = p4[d2];
        part = fmaf(qv[2 * d2], nib_f(byte, 0), part);
        part = fmaf(qv[2 * d2 + 1], nib_f(byte, 1), part);
      }
      part = wave_sum_f(part);
      if (lane == 0) s_z[s] = part * ks4[sl * H + h] * inv_sqrt_d;
    }
  }
  __syncthreads();

  // softmax: max, exp, sum
  float mx = -INFINITY;
  for (int64_t s = tid; s < S; s += kAttnThreads) mx = fmaxf(mx, s_z[s]);
  mx = wave_max_f(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < kAttnThreads / 64; ++w) mx = fmaxf(mx, s_red[w]);
  __syncthreads();
  float tot = 0.0f;
  for (int64_t s = tid; s < S; s += kAttnThreads) {
    const float e = expf(s_z[s] - mx);
    s_z[s] = e;
    tot += e;
  }
  tot = wave_sum_f(tot);
  if (lane == 0) s_red[wave] = tot;
  __syncthreads();
  tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kAttnThreads / 64; ++w) tot += s_red[w];

  // pass 2: weighted values from the 3-bit codes (special positions weigh 0)
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
  float wsum = 0.0f;
  for (int64_t s = slice; s < S; s += SL) {
    const int64_t vec = (b * S + s) * H + h;
    const uint32_t* __restrict__ pw = reinterpret_cast<const uint32_t*>(vp3 + vec * VB) + 3 * g;
    const bool sp = (s_spec[s >> 5] >> (s & 31)) & 1u;
    const float w = sp ? 0.0f : s_z[s] * vs3[vec];
    uint32_t u[8];
    unpack_group(pw[0], pw[1], pw[2], u);
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int by = 0; by < 4; ++by) acc[k + 8 * by] = fmaf(w, byte_f(u[k], by), acc[k + 8 * by]);
    wsum += w;
  }
  // remove the +4 of the codes, then sum the lanes of each group within the wave
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float v = acc[i] - 4.0f * wsum;
#pragma unroll
    for (int o = G; o < 64; o <<= 1) v += __shfl_xor(v, o);
    acc[i] = v;
  }
  if (lane < G) {
#pragma unroll
    for (int i = 0; i < 32; ++i) s_acc[wave][32 * g + i] = acc[i];
  }

  // special positions from their 4-bit codes, one wave per position
  float fix[D / 64 > 0 ? D / 64 : 1][2];
#pragma unroll
  for (int j = 0; j < (D / 64 > 0 ? D / 64 : 1); ++j) fix[j][0] = fix[j][1] = 0.0f;
  for (int w = wave; w < nwords; w += kAttnThreads / 64) {
    uint32_t bits = s_spec[w];
    while (bits) {
      const int i = __builtin_ctz(bits);
      bits &= bits - 1;
      const int64_t s = 32 * static_cast<int64_t>(w) + i;
      const int64_t sl = slots[s];
      const uint8_t* __restrict__ p4 = vp4 + (sl * H + h) * (D / 2);
      const float wt = s_z[s] * vs4[sl * H + h];
#pragma unroll
      for (int j = 0; j < (D / 64 > 0 ? D / 64 : 1); ++j) {
        const int d2 = lane + 64 * j;
        if (d2 < D / 2) {
          const uint32_t byte = p4[d2];
          fix[j][0] = fmaf(wt, nib_f(byte, 0), fix[j][0]);
          fix[j][1] = fmaf(wt, nib_f(byte, 1), fix[j][1]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < (D / 64 > 0 ? D / 64 : 1); ++j) {
    const int d2 = lane + 64 * j;
    if (d2 < D / 2) {
      s_fix[wave][2 * d2] = fix[j][0];
      s_fix[wave][2 * d2 + 1] = fix[j][1];
    }
  }
  __syncthreads();
  if (tid < D) {
    // byte `by` of u[k] is code k + 8 by of its group, so acc[i] (written to
    // s_acc[.][32 g + i]) is dimension 32 g + i
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) a += s_acc[w][tid] + s_fix[w][tid];
    out[(b * H + h) * D + tid] = a / tot;
  }
}

}  // namespace

hipError_t launch_attn_decode3(const float* q, const uint8_t* kp3, const float* ks3, const uint8_t* kp4,
                               const float* ks4, const uint8_t* vp3, const float* vs3, const uint8_t* vp4,
                               const float* vs4, const int32_t* slot_of, int64_t n_special, int64_t B, int64_t S,
                               int64_t H, int64_t D, float* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(B * H));
  const size_t lds = static_cast<size_t>(S) * sizeof(float);
  if (D == 64) {
    hipLaunchKernelGGL(k_attn_decode3<64>, grid, dim3(kAttnThreads), lds, s, q, kp3, ks3, kp4, ks4, vp3, vs3, vp4,
                       vs4, slot_of, n_special, B, S, H, out);
  } else {
    hipLaunchKernelGGL(k_attn_decode3<128>, grid, dim3(kAttnThreads), lds, s, q, kp3, ks3, kp4, ks4, vp3, vs3, vp4,
                       vs4, slot_of, n_special, B, S, H, out);
  }
  return hipGetLastError();
}

}  // namespace bw
