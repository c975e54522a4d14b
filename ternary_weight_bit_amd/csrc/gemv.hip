// Decode-shape BitLinear (M <= 16 tokens) for gfx950: streams the 2-bit
// weights once from HBM.
//
// BitNet a4.8 abstract: ternary layers on 4-bit activations (INT4/FP4
// kernels) and on 8-bit sparsified states.  At decode the weight bytes are
// the whole cost, so the kernel is shaped for HBM streaming:
//   * one workgroup per 16 output channels (one packed tile column); its
//     K/64 tiles are one contiguous run of K*4 bytes;
//   * the waves split the tiles; a wave's lane group g (16 lanes) reads tile
//     base+g, so one wave load moves 1 KB of contiguous weights, 16 B per lane,
//     and all of a wave's loads are issued before any is consumed.  A grid of
//     few workgroups with a long K (N = 4096, K = 11008) takes 8 waves per
//     workgroup so that each wave's share of K is two rounds of loads;
//   * the tokens (M <= 16, zero-padded) are the rows of 16x16 MFMAs
//     (i8 16x16x64, or scaled f8f6f4 16x16x128 for e2m1); activations are read
//     straight from L2-resident global memory;
//   * the waves' partial int32/fp32 tiles are summed through LDS (exact) and
//     the epilogue writes y for the M real rows; optionally it adds a residual
//     (y = r + W x, the decoder layer's skip connections) and splits the
//     columns into row-major planes (a fused gate/up product written as two
//     [M][F] arrays).
#include "bw_internal.h"
#include "bw_widen.h"

namespace bw {
namespace {

constexpr int kUnroll = 4;  // tile groups in flight per lane

template <int MODE, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(const uint8_t* __restrict__ A,
                                                   const float* __restrict__ sx, int M, int64_t K,
                                                   const uint8_t* __restrict__ Wp,
                                                   const float* __restrict__ beta, int64_t N,
                                                   float* __restrict__ y, void* __restrict__ acc_dbg,
                                                   const float* __restrict__ resid, int64_t split) {
  using acc_t = typename std::conditional<MODE == MODE_FP4, v4f, v4i>::type;
  __shared__ acc_t part[WAVES][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;  // token row (A) / output channel (B) of this lane
  const int g = lane >> 4;   // lane group: which tile of a group of four
  const int64_t nb = blockIdx.x;
  const int64_t T = K >> 6;  // tiles along K
  const int64_t a_row = (MODE == MODE_INT8) ? K : (K >> 1);
  const uint8_t* __restrict__ wcol = Wp + nb * T * 256 + li * 16;
  const bool row_ok = li < M;

  // wave w handles tiles [t0, t1)
  const int64_t per = (T + WAVES - 1) / WAVES;
  const int64_t t0 = wave * per;
  const int64_t t1 = (t0 + per < T) ? t0 + per : T;

  acc_t acc;
  acc[0] = 0; acc[1] = 0; acc[2] = 0; acc[3] = 0;

  // Epilogue scales, loaded first so their latency hides under the weight
  // stream (16x16 accumulator layout: lane holds column lane % 16, rows
  // 4*(lane/16) + e).
  const int64_t n_out = nb * 16 + li;
  const float bn = beta[n_out];
  float sxm[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sxm[e] = sx[(4 * g + e < M) ? 4 * g + e : 0];

  // Every load is issued unconditionally from an in-bounds address (rows past M
  // read row 0, tiles past t1 read tile T-1) and masked to zero afterwards, so
  // all of a lane's weight and activation loads are in flight before the first
  // wait.
  const uint8_t* __restrict__ arow = A + static_cast<int64_t>(row_ok ? li : 0) * a_row;
  constexpr int AW = (MODE == MODE_INT8) ? 4 : 2;  // 16-byte activation loads per tile
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t base = t0; base < t1; base += 4 * kUnroll) {
    uint4 wr[kUnroll];
    uint4 ar[kUnroll][AW];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t kt = base + 4 * u + g;
      ok[u] = kt < t1;
      const int64_t kc = ok[u] ? kt : T - 1;
      wr[u] = *reinterpret_cast<const uint4*>(wcol + kc * 256);
#pragma unroll
      for (int w = 0; w < AW; ++w)
        ar[u][w] = *reinterpret_cast<const uint4*>(arow + kc * (16 * AW) + 16 * w);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint4 wv = ok[u] ? wr[u] : z;
      uint4 a[AW];
#pragma unroll
      for (int w = 0; w < AW; ++w) a[w] = (ok[u] && row_ok) ? ar[u][w] : z;
      if constexpr (MODE == MODE_INT4) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4(a[0].x, a[0].y), widen_w_a4(wv.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4(a[0].z, a[0].w), widen_w_a4(wv.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4(a[1].x, a[1].y), widen_w_a4(wv.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4(a[1].z, a[1].w), widen_w_a4(wv.w), acc, 0, 0, 0);
      } else if constexpr (MODE == MODE_INT8) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(a[0]), widen_w_a8(wv.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(a[1]), widen_w_a8(wv.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(a[2]), widen_w_a8(wv.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(a[3]), widen_w_a8(wv.w), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(a[0].x, a[0].y, a[0].z, a[0].w),
                                                               fp4_weights(wv.x, wv.y), acc, 4, 4, 0, 127, 0, 127);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(a[1].x, a[1].y, a[1].z, a[1].w),
                                                               fp4_weights(wv.z, wv.w), acc, 4, 4, 0, 127, 0, 127);
      }
    }
  }

  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc_t s = part[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const acc_t p = part[w][lane];
    s[0] += p[0]; s[1] += p[1]; s[2] += p[2]; s[3] += p[3];
  }
  const int64_t n = n_out;
  // output plane of this column: columns [p*split, (p+1)*split) go to the
  // row-major [M][split] plane p (split = N: the plain [M][N] layout)
  const int64_t plane = n / split;
  float* __restrict__ yp = y + plane * M * split;
  const int64_t nc = n - plane * split;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * g + e;
    if (m >= M) continue;
    float accf;
    if constexpr (MODE == MODE_FP4) {
      accf = s[e];
      if (acc_dbg) static_cast<float*>(acc_dbg)[m * N + n] = accf;
    } else {
      const int32_t a = s[e] >> acc_shift<MODE>();
      if (acc_dbg) static_cast<int32_t*>(acc_dbg)[m * N + n] = a;
      accf = static_cast<float>(a);
    }
    float o = dequant(accf, sxm[e], bn);
    if (resid) o = o + resid[m * N + n];  // residual: one fp32 rounding
    yp[m * split + nc] = o;
  }
}

template <int MODE>
void launch_waves(int waves, const uint8_t* A, const float* sx, int m, int64_t K, const uint8_t* w,
                  const float* beta, int64_t N, float* y, void* acc_dbg, const float* resid, int64_t split,
                  hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(N / 16));
  if (waves == 8) {
    hipLaunchKernelGGL((k_gemv<MODE, 8>), grid, dim3(512), 0, s, A, sx, m, K, w, beta, N, y, acc_dbg, resid, split);
  } else {
    hipLaunchKernelGGL((k_gemv<MODE, 4>), grid, dim3(256), 0, s, A, sx, m, K, w, beta, N, y, acc_dbg, resid, split);
  }
}

// Waves per workgroup.  Measured at M = 1 over 32 layers: 8 waves help only
// where the grid is small and K long (down_proj, N = 4096, K = 11008:
// 8.3 -> 7.3 us); at K = 4096 (q/k/v, out_proj) and at N = 22016 (gate/up)
// 4-wave workgroups, several per CU, are faster, and 16 waves are slower
// everywhere.
int gemv_waves(int64_t K, int64_t N) {
  const int64_t T = K >> 6;
  const int64_t blocks = N / 16;
  return (blocks <= 512 && T >= 128) ? 8 : 4;
}

}  // namespace

hipError_t launch_gemv_ex(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                          const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                          const float* resid, int64_t split, hipStream_t s) {
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  const int m = static_cast<int>(M);
  const int waves = gemv_waves(K, N);
  switch (mode) {
    case MODE_INT4:
      launch_waves<MODE_INT4>(waves, A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
    case MODE_FP4:
      launch_waves<MODE_FP4>(waves, A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
    default:
      launch_waves<MODE_INT8>(waves, A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                       const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                       hipStream_t s) {
  return launch_gemv_ex(mode, codes, sx, M, K, w_packed, beta, N, y, acc_dbg, nullptr, N, s);
}

}  // namespace bw
