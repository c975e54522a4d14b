// Decode-shape BitLinear (M <= 16 tokens) for gfx950: streams the 2-bit
// weights once from HBM.
//
// BitNet a4.8 abstract: ternary layers on 4-bit activations (INT4/FP4
// kernels) and on 8-bit sparsified states.  At decode the weight bytes are
// the whole cost, so the kernel is shaped for HBM streaming:
//   * one workgroup per 16 output channels (one packed tile column); its
//     K/64 tiles are one contiguous run of K*4 bytes;
//   * the waves split the tiles; a wave's lane group g (16 lanes) reads tile
//     base+g, so one wave load moves 1 KB of contiguous weights, 16 B per lane;
//     each lane keeps two tiles' loads in flight per round (4 waves for 4-bit
//     codes, 8 for INT8 codes, whose activation operand is twice as wide);
//   * every load is a buffer load through a resource that covers exactly its
//     operand: lanes whose token row is past M, or whose tile is past the
//     wave's range, use an out-of-range offset and read zeros without a
//     memory access (no clamped re-reads, no selects after the load).  INT8
//     activation loads are issued only by the lanes of real rows;
//   * the tokens (zero-padded to 16) are the rows of 16x16 MFMAs (i8 16x16x64,
//     or scaled f8f6f4 16x16x128 for e2m1 codes and for INT4 values stored as
//     e2m3 fields; those use the weights as e2m1 +-2.0 by one mask, so a
//     4-tile round costs a few VALU operations instead of widening every
//     nibble and 2-bit code to a byte, and the fp32 sums are exact integers);
//   * the waves' partial int32/fp32 tiles are summed through LDS (exact) and
//     the epilogue writes y for the M real rows; optionally it adds a residual
//     (y = r + W x, the decoder layer's skip connections) and splits the
//     columns into row-major planes (a fused gate/up product written as two
//     [M][F] arrays).
//
// Quantize + GEMV in one launch (M <= 2): every workgroup quantizes the M
// token rows itself (thread t holds chunks t + 256 i of 8 elements of every
// row; row maxima by DPP and one LDS exchange), writes the codes to LDS and
// contracts them there; the x loads are issued before the weight loads and
// the quantization runs while the weights are in flight.  Workgroup 0 also
// stores the codes and scales.  The codes are the standalone quantizer's
// (same absmax, same correctly-rounded operations).
#include "bw_internal.h"
#include "bw_quant.h"
#include "bw_widen.h"

namespace bw {
namespace {

template <int MODE>
struct TileOps {
  // 16-byte activation parts per tile: 64 codes of 8, 6 (e2m3 fields) or 4 bits
  static constexpr int AW = (MODE == MODE_INT8) ? 4 : (MODE == MODE_E2M3) ? 3 : 2;
  using acc_t = typename std::conditional<MODE == MODE_FP4 || MODE == MODE_E2M3, v4f, v4i>::type;
};

// One 64-k tile of lane group g: activation parts a (this lane's token row) x
// the lane's 16 bytes of packed weights.
template <int MODE>
__device__ __forceinline__ void mfma_tile(typename TileOps<MODE>::acc_t& acc, const uint4 (&a)[TileOps<MODE>::AW],
                                          uint4 wv) {
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
  } else if constexpr (MODE == MODE_E2M3) {
    // the tile's 48 bytes: the first 16 bytes of the fields of values 0..31,
    // the same of values 32..63, then the last 8 bytes of each.  An fp6
    // operand is the first six words of its vector, so each is the
    // concatenation of one 16-byte part and the tail part (words 6, 7 unused)
    const v4i p0 = as_v4i(a[0]), p1 = as_v4i(a[1]), p2 = as_v4i(a[2]);
    const v8i x0 = __builtin_shufflevector(p0, p2, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i x1 = __builtin_shufflevector(p1, p2, 0, 1, 2, 3, 6, 7, 4, 5);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x0, fp4_weights(wv.x, wv.y), acc, 2, 4, 0, kE2m3ActScale, 0,
                                                           kE2m1WeightScale);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x1, fp4_weights(wv.z, wv.w), acc, 2, 4, 0, kE2m3ActScale, 0,
                                                           kE2m1WeightScale);
  } else {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(a[0].x, a[0].y, a[0].z, a[0].w),
                                                           fp4_weights(wv.x, wv.y), acc, 4, 4, 0, 127, 0,
                                                           kE2m1WeightScale);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(a[1].x, a[1].y, a[1].z, a[1].w),
                                                           fp4_weights(wv.z, wv.w), acc, 4, 4, 0, 127, 0,
                                                           kE2m1WeightScale);
  }
}

// Sum of the waves' partial tiles and the epilogue (16x16 accumulator layout:
// lane holds column lane % 16, rows 4 * (lane / 16) + e).
template <int MODE, int WAVES>
__device__ __forceinline__ void gemv_epilogue(typename TileOps<MODE>::acc_t acc,
                                              typename TileOps<MODE>::acc_t (&part)[WAVES][64], int M, int64_t N,
                                              int64_t nb, const float (&sxm)[4], float bn, float* __restrict__ y,
                                              void* __restrict__ acc_dbg, const float* __restrict__ resid,
                                              int64_t split) {
  using acc_t = typename TileOps<MODE>::acc_t;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc_t s = part[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const acc_t p = part[w][lane];
    s[0] += p[0]; s[1] += p[1]; s[2] += p[2]; s[3] += p[3];
  }
  const int g = lane >> 4;
  const int64_t n = nb * 16 + (lane & 15);
  // output plane of this column: columns [p*split, (p+1)*split) go to the
  // row-major [M][split] plane p (split = N: the plain [M][N] layout; 32-bit
  // division, N < 2^31)
  const int64_t plane =
      (split == N) ? 0 : static_cast<int64_t>(static_cast<uint32_t>(n) / static_cast<uint32_t>(split));
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
    } else if constexpr (MODE == MODE_E2M3) {
      accf = s[e];  // an exact integer: |sum q*t| <= 8K < 2^24
      if (acc_dbg) static_cast<int32_t*>(acc_dbg)[m * N + n] = static_cast<int32_t>(accf);
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

template <int MODE, int WAVES, int UNR>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(const uint8_t* __restrict__ A, const float* __restrict__ sx,
                                                   int M, int64_t K, const uint8_t* __restrict__ Wp,
                                                   const float* __restrict__ beta, int64_t N, float* __restrict__ y,
                                                   void* __restrict__ acc_dbg, const float* __restrict__ resid,
                                                   int64_t split) {
  using Ops = TileOps<MODE>;
  constexpr int AW = Ops::AW;
  __shared__ typename Ops::acc_t part[WAVES][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;  // token row (A) / output channel (B) of this lane
  const int g = lane >> 4;   // lane group: which tile of a group of four
  const int64_t nb = blockIdx.x;
  const int64_t T = K >> 6;  // tiles along K
  const int64_t a_row = 16 * AW * T;
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wp + nb * T * 256, T * 256);
  const __amdgpu_buffer_rsrc_t ar = rsrc(A, M * a_row);
  const bool row_ok = li < M;
  const uint32_t a_base = row_ok ? static_cast<uint32_t>(li * a_row) : 0u;

  // wave w handles tiles [t0, t1)
  const int64_t per = (T + WAVES - 1) / WAVES;
  const int64_t t0 = wave * per;
  const int64_t t1 = (t0 + per < T) ? t0 + per : T;

  // epilogue scales first, so their latency hides under the weight stream
  const float bn = beta[nb * 16 + li];
  float sxm[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sxm[e] = sx[(4 * g + e < M) ? 4 * g + e : 0];

  typename Ops::acc_t acc;
  acc[0] = 0; acc[1] = 0; acc[2] = 0; acc[3] = 0;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t base = t0; base < t1; base += 4 * UNR) {
    uint4 wv[UNR];
    uint4 av[UNR][AW];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t kt = base + 4 * u + g;
      const bool ok = kt < t1;
      wv[u] = bload16(wr, ok ? static_cast<uint32_t>(kt * 256 + li * 16) : kOutOfRange);
      if constexpr (MODE == MODE_INT8) {
        // 64-byte activation parts: only the lanes of real rows load
#pragma unroll
        for (int w = 0; w < AW; ++w) av[u][w] = z;
        if (ok && row_ok) {
#pragma unroll
          for (int w = 0; w < AW; ++w) av[u][w] = bload16(ar, a_base + static_cast<uint32_t>(kt * (16 * AW) + 16 * w));
        }
      } else {
#pragma unroll
        for (int w = 0; w < AW; ++w)
          av[u][w] = bload16(ar, (ok && row_ok) ? a_base + static_cast<uint32_t>(kt * (16 * AW) + 16 * w)
                                                : kOutOfRange);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) mfma_tile<MODE>(acc, av[u], wv[u]);
  }
  gemv_epilogue<MODE, WAVES>(acc, part, M, N, nb, sxm, bn, y, acc_dbg, resid, split);
}

// Quantize the M (<= MR) token rows of x in every workgroup, then contract.
// CPR chunks of 8 elements per thread and row (K <= 2048 * CPR).
template <int FMT, bool BF16, int MR, int CPR>
__global__ __launch_bounds__(256) void k_gemv_quant(const void* __restrict__ X, int M, int64_t K,
                                                    const uint8_t* __restrict__ Wp, const float* __restrict__ beta,
                                                    int64_t N, float* __restrict__ y, uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales, void* __restrict__ acc_dbg,
                                                    const float* __restrict__ resid, int64_t split) {
  constexpr int MODE = (FMT == 0) ? MODE_INT4 : MODE_FP4;
  constexpr int WAVES = 4, UNR = 4;
  constexpr int XW = BF16 ? 1 : 2;  // 16-byte loads per chunk of 8 elements
  using Ops = TileOps<MODE>;
  __shared__ typename Ops::acc_t part[WAVES][64];
  __shared__ uint32_t s_wmax[MR][WAVES];
  __shared__ float s_sx[MR];
  extern __shared__ __attribute__((aligned(16))) uint8_t s_codes[];  // [M][K/2 + 16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int64_t nb = blockIdx.x;
  const int64_t T = K >> 6;
  const int nch = static_cast<int>(K >> 3);
  const int cstride = static_cast<int>(K >> 1) + 16;  // padded row of codes (16-byte aligned)

  // x rows first (chunks past the row or rows past M read zeros, no access)
  const __amdgpu_buffer_rsrc_t xr = rsrc(X, M * K * (BF16 ? 2 : 4));
  uint4 xv[MR][CPR][XW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int c = tid + 256 * i;
      const bool in = m < M && c < nch;
#pragma unroll
      for (int h = 0; h < XW; ++h)
        xv[m][i][h] = bload16(xr, in ? static_cast<uint32_t>((m * K + c * 8) * (BF16 ? 2 : 4) + 16 * h) : kOutOfRange);
    }
  asm volatile("" ::: "memory");
  // then the first round of weights and the epilogue's beta
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wp + nb * T * 256, T * 256);
  const int64_t per = (T + WAVES - 1) / WAVES;
  const int64_t t0 = wave * per;
  const int64_t t1 = (t0 + per < T) ? t0 + per : T;
  uint4 wv0[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int64_t kt = t0 + 4 * u + g;
    wv0[u] = bload16(wr, kt < t1 ? static_cast<uint32_t>(kt * 256 + li * 16) : kOutOfRange);
  }
  const float bn = beta[nb * 16 + li];
  // keep the quantization below the weight loads: it waits for x only
  __builtin_amdgcn_sched_barrier(0);

  // element e (0..7) of a chunk as fp32
  auto elem = [&](const uint4 (&v)[XW], int e) -> float {
    if constexpr (BF16) {
      const uint32_t w = (e < 2) ? v[0].x : (e < 4) ? v[0].y : (e < 6) ? v[0].z : v[0].w;
      return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
      const uint4 q = v[e >> 2];
      const uint32_t w = ((e & 3) == 0) ? q.x : ((e & 3) == 1) ? q.y : ((e & 3) == 2) ? q.z : q.w;
      return __uint_as_float(w);
    }
  };
  // row maxima of |x| (as bits: non-negative floats order as integers)
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < CPR; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = max(amax, __float_as_uint(elem(xv[m][i], e)) & 0x7FFFFFFFu);
    amax = wave_incl_umax(amax);
    if (lane == 63) s_wmax[m][wave] = amax;
  }
  __syncthreads();
  constexpr float qmax = act4_qmax<FMT>();
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t amax = s_wmax[m][0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) amax = max(amax, s_wmax[m][w]);
    const float a = fmaxf(__uint_as_float(amax), 1e-5f);
    const float inv = div_rn(qmax, a);
    if (tid == 0 && m < M) {
      const float sc = div_rn(a, qmax);
      s_sx[m] = sc;
      if (nb == 0) scales[m] = sc;
    }
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int c = tid + 256 * i;
      float xe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xe[e] = elem(xv[m][i], e);
      const uint32_t word = act4_word<FMT>(xe, inv);
      if (m < M && c < nch) {
        *reinterpret_cast<uint32_t*>(s_codes + m * cstride + c * 4) = word;
        if (nb == 0) reinterpret_cast<uint32_t*>(codes + m * (K >> 1))[c] = word;
      }
    }
  }
  __syncthreads();

  float sxm[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sxm[e] = s_sx[(4 * g + e < M) ? 4 * g + e : 0];
  typename Ops::acc_t acc;
  acc[0] = 0; acc[1] = 0; acc[2] = 0; acc[3] = 0;
  const bool row_ok = li < M;
  const uint4* __restrict__ arow = reinterpret_cast<const uint4*>(s_codes + (row_ok ? li : 0) * cstride);
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t base = t0; base < t1; base += 4 * UNR) {
    uint4 wv[UNR];
    if (base == t0) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) wv[u] = wv0[u];
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t kt = base + 4 * u + g;
        wv[u] = bload16(wr, kt < t1 ? static_cast<uint32_t>(kt * 256 + li * 16) : kOutOfRange);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t kt = base + 4 * u + g;
      const bool ok = row_ok && kt < t1;
      uint4 av[2];
      av[0] = ok ? arow[2 * kt] : z;
      av[1] = ok ? arow[2 * kt + 1] : z;
      mfma_tile<MODE>(acc, av, wv[u]);
    }
  }
  gemv_epilogue<MODE, WAVES>(acc, part, M, N, nb, sxm, bn, y, acc_dbg, resid, split);
}

constexpr int64_t kGemvWideN = 16384;

template <int MODE, int WAVES>
void launch_modes(const uint8_t* A, const float* sx, int m, int64_t K, const uint8_t* w, const float* beta,
                  int64_t N, float* y, void* acc_dbg, const float* resid, int64_t split, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv<MODE, WAVES, 2>), dim3(static_cast<unsigned>(N / 16)), dim3(64 * WAVES), 0, s, A, sx, m,
                     K, w, beta, N, y, acc_dbg, resid, split);
}

template <int FMT, bool BF16, int MR>
void launch_quant_cpr(const void* x, int m, int64_t K, const uint8_t* w, const float* beta, int64_t N, float* y,
                      uint8_t* codes, float* scales, void* acc_dbg, const float* resid, int64_t split,
                      hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(N / 16)), block(256);
  const size_t lds = static_cast<size_t>(m) * ((K >> 1) + 16);
  const int64_t cpr = (K + 2047) / 2048;
#define BW_GQ(C)                                                                                                    \
  hipLaunchKernelGGL((k_gemv_quant<FMT, BF16, MR, C>), grid, block, lds, s, x, m, K, w, beta, N, y, codes, scales, \
                     acc_dbg, resid, split)
  if (cpr <= 1) BW_GQ(1);
  else if (cpr <= 2) BW_GQ(2);
  else if (cpr <= 3) BW_GQ(3);
  else BW_GQ(4);
#undef BW_GQ
}

template <int FMT, bool BF16>
void launch_quant_m(const void* x, int m, int64_t K, const uint8_t* w, const float* beta, int64_t N, float* y,
                    uint8_t* codes, float* scales, void* acc_dbg, const float* resid, int64_t split, hipStream_t s) {
  if (m <= 1) launch_quant_cpr<FMT, BF16, 1>(x, m, K, w, beta, N, y, codes, scales, acc_dbg, resid, split, s);
  else launch_quant_cpr<FMT, BF16, 2>(x, m, K, w, beta, N, y, codes, scales, acc_dbg, resid, split, s);
}

}  // namespace

hipError_t launch_gemv_ex(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                          const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                          const float* resid, int64_t split, hipStream_t s) {
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  const int m = static_cast<int>(M);
  // 4-bit codes: four waves split K; from N = 16384 on (1024 workgroups and
  // more, e.g. the fused gate/up width) eight waves, measured faster there and
  // slower on the 768 workgroups of the fused q/k/v width
  const bool wide = N >= kGemvWideN;
  switch (mode) {
    case MODE_INT4:
      if (wide) launch_modes<MODE_INT4, 8>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      else launch_modes<MODE_INT4, 4>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
    case MODE_FP4:
      launch_modes<MODE_FP4, 4>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
    case MODE_E2M3:
      if (wide) launch_modes<MODE_E2M3, 8>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      else launch_modes<MODE_E2M3, 4>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
    default:
      launch_modes<MODE_INT8, 8>(A, sx, m, K, w_packed, beta, N, y, acc_dbg, resid, split, s);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                       const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                       hipStream_t s) {
  return launch_gemv_ex(mode, codes, sx, M, K, w_packed, beta, N, y, acc_dbg, nullptr, N, s);
}

bool gemv_quant_supported(int64_t M, int64_t K) { return M >= 1 && M <= kGemvQuantMaxM && K <= kGemvQuantMaxK; }

hipError_t launch_gemv_quant(const void* x, bool bf16, int fmt, int64_t M, int64_t K, const uint8_t* w_packed,
                             const float* beta, int64_t N, float* y, uint8_t* codes, float* scales, void* acc_dbg,
                             const float* resid, int64_t split, hipStream_t s) {
  const int m = static_cast<int>(M);
  if (fmt == 0) {
    if (bf16) launch_quant_m<0, true>(x, m, K, w_packed, beta, N, y, codes, scales, acc_dbg, resid, split, s);
    else launch_quant_m<0, false>(x, m, K, w_packed, beta, N, y, codes, scales, acc_dbg, resid, split, s);
  } else {
    if (bf16) launch_quant_m<1, true>(x, m, K, w_packed, beta, N, y, codes, scales, acc_dbg, resid, split, s);
    else launch_quant_m<1, false>(x, m, K, w_packed, beta, N, y, codes, scales, acc_dbg, resid, split, s);
  }
  return hipGetLastError();
}

}  // namespace bw
