// Prefill-shape BitLinear (M > 16 tokens) for gfx950: MFMA-bound contraction.
// This register-staged kernel serves the shapes the LDS-streaming kernel
// (gemm_lds.hip) does not take: K not a multiple of 128, or operands of 2 GiB
// and more.
//
// BitNet a4.8 abstract: ternary layers consume 4-bit activations (INT4/FP4
// kernels) and sparsified 8-bit states.
//
//   acc[m][n] = sum_k v(code[m][k]) * t[n][k],   y = fl(fl(acc * sx[m]) * beta[n])
//
// Workgroup tile 128 tokens x 256 channels, eight waves (2 x 4) of 64 x 64,
// each holding 2 x 2 accumulator tiles of 32 x 32.  The small per-wave tile
// keeps a wave under 128 VGPRs, so four waves share each SIMD and hide each
// other's LDS and barrier waits; the operand widening it costs (about six
// VALU ops per MFMA) co-issues with the matrix instructions.  A stage brings
// 128 k of packed activations and weights into LDS
// through registers, double-buffered with one barrier per stage; operands are
// widened in registers right before v_mfma_i32_32x32x32_i8 (INT4/INT8 codes)
// or v_mfma_scale_f32_32x32x64_f8f6f4 (e2m1 codes; block scales 2^0 for the
// activations, 2^-1 for the weights, which enter as +-2.0).
// LDS rows are padded (A by 16 bytes, B by 8) so the 32 lanes of a fragment
// read hit distinct banks.  Tiles are numbered so that each of the 8 XCDs
// (workgroup id mod 8) works through a contiguous range of tiles.
#include "bw_internal.h"
#include "bw_widen.h"

namespace bw {
namespace {

constexpr int WM = 2;                    // wave rows
constexpr int WN = 4;                    // wave columns
constexpr int kThreads = 64 * WM * WN;   // 512
constexpr int BM = WM * 64;              // 128 tokens
constexpr int BN = WN * 64;              // 256 channels

template <int MODE>
struct Cfg {
  static constexpr int SLABS = 2;                                 // 64-k slabs per stage
  static constexpr int AB = (MODE == MODE_INT8) ? 64 : 32;        // A bytes per row per slab
  static constexpr int AROW = AB * SLABS;                         // A bytes per row per stage
  static constexpr int ASTR = AROW + 16;                          // padded LDS row stride
  static constexpr int BROW = 16 * SLABS;                         // B bytes per column per stage
  static constexpr int BSTR = BROW + 8;                           // padded LDS column stride
  static constexpr int ACH = BM * AROW / 16 / kThreads;           // 16-B A chunks per thread
  static constexpr int BCHUNKS = BN * SLABS;                      // 16-B B chunks per stage
  static constexpr int BCH = (BCHUNKS + kThreads - 1) / kThreads;  // per thread (last may idle)
  static_assert(ACH * 16 * kThreads == BM * AROW, "A stage must split evenly");
};

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemm(const uint8_t* __restrict__ A,
                                                   const float* __restrict__ sx, int64_t M, int64_t K,
                                                   const uint8_t* __restrict__ Wp,
                                                   const float* __restrict__ beta, int64_t N,
                                                   float* __restrict__ y, void* __restrict__ acc_dbg,
                                                   int MT, int NT) {
  using C = Cfg<MODE>;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * C::ASTR];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * C::BSTR];
  __shared__ float sxs[BM];  // token scales of this tile (read by the epilogue)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 31;
  const int lh = lane >> 5;

  // XCD-aware tile order: workgroups b, b+8, b+16, ... share an XCD
  const int T = MT * NT;
  const int b = blockIdx.x;
  const int t = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int64_t m0 = static_cast<int64_t>(t % MT) * BM;
  const int64_t n0 = static_cast<int64_t>(t / MT) * BN;

  const int64_t kblocks = K >> 6;
  const int64_t nst = (kblocks + C::SLABS - 1) / C::SLABS;
  const int64_t a_row = (MODE == MODE_INT8) ? K : (K >> 1);

  uint4 ra[C::ACH];
  uint4 rb[C::BCH];

  auto gload = [&](int64_t st) {
#pragma unroll
    for (int c = 0; c < C::ACH; ++c) {
      const int q = tid + c * kThreads;
      const int row = q / (C::AROW / 16);
      const int part = q % (C::AROW / 16);
      const int64_t gm = m0 + row;
      const int64_t kb = st * C::SLABS + part / (C::AB / 16);
      ra[c] = (gm < M && kb < kblocks)
                  ? *reinterpret_cast<const uint4*>(A + gm * a_row + st * C::AROW + part * 16)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < C::BCH; ++c) {
      const int q = tid + c * kThreads;
      const int col = q / C::SLABS;
      const int slab = q % C::SLABS;
      const int64_t gn = n0 + col;
      const int64_t kb = st * C::SLABS + slab;
      rb[c] = (q < C::BCHUNKS && gn < N && kb < kblocks)
                  ? *reinterpret_cast<const uint4*>(Wp + ((gn >> 4) * kblocks + kb) * 256 + (gn & 15) * 16)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < C::ACH; ++c) {
      const int q = tid + c * kThreads;
      const int row = q / (C::AROW / 16);
      const int part = q % (C::AROW / 16);
      *reinterpret_cast<uint4*>(&As[buf][row * C::ASTR + part * 16]) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < C::BCH; ++c) {
      const int q = tid + c * kThreads;
      if (q >= C::BCHUNKS) continue;
      const int col = q / C::SLABS;
      const int slab = q % C::SLABS;
      // the column stride is a multiple of 8 bytes: two 8-byte stores
      *reinterpret_cast<uint2*>(&Bs[buf][col * C::BSTR + slab * 16]) = make_uint2(rb[c].x, rb[c].y);
      *reinterpret_cast<uint2*>(&Bs[buf][col * C::BSTR + slab * 16 + 8]) = make_uint2(rb[c].z, rb[c].w);
    }
  };

  using acc_t = typename std::conditional<MODE == MODE_FP4, v16f, v16i>::type;
  acc_t acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0;

  if (tid < BM) sxs[tid] = sx[(m0 + tid < M) ? m0 + tid : M - 1];
  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int cur = static_cast<int>(st & 1);
    if (st + 1 < nst) gload(st + 1);
#pragma unroll
    for (int s = 0; s < C::SLABS; ++s) {
      uint2 wq[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wn * 64 + c * 32 + li;
        wq[c] = *reinterpret_cast<const uint2*>(&Bs[cur][col * C::BSTR + s * 16 + 8 * lh]);
      }
      if constexpr (MODE == MODE_INT4) {
        const v4i b00 = widen_w_a4(wq[0].x), b01 = widen_w_a4(wq[0].y);
        const v4i b10 = widen_w_a4(wq[1].x), b11 = widen_w_a4(wq[1].y);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = wm * 64 + r * 32 + li;
          const uint4 x = *reinterpret_cast<const uint4*>(&As[cur][row * C::ASTR + s * 32 + 16 * lh]);
          const v4i a0 = widen_int4(x.x, x.y);
          const v4i a1 = widen_int4(x.z, x.w);
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b00, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b10, acc[r][1], 0, 0, 0);
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b01, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b11, acc[r][1], 0, 0, 0);
        }
      } else if constexpr (MODE == MODE_INT8) {
        const v4i b00 = widen_w_a8(wq[0].x), b01 = widen_w_a8(wq[0].y);
        const v4i b10 = widen_w_a8(wq[1].x), b11 = widen_w_a8(wq[1].y);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = wm * 64 + r * 32 + li;
          const uint4 x0 = *reinterpret_cast<const uint4*>(&As[cur][row * C::ASTR + s * 64 + 32 * lh]);
          const uint4 x1 = *reinterpret_cast<const uint4*>(&As[cur][row * C::ASTR + s * 64 + 32 * lh + 16]);
          const v4i a0 = as_v4i(x0);
          const v4i a1 = as_v4i(x1);
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b00, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b10, acc[r][1], 0, 0, 0);
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b01, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b11, acc[r][1], 0, 0, 0);
        }
      } else {
        const v8i b0 = fp4_weights(wq[0].x, wq[0].y);
        const v8i b1 = fp4_weights(wq[1].x, wq[1].y);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = wm * 64 + r * 32 + li;
          const uint4 x = *reinterpret_cast<const uint4*>(&As[cur][row * C::ASTR + s * 32 + 16 * lh]);
          const v8i a = fp4_operand(x.x, x.y, x.z, x.w);
          acc[r][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b0, acc[r][0], 4, 4, 0, 127, 0, kE2m1WeightScale);
          acc[r][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b1, acc[r][1], 4, 4, 0, 127, 0, kE2m1WeightScale);
        }
      }
    }
    if (st + 1 < nst) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32) and rows
  // 8*(e/4) + 4*(lane/32) + (e%4) for its 16 elements e.  Token scales come
  // from LDS (staged at kernel start); the two channel scales are loaded
  // together before any store.
  float bn[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t gn = n0 + wn * 64 + c * 32 + li;
    bn[c] = beta[gn < N ? gn : N - 1];
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t gn = n0 + wn * 64 + c * 32 + li;
    if (gn >= N) continue;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t gm = m0 + wm * 64 + r * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (gm >= M) continue;
        float accf;
        if constexpr (MODE == MODE_FP4) {
          accf = acc[r][c][e];
          if (acc_dbg) static_cast<float*>(acc_dbg)[gm * N + gn] = accf;
        } else {
          const int32_t a = acc[r][c][e] >> acc_shift<MODE>();
          if (acc_dbg) static_cast<int32_t*>(acc_dbg)[gm * N + gn] = a;
          accf = static_cast<float>(a);
        }
        y[gm * N + gn] = dequant(accf, sxs[wm * 64 + r * 32 + 8 * (e >> 2) + 4 * lh + (e & 3)], bn[c]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                       const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                       hipStream_t s) {
  if (gemm_lds_supported(mode, M, K, N)) return launch_gemm_lds(mode, codes, sx, M, K, w_packed, beta, N, y, acc_dbg, s);
  const int MT = static_cast<int>((M + BM - 1) / BM);
  const int NT = static_cast<int>((N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(MT * NT)), block(kThreads);
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  switch (mode) {
    case MODE_INT4:
      hipLaunchKernelGGL(k_gemm<MODE_INT4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
    case MODE_FP4:
      hipLaunchKernelGGL(k_gemm<MODE_FP4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
    default:
      hipLaunchKernelGGL(k_gemm<MODE_INT8>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
  }
  return hipGetLastError();
}

}  // namespace bw
