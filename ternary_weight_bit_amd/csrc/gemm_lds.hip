// Prefill-shape BitLinear for gfx950 with operands streamed straight into LDS.
//
// BitNet a4.8 abstract: ternary layers consume 4-bit activations (INT4/FP4
// kernels) and sparsified 8-bit states.
//
//   acc[m][n] = sum_k v(code[m][k]) * t[n][k],   y = fl(fl(acc * sx[m]) * beta[n])
//
// Same tiling as the register-staged kernel (128 tokens x 256 channels per
// workgroup, eight waves of 64 x 64, 2 x 2 tiles of 32 x 32 per wave, stages of
// 128 k), but the global -> LDS copies are buffer_load ... lds operations: the
// data lands in LDS without passing through VGPRs, so there is no register
// staging and no ds_write phase, and the loads of a stage are issued two
// stages ahead into a ring of three LDS buffers (one barrier per stage).
//
//   * Each wave's load writes 1 KB of consecutive LDS (16 bytes per lane), so
//     the LDS layout is fixed by the lane -> source mapping.  Activation rows
//     are unpadded; the 16-byte parts of a row are XOR-swizzled by the row
//     index so that the 32 rows of a fragment read fall in distinct banks.
//     Weights keep their packed order (16 columns x 64 k per 256 bytes).
//   * Load addresses are a scalar base per stage plus a fixed 32-bit lane
//     offset (buffer resource + soffset), so no VGPR is rewritten while a load
//     is in flight.  Rows past M and column groups past N repeat the last
//     valid one, and stages past the end reload the last stage: every access
//     stays inside the operand.
//   * Each LDS buffer is its own object and the fragment reads use explicit
//     offsets, which keeps the compiler's alias information intact: a read of
//     buffer b waits only for the loads into b.
//   * The MFMA operands are (weights, activations), so the accumulator tile is
//     y^T: each group of four accumulator elements holds four consecutive
//     channels of one token, stored as one 16-byte write.
//
// Requirements (checked by the launcher): K a multiple of 128, activation and
// packed-weight byte sizes below 2^31.
#include "bw_internal.h"
#include "bw_widen.h"

namespace bw {
namespace {

constexpr int kThreads = 512;
constexpr int BM = 128;
constexpr int BN = 256;
constexpr int WN = 4;
constexpr int kBStage = BN * 2 * 16;  // [group 16][slab 2][column 16] x 16 B
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

#define BW_GP(p) ((const __attribute__((address_space(1))) void*)(p))
#define BW_LP(p) ((__attribute__((address_space(3))) void*)(p))

template <int MODE>
struct LdsCfg {
  static constexpr int AROW = (MODE == MODE_INT8) ? 128 : 64;  // A bytes per row per stage
  static constexpr int AStage = BM * AROW;
  static constexpr int ALOADS = AStage / (8 * 1024);           // 1 KB loads per wave per stage
  static constexpr int LPS = ALOADS + 1;                       // loads per wave per stage
  static constexpr int PARTS = AROW / 16;
};

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence (the fence would wait for every
// load in flight); the empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Swizzle of the 16-byte part p of activation row `row` (one stage's bytes).
template <int MODE>
__device__ __forceinline__ int a_slot(int row, int p) {
  if constexpr (MODE == MODE_INT8) return p ^ ((row >> 1) & 7);
  else return p ^ ((row >> 2) & 3);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemm_lds(
    const uint8_t* __restrict__ A, const float* __restrict__ sx, int64_t M, int64_t K,
    const uint8_t* __restrict__ Wp, const float* __restrict__ beta, int64_t N, float* __restrict__ y,
    void* __restrict__ acc_dbg, int MT, int NT) {
  using C = LdsCfg<MODE>;
  __shared__ __attribute__((aligned(1024))) uint8_t A0[C::AStage];
  __shared__ __attribute__((aligned(1024))) uint8_t A1[C::AStage];
  __shared__ __attribute__((aligned(1024))) uint8_t A2[C::AStage];
  __shared__ __attribute__((aligned(1024))) uint8_t B0[kBStage];
  __shared__ __attribute__((aligned(1024))) uint8_t B1[kBStage];
  __shared__ __attribute__((aligned(1024))) uint8_t B2[kBStage];
  __shared__ float sxs[BM];

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
  const int64_t nst = kblocks >> 1;
  const int64_t a_row = (MODE == MODE_INT8) ? K : (K >> 1);

  // ---- load sources.  A: load j of wave w fills rows R = 16w + (16/ALOADS) j
  // onward; lane i -> row R + i / PARTS, LDS slot i % PARTS, which holds the
  // row's 16-byte part a_slot(row, i % PARTS) (the swizzle is an involution).
  const int64_t m_last = (M - 1 - m0 < BM - 1) ? M - 1 - m0 : BM - 1;
  uint32_t aoff[C::ALOADS];
#pragma unroll
  for (int j = 0; j < C::ALOADS; ++j) {
    const int row = 16 * wave + (16 / C::ALOADS) * j + lane / C::PARTS;
    const int part = a_slot<MODE>(row, lane % C::PARTS);
    aoff[j] = static_cast<uint32_t>((row < m_last ? row : m_last) * a_row + part * 16);
  }
  // B: wave w fills column groups 2w, 2w+1 for both slabs, in packed order:
  // lane i -> group 2w + i/32, slab (i/16) % 2, column i % 16.
  const int64_t ng = N >> 4;
  const int64_t g_first = n0 >> 4;
  const int64_t g_lane0 = 2 * wave + (lane >> 5);
  const int64_t g_lane = (g_first + g_lane0 < ng) ? g_lane0 : ng - 1 - g_first;
  const uint32_t boff = static_cast<uint32_t>((g_lane * kblocks + ((lane >> 4) & 1)) * 256 + (lane & 15) * 16);

  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A + m0 * a_row), 0, static_cast<int>((M - m0) * a_row), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wp + g_first * kblocks * 256), 0, static_cast<int>((ng - g_first) * kblocks * 256),
      kRsrcWord3);

  // Rows of tiles start their k walk at one of four stage offsets (the sums are
  // exact in any order), so the workgroups in flight do not all read the same
  // k range of cold operands at once; tiles that share activation rows stay in
  // step and share them through L2.
  const int64_t rot = ((t % MT) % 4) * (nst / 4);
  auto issue = [&](int64_t st_req, uint8_t* As, uint8_t* Bs) {
    int64_t sp = (st_req < nst ? st_req : nst - 1) + rot;  // past the end: reload the last stage
    if (sp >= nst) sp -= nst;
    const int st = static_cast<int>(sp);
    // the builtin's operands are plain local values: an array element or a
    // static member in them silently drops the kernel's host-side launch stub
    const int sa = st * C::AROW;
    const int sb = st * 512;
#pragma unroll
    for (int j = 0; j < C::ALOADS; ++j) {
      const uint32_t voff = aoff[j];
      uint8_t* const dst = As + wave * (1024 * C::ALOADS) + 1024 * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, BW_LP(dst), 16, voff, sa, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, BW_LP(Bs + wave * 1024), 16, boff, sb, 0, 0);
  };

  using acc_t = typename std::conditional<MODE == MODE_FP4, v16f, v16i>::type;
  acc_t acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0;

  auto compute = [&](const uint8_t* As, const uint8_t* Bs) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // weight fragments of columns wn*64 + li and +32; the offsets are opaque
      // so each read keeps its own LDS object in the alias information
      const int col = wn * 64 + li;
      int o0 = ((col >> 4) * 2 + s) * 256 + (col & 15) * 16 + 8 * lh;
      int o1 = o0 + 1024;
      asm volatile("" : "+v"(o0), "+v"(o1));
      const uint2 w0 = *reinterpret_cast<const uint2*>(Bs + o0);
      const uint2 w1 = *reinterpret_cast<const uint2*>(Bs + o1);
      if constexpr (MODE == MODE_FP4) {
        const v8i b0 = fp4_weights(w0.x, w0.y);
        const v8i b1 = fp4_weights(w1.x, w1.y);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = wm * 64 + r * 32 + li;
          const uint4 x = *reinterpret_cast<const uint4*>(As + row * 64 + 16 * a_slot<MODE>(row, 2 * s + lh));
          const v8i a = fp4_operand(x.x, x.y, x.z, x.w);
          acc[r][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a, acc[r][0], 4, 4, 0, 127, 0, 127);
          acc[r][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a, acc[r][1], 4, 4, 0, 127, 0, 127);
        }
      } else {
        v4i b00, b01, b10, b11;
        if constexpr (MODE == MODE_INT4) {
          b00 = widen_w_a4(w0.x); b01 = widen_w_a4(w0.y);
          b10 = widen_w_a4(w1.x); b11 = widen_w_a4(w1.y);
        } else {
          b00 = widen_w_a8(w0.x); b01 = widen_w_a8(w0.y);
          b10 = widen_w_a8(w1.x); b11 = widen_w_a8(w1.y);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = wm * 64 + r * 32 + li;
          v4i a0, a1;
          if constexpr (MODE == MODE_INT4) {
            const uint4 x = *reinterpret_cast<const uint4*>(As + row * 64 + 16 * a_slot<MODE>(row, 2 * s + lh));
            a0 = widen_int4(x.x, x.y);
            a1 = widen_int4(x.z, x.w);
          } else {
            a0 = as_v4i(*reinterpret_cast<const uint4*>(As + row * 128 + 16 * a_slot<MODE>(row, 4 * s + 2 * lh)));
            a1 = as_v4i(*reinterpret_cast<const uint4*>(As + row * 128 + 16 * a_slot<MODE>(row, 4 * s + 2 * lh + 1)));
          }
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b00, a0, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b10, a0, acc[r][1], 0, 0, 0);
          acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b01, a1, acc[r][0], 0, 0, 0);
          acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b11, a1, acc[r][1], 0, 0, 0);
        }
      }
    }
  };

  if (tid < BM) sxs[tid] = sx[(m0 + tid < M) ? m0 + tid : M - 1];

  // Ring of three stage buffers.  Stage st: wait for this wave's loads of
  // stage st (those of st + 1 stay in flight), barrier (stage st is complete
  // in LDS and everyone is done with buffer st - 1), issue stage st + 2 into
  // that buffer, compute stage st.  The loop is unrolled by three so every
  // buffer reference is static.
  issue(0, A0, B0);
  issue(1, A1, B1);
  auto step = [&](int64_t st, uint8_t* Ac, uint8_t* Bc, uint8_t* An, uint8_t* Bn) {
    wait_vm<C::LPS>();
    block_barrier();
    issue(st + 2, An, Bn);
    compute(Ac, Bc);
  };
  for (int64_t st = 0; st < nst; st += 3) {
    step(st, A0, B0, A2, B2);
    if (st + 1 < nst) step(st + 1, A1, B1, A0, B0);
    if (st + 2 < nst) step(st + 2, A2, B2, A1, B1);
  }
  wait_vm<0>();  // no load into LDS outlives the workgroup

  // Epilogue.  Accumulator tile = y^T: lane l holds token (l % 32) and channels
  // 8*(e/4) + 4*(l/32) + (e%4), so elements 4g..4g+3 are four consecutive
  // channels of one token.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int mt = wm * 64 + r * 32 + li;
    const int64_t gm = m0 + mt;
    const float sm = sxs[mt];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t gn = n0 + wn * 64 + c * 32 + 8 * g + 4 * lh;
        if (gn >= N || gm >= M) continue;
        const float4 bq = *reinterpret_cast<const float4*>(beta + gn);
        const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
        float o[4];
        if constexpr (MODE == MODE_FP4) {
          if (acc_dbg)
            *reinterpret_cast<float4*>(static_cast<float*>(acc_dbg) + gm * N + gn) =
                make_float4(acc[r][c][4 * g], acc[r][c][4 * g + 1], acc[r][c][4 * g + 2], acc[r][c][4 * g + 3]);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = dequant(acc[r][c][4 * g + j], sm, bv[j]);
        } else {
          int32_t q[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) q[j] = acc[r][c][4 * g + j] >> acc_shift<MODE>();
          if (acc_dbg)
            *reinterpret_cast<int4*>(static_cast<int32_t*>(acc_dbg) + gm * N + gn) = make_int4(q[0], q[1], q[2], q[3]);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = dequant(static_cast<float>(q[j]), sm, bv[j]);
        }
        *reinterpret_cast<float4*>(y + gm * N + gn) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

}  // namespace

bool gemm_lds_supported(int mode, int64_t M, int64_t K, int64_t N) {
  const int64_t a_bytes = M * ((mode == 2) ? K : K / 2);
  const int64_t w_bytes = N * K / 4;
  return K % 128 == 0 && a_bytes < (int64_t{1} << 31) && w_bytes < (int64_t{1} << 31);
}

hipError_t launch_gemm_lds(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                           const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                           hipStream_t s) {
  const int MT = static_cast<int>((M + BM - 1) / BM);
  const int NT = static_cast<int>((N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(MT * NT)), block(kThreads);
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  switch (mode) {
    case MODE_INT4:
      hipLaunchKernelGGL(k_gemm_lds<MODE_INT4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
    case MODE_FP4:
      hipLaunchKernelGGL(k_gemm_lds<MODE_FP4>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
    default:
      hipLaunchKernelGGL(k_gemm_lds<MODE_INT8>, grid, block, 0, s, A, sx, M, K, w_packed, beta, N, y, acc_dbg, MT, NT);
      break;
  }
  return hipGetLastError();
}

}  // namespace bw
