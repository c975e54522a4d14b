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

// Field of group g (g < kMaxGroups) without indexing the kernel argument
// array by a variable (which would copy it to scratch).
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[kMaxGroups], int g) {
  static_assert(kMaxGroups == 4, "pick covers four groups");
  return g == 0 ? a[0] : g == 1 ? a[1] : g == 2 ? a[2] : a[3];
}

// Group of grid tile tg (tiles in group order), and tg's index inside it.
__device__ __forceinline__ int group_of(const GemmGroups& G, int tg, int& t_local) {
  int gi = 0;
  if (G.n > 1 && tg >= G.tile_end[0]) gi = 1;
  if (G.n > 2 && tg >= G.tile_end[1]) gi = 2;
  if (G.n > 3 && tg >= G.tile_end[2]) gi = 3;
  t_local = tg - (gi == 0 ? 0 : pick(G.tile_end, gi - 1));
  return gi;
}

// Epilogue of one wave's 64 x 64 accumulator block, y = fl(fl(q * sx) * beta).
// The accumulator tile is y^T: lane l holds token l % 32 and channels
// 8*(e/4) + 4*(l/32) + (e%4) of each 32 x 32 product, so elements 4g..4g+3 are
// four consecutive channels of one token. Stores of that layout write 16-byte
// pieces of 32 rows; instead the block goes through `stage`, LDS that only this
// wave uses, and each store writes whole rows: WIDE = true stages 32 tokens x
// 64 channels (8 KB) per round and stores 4 rows x 256 bytes; WIDE = false
// stages 32 tokens x 32 channels (4 KB) and stores 8 rows x 128 bytes. Every
// lane takes part in every LDS access (no divergent branch around them); the
// 16-byte units of a staged row are XOR-swizzled by the row. LDS accesses of
// one wave complete in issue order.
template <int MODE, bool WIDE, typename AccT>
__device__ __forceinline__ void epilogue_staged(const AccT (&acc)[2][2], uint8_t* stage, int lane, int wm, int wn,
                                                int64_t m0, int64_t n0, int64_t M, int64_t N, const float* sxs,
                                                const float* __restrict__ beta, float* __restrict__ y,
                                                void* __restrict__ acc_dbg) {
  using stage_t = typename std::conditional<MODE == MODE_FP4 || MODE == MODE_E2M3, float4, int4>::type;
  constexpr int ROWB = WIDE ? 256 : 128;   // staged bytes per token
  constexpr int UNITS = ROWB / 16;         // 16-byte units per staged token
  constexpr int LPR = UNITS;               // lanes reading one token
  constexpr int RPI = 64 / LPR;            // tokens per read instruction
  constexpr int NC = WIDE ? 1 : 2;         // rounds over the two 32-channel halves
  const int li = lane & 31;
  const int lh = lane >> 5;
  const int u = lane % LPR;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int cr = 0; cr < NC; ++cr) {
      // write: token li, units of channel halves c (all of them when WIDE)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (!WIDE && c != cr) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int unit = (WIDE ? c * 8 : 0) + 2 * g + lh;
          stage_t v;
          v.x = acc[r][c][4 * g];
          v.y = acc[r][c][4 * g + 1];
          v.z = acc[r][c][4 * g + 2];
          v.w = acc[r][c][4 * g + 3];
          *reinterpret_cast<stage_t*>(stage + li * ROWB + ((unit ^ (li % UNITS)) << 4)) = v;
        }
      }
      const int64_t gn = n0 + wn * 64 + (WIDE ? 0 : cr * 32) + 4 * u;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (gn < N) {
        const float4 bq = *reinterpret_cast<const float4*>(beta + gn);
        bv[0] = bq.x;
        bv[1] = bq.y;
        bv[2] = bq.z;
        bv[3] = bq.w;
      }
      // read: token m, unit u; store 16 bytes of y
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int m = RPI * k + lane / LPR;
        const stage_t v = *reinterpret_cast<const stage_t*>(stage + m * ROWB + ((u ^ (m % UNITS)) << 4));
        const int mt = wm * 64 + r * 32 + m;
        const int64_t gm = m0 + mt;
        const float sm = sxs[mt];
        float o[4];
        if constexpr (MODE == MODE_FP4) {
          if (acc_dbg && gm < M && gn < N) *reinterpret_cast<float4*>(static_cast<float*>(acc_dbg) + gm * N + gn) = v;
          o[0] = dequant(v.x, sm, bv[0]);
          o[1] = dequant(v.y, sm, bv[1]);
          o[2] = dequant(v.z, sm, bv[2]);
          o[3] = dequant(v.w, sm, bv[3]);
        } else if constexpr (MODE == MODE_E2M3) {
          // exact integers in fp32: the int32 accumulator and the same y as the INT4 path
          if (acc_dbg && gm < M && gn < N)
            *reinterpret_cast<int4*>(static_cast<int32_t*>(acc_dbg) + gm * N + gn) =
                make_int4(static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w));
          o[0] = dequant(v.x, sm, bv[0]);
          o[1] = dequant(v.y, sm, bv[1]);
          o[2] = dequant(v.z, sm, bv[2]);
          o[3] = dequant(v.w, sm, bv[3]);
        } else {
          const int32_t q[4] = {v.x >> acc_shift<MODE>(), v.y >> acc_shift<MODE>(), v.z >> acc_shift<MODE>(),
                                v.w >> acc_shift<MODE>()};
          if (acc_dbg && gm < M && gn < N)
            *reinterpret_cast<int4*>(static_cast<int32_t*>(acc_dbg) + gm * N + gn) = make_int4(q[0], q[1], q[2], q[3]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) o[jj] = dequant(static_cast<float>(q[jj]), sm, bv[jj]);
        }
        if (gm < M && gn < N) *reinterpret_cast<float4*>(y + gm * N + gn) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemm_lds(
    const uint8_t* __restrict__ A, const float* __restrict__ sx, int64_t M, int64_t K, const GemmGroups G,
    int MT) {
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

  // XCD-aware tile order over all groups: workgroups b, b+8, b+16, ... share an XCD
  const int T = pick(G.tile_end, G.n - 1);
  const int b = blockIdx.x;
  const int tg = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  int t;
  const int gi = group_of(G, tg, t);
  const uint8_t* __restrict__ const Wp = pick(G.w, gi);
  const float* __restrict__ const beta = pick(G.beta, gi);
  float* __restrict__ const y = pick(G.y, gi);
  void* __restrict__ const acc_dbg = pick(G.acc_dbg, gi);
  const int64_t N = pick(G.N, gi);
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
          acc[r][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a, acc[r][0], 4, 4, 0, kE2m1WeightScale, 0, 127);
          acc[r][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a, acc[r][1], 4, 4, 0, kE2m1WeightScale, 0, 127);
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
  __syncthreads();  // every wave is done with the operand buffers

  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));  // derive the epilogue's indices here, not before the loop
  static_assert(MODE == MODE_INT8 ? (C::AStage >= 16384 && kBStage >= 8192) : (C::AStage >= 8192 && kBStage >= 4096),
                "epilogue staging regions");
  if constexpr (MODE == MODE_INT8) {
    // 8 KB of LDS per wave: waves 2i, 2i+1 take A_i (16 KB each), waves 6, 7 take B0, B1
    uint8_t* const stage = wave < 6 ? (wave < 2 ? A0 : wave < 4 ? A1 : A2) + (wave & 1) * 8192 : (wave == 6 ? B0 : B1);
    epilogue_staged<MODE, true>(acc, stage, lane_e, wm, wn, m0, n0, M, N, sxs, beta, y, acc_dbg);
  } else {
    // 4 KB of LDS per wave: waves 2i, 2i+1 take A_i (8 KB each), waves 6, 7 take B0
    uint8_t* const stage = (wave < 2 ? A0 : wave < 4 ? A1 : wave < 6 ? A2 : B0) + (wave & 1) * 4096;
    epilogue_staged<MODE, false>(acc, stage, lane_e, wm, wn, m0, n0, M, N, sxs, beta, y, acc_dbg);
  }
}


// 4-bit codes with K a multiple of 256, and INT4 values stored as e2m3 fields
// (any K % 64 == 0): stages of 256 k in two LDS buffers.
// The same prefetch window as the three-buffer ring of 128-k stages (stage
// st + 1 loads while stage st computes) with half the workgroup barriers.
// Nibble activation rows hold 128 bytes per stage (eight 16-byte parts,
// swizzled by row / 2).  e2m3 rows hold 192 bytes per stage (twelve 16-byte
// parts) and are stored by bands of 16 rows, part-major: part c of row r at
// (r / 16) * 3072 + c * 256 + (r % 16) * 16, so one wave's copy is 16 rows x
// four parts and the fragment reads of 16 rows are 16 bytes apart (no bank
// conflict).  Weights keep their packed order, four 64-k slabs per column
// group.
// The copies into LDS are issued from inline asm (`lds_copy16`): the
// compiler then adds no wait for them before the fragment reads, which with
// two buffers would stall each stage on the loads just issued for the next;
// the wait for a stage's own copies is explicit (vmcnt before the barrier).
__device__ __forceinline__ int a_slot256(int row, int p) { return p ^ ((row >> 1) & 7); }

constexpr int kGroupRows = 4;  // row tiles per block of the e2m3 tile order

// 16 bytes per lane from a buffer resource into LDS at `lds` + 16 * lane.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_addr), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}

// LDS byte address of a __shared__ pointer (the low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Fragments of one 64-k block: weight words of two columns and the activation
// bits of two rows (16 bytes of nibbles, or 24 bytes of e2m3 fields, each).
template <bool E6>
struct Frag256 {
  uint2 w0, w1;
  uint4 x0, x1;
};
template <>
struct Frag256<true> {
  uint2 w0, w1;
  v8i a0, a1;  // the two rows' e2m3 operands
};

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemm_lds256(
    const uint8_t* __restrict__ A, const float* __restrict__ sx, int64_t M, int64_t K, const GemmGroups G,
    int MT) {
  static_assert(MODE != MODE_INT8, "4-bit codes only");
  constexpr bool E6 = MODE == MODE_E2M3;
  constexpr int AROW = E6 ? 192 : 128;   // bytes per activation row per stage (256 values)
  constexpr int AStage = BM * AROW;      // 24 KB / 16 KB
  constexpr int ACOPIES = AStage / 8192; // 1 KB copies per wave per stage
  constexpr int BStage = BN * 64;        // 16 KB: [group 16][slab 4][column 16] x 16 B
  __shared__ __attribute__((aligned(1024))) uint8_t A0[AStage];
  __shared__ __attribute__((aligned(1024))) uint8_t A1[AStage];
  __shared__ __attribute__((aligned(1024))) uint8_t B0[BStage];
  __shared__ __attribute__((aligned(1024))) uint8_t B1[BStage];
  // Token scales: their own 512 bytes, except for e2m3 rows, whose buffers
  // fill exactly half of the CU's LDS (two workgroups per CU); there the
  // scales go to B1 after the main loop.
  float* sxs;
  if constexpr (E6) {
    sxs = reinterpret_cast<float*>(B1);
  } else {
    __shared__ float sxs_own[BM];
    sxs = sxs_own;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 31;
  const int lh = lane >> 5;

  // XCD-aware tile order over all groups, as in k_gemm_lds
  const int T = pick(G.tile_end, G.n - 1);
  const int b = blockIdx.x;
  const int tg = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  int t;
  const int gi = group_of(G, tg, t);
  const uint8_t* __restrict__ const Wp = pick(G.w, gi);
  const float* __restrict__ const beta = pick(G.beta, gi);
  float* __restrict__ const y = pick(G.y, gi);
  void* __restrict__ const acc_dbg = pick(G.acc_dbg, gi);
  const int64_t N = pick(G.N, gi);
  // Tile -> (row tile, column tile).  e2m3 rows: blocks of kGroupRows row
  // tiles, column by column inside a block, so the tiles an XCD holds at once
  // share both their rows and their columns (its slice of consecutive tiles
  // is about kGroupRows rows by a few columns, not every row).
  int mt = t % MT, nt = t / MT;
  if constexpr (E6 && kGroupRows > 0) {
    const int NT = static_cast<int>((N + BN - 1) / BN);
    const int bm = t / (kGroupRows * NT);
    const int rows = MT - bm * kGroupRows < kGroupRows ? MT - bm * kGroupRows : kGroupRows;
    const int rem = t - bm * kGroupRows * NT;
    mt = bm * kGroupRows + rem % rows;
    nt = rem / rows;
  }
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int64_t n0 = static_cast<int64_t>(nt) * BN;
  const int64_t kblocks = K >> 6;
  const int nst = static_cast<int>((K + 255) >> 8);
  // 64-k blocks in the last stage (K % 256 != 0 happens for e2m3 rows only)
  const int nb_last = (kblocks & 3) ? static_cast<int>(kblocks & 3) : 4;
  const int64_t a_row = E6 ? (K >> 2) * 3 : (K >> 1);

  // A copies.  Nibble rows: copy j of wave w fills rows 8 (2w + j) .. + 7;
  // lane i -> row + i / 8, LDS slot i % 8, which holds the row's part
  // a_slot256(row, i % 8) (an involution).  e2m3 rows: copy j of wave w fills
  // parts 4j .. 4j + 3 of rows 16w .. 16w + 15 (lane i -> row 16w + i % 16,
  // part 4j + i / 16): one lane offset, the copies 64 bytes apart.
  const int64_t m_last = (M - 1 - m0 < BM - 1) ? M - 1 - m0 : BM - 1;
  uint32_t aoff[E6 ? 1 : ACOPIES];
  if constexpr (E6) {
    const int row = 16 * wave + (lane & 15);
    aoff[0] = static_cast<uint32_t>((row < m_last ? row : m_last) * a_row + (lane >> 4) * 16);
  } else {
#pragma unroll
    for (int j = 0; j < ACOPIES; ++j) {
      const int row = 8 * (2 * wave + j) + lane / 8;
      const int part = a_slot256(row, lane % 8);
      aoff[j] = static_cast<uint32_t>((row < m_last ? row : m_last) * a_row + part * 16);
    }
  }
  // B: copy j of wave w fills column group 2w + j (wave-uniform), all four
  // slabs: lane i -> slab i / 16, column i % 16.
  const int64_t ng = N >> 4;
  const int64_t g_first = n0 >> 4;
  const uint32_t boff = static_cast<uint32_t>((lane >> 4) * 256 + (lane & 15) * 16);
  int bgrp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t g0 = 2 * wave + j;
    const int64_t gl = (g_first + g0 < ng) ? g0 : ng - 1 - g_first;
    bgrp[j] = __builtin_amdgcn_readfirstlane(static_cast<int>(gl * kblocks * 256));
  }
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(A + m0 * a_row), 0, static_cast<int>((M - m0) * a_row), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wp + g_first * kblocks * 256), 0, static_cast<int>((ng - g_first) * kblocks * 256),
      kRsrcWord3);
  const int rot = (mt % 4) * (nst / 4);  // as in k_gemm_lds
  auto stage_of = [&](int st) {
    const int sp = st + rot;
    return sp >= nst ? sp - nst : sp;
  };
  // this wave's part of each stage buffer, as wave-uniform (scalar) offsets
  const uint32_t wbase_a = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ACOPIES * wave * 1024));
  const uint32_t wbase_b = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(2 * wave * 1024));
  // The last stage of a K that is not a multiple of 256 (e2m3 rows) holds
  // nb_last < 4 blocks: the copies of the parts and slabs past K read the
  // stage's first part and slab instead, so no copy leaves the row or the
  // column group (the copies are not range-checked against the scalar
  // offset); the blocks they fill are skipped.
  auto issue = [&](int st_req, uint8_t* As, uint8_t* Bs) {
    const int st = stage_of(st_req);
    const int sa = st * AROW;
    const int sb = st * 1024;
    const uint32_t la = lds_addr(As) + wbase_a;
    const uint32_t lb = lds_addr(Bs) + wbase_b;
    if (E6 && nb_last < 4 && st == nst - 1) {
      // derived here (once per workgroup), not kept in registers across the loop
      uint32_t a0 = aoff[0], b0 = boff, q = static_cast<uint32_t>(lane >> 4);
      asm volatile("" : "+v"(a0), "+v"(b0), "+v"(q));
#pragma unroll
      for (int j = 0; j < ACOPIES; ++j) {
        const bool in_k = static_cast<int>(4 * j + q) < 3 * nb_last;
        lds_copy16(arsrc, la + 1024 * j, in_k ? a0 + 64 * j : a0 - 16 * q, sa);
      }
      const uint32_t bo = static_cast<int>(q) < nb_last ? b0 : b0 - 256 * q;
#pragma unroll
      for (int j = 0; j < 2; ++j) lds_copy16(brsrc, lb + 1024 * j, bo, bgrp[j] + sb);
      return;
    }
#pragma unroll
    for (int j = 0; j < ACOPIES; ++j) {
      if constexpr (E6) lds_copy16(arsrc, la + 1024 * j, aoff[0], sa + 64 * j);
      else lds_copy16(arsrc, la + 1024 * j, aoff[j], sa);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) lds_copy16(brsrc, lb + 1024 * j, boff, bgrp[j] + sb);
  };

  using acc_t = typename std::conditional<MODE == MODE_INT4, v16i, v16f>::type;
  acc_t acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0;

  // e2m3 rows: the 48 bytes of 64-k block s are parts 3s, 3s+1, 3s+2 (the
  // first 16 bytes of the fields of values 0..31, the same of values 32..63,
  // then the last 8 of each): this lane's 24 bytes are 16 at e6_x and 8 at
  // e6_y, plus 768 s; row + 32 is two bands further on.
  int e6_x = 0, e6_y = 0;
  if constexpr (E6) {
    const int base = (wm * 4 + (li >> 4)) * 3072 + (li & 15) * 16;
    e6_x = base + 256 * lh;
    e6_y = base + 512 + 8 * lh;
  }

  // Fragments of one 64-k block s of a stage: the weight words of columns
  // wn*64 + li and + 32, and the activation bits of rows wm*64 + li and + 32.
  using Frag = Frag256<E6>;
  auto load_frag = [&](const uint8_t* As, const uint8_t* Bs, int s) {
    Frag f;
    const int col = wn * 64 + li;
    int o0 = ((col >> 4) * 4 + s) * 256 + (col & 15) * 16 + 8 * lh;
    int o1 = o0 + 2048;
    if constexpr (!E6) asm volatile("" : "+v"(o0), "+v"(o1));
    f.w0 = *reinterpret_cast<const uint2*>(Bs + o0);
    f.w1 = *reinterpret_cast<const uint2*>(Bs + o1);
    if constexpr (E6) {
      const uint8_t* p = As + 768 * s;
      const uint4 x0 = *reinterpret_cast<const uint4*>(p + e6_x);
      const uint2 x0t = *reinterpret_cast<const uint2*>(p + e6_y);
      const uint4 x1 = *reinterpret_cast<const uint4*>(p + e6_x + 6144);
      const uint2 x1t = *reinterpret_cast<const uint2*>(p + e6_y + 6144);
      f.a0 = fp6_operand(x0.x, x0.y, x0.z, x0.w, x0t.x, x0t.y);
      f.a1 = fp6_operand(x1.x, x1.y, x1.z, x1.w, x1t.x, x1t.y);
    } else {
      const int row0 = wm * 64 + li;
      const int row1 = row0 + 32;
      f.x0 = *reinterpret_cast<const uint4*>(As + row0 * AROW + 16 * a_slot256(row0, 2 * s + lh));
      f.x1 = *reinterpret_cast<const uint4*>(As + row1 * AROW + 16 * a_slot256(row1, 2 * s + lh));
    }
    return f;
  };
  auto mma_frag = [&](const Frag& f) {
    if constexpr (MODE == MODE_FP4 || MODE == MODE_E2M3) {
      const v8i b0 = fp4_weights(f.w0.x, f.w0.y);
      const v8i b1 = fp4_weights(f.w1.x, f.w1.y);
      if constexpr (E6) {
        const v8i a0 = f.a0;
        const v8i a1 = f.a1;
        acc[0][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a0, acc[0][0], 4, 2, 0, kE2m1WeightScale, 0,
                                                                    kE2m3ActScale);
        acc[0][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a0, acc[0][1], 4, 2, 0, kE2m1WeightScale, 0,
                                                                    kE2m3ActScale);
        acc[1][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a1, acc[1][0], 4, 2, 0, kE2m1WeightScale, 0,
                                                                    kE2m3ActScale);
        acc[1][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a1, acc[1][1], 4, 2, 0, kE2m1WeightScale, 0,
                                                                    kE2m3ActScale);
      } else {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint4 x = r ? f.x1 : f.x0;
          const v8i a = fp4_operand(x.x, x.y, x.z, x.w);
          acc[r][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a, acc[r][0], 4, 4, 0, kE2m1WeightScale, 0, 127);
          acc[r][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a, acc[r][1], 4, 4, 0, kE2m1WeightScale, 0, 127);
        }
      }
    } else {
      const v4i b00 = widen_w_a4(f.w0.x), b01 = widen_w_a4(f.w0.y);
      const v4i b10 = widen_w_a4(f.w1.x), b11 = widen_w_a4(f.w1.y);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint4 x = r ? f.x1 : f.x0;
        const v4i a0 = widen_int4(x.x, x.y);
        const v4i a1 = widen_int4(x.z, x.w);
        acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b00, a0, acc[r][0], 0, 0, 0);
        acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b10, a0, acc[r][1], 0, 0, 0);
        acc[r][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b01, a1, acc[r][0], 0, 0, 0);
        acc[r][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b11, a1, acc[r][1], 0, 0, 0);
      }
    }
  };
  // The four 64-k blocks of a stage, each block's LDS reads issued before the
  // previous block's products (the scheduling barriers keep that order; left to
  // itself the compiler sinks each read next to its first use, which exposes the
  // LDS latency once per block).  nb < 4 only in the last stage of a K that is
  // not a multiple of 256: the blocks past K hold other rows' bytes and are
  // skipped (wave-uniform branch).
  auto compute = [&](const uint8_t* As, const uint8_t* Bs, int nb) {
    if constexpr (E6) {
      const Frag f0 = load_frag(As, Bs, 0);
      const Frag f1 = load_frag(As, Bs, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_frag(f0);
      __builtin_amdgcn_sched_barrier(0);
      const Frag f2 = load_frag(As, Bs, 2);
      __builtin_amdgcn_sched_barrier(0);
      if (nb > 1) mma_frag(f1);
      __builtin_amdgcn_sched_barrier(0);
      const Frag f3 = load_frag(As, Bs, 3);
      __builtin_amdgcn_sched_barrier(0);
      if (nb > 2) mma_frag(f2);
      __builtin_amdgcn_sched_barrier(0);
      if (nb > 3) mma_frag(f3);
    } else {
      Frag f = load_frag(As, Bs, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag g;
        if (s < 3) g = load_frag(As, Bs, s + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_frag(f);
        __builtin_amdgcn_sched_barrier(0);
        f = g;
      }
    }
  };

  if constexpr (!E6) {
    if (tid < BM) sxs[tid] = sx[(m0 + tid < M) ? m0 + tid : M - 1];
  }

  // Stage st: wait for this wave's copies of stage st (none other is in
  // flight), barrier (stage st is complete in LDS and everyone is done with
  // the other buffer), copy stage st + 1 into it, compute stage st.
  issue(0, A0, B0);
  auto step = [&](int st, uint8_t* Ac, uint8_t* Bc, uint8_t* An, uint8_t* Bn) {
    wait_vm<0>();
    block_barrier();
    if (st + 1 < nst) issue(st + 1, An, Bn);
    int nb = 4;
    if constexpr (E6) nb = stage_of(st) == nst - 1 ? nb_last : 4;
    compute(Ac, Bc, nb);
  };
  for (int st = 0; st < nst; st += 2) {
    step(st, A0, B0, A1, B1);
    if (st + 1 < nst) step(st + 1, A1, B1, A0, B0);
  }
  wait_vm<0>();  // (every copy was waited for at its stage)
  __syncthreads();

  // 8 KB of LDS per wave for the epilogue: nibble rows: waves 2i, 2i+1 take
  // A0, A1, B0, B1; e2m3 rows: waves 0-2 take A0, 3-5 A1, 6-7 B0 (the scales
  // are in B1).
  static_assert(AStage >= 16384 && BStage >= 16384, "epilogue staging regions");
  uint8_t* stage;
  if constexpr (E6) {
    if (tid < BM) sxs[tid] = sx[(m0 + tid < M) ? m0 + tid : M - 1];
    __syncthreads();
    stage = (wave < 3 ? A0 + wave * 8192 : wave < 6 ? A1 + (wave - 3) * 8192 : B0 + (wave - 6) * 8192);
  } else {
    stage = (wave < 2 ? A0 : wave < 4 ? A1 : wave < 6 ? B0 : B1) + (wave & 1) * 8192;
  }
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));  // derive the epilogue's indices here, not before the loop
  epilogue_staged<MODE, true>(acc, stage, lane_e, wm, wn, m0, n0, M, N, sxs, beta, y, acc_dbg);
}

}  // namespace

int64_t gemm_lds_tiles(int64_t M, int64_t N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

bool gemm_lds_supported(int mode, int64_t M, int64_t K, int64_t N) {
  const int64_t a_bytes = M * (mode == MODE_INT8 ? K : mode == MODE_E2M3 ? K / 4 * 3 : K / 2);
  const int64_t w_bytes = N * K / 4;
  return K % (mode == MODE_E2M3 ? 64 : 128) == 0 && a_bytes < (int64_t{1} << 31) && w_bytes < (int64_t{1} << 31) &&
         gemm_lds_tiles(M, N) < (int64_t{1} << 30);
}

hipError_t launch_gemm_lds_grouped(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                                   GemmGroups G, hipStream_t s) {
  const int MT = static_cast<int>((M + BM - 1) / BM);
  int T = 0;
  for (int g = 0; g < kMaxGroups; ++g) {
    if (g < G.n) {
      T += MT * static_cast<int>((G.N[g] + BN - 1) / BN);
    } else {  // unused slots: valid values, never selected
      G.w[g] = G.w[0];
      G.beta[g] = G.beta[0];
      G.y[g] = G.y[0];
      G.acc_dbg[g] = G.acc_dbg[0];
      G.N[g] = G.N[0];
    }
    G.tile_end[g] = T;
  }
  const dim3 grid(static_cast<unsigned>(T)), block(kThreads);
  const uint8_t* A = static_cast<const uint8_t*>(codes);
  const bool k256 = K % 256 == 0;
  switch (mode) {
    case MODE_INT4:
      if (k256)
        hipLaunchKernelGGL(k_gemm_lds256<MODE_INT4>, grid, block, 0, s, A, sx, M, K, G, MT);
      else
        hipLaunchKernelGGL(k_gemm_lds<MODE_INT4>, grid, block, 0, s, A, sx, M, K, G, MT);
      break;
    case MODE_FP4:
      if (k256)
        hipLaunchKernelGGL(k_gemm_lds256<MODE_FP4>, grid, block, 0, s, A, sx, M, K, G, MT);
      else
        hipLaunchKernelGGL(k_gemm_lds<MODE_FP4>, grid, block, 0, s, A, sx, M, K, G, MT);
      break;
    case MODE_E2M3:
      hipLaunchKernelGGL(k_gemm_lds256<MODE_E2M3>, grid, block, 0, s, A, sx, M, K, G, MT);
      break;
    default:
      hipLaunchKernelGGL(k_gemm_lds<MODE_INT8>, grid, block, 0, s, A, sx, M, K, G, MT);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_lds(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                           const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                           hipStream_t s) {
  GemmGroups G{};
  G.n = 1;
  G.w[0] = w_packed;
  G.beta[0] = beta;
  G.y[0] = y;
  G.acc_dbg[0] = acc_dbg;
  G.N[0] = N;
  return launch_gemm_lds_grouped(mode, codes, sx, M, K, G, s);
}

}  // namespace bw
