// Single-token W1.58A8 product that reads only the weight rows of the inputs
// that survived sparsification, for gfx950.
//
// BitNet a4.8 abstract: only 55 % of the parameters are active, because the
// inputs of out_proj (top-k at 50 %) and down_proj (ReLU^2 gate) are mostly
// zeros.  toshoseti review, "Method": the kept positions change from token to
// token, so a tiled weight layout cannot skip anything.  With the K-major
// layout (input k owns one contiguous run of N/4 bytes, codes t + 1) a single
// token's product touches only the runs of its nonzero codes, which halves
// the weight bytes at 50 % sparsity.
//
// One launch, grid (segments x column chunks, tokens):
//   * a workgroup takes a segment of up to kMaxSeg inputs of one token and a
//     chunk of kCols = 512 outputs (128 bytes of every row);
//   * it lists the nonzero codes of its segment in LDS (wave ballots, order
//     free: the sum is exact integer arithmetic);
//   * each half-wave (row group) walks every eighth listed row; lane c of the
//     group loads the 4-byte word of outputs 16c..16c+15 of that row, 16 rows
//     in flight, and accumulates q * (t + 1) two outputs per 32-bit register
//     (16-bit fields, exact while a group sees at most 127 rows, which the
//     segment bound guarantees), subtracting sum(q) at the end;
//   * the eight row groups are summed in LDS and added into an int32
//     accumulator in the workspace with device-scope atomics;
//   * the last workgroup of a (token, chunk) -- counted with a wrapping atomic
//     counter -- reads and clears the accumulators and writes
//     y = fl(fl(acc * s_x) * beta).
// The workspace must be zero before the first call; every completed call
// leaves it zero again.
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 512;   // outputs per workgroup
constexpr int kGroups = 8;   // row groups (half-waves) per workgroup
constexpr int kBatch = 16;   // rows per lane with loads in flight together
constexpr int kMaxSeg = 960; // inputs per workgroup: multiple of 64, at most 8 * 127 nonzero
constexpr int kTargetBlocks = 512;

static_assert(kMaxSeg % 64 == 0 && kMaxSeg / 4 <= kThreads, "segment scan: one dword per thread");
static_assert((kMaxSeg + kGroups - 1) / kGroups <= 127, "16-bit accumulator fields");

__global__ __launch_bounds__(kThreads) void k_gather_a8(
    const int8_t* __restrict__ codes, const float* __restrict__ sx, int64_t K,
    const uint8_t* __restrict__ Wk, const float* __restrict__ beta, int64_t N, int seg, int nseg,
    int chunks, float* __restrict__ y, int32_t* __restrict__ acc_dbg, int32_t* __restrict__ acc_ws,
    uint32_t* __restrict__ cnt_ws) {
  __shared__ int2 s_row[kMaxSeg];  // (byte offset of the row, code)
  __shared__ int32_t s_red[kGroups][kCols];
  __shared__ uint32_t s_count;
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t m = blockIdx.y;
  const int chunk = static_cast<int>(blockIdx.x % chunks);
  const int64_t k0 = static_cast<int64_t>(blockIdx.x / chunks) * seg;
  const int64_t k1 = (k0 + seg < K) ? k0 + seg : K;
  const uint32_t row_bytes = static_cast<uint32_t>(N >> 2);

  if (tid == 0) s_count = 0;
  __syncthreads();

  // 1. list the nonzero codes of [k0, k1): four per thread
  const int nq = static_cast<int>((k1 - k0) >> 2);
  const int word = (tid < nq) ? *reinterpret_cast<const int*>(codes + m * K + k0 + 4 * tid) : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = static_cast<int>(static_cast<int8_t>(word >> (8 * j)));
    const bool nz = q != 0;
    const uint64_t bal = __ballot(nz);
    uint32_t base = 0;
    if (lane == 0 && bal != 0) base = atomicAdd(&s_count, static_cast<uint32_t>(__popcll(bal)));
    base = __shfl(base, 0);
    if (nz) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
      const uint32_t k = static_cast<uint32_t>(k0 + 4 * tid + j);
      s_row[base + below] = make_int2(static_cast<int>(k * row_bytes), q);
    }
  }
  __syncthreads();
  const int R = static_cast<int>(s_count);

  // 2. gather: row group g = half-wave, lane c of the group owns 16 outputs
  // Loads are unconditional so that all of a batch is in flight at once: a
  // slot past the list end re-reads listed row 0 with q = 0, and a lane past
  // the last output reads the chunk's first word (its sums are never stored).
  const int g = tid >> 5;
  const int c = tid & 31;
  const bool col_ok = static_cast<int64_t>(chunk) * kCols + 16 * c < N;
  const uint8_t* __restrict__ wchunk = Wk + static_cast<int64_t>(chunk) * (kCols / 4);
  const uint32_t lane_off = col_ok ? 4u * static_cast<uint32_t>(c) : 0u;
  int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // fields: output p (low 16 bits), p + 8 (high)
  int qsum = 0;
  for (int i0 = g; i0 < R; i0 += kGroups * kBatch) {
    uint32_t d[kBatch];
    int qv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + b * kGroups;
      const bool ok = i < R;
      const int2 e = s_row[ok ? i : 0];
      qv[b] = ok ? e.y : 0;
      d[b] = *reinterpret_cast<const uint32_t*>(wchunk + (static_cast<uint32_t>(e.x) + lane_off));
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      qsum += qv[b];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        acc[p] += __mul24(qv[b], static_cast<int>((d[b] >> (2 * p)) & 0x00030003u));
    }
  }

  // 3. unpack the fields, remove the +1 of the codes, sum the row groups
  int sums[16];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int lo = (acc[p] << 16) >> 16;  // exact: |field| < 2^15
    const int hi = (acc[p] - lo) >> 16;
    sums[p] = lo - qsum;
    sums[p + 8] = hi - qsum;
  }
  int4* dst = reinterpret_cast<int4*>(&s_red[g][16 * c]);
#pragma unroll
  for (int v = 0; v < 4; ++v) dst[v] = make_int4(sums[4 * v], sums[4 * v + 1], sums[4 * v + 2], sums[4 * v + 3]);
  __syncthreads();
  const int col = 2 * tid;
  int s0 = 0, s1 = 0;
#pragma unroll
  for (int gg = 0; gg < kGroups; ++gg) {
    const int2 v = *reinterpret_cast<const int2*>(&s_red[gg][col]);
    s0 += v.x;
    s1 += v.y;
  }
  const int64_t n = static_cast<int64_t>(chunk) * kCols + col;
  const bool out_ok = n < N;  // N % 16 == 0: n + 1 < N too
  int32_t* __restrict__ acc_row = acc_ws + m * N;
  if (R > 0 && out_ok) {
    atomicAdd(&acc_row[n], s0);
    atomicAdd(&acc_row[n + 1], s1);
  }

  // 4. the last workgroup of this (token, chunk) finishes the outputs
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t last = static_cast<uint32_t>(nseg - 1);
    s_last = (atomicInc(&cnt_ws[m * chunks + chunk], last) == last) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0) return;
  __threadfence();
  if (out_ok) {
    const int a0 = atomicExch(&acc_row[n], 0);
    const int a1 = atomicExch(&acc_row[n + 1], 0);
    const float s = sx[m];
    float2 out;
    out.x = __fmul_rn(__fmul_rn(static_cast<float>(a0), s), beta[n]);
    out.y = __fmul_rn(__fmul_rn(static_cast<float>(a1), s), beta[n + 1]);
    *reinterpret_cast<float2*>(y + m * N + n) = out;
    if (acc_dbg) *reinterpret_cast<int2*>(acc_dbg + m * N + n) = make_int2(a0, a1);
  }
}

struct GatherGrid {
  int seg, nseg, chunks;
};

GatherGrid gather_grid(int64_t M, int64_t K, int64_t N) {
  GatherGrid gg;
  gg.chunks = static_cast<int>((N + kCols - 1) / kCols);
  const int64_t per_token = static_cast<int64_t>(gg.chunks) * M;
  int64_t want = kTargetBlocks / per_token;  // segments per (token, chunk)
  if (want < 1) want = 1;
  const int64_t blocks64 = K / 64;
  int64_t seg = 64 * ((blocks64 + want - 1) / want);
  if (seg > kMaxSeg) seg = kMaxSeg;
  gg.seg = static_cast<int>(seg);
  gg.nseg = static_cast<int>((K + seg - 1) / seg);
  return gg;
}

}  // namespace

size_t gather_a8_workspace_bytes(int64_t M, int64_t N) {
  const int64_t chunks = (N + kCols - 1) / kCols;
  const size_t bytes = static_cast<size_t>(M) * static_cast<size_t>(N) * 4 + static_cast<size_t>(M * chunks) * 4;
  return (bytes + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_gather_a8(const int8_t* codes, const float* sx, int64_t M, int64_t K, const uint8_t* w_kmajor,
                            const float* beta, int64_t N, float* y, int32_t* acc_dbg, void* ws, hipStream_t s) {
  const GatherGrid gg = gather_grid(M, K, N);
  int32_t* acc_ws = static_cast<int32_t*>(ws);
  uint32_t* cnt_ws = reinterpret_cast<uint32_t*>(acc_ws + M * N);
  hipLaunchKernelGGL(k_gather_a8, dim3(static_cast<unsigned>(gg.nseg * gg.chunks), static_cast<unsigned>(M)),
                     dim3(kThreads), 0, s, codes, sx, K, w_kmajor, beta, N, gg.seg, gg.nseg, gg.chunks, y, acc_dbg,
                     acc_ws, cnt_ws);
  return hipGetLastError();
}

}  // namespace bw
