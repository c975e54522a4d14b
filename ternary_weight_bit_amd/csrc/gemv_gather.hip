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
// Two launches:
//   1. grid (segments x column chunks, tokens): a workgroup takes a segment of
//      up to kMaxSeg inputs of one token and a chunk of kCols = 512 outputs
//      (128 bytes of every row).  It lists the nonzero codes of its segment in
//      LDS (order free: the sum is exact integer arithmetic); each half-wave
//      (row group) walks every sixteenth listed row, lane c of the group
//      loading the 4-byte word of outputs 16c..16c+15 of that row, and
//      accumulates q * (t + 1) two outputs per 32-bit register (16-bit fields,
//      exact while a group sees at most 127 rows, which the segment bound
//      guarantees), subtracting sum(q) at the end.  The sixteen row groups are
//      summed in LDS and the segment's int32 partial sums are stored to the
//      workspace.
//   2. grid (64-output chunks, tokens): sums the partials of every segment
//      and writes y = fl(fl(acc * s_x) * beta).
// Plain stores and a kernel boundary replace device-scope atomics, whose
// round trips to the coherence point cost more than the weight reads here.
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 512;
constexpr int kCols = 512;    // outputs per workgroup
constexpr int kGroups = 16;   // row groups (half-waves) per workgroup
constexpr int kBatch = 8;     // rows per lane with loads in flight together
constexpr int kMaxSeg = 1024; // inputs per workgroup: multiple of 64, at most 16 * 64 nonzero
constexpr int kTargetBlocks = 256;
constexpr int kFinishThreads = 256;
constexpr int kFinishCols = 64;                                 // outputs per finishing workgroup
constexpr int kFinishSlices = kFinishThreads / (kFinishCols / 2);  // segment slices per output pair

static_assert(kMaxSeg % 64 == 0 && kMaxSeg / 4 <= kThreads, "segment scan: one dword per thread");
static_assert((kMaxSeg + kGroups - 1) / kGroups <= 127, "16-bit accumulator fields");
static_assert(kCols == kThreads, "one output per thread in the row-group sum");

__global__ __launch_bounds__(kThreads) void k_gather_a8(const int8_t* __restrict__ codes, int64_t M, int64_t K,
                                                         const uint8_t* __restrict__ Wk, int64_t N, int seg,
                                                         int chunks, int32_t* __restrict__ part) {
  __shared__ int2 s_row[kMaxSeg];  // (byte offset of the row, code)
  __shared__ int32_t s_red[kGroups][kCols];
  __shared__ int s_wtot[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m = blockIdx.y;
  const int chunk = static_cast<int>(blockIdx.x % chunks);
  const int sgi = static_cast<int>(blockIdx.x / chunks);
  const int64_t k0 = static_cast<int64_t>(sgi) * seg;
  const int64_t k1 = (k0 + seg < K) ? k0 + seg : K;
  const uint32_t row_bytes = static_cast<uint32_t>(N >> 2);

  // 1. list the nonzero codes of [k0, k1), four per thread: wave ballots give
  //    each code its slot inside the wave, wave totals the wave's base.
  const int nq = static_cast<int>((k1 - k0) >> 2);
  const int word = (tid < nq) ? *reinterpret_cast<const int*>(codes + m * K + k0 + 4 * tid) : 0;
  uint64_t bal[4];
  int wsum = 0;
  int before[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bal[j] = __ballot(static_cast<int8_t>(word >> (8 * j)) != 0);
    before[j] = wsum;
    wsum += __popcll(bal[j]);
  }
  if (lane == 0) s_wtot[wave] = wsum;
  __syncthreads();
  int base = 0, R = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int t = s_wtot[w];
    base += (w < wave) ? t : 0;
    R += t;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = static_cast<int>(static_cast<int8_t>(word >> (8 * j)));
    if (q != 0) {
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(bal[j] >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[j]), 0u)));
      const uint32_t k = static_cast<uint32_t>(k0 + 4 * tid + j);
      s_row[base + before[j] + below] = make_int2(static_cast<int>(k * row_bytes), q);
    }
  }
  __syncthreads();

  // 2. gather: row group g = half-wave, lane c of the group owns 16 outputs.
  // Loads are unconditional so that a whole batch is in flight at once: a slot
  // past the list end re-reads listed row 0 with q = 0, and a lane past the
  // last output reads the chunk's first word (its sums are never stored).
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
  int total = 0;
#pragma unroll
  for (int gg = 0; gg < kGroups; ++gg) total += s_red[gg][tid];
  const int64_t n = static_cast<int64_t>(chunk) * kCols + tid;
  if (n < N) part[(static_cast<int64_t>(sgi) * M + m) * N + n] = total;
}

// Sum the segments' partials of 64 outputs of one token and apply the
// epilogue.  Thread (r, p) adds output pair p of every eighth segment starting
// at r, so each thread's loads (at most eight per pass) are all in flight at
// once; the eight slices are then summed in LDS.
__global__ __launch_bounds__(kFinishThreads) void k_gather_finish(const int32_t* __restrict__ part, int nseg,
                                                                  const float* __restrict__ sx, int64_t M,
                                                                  const float* __restrict__ beta, int64_t N,
                                                                  float* __restrict__ y,
                                                                  int32_t* __restrict__ acc_dbg) {
  __shared__ int2 s_sum[kFinishSlices][kFinishCols / 2];
  const int tid = threadIdx.x;
  const int pi = tid & (kFinishCols / 2 - 1);
  const int r = tid / (kFinishCols / 2);
  const int64_t m = blockIdx.y;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kFinishCols + 2 * pi;
  const bool ok = n < N;  // N % 16 == 0: n + 1 < N too
  const int32_t* __restrict__ src = part + m * N + (ok ? n : 0);
  const int64_t stride = M * N;
  int a0 = 0, a1 = 0;
  for (int s0 = r; s0 < nseg; s0 += kFinishSlices * 8) {
    int2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sg = s0 + u * kFinishSlices;
      v[u] = (sg < nseg) ? *reinterpret_cast<const int2*>(src + sg * stride) : make_int2(0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 += v[u].x;
      a1 += v[u].y;
    }
  }
  s_sum[r][pi] = make_int2(a0, a1);
  __syncthreads();
  if (r != 0 || !ok) return;
#pragma unroll
  for (int q = 1; q < kFinishSlices; ++q) {
    const int2 v = s_sum[q][pi];
    a0 += v.x;
    a1 += v.y;
  }
  const float s = sx[m];
  float2 out;
  out.x = __fmul_rn(__fmul_rn(static_cast<float>(a0), s), beta[n]);
  out.y = __fmul_rn(__fmul_rn(static_cast<float>(a1), s), beta[n + 1]);
  *reinterpret_cast<float2*>(y + m * N + n) = out;
  if (acc_dbg) *reinterpret_cast<int2*>(acc_dbg + m * N + n) = make_int2(a0, a1);
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

size_t gather_a8_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  const GatherGrid gg = gather_grid(M, K, N);
  const size_t bytes = static_cast<size_t>(gg.nseg) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
  return (bytes + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_gather_a8(const int8_t* codes, const float* sx, int64_t M, int64_t K, const uint8_t* w_kmajor,
                            const float* beta, int64_t N, float* y, int32_t* acc_dbg, void* ws, hipStream_t s) {
  const GatherGrid gg = gather_grid(M, K, N);
  int32_t* part = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_gather_a8, dim3(static_cast<unsigned>(gg.nseg * gg.chunks), static_cast<unsigned>(M)),
                     dim3(kThreads), 0, s, codes, M, K, w_kmajor, N, gg.seg, gg.chunks, part);
  const unsigned fblocks = static_cast<unsigned>((N + kFinishCols - 1) / kFinishCols);
  hipLaunchKernelGGL(k_gather_finish, dim3(fblocks, static_cast<unsigned>(M)), dim3(kFinishThreads), 0, s, part,
                     gg.nseg, sx, M, beta, N, y, acc_dbg);
  return hipGetLastError();
}

}  // namespace bw
