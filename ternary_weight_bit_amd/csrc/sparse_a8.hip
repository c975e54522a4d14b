// Fused ReLU^2 gate + per-token top-k + INT8 absmax quantizer for gfx950.
//
// BitNet a4.8 abstract: intermediate states are sparsified, then quantized to
// 8 bits.  toshoseti review «Метод»: top-k at 50 % sparsity for the out
// projection input; ReLU^2 replaces swish in the FFN gate to sparsify the
// down projection input.  9pt.com article, methodology: the low-magnitude
// entries are the ones dropped.
//
// Two kernels share one selection scheme.  Rows of up to 4096 entries, when
// there are more than 256 of them: one wave per token row, no workgroup
// barrier.  Every other shape (rows up to 16384 entries): one workgroup of 8
// waves per row, each wave holding 512-entry chunks in the same per-lane
// arrangement; measured at 2048 rows of 11008 this is 43.5 us cold against
// 65 us for a wave per row, while at 2048 rows of 4096 a wave per row stays
// faster (18 vs 23 us warm).  A third kernel takes the one-wave shapes when
// the input is bf16 without a gate: it selects on the 15-bit bf16 magnitudes
// themselves (two radix passes, described at the kernel).
//
// Lane l of a wave holds entries 512c + 8l + i (i < 8) of its 512-entry
// chunks c in registers as the fp32 bits of h, read once with 16-byte loads
// that are all in flight before the first use.  The k-th largest magnitude
// tau is found by a three-pass radix select over the 31 magnitude bits (11,
// 10, 10 bits): each pass histograms the still-possible entries into an LDS
// array with LDS atomics, and a wave scan over the bins picks the bin holding
// the k-th largest.  Zeros (half of a ReLU^2 row) never enter a histogram:
// when fewer than k entries are nonzero, tau = 0 and no pass runs.  Entries
// equal to tau are taken lowest index first: their rank in index order comes
// from one ballot per register slot, counted with mbcnt, chunk by chunk.
// Codes are written as 8-byte runs per lane.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ one wave per row
constexpr int kRowsPerBlock = kThreads / kWave;  // 4 rows (waves) per workgroup
constexpr int kBins = 2048;                      // first radix pass: bits 30..20
constexpr int kHist = kBins + kWave;             // + one private discard bin per lane

// Register budget: CH*8 keys per lane stay live through the whole kernel.
template <int CH>
constexpr int wave_occupancy() { return CH <= 8 ? 4 : 2; }

template <bool BF16, bool GATED, int CH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(wave_occupancy<CH>(), 8)))
void k_sparse_a8_wave(const void* __restrict__ g,
                                                             const void* __restrict__ u, int M, int K,
                                                             int k_keep, int8_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             uint32_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) int hist_all[kRowsPerBlock][kHist];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x * kRowsPerBlock + wave;
  if (m >= M) return;  // whole wave leaves together
  int* hist = hist_all[wave];
  const int64_t row = static_cast<int64_t>(m) * K;
  constexpr int SW = (CH + 3) / 4;

  // ---- |h| bits (key) and sign bits of every entry of this lane; entries past
  // K hold key 0 and are never counted or written
  uint32_t key[CH][8];
  uint32_t sg[SW];
#pragma unroll
  for (int w = 0; w < SW; ++w) sg[w] = 0;
  auto put = [&](int c, int i, float v, bool ok) {
    const uint32_t b = __float_as_uint(v);
    key[c][i] = ok ? (b & 0x7FFFFFFFu) : 0u;
    sg[c >> 2] |= (b >> 31) << (8 * (c & 3) + i);
  };
  if constexpr (BF16) {
    uint4 rg[CH], ru[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = c * 512 + 8 * lane;
      const int64_t off = row + ((e < K) ? e : 0);
      rg[c] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(g) + off);
      if constexpr (GATED) ru[c] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(u) + off);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool ok = c * 512 + 8 * lane < K;
      const uint32_t wg[4] = {rg[c].x, rg[c].y, rg[c].z, rg[c].w};
      uint32_t wu[4] = {0, 0, 0, 0};
      if constexpr (GATED) { wu[0] = ru[c].x; wu[1] = ru[c].y; wu[2] = ru[c].z; wu[3] = ru[c].w; }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = (i & 1) ? bf16_hi(wg[i >> 1]) : bf16_lo(wg[i >> 1]);
        if constexpr (GATED) {
          const float up = (i & 1) ? bf16_hi(wu[i >> 1]) : bf16_lo(wu[i >> 1]);
          const float r = v > 0.0f ? v : 0.0f;
          v = mul_rn(mul_rn(r, r), up);
        }
        put(c, i, v, ok);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = c * 512 + 8 * lane;
      const bool ok = e < K;
      const int64_t off = row + (ok ? e : 0);
      float gv[8], uv[8];
      load8<false>(g, off, gv);
      if constexpr (GATED) load8<false>(u, off, uv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = gv[i];
        if constexpr (GATED) {
          const float r = v > 0.0f ? v : 0.0f;
          v = mul_rn(mul_rn(r, r), uv[i]);
        }
        put(c, i, v, ok);
      }
    }
  }

  // The sign words go through an empty asm statement: otherwise the compiler
  // sees that key | sign rebuilds the loaded bits and keeps those live too,
  // doubling the registers held through the selection.
#pragma unroll
  for (int w = 0; w < SW; ++w) asm volatile("" : "+v"(sg[w]));

  // ---- row maximum (exact, order-free) and count of nonzero magnitudes
  uint32_t kmax = 0;
  int nz = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kmax = max(kmax, key[c][i]);
      nz += static_cast<int>(min(key[c][i], 1u));
    }
  const float amax = __uint_as_float(static_cast<uint32_t>(lane_value(static_cast<int>(wave_incl_umax(kmax)), kWave - 1)));
  const int nnz = lane_value(wave_incl_scan(nz, lane), kWave - 1);

  // ---- tau = the k_keep-th largest magnitude; n_gt = entries above it
  uint32_t tau = 0;
  int n_gt = nnz;
  int n_eq = K - nnz;  // entries equal to tau (tau = 0: the valid zeros)
  if (nnz >= k_keep && k_keep < K) {  // keep-all (the b1.58 INT8 absmax): no selection
    // Radix passes over the nonzero magnitudes: bits 30..20, then 19..10 and
    // 9..0.  After the first pass the entries left in the chosen bin (usually
    // a few dozen) are gathered into an LDS list and the last two passes run
    // over that list alone.
    int need = k_keep;  // rank of tau among the entries that share the prefix
    int above = 0;      // entries known to lie above the current prefix range
    // Bin of the current histogram (per bins a lane) holding the need-th
    // largest; returns it with the count above it and its own count.
    auto find_bin = [&](int per, int& bin, int& cum, int& cnt_bin) {
      int sum = 0;
      for (int b = 0; b < per; b += 4) {
        const int4 q = *reinterpret_cast<const int4*>(&hist[lane * per + b]);
        sum += q.x + q.y + q.z + q.w;
      }
      const int incl = wave_incl_scan(sum, lane);
      const int total = lane_value(incl, kWave - 1);
      const int over_l = total - incl;  // candidates in higher lanes' bins
      const int L = __ffsll(static_cast<long long>(__ballot(over_l < need && need <= over_l + sum))) - 1;
      const int over = lane_value(over_l, L);
      // within lane L's bins, lane j takes bin L*per + per-1-j (top first)
      const int cnt = (lane < per) ? hist[L * per + per - 1 - lane] : 0;
      const int run = wave_incl_scan(cnt, lane);
      const int J = __ffsll(static_cast<long long>(__ballot(lane < per && over + run >= need))) - 1;
      bin = L * per + per - 1 - J;
      cum = over + lane_value(run - cnt, J);
      cnt_bin = lane_value(cnt, J);
    };
    const uint32_t discard = static_cast<uint32_t>(kBins + lane);  // this lane's own bin: no conflicts

    // pass 1: bits 30..20 of every nonzero magnitude.  The candidate test is
    // plain arithmetic on purpose (the top bit of (k - 1) is set iff k == 0):
    // lane masks per entry would be kept live and exhaust the scalar registers.
    for (int b = 0; b < kBins / kWave; b += 4)
      *reinterpret_cast<int4*>(&hist[lane * (kBins / kWave) + b]) = make_int4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t k = key[c][i];
        const uint32_t nzf = 1u - ((k - 1u) >> 31);
        atomicAdd(&hist[discard + nzf * ((k >> 20) - discard)], 1);
      }
    int bin1, cum1, c1;
    find_bin(kBins / kWave, bin1, cum1, c1);
    need -= cum1;
    above += cum1;
    uint32_t prefix = static_cast<uint32_t>(bin1) << 20;

    // gather the c1 entries of that bin into list[0, c1) (LDS words 1024..2047,
    // unused by the 1024-bin passes), one ballot + mbcnt per register slot
    constexpr int kList = 1024;
    int* list = hist + 1024;
    const bool gathered = c1 <= kList;
    if (gathered) {
      int base = 0;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t k = key[c][i];
          const bool f = k != 0u && (k >> 20) == static_cast<uint32_t>(bin1);
          const uint64_t bm = __ballot(f);
          const int pos = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                     static_cast<uint32_t>(bm >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0u)));
          hist[f ? 1024 + pos : static_cast<int>(discard)] = static_cast<int>(k);
          base += __popcll(bm);
        }
    }
    // passes 2 and 3: bits 19..10, then 9..0, over the list (or every entry)
#pragma unroll 1
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = (pass == 1) ? 10 : 0;
      const uint32_t want = prefix >> (shift + 10);
      for (int b = 0; b < 1024 / kWave; b += 4)
        *reinterpret_cast<int4*>(&hist[lane * (1024 / kWave) + b]) = make_int4(0, 0, 0, 0);
      if (gathered) {
        for (int t = lane; t < c1; t += kWave) {
          const uint32_t k = static_cast<uint32_t>(list[t]);
          const bool cand = (k >> (shift + 10)) == want;
          atomicAdd(&hist[cand ? static_cast<int>((k >> shift) & 1023u) : static_cast<int>(discard)], 1);
        }
      } else {
        // (`zero` is opaque so that -k is not hoisted out of the pass loop as
        // a second register copy of every key)
        uint32_t zero = 0;
        asm volatile("" : "+s"(zero));
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t k = key[c][i];
            const uint32_t cand = ((((k >> (shift + 10)) ^ want) - 1u) & (zero - k)) >> 31;
            const uint32_t digit = (k >> shift) & 1023u;
            atomicAdd(&hist[discard + cand * (digit - discard)], 1);
          }
      }
      int bin, cum, cnt_bin;
      find_bin(1024 / kWave, bin, cum, cnt_bin);
      prefix |= static_cast<uint32_t>(bin) << shift;
      need -= cum;
      above += cum;
      n_eq = cnt_bin;  // after the last pass: entries whose 31 bits all equal tau
    }
    tau = prefix;
    n_gt = above;
  }
  const int need = k_keep - n_gt;  // >= 1 entries equal to tau, lowest index first

  // ---- tie cut in index order, quantize, write codes (and the keep mask).
  // Entries past K hold key 0 and come last in index order, after K - nnz >=
  // need valid zeros, so the cut never reaches them: no per-entry bounds test.
  const float a = fmaxf(amax, 1e-5f);
  const float inv = div_rn(127.0f, a);
  // When every entry equal to tau survives (no tie straddles the cut, the
  // usual case for tau > 0) no ranking is needed.  Nor is it when tau = 0 and
  // no keep mask is asked for: the entries equal to tau are then zeros, whose
  // code is 0 whether they are kept or not.
  const bool all_eq = n_eq == need;
  const bool no_rank = all_eq || (tau == 0u && mask == nullptr);
  // Output addresses from an opaque copy of the lane's offset: shared with the
  // load addresses, they would be kept live (one per chunk) through the whole
  // selection.
  int lane_off = 8 * lane;
  asm volatile("" : "+v"(lane_off));
  int8_t* out = codes + row;
  // |h| <= a' keeps |h * fl(127/a')| below 127.5, so rne() lands in [-127, 127]
  // and the clamp to [-128, 127] never acts; adding 1.5 * 2^23 rounds to an
  // integer (ties to even) left, two's complement, in the low mantissa byte.
  // A dropped entry is quantized as 0.
  auto code_of = [&](int c, int i, uint32_t keep) {
    const uint32_t k = key[c][i];
    const float h = __uint_as_float(k | (((sg[c >> 2] >> (8 * (c & 3) + i)) & 1u) << 31));
    return __float_as_uint(mul_rn(keep ? h : 0.0f, inv) + 12582912.0f);
  };
  // low bytes of four codes -> one word (byte i = code i)
  auto pack4 = [](uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u) | __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);
  };
  if (no_rank) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t q[8];
      uint32_t kbits = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t keep = static_cast<uint32_t>(key[c][i] >= tau);
        q[i] = code_of(c, i, keep);
        kbits |= keep << i;
      }
      const int e = c * 512 + lane_off;
      if (e < K) {
        *reinterpret_cast<uint2*>(out + e) = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
        if (mask) reinterpret_cast<uint8_t*>(mask)[(row + e) >> 3] = static_cast<uint8_t>(kbits);
      }
    }
  } else {
    int taken = 0;  // entries equal to tau in earlier chunks (index order)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // rank of this lane's first tau-equal entry in the chunk: equal entries
      // of lower lanes (one ballot per slot i, counted with mbcnt)
      int rank = taken;
      int lower = 0, total = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint64_t bm = __ballot(key[c][i] == tau);
        lower = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), lower));
        total += __popcll(bm);
      }
      rank += lower;
      taken += total;
      uint32_t q[8];
      uint32_t kbits = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t k = key[c][i];
        const int is_eq = static_cast<int>(k == tau);
        const uint32_t keep = static_cast<uint32_t>(k > tau) | static_cast<uint32_t>(is_eq & (rank < need));
        rank += is_eq;
        q[i] = code_of(c, i, keep);
        kbits |= keep << i;
      }
      const int e = c * 512 + lane_off;
      if (e < K) {
        *reinterpret_cast<uint2*>(out + e) = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
        if (mask) reinterpret_cast<uint8_t*>(mask)[(row + e) >> 3] = static_cast<uint8_t>(kbits);
      }
    }
  }
  if (lane == 0) scales[m] = div_rn(a, 127.0f);
}

// ------------------------------------------------------ one workgroup per row
// A row is spread over NW waves: wave w holds the 512-entry chunks w, w + NW,
// ... in the same per-lane arrangement as the one-wave kernel (entries
// 512c + 8l + i).  Against one wave per row this cuts each row's latency (a
// decode step's few rows would otherwise leave the chip idle) and, for long
// rows, the registers each wave keeps through the selection.  The radix
// passes share one LDS histogram (LDS atomics); wave 0 scans it and the
// result goes to every wave through LDS.  Ties at tau are ranked in index
// order with per-chunk counts exchanged through LDS and one ballot + mbcnt per
// register slot inside a chunk.
constexpr int kBlkList = 1024;  // capacity of the list of entries in the chosen first-pass bin
constexpr int64_t kBlockRowsMax = 256;  // rows of <= 4096 entries: a workgroup per row up to this many rows

// Bin of hist[0, 64 * per) holding the need-th largest (bins scanned from the
// top); returns the bin, the count in bins above it and its own count.
// Called by one whole wave.
__device__ __forceinline__ void find_bin_wave(const int* hist, int per, int need, int lane, int& bin,
                                              int& cum, int& cnt_bin) {
  int sum = 0;
  for (int b = 0; b < per; b += 4) {
    const int4 q = *reinterpret_cast<const int4*>(&hist[lane * per + b]);
    sum += q.x + q.y + q.z + q.w;
  }
  const int incl = wave_incl_scan(sum, lane);
  const int total = lane_value(incl, kWave - 1);
  const int over_l = total - incl;
  const int L = __ffsll(static_cast<long long>(__ballot(over_l < need && need <= over_l + sum))) - 1;
  const int over = lane_value(over_l, L);
  const int cnt = (lane < per) ? hist[L * per + per - 1 - lane] : 0;
  const int run = wave_incl_scan(cnt, lane);
  const int J = __ffsll(static_cast<long long>(__ballot(lane < per && over + run >= need))) - 1;
  bin = L * per + per - 1 - J;
  cum = over + lane_value(run - cnt, J);
  cnt_bin = lane_value(cnt, J);
}

// ------------------------------------ one wave per row, bf16 input without a gate
// When h is a bf16 input itself, |h| is the low 15 bits of its bf16 word and
// the fp32 magnitudes order exactly as those bits.  The row then stays in
// registers as loaded, two entries per word (32 registers for 4096 entries),
// and tau comes from two radix passes over the 15-bit keys: bits 14..4 (2048
// bins) over every entry, then bits 3..0 (16 bins) over the entries of the
// chosen bin.  Zeros are counted like any other key, so tau = 0 falls out
// when fewer than k_keep entries are nonzero; the lanes' entries past K read
// as zero (buffer loads past the row) and are taken out of bin 0.  Ties at
// tau, lowest index first: per 512-entry chunk one ballot per register slot
// counts the entries equal to tau, and only the chunk where the cut falls
// ranks them (ballot + mbcnt); the other chunks keep key >= tau or key > tau.
template <int CH, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void k_sparse_a8_wave_bf16(const uint16_t* __restrict__ x, int M, int K, int k_keep, int8_t* __restrict__ codes,
                           float* __restrict__ scales, uint32_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) int hist_all[kRowsPerBlock][kHist];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: LDS and row bases in SGPRs
  const int m = blockIdx.x * kRowsPerBlock + wave;
  if (m >= M) return;  // whole wave leaves together
  int* hist = hist_all[wave];
  const int64_t row = static_cast<int64_t>(m) * K;

  // w[c][j]: entry 512c + 8 lane + 2j in the low half, 2j + 1 in the high half
  const auto rs = rsrc(x + row, 2 * static_cast<int64_t>(K));
  uint32_t w[CH][4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = c * 512 + 8 * lane;
    const uint4 v = bload16(rs, e < K ? static_cast<uint32_t>(2 * e) : kOutOfRange);
    w[c][0] = v.x;
    w[c][1] = v.y;
    w[c][2] = v.z;
    w[c][3] = v.w;
  }

  // ---- row maximum on packed 16-bit magnitudes (exact, order-free)
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 m2 = {0, 0};
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, w[c][j] & 0x7FFF7FFFu));
  const uint32_t kmax = lane_value(static_cast<int>(wave_incl_umax(m2.x > m2.y ? m2.x : m2.y)), kWave - 1);
  const float amax = __uint_as_float(kmax << 16);

  // ---- tau = the k_keep-th largest key; n_gt entries above it, n_eq equal
  const bool keep_all = k_keep >= K;
  uint32_t tau = 0;
  int n_gt = 0, n_eq = K;
  if (!keep_all) {
    const int n_pad = 512 * CH - K;  // entries past K, all in bin 0
#pragma unroll
    for (int b = 0; b < kBins / kWave; b += 4)
      *reinterpret_cast<int4*>(&hist[lane * (kBins / kWave) + b]) = make_int4(0, 0, 0, 0);
    // (each bin index goes through an empty asm statement so that it stays one
    // bit-field extract followed by one shift-and-add into the LDS address)
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t b0 = __builtin_amdgcn_ubfe(w[c][j], 4, 11), b1 = __builtin_amdgcn_ubfe(w[c][j], 20, 11);
        asm volatile("" : "+v"(b0), "+v"(b1));
        atomicAdd(&hist[b0], 1);
        atomicAdd(&hist[b1], 1);
      }
    if (lane == 0 && n_pad > 0) atomicSub(&hist[0], n_pad);
    int bin1, cum1, c1;
    find_bin_wave(hist, kBins / kWave, k_keep, lane, bin1, cum1, c1);
    // pass 2: bits 3..0 of the keys in bin1 (16 bins in words 0..15; every
    // other key goes to this lane's own bin, so no conflicts)
    const int need2 = k_keep - cum1;
    if (lane < 4) *reinterpret_cast<int4*>(&hist[4 * lane]) = make_int4(0, 0, 0, 0);
    // Per word, with packed 16-bit operations: d = key - 16 bin1 (wrapping
    // below), then min(d, 16 + lane): a key of the chosen bin lands on its
    // digit, every other key on a word >= 16 (this lane's own word 16 + lane
    // unless it lies less than 16 + lane above the bin; the bins past 15 are
    // never read).
    const uint32_t lo16 = static_cast<uint32_t>(bin1) << 4;
    typedef unsigned short us2v __attribute__((ext_vector_type(2)));
    const us2v base2 = {static_cast<unsigned short>(lo16), static_cast<unsigned short>(lo16)};
    const us2v disc2 = {static_cast<unsigned short>(16 + lane), static_cast<unsigned short>(16 + lane)};
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const us2v k2 = __builtin_bit_cast(us2v, w[c][j] & 0x7FFF7FFFu);
        const us2v d2 = __builtin_elementwise_min(k2 - base2, disc2);
        const uint32_t dd = __builtin_bit_cast(uint32_t, d2);
        atomicAdd(&hist[dd & 0xFFFFu], 1);
        atomicAdd(&hist[dd >> 16], 1);
      }
    if (lane == 0 && n_pad > 0 && bin1 == 0) atomicSub(&hist[0], n_pad);
    const int cnt = (lane < 16) ? hist[15 - lane] : 0;
    const int run = wave_incl_scan(cnt, lane);
    const int J = __ffsll(static_cast<long long>(__ballot(lane < 16 && run >= need2))) - 1;
    tau = lo16 | static_cast<uint32_t>(15 - J);
    n_gt = cum1 + lane_value(run - cnt, J);
    n_eq = lane_value(cnt, J);
  }
  const int need = keep_all ? n_eq : k_keep - n_gt;  // entries equal to tau that survive

  // ---- quantize and write codes (and the keep mask)
  const float a = fmaxf(amax, 1e-5f);
  const float inv = div_rn(127.0f, a);
  int lane_off = 8 * lane;
  asm volatile("" : "+v"(lane_off));
  int8_t* out = codes + row;
  // |h| <= a' keeps |h * fl(127/a')| below 127.5: rne() lands in [-127, 127];
  // adding 1.5 * 2^23 leaves it, two's complement, in the low mantissa byte.
  // A dropped entry is quantized as 0.
  auto q_of = [&](float h, bool keep) { return __float_as_uint(mul_rn(keep ? h : 0.0f, inv) + 12582912.0f); };
  auto pack4 = [](uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u) | __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);
  };
  auto store = [&](int c, const uint32_t (&q)[8], uint32_t kbits) {
    const int e = c * 512 + lane_off;
    if (e < K) {
      *reinterpret_cast<uint2*>(out + e) = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      if constexpr (MASK) reinterpret_cast<uint8_t*>(mask)[(row + e) >> 3] = static_cast<uint8_t>(kbits);
    }
  };
  // keep = key >= thr for a whole chunk
  auto encode_thr = [&](int c, uint32_t thr) {
    uint32_t q[8];
    uint32_t kbits = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[c][j];
      const bool k0 = (v & 0x7FFFu) >= thr;
      const bool k1 = __builtin_amdgcn_ubfe(v, 16, 15) >= thr;
      q[2 * j] = q_of(bf16_lo(v), k0);
      q[2 * j + 1] = q_of(bf16_hi(v), k1);
      if constexpr (MASK) kbits |= (static_cast<uint32_t>(k0) << (2 * j)) | (static_cast<uint32_t>(k1) << (2 * j + 1));
    }
    store(c, q, kbits);
  };
  // when tau = 0 and no mask is asked for, the entries equal to tau are zeros,
  // whose code is 0 whether they are kept or not
  if (n_eq == need || (!MASK && tau == 0u)) {
#pragma unroll
    for (int c = 0; c < CH; ++c) encode_thr(c, tau);
  } else {
    int taken = 0;  // entries equal to tau in earlier chunks (index order)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (taken >= need) {  // every later tie is dropped
        encode_thr(c, tau + 1u);
        continue;
      }
      uint64_t eq[8];
      int total = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        eq[2 * j] = __ballot((w[c][j] & 0x7FFFu) == tau);
        eq[2 * j + 1] = __ballot(__builtin_amdgcn_ubfe(w[c][j], 16, 15) == tau);
        total += __popcll(eq[2 * j]) + __popcll(eq[2 * j + 1]);
      }
      if (taken + total <= need) {  // every tie of this chunk survives
        encode_thr(c, tau);
        taken += total;
        continue;
      }
      // the cut falls in this chunk: rank = ties at lower indices
      int rank = taken;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(eq[i] >> 32),
                                         __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(eq[i]), rank));
      uint32_t q[8];
      uint32_t kbits = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t v = w[c][i >> 1];
        const uint32_t k = (i & 1) ? __builtin_amdgcn_ubfe(v, 16, 15) : (v & 0x7FFFu);
        const bool is_eq = k == tau;
        const bool keep = k > tau || (is_eq && rank < need);
        rank += static_cast<int>(is_eq);
        q[i] = q_of((i & 1) ? bf16_hi(v) : bf16_lo(v), keep);
        if constexpr (MASK) kbits |= static_cast<uint32_t>(keep) << i;
      }
      store(c, q, kbits);
      taken += total;
    }
  }
  if (lane == 0) scales[m] = div_rn(a, 127.0f);
}

template <bool BF16, bool GATED, int CH, int NW>
__global__ __launch_bounds__(NW * kWave) void k_sparse_a8_block(const void* __restrict__ g,
                                                                 const void* __restrict__ u, int K, int k_keep,
                                                                 int8_t* __restrict__ codes,
                                                                 float* __restrict__ scales,
                                                                 uint32_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) int hist[kHist];
  __shared__ int list[kBlkList];
  constexpr int kBlkWaves = NW;
  constexpr int kBlkThreads = NW * kWave;
  __shared__ uint32_t w_max[kBlkWaves];
  __shared__ int w_nz[kBlkWaves];
  __shared__ int sel[4];  // list fill, then (bin, count above, count in bin) of the last scan
  __shared__ int tiecnt[kBlkWaves * CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = blockIdx.x;
  const int64_t row = static_cast<int64_t>(m) * K;
  constexpr int SW = (CH + 3) / 4;

  // ---- |h| bits and sign bits of this lane's entries (same scheme as above)
  uint32_t key[CH][8];
  uint32_t sg[SW];
#pragma unroll
  for (int w = 0; w < SW; ++w) sg[w] = 0;
  auto ent = [&](int c) { return 512 * (wave + kBlkWaves * c) + 8 * lane; };
  auto put = [&](int c, int i, float v, bool ok) {
    const uint32_t b = __float_as_uint(v);
    key[c][i] = ok ? (b & 0x7FFFFFFFu) : 0u;
    sg[c >> 2] |= (b >> 31) << (8 * (c & 3) + i);
  };
  {
    float gv[CH][8], uv[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = ent(c);
      const int64_t off = row + ((e < K) ? e : 0);
      load8<BF16>(g, off, gv[c]);
      if constexpr (GATED) load8<BF16>(u, off, uv[c]);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool ok = ent(c) < K;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = gv[c][i];
        if constexpr (GATED) {
          const float r = v > 0.0f ? v : 0.0f;
          v = mul_rn(mul_rn(r, r), uv[c][i]);
        }
        put(c, i, v, ok);
      }
    }
  }

  // ---- clear the histogram; per-wave maximum and nonzero count
  for (int i = tid; i < kHist; i += kBlkThreads) hist[i] = 0;
  if (tid == 0) sel[0] = 0;
  {
    uint32_t kmax = 0;
    int nz = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kmax = max(kmax, key[c][i]);
        nz += static_cast<int>(min(key[c][i], 1u));
      }
    kmax = static_cast<uint32_t>(lane_value(static_cast<int>(wave_incl_umax(kmax)), kWave - 1));
    nz = lane_value(wave_incl_scan(nz, lane), kWave - 1);
    if (lane == 0) {
      w_max[wave] = kmax;
      w_nz[wave] = nz;
    }
  }
  __syncthreads();

  // ---- first radix pass (bits 30..20 of the nonzero magnitudes) by every wave
  const uint32_t discard = static_cast<uint32_t>(kBins + lane);
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t k = key[c][i];
      const uint32_t nzf = 1u - ((k - 1u) >> 31);
      atomicAdd(&hist[discard + nzf * ((k >> 20) - discard)], 1);
    }
  __syncthreads();
  uint32_t kmax = 0;
  int nnz = 0;
#pragma unroll
  for (int w = 0; w < kBlkWaves; ++w) {
    kmax = max(kmax, w_max[w]);
    nnz += w_nz[w];
  }
  const float amax = __uint_as_float(kmax);

  uint32_t tau = 0;
  int n_gt = nnz;
  int n_eq = K - nnz;
  if (nnz >= k_keep && k_keep < K) {  // uniform over the workgroup
    int need = k_keep;
    int above = 0;
    if (wave == 0) {
      int bin, cum, cnt;
      find_bin_wave(hist, kBins / kWave, need, lane, bin, cum, cnt);
      if (lane == 0) {
        sel[1] = bin;
        sel[2] = cum;
        sel[3] = cnt;
      }
    }
    __syncthreads();
    const int bin1 = sel[1];
    const int cum1 = sel[2];
    const int c1 = sel[3];
    need -= cum1;
    above += cum1;
    uint32_t prefix = static_cast<uint32_t>(bin1) << 20;
    // entries of the chosen bin -> list[0, c1) when they fit
    const bool gathered = c1 <= kBlkList;
    if (gathered) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t k = key[c][i];
          const bool f = k != 0u && (k >> 20) == static_cast<uint32_t>(bin1);
          const uint64_t bm = __ballot(f);
          if (bm != 0) {  // wave-uniform
            int base = 0;
            if (lane == 0) base = atomicAdd(&sel[0], __popcll(bm));
            base = __shfl(base, 0, kWave);
            const int pos = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                       static_cast<uint32_t>(bm >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0u)));
            if (f) list[pos] = static_cast<int>(k);
          }
        }
    }
    // passes 2 and 3: bits 19..10, then 9..0, over the list (or every entry)
#pragma unroll 1
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = (pass == 1) ? 10 : 0;
      const uint32_t want = prefix >> (shift + 10);
      __syncthreads();  // the previous scan's reads (and the list writes) are done
      for (int i = tid; i < 1024; i += kBlkThreads) hist[i] = 0;
      if (tid < kWave) hist[kBins + tid] = 0;
      __syncthreads();
      if (gathered) {
        for (int t = tid; t < c1; t += kBlkThreads) {
          const uint32_t k = static_cast<uint32_t>(list[t]);
          const bool cand = (k >> (shift + 10)) == want;
          atomicAdd(&hist[cand ? static_cast<int>((k >> shift) & 1023u) : static_cast<int>(discard)], 1);
        }
      } else {
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t k = key[c][i];
            const bool cand = k != 0u && (k >> (shift + 10)) == want;
            atomicAdd(&hist[cand ? static_cast<int>((k >> shift) & 1023u) : static_cast<int>(discard)], 1);
          }
      }
      __syncthreads();
      if (wave == 0) {
        int bin, cum, cnt;
        find_bin_wave(hist, 1024 / kWave, need, lane, bin, cum, cnt);
        if (lane == 0) {
          sel[1] = bin;
          sel[2] = cum;
          sel[3] = cnt;
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(sel[1]) << shift;
      need -= sel[2];
      above += sel[2];
      n_eq = sel[3];
    }
    tau = prefix;
    n_gt = above;
  }
  const int need = k_keep - n_gt;  // >= 1 entries equal to tau, lowest index first

  const float a = fmaxf(amax, 1e-5f);
  const float inv = div_rn(127.0f, a);
  const bool no_rank = n_eq == need || (tau == 0u && mask == nullptr);  // uniform
  auto code_of = [&](int c, int i, uint32_t keep) {
    const uint32_t k = key[c][i];
    const float h = __uint_as_float(k | (((sg[c >> 2] >> (8 * (c & 3) + i)) & 1u) << 31));
    return __float_as_uint(mul_rn(keep ? h : 0.0f, inv) + 12582912.0f);
  };
  auto pack4 = [](uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u) | __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);
  };
  int8_t* out = codes + row;
  // entries equal to tau in lower chunks (index order) of each chunk of this wave
  int taken[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) taken[c] = 0;
  if (!no_rank) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      int tc = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) tc += __popcll(__ballot(key[c][i] == tau && ent(c) < K));
      if (lane == 0) tiecnt[wave + kBlkWaves * c] = tc;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int gc = wave + kBlkWaves * c;
      int t = 0;
      for (int j = 0; j < gc; ++j) t += tiecnt[j];
      taken[c] = t;
    }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = ent(c);
    uint32_t q[8];
    uint32_t kbits = 0;
    if (no_rank) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t keep = static_cast<uint32_t>(key[c][i] >= tau);
        q[i] = code_of(c, i, keep);
        kbits |= keep << i;
      }
    } else {
      int rank = taken[c];
      int lower = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint64_t bm = __ballot(key[c][i] == tau && e < K);
        lower = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), lower));
      }
      rank += lower;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t k = key[c][i];
        const int is_eq = static_cast<int>(k == tau);
        const uint32_t keep = static_cast<uint32_t>(k > tau) | static_cast<uint32_t>(is_eq & (rank < need));
        rank += is_eq;
        q[i] = code_of(c, i, keep);
        kbits |= keep << i;
      }
    }
    if (e < K) {
      *reinterpret_cast<uint2*>(out + e) = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      if (mask) reinterpret_cast<uint8_t*>(mask)[(row + e) >> 3] = static_cast<uint8_t>(kbits);
    }
  }
  if (tid == 0) scales[m] = div_rn(a, 127.0f);
}

template <bool BF16, bool GATED>
hipError_t launch_t(const void* g, const void* u, int64_t M, int64_t K, int64_t k_keep, int8_t* codes,
                    float* scales, uint32_t* mask, hipStream_t s) {
  const int m = static_cast<int>(M), k = static_cast<int>(K), kk = static_cast<int>(k_keep);
  const dim3 wgrid(static_cast<unsigned>((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  const dim3 bgrid(static_cast<unsigned>(M)), bblock(8 * kWave);
  if (K <= 4096) {
    // short rows: a workgroup per row while few rows, else a wave per row
    if (M <= kBlockRowsMax)
      hipLaunchKernelGGL((k_sparse_a8_block<BF16, GATED, 1, 8>), bgrid, bblock, 0, s, g, u, k, kk, codes, scales, mask);
    else if (BF16 && !GATED && mask)
      hipLaunchKernelGGL((k_sparse_a8_wave_bf16<8, true>), wgrid, block, 0, s, static_cast<const uint16_t*>(g), m, k, kk,
                         codes, scales, mask);
    else if (BF16 && !GATED)
      hipLaunchKernelGGL((k_sparse_a8_wave_bf16<8, false>), wgrid, block, 0, s, static_cast<const uint16_t*>(g), m, k,
                         kk, codes, scales, mask);
    else
      hipLaunchKernelGGL((k_sparse_a8_wave<BF16, GATED, 8>), wgrid, block, 0, s, g, u, m, k, kk, codes, scales, mask);
  } else if (K <= 8192) {
    hipLaunchKernelGGL((k_sparse_a8_block<BF16, GATED, 2, 8>), bgrid, bblock, 0, s, g, u, k, kk, codes, scales, mask);
  } else if (K <= 12288) {
    hipLaunchKernelGGL((k_sparse_a8_block<BF16, GATED, 3, 8>), bgrid, bblock, 0, s, g, u, k, kk, codes, scales, mask);
  } else {
    hipLaunchKernelGGL((k_sparse_a8_block<BF16, GATED, 4, 8>), bgrid, bblock, 0, s, g, u, k, kk, codes, scales, mask);
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
