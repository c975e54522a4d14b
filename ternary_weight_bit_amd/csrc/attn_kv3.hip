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
// Two launches (split over positions, then merged):
//   1. grid (position chunks x batches): a workgroup takes CH positions of
//      one batch for every head, so each position's H vectors (H * 3D/8
//      contiguous bytes) and H scales are read whole.  A lane owns head h and
//      32-dim group g (lanes G h' + g: one wave load covers 64 / G whole
//      vectors of one position, contiguous); the 8 waves are 2 head slices x
//      4 position phases (wave w takes positions 4j + w / 2).  The slabs are
//      read through buffer resources bounded at the chunk's end:
//      pass 1: the group's three words are unpacked four codes per 32-bit
//        word (u = code + 4 of codes k, k+8, k+16, k+24 in its bytes, mostly
//        one shift and one mask each); with q in fixed point (four
//        base-256 digits of q * 2^30 / max|q|) sum q*u is four integer dot4
//        per word, exact; minus 4 * sum q it is summed over the G groups and
//        scaled.  Special positions (slot_of in [0, n_special)) are rescored
//        from their 4-bit codes by the same threads;
//      per head: m = max z, e = exp(z - m), l = sum e over the chunk;
//      pass 2: acc[d] += w * u_d with w = e * s3 (0 at special positions;
//        u_d converted two at a time as fp8 subnormals, the unit folded into w),
//        minus 4 * sum w, plus the special positions' 4-bit terms; summed
//        over the four phase waves through LDS, then (acc[D], m, l) per
//        (chunk, head) go to the workspace.
//   2. grid (batch x head): M = max m_c, out = sum_c acc_c e^(m_c - M) /
//      sum_c l_c e^(m_c - M).
// Every sum runs in a fixed order, so results are deterministic.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

constexpr int kAttnThreads = 512;
constexpr int kUnroll = 4;  // positions per thread with loads in flight together (8 measured slower)
constexpr int kAttnMergeMax = 4096;  // chunks per (batch, head) the merge holds in LDS
// Workgroups the chunking aims at: about one per CU (twice as many, with the
// per-chunk set-up repeated, measured slower).
constexpr int64_t kAttnTargetWgs = 256;
// LDS for summing the four position phases of pass 2: four slots of one
// wave's 32 accumulators per lane.
constexpr int kAttnRedFloats = 4 * 32 * kWave;

// Unpacked codes of one 32-code group: u[k] holds code+4 of codes k, k+8,
// k+16, k+24 in bytes 0..3.  Byte i of the group's words w0, w1, w2 carries
// the fields u = code + 4 of codes 8i .. 8i+7 (w0: u0 | u1 << 3 | low two bits
// of u6 at 6; w1: u2 | u3 << 3 | bit 2 of u6 at 6 | bit 0 of u7 at 7; w2:
// u4 | u5 << 3 | bits 1..2 of u7 at 6), so six slices are one shift and one
// mask of a word and the other two take two of each and an OR.
__device__ __forceinline__ void unpack_group(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t (&u)[8]) {
  constexpr uint32_t M7 = 0x07070707u;
  u[0] = w0 & M7;
  u[1] = (w0 >> 3) & M7;
  u[2] = w1 & M7;
  u[3] = (w1 >> 3) & M7;
  u[4] = w2 & M7;
  u[5] = (w2 >> 3) & M7;
  u[6] = ((w0 >> 6) & 0x03030303u) | ((w1 >> 4) & 0x04040404u);
  u[7] = ((w1 >> 7) & 0x01010101u) | ((w2 >> 5) & 0x06060606u);
}

// bytes 2w and 2w+1 of x (w = HI_WORD) read as fp8 values: a byte 0..7 is an fp8 subnormal,
// so the pair is (x_b * unit) exactly, unit being the fp8 value of byte 1
template <bool HI_WORD>
__device__ __forceinline__ float2 byte_pair_fp8(uint32_t x) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x), HI_WORD);
  return make_float2(v[0], v[1]);
}

// 4-bit two's-complement nibble (low or high half of a byte) -> value
__device__ __forceinline__ float nib_f(uint32_t byte, int hi) {
  const int n = static_cast<int>((byte >> (4 * hi)) & 0xFu);
  return static_cast<float>(n >= 8 ? n - 16 : n);
}

// DPP move of a float with bound control (lanes whose source is outside the
// row read 0): row_shr:n is 0x110 + n, quad_perm(a,b,c,d) is a|b<<2|c<<4|d<<6
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112;
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;  // quad_perm [1,0,3,2] and [2,3,0,1]

// Sum over the G adjacent lanes of one head (lanes G h' + g of a 16-lane
// row): after the row shifts the lane with g = G - 1 holds
// (v3 + v2) + (v1 + v0) (others hold partial sums).
template <int G>
__device__ __forceinline__ float groups_sum_last(float v) {
  v += dpp_f<kRowShr1>(v);
  if constexpr (G == 4) v += dpp_f<kRowShr2>(v);
  return v;
}

// Sum or maximum over the 64 lanes with DPP moves (no LDS round trips): row
// totals by row_shr 1, 2, 4, 8 (lanes without a source take the identity),
// carried into the last row by row_bcast 15 and 31; every lane gets lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_id(float v, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ float wave_total_f(float v) {
  const float id = MAX ? -INFINITY : 0.0f;
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_id<0x111, 0xF>(v, id));
  v = op(v, dpp_id<0x112, 0xF>(v, id));
  v = op(v, dpp_id<0x114, 0xF>(v, id));
  v = op(v, dpp_id<0x118, 0xF>(v, id));
  v = op(v, dpp_id<0x142, 0xA>(v, id));  // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_id<0x143, 0xC>(v, id));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_chunk(
    const float* __restrict__ q, const uint8_t* __restrict__ kp3, const float* __restrict__ ks3,
    const uint8_t* __restrict__ kp4, const float* __restrict__ ks4, const uint8_t* __restrict__ vp3,
    const float* __restrict__ vs3, const uint8_t* __restrict__ vp4, const float* __restrict__ vs4,
    const int32_t* __restrict__ slot_of, int64_t n_special, int64_t B, int64_t S, int64_t S_cap, int64_t H,
    int64_t q_stride, int CH, int nch, float* __restrict__ part) {
  constexpr int G = D / 32;                   // 32-dim groups per vector
  constexpr int HW = kWave / G;               // heads per wave
  constexpr int HS = 2 * HW;                  // heads per head block (two head slices)
  constexpr int VB = 3 * D / 8;               // 3-bit code bytes per vector
  extern __shared__ float s_dyn[];            // s_red[kAttnRedFloats], s_z[CH][H + 1], s_m[H], s_l[H]
  __shared__ uint16_t s_list[kAttnMaxChunk];  // special positions of the chunk, ascending
  __shared__ uint32_t s_spec[kAttnMaxChunk / 32];
  __shared__ int s_wscan[kAttnThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar loop bounds)
  const int phase = wave >> 1;                  // positions phase, phase + 4, ...
  const int g = lane % G;                       // 32-dim group
  const int hl = (wave & 1) * HW + lane / G;    // head within the head block
  const int64_t b = blockIdx.x % B;
  const int64_t c = blockIdx.x / B;
  const int64_t p0 = c * CH;
  const int np = static_cast<int>((S - p0 < CH) ? S - p0 : CH);  // positions in this chunk
  const int HP = static_cast<int>(H) + 1;
  float* __restrict__ s_red = s_dyn;
  float* __restrict__ s_z = s_dyn + kAttnRedFloats;
  float* __restrict__ s_m = s_z + static_cast<int64_t>(CH) * HP;
  float* __restrict__ s_l = s_m + H;
  const int32_t* __restrict__ slots = slot_of + b * S_cap + p0;
  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
  // The chunk's 3-bit slabs and scales as buffers: position p (0 <= p < np),
  // head h at byte (p H + h) VB of a slab and (p H + h) 4 of a scale array.  An
  // offset at or past np positions reads zeros without memory traffic.
  const int64_t vec0 = (b * S_cap + p0) * H;
  const int nvh = np * static_cast<int>(H);
  const __amdgpu_buffer_rsrc_t kr = rsrc(kp3 + vec0 * VB, static_cast<int64_t>(nvh) * VB);
  const __amdgpu_buffer_rsrc_t vr = rsrc(vp3 + vec0 * VB, static_cast<int64_t>(nvh) * VB);
  const __amdgpu_buffer_rsrc_t ksr = rsrc(ks3 + vec0, static_cast<int64_t>(nvh) * 4);
  const __amdgpu_buffer_rsrc_t vsr = rsrc(vs3 + vec0, static_cast<int64_t>(nvh) * 4);
  const uint32_t pstride = static_cast<uint32_t>(H) * VB;  // slab bytes from one position to the next
  const uint32_t sstride = static_cast<uint32_t>(H) * 4;

  // special positions of the chunk (slot id in [0, n_special)): the ids are
  // loaded here, the bitmask (wave ballots) and the ordered list are built
  // after the first pass-1 loop, whose loads hide this one's latency
  const int nwords = (np + 31) / 32;
  const int32_t sl_first = (64 * wave + lane < np) ? slots[64 * wave + lane] : -1;
  int nspec = 0;
  auto scan_specials = [&]() {
    for (int s0 = 64 * wave; s0 < np; s0 += kAttnThreads) {
      const int s = s0 + lane;
      const int32_t sl = (s0 == 64 * wave) ? sl_first : ((s < np) ? slots[s] : -1);
      const uint64_t bal = __ballot(sl >= 0 && sl < n_special);
      if (lane == 0) {
        s_spec[s0 >> 5] = static_cast<uint32_t>(bal);
        if (s0 + 32 < np) s_spec[(s0 >> 5) + 1] = static_cast<uint32_t>(bal >> 32);
      }
    }
    __syncthreads();
    const uint32_t word = (tid < nwords) ? s_spec[tid] : 0u;
    const int cnt = __popc(word);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wscan[wave] = incl;
    __syncthreads();
    int pos = incl - cnt;
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) pos += (w < wave) ? s_wscan[w] : 0;
    uint32_t bits = word;
    while (bits) {
      const int i = __builtin_ctz(bits);
      bits &= bits - 1;
      s_list[pos++] = static_cast<uint16_t>(32 * tid + i);
    }
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) nspec += s_wscan[w];
    __syncthreads();
  };

  // ---- pass 1: scores, one head block at a time
  for (int hb = 0; hb < H; hb += HS) {
    const int64_t h = hb + hl;
    const bool hok = h < H;
    const int64_t hc = hok ? h : H - 1;
    // A batch's loads are issued together; positions past the chunk read
    // zeros and are not stored.  The next batch's loads are issued before this
    // batch is computed (two register buffers); the first batch is issued
    // before the query is converted, which hides its latency.
    const uint32_t t3 = static_cast<uint32_t>(hc) * VB + 12 * g;  // this lane's words at position 0
    const uint32_t ts = static_cast<uint32_t>(hc) * 4;
    uint32_t pl[kUnroll][3], nl[kUnroll][3];
    float sc[kUnroll], ns[kUnroll];
    auto load_k = [&](int j0, uint32_t (&dl)[kUnroll][3], float (&ds)[kUnroll]) {
      const uint32_t o3 = t3 + static_cast<uint32_t>(j0) * pstride;
      const uint32_t os = ts + static_cast<uint32_t>(j0) * sstride;
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        bload12(kr, o3 + 4 * j * pstride, dl[j]);
        ds[j] = bload_f32(ksr, os + 4 * j * sstride);
      }
    };
    load_k(phase, pl, sc);
    const float* __restrict__ qv = q + b * q_stride + hc * D + 32 * g;
    // fixed-point query: Q_i = rne(q_i * 2^30 / max|q|) (fp64 product), four
    // balanced base-256 digits; its deviation from q is at most 2^-31 max|q|
    float qmax = 0.0f;
    uint32_t qd[4][8];  // digit j of codes k, k+8, k+16, k+24 in bytes 0..3
    int dsum[4] = {0, 0, 0, 0};  // sum of digit j over the group's 32 codes
    {
      float qg[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) qg[i] = qv[i];
#pragma unroll
      for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qg[i]));
      qmax = fmaxf(qmax, dpp_f<kQuadXor1>(qmax));  // over the G lanes of the head
      if constexpr (G == 4) qmax = fmaxf(qmax, dpp_f<kQuadXor2>(qmax));
      const double qscale = qmax > 0.0f ? 1073741824.0 / static_cast<double>(qmax) : 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) qd[j][k] = 0u;
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          int Q = static_cast<int>(rint(static_cast<double>(qg[k + 8 * by]) * qscale));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int dg = (j < 3) ? static_cast<int>(static_cast<int8_t>(Q & 0xFF)) : Q;
            qd[j][k] |= (static_cast<uint32_t>(dg) & 0xFFu) << (8 * by);
            dsum[j] += dg;
            Q = (Q - dg) >> 8;
          }
        }
      }
    }
    const float qunit = qmax * (1.0f / 1073741824.0f);  // exact: a power-of-two scaling
    // sum Q = D0 + 2^8 D1 + 2^16 D2 + 2^24 D3 over the group (D_j: digit sums,
    // |D_j| <= 4096), so 4 sum Q = T + 2^26 D3 with T in int32; split as
    // 2^24 q4hi + q4lo with 0 <= q4lo < 2^24 so that the exact sum below
    // splits into two int32 parts
    const int T = 4 * dsum[0] + 1024 * dsum[1] + 262144 * dsum[2];
    const int q4lo = T & 0xFFFFFF;
    const int q4hi = ((T - q4lo) >> 24) + 4 * dsum[3];

    auto score = [&](int j0, const uint32_t (&kl)[kUnroll][3], const float (&ks)[kUnroll]) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        uint32_t u[8];
        unpack_group(kl[j][0], kl[j][1], kl[j][2], u);
        int dg[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int d = 0; d < 4; ++d)
            dg[d] = __builtin_amdgcn_sdot4(static_cast<int>(u[k]), static_cast<int>(qd[d][k]), dg[d], false);
        // sum Q u - 4 sum Q = lo + 2^24 hi, both exact in int32
        // (|dg[d]| <= 32 * 7 * 128, so |lo| < 1.96e9); one rounding each to fp32
        const int lo = dg[0] + (dg[1] << 8) + (dg[2] << 16) - q4lo;
        const int hi = dg[3] - q4hi;
        const float tf = fmaf(static_cast<float>(hi), 16777216.0f, static_cast<float>(lo));
        const float dot = groups_sum_last<G>(tf);
        const int p = j0 + 4 * j;
        if (g == G - 1 && hok && p < np) s_z[p * HP + h] = dot * qunit * ks[j] * inv_sqrt_d;
      }
    };
    // two register buffers in alternation (no copy from one to the other, which
    // would wait for the batch just issued): batch i + 1 loads while batch i
    // is scored
    for (int j0 = phase; j0 < np;) {
      load_k(j0 + 4 * kUnroll, nl, ns);
      score(j0, pl, sc);
      j0 += 4 * kUnroll;
      if (j0 >= np) break;
      load_k(j0 + 4 * kUnroll, pl, sc);
      score(j0, nl, ns);
      j0 += 4 * kUnroll;
    }
    if (hb == 0) scan_specials();  // uniform: every thread takes the barriers
    // special positions: rescored from their 4-bit codes by the lanes of the
    // same phase (the g = G - 1 lane wrote the 3-bit score: program order)
    for (int e = 0; e < nspec; ++e) {
      const int p = s_list[e];
      if ((p & 3) != phase) continue;
      const int64_t sl = slots[p];
      const uint4 nb = *reinterpret_cast<const uint4*>(kp4 + (sl * H + hc) * (D / 2) + 16 * g);
      const uint32_t w4[4] = {nb.x, nb.y, nb.z, nb.w};
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (w4[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        dot = fmaf(qv[2 * i], nib_f(byte, 0), dot);
        dot = fmaf(qv[2 * i + 1], nib_f(byte, 1), dot);
      }
      dot = groups_sum_last<G>(dot);
      if (g == G - 1 && hok) s_z[p * HP + h] = dot * ks4[sl * H + hc] * inv_sqrt_d;
    }
  }
  __syncthreads();

  // the first batch of pass 2's values (head block 0) loads during the softmax
  uint32_t v0l[kUnroll][3];
  float v0s[kUnroll];
  {
    const int64_t hc0 = hl < H ? hl : H - 1;
    const uint32_t o3 = static_cast<uint32_t>(hc0) * VB + 12 * g + static_cast<uint32_t>(phase) * pstride;
    const uint32_t os = static_cast<uint32_t>(hc0) * 4 + static_cast<uint32_t>(phase) * sstride;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      bload12(vr, o3 + 4 * j * pstride, v0l[j]);
      v0s[j] = bload_f32(vsr, os + 4 * j * sstride);
    }
  }

  // ---- per head over the chunk: m = max z, e = exp(z - m), l = sum e
  for (int64_t h = wave; h < H; h += kAttnThreads / 64) {
    float mx = -INFINITY;
    for (int p = lane; p < np; p += 64) mx = fmaxf(mx, s_z[p * HP + h]);
    mx = wave_total_f<true>(mx);
    float tot = 0.0f;
    for (int p = lane; p < np; p += 64) {
      const float e = expf(s_z[p * HP + h] - mx);
      s_z[p * HP + h] = e;
      tot += e;
    }
    tot = wave_total_f<false>(tot);
    if (lane == 0) {
      s_m[h] = mx;
      s_l[h] = tot;
    }
  }
  __syncthreads();

  // ---- pass 2: weighted values, one head block at a time
  for (int hb = 0; hb < H; hb += HS) {
    const int64_t h = hb + hl;
    const bool hok = h < H;
    const int64_t hc = hok ? h : H - 1;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
    float wsum = 0.0f;
    // codes enter as fp8 subnormals (byte * unit); 1 / unit is a power of two
    const float inv_unit = 1.0f / byte_pair_fp8<false>(1u).x;
    const uint32_t t3 = static_cast<uint32_t>(hc) * VB + 12 * g;
    const uint32_t ts = static_cast<uint32_t>(hc) * 4;
    uint32_t pl[kUnroll][3], nl[kUnroll][3];
    float sc[kUnroll], ns[kUnroll];
    auto load_v = [&](int j0, uint32_t (&dl)[kUnroll][3], float (&ds)[kUnroll]) {
      const uint32_t o3 = t3 + static_cast<uint32_t>(j0) * pstride;
      const uint32_t os = ts + static_cast<uint32_t>(j0) * sstride;
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        bload12(vr, o3 + 4 * j * pstride, dl[j]);
        ds[j] = bload_f32(vsr, os + 4 * j * sstride);
      }
    };
    auto accumulate = [&](int j0, const uint32_t (&vl)[kUnroll][3], const float (&vsc)[kUnroll]) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int p = j0 + 4 * j;
        const int pc = p < np ? p : 0;
        const bool live = p < np && !((s_spec[pc >> 5] >> (pc & 31)) & 1u);
        const float w = live ? s_z[pc * HP + hc] * vsc[j] : 0.0f;
        const float wu = w * inv_unit;  // exact: power-of-two scaling
        uint32_t u[8];
        unpack_group(vl[j][0], vl[j][1], vl[j][2], u);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float2 lo2 = byte_pair_fp8<false>(u[k]);  // codes k, k + 8
          const float2 hi2 = byte_pair_fp8<true>(u[k]);   // codes k + 16, k + 24
          acc[k] = fmaf(wu, lo2.x, acc[k]);
          acc[k + 8] = fmaf(wu, lo2.y, acc[k + 8]);
          acc[k + 16] = fmaf(wu, hi2.x, acc[k + 16]);
          acc[k + 24] = fmaf(wu, hi2.y, acc[k + 24]);
        }
        wsum += w;
      }
    };
    if (hb == 0) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        pl[j][0] = v0l[j][0];
        pl[j][1] = v0l[j][1];
        pl[j][2] = v0l[j][2];
        sc[j] = v0s[j];
      }
    } else {
      load_v(phase, pl, sc);
    }
    for (int j0 = phase; j0 < np;) {
      load_v(j0 + 4 * kUnroll, nl, ns);
      accumulate(j0, pl, sc);
      j0 += 4 * kUnroll;
      if (j0 >= np) break;
      load_v(j0 + 4 * kUnroll, pl, sc);
      accumulate(j0, nl, ns);
      j0 += 4 * kUnroll;
    }
    // remove the +4 of the codes, add the special positions' 4-bit terms
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] -= 4.0f * wsum;
    for (int e = 0; e < nspec; ++e) {
      const int p = s_list[e];
      if ((p & 3) != phase) continue;
      const int64_t sl = slots[p];
      const uint4 nb = *reinterpret_cast<const uint4*>(vp4 + (sl * H + hc) * (D / 2) + 16 * g);
      const uint32_t w4[4] = {nb.x, nb.y, nb.z, nb.w};
      const float w = s_z[p * HP + hc] * vs4[sl * H + hc];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (w4[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        acc[2 * i] = fmaf(w, nib_f(byte, 0), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, nib_f(byte, 1), acc[2 * i + 1]);
      }
    }
    // sum the four phases (wave = 2 phase + head slice) through LDS in the
    // order (p0 + p1) + (p2 + p3); slot `a` of s_red holds 32 floats per lane
    // of one wave.  Phase 0 then writes dims 32 g .. 32 g + 31 of head h (byte
    // `by` of u[k] is code k + 8 by of its group, so acc[i] is dim 32 g + i).
    const int slice = wave & 1;
    float* __restrict__ pair = s_red + ((phase >> 1) * 2 + slice) * 32 * kWave + lane;  // phases 1 -> 0, 3 -> 2
    float* __restrict__ half = s_red + slice * 32 * kWave + lane;                        // phase 2 -> 0
    __syncthreads();  // readers of the previous head block are done with s_red
    if (phase & 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) pair[i * kWave] = acc[i];
    }
    __syncthreads();
    if (!(phase & 1)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] += pair[i * kWave];
    }
    __syncthreads();
    if (phase == 2) {
#pragma unroll
      for (int i = 0; i < 32; ++i) half[i * kWave] = acc[i];
    }
    __syncthreads();
    if (phase == 0 && hok) {
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] += half[i * kWave];
      float4* dst = reinterpret_cast<float4*>(part + ((b * nch + c) * H + h) * (D + 4) + 32 * g);
#pragma unroll
      for (int v = 0; v < 8; ++v) dst[v] = make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]);
    }
  }
  for (int64_t h = tid; h < H; h += kAttnThreads) {
    float* dst = part + ((b * nch + c) * H + h) * (D + 4) + D;
    dst[0] = s_m[h];
    dst[1] = s_l[h];
  }
}

// Merge the chunks of one (batch, head): the chunk maxima and sums go to LDS
// (one thread per chunk), then one thread per dimension adds the chunks'
// rescaled sums in chunk order.  The first kMergePre chunks' values are loaded
// together with the maxima and sums, later ones eight at a time.
constexpr int kMergePre = 32;
template <int D>
__global__ __launch_bounds__(D) void k_attn_merge(const float* __restrict__ part, int64_t B, int64_t H, int nch,
                                                  float* __restrict__ out) {
  __shared__ float s_mc[kAttnMergeMax];
  __shared__ float s_f[kAttnMergeMax];
  __shared__ float s_L;
  const int d = threadIdx.x;
  const int64_t b = blockIdx.x % B;
  const int64_t h = blockIdx.x / B;
  const int64_t stride = H * (D + 4);
  const float* __restrict__ base = part + (b * nch * H + h) * (D + 4);
  float pre[kMergePre];
#pragma unroll
  for (int u = 0; u < kMergePre; ++u) pre[u] = base[(u < nch ? u : 0) * stride + d];
  for (int c = d; c < nch; c += D) {
    s_mc[c] = base[c * stride + D];
    s_f[c] = base[c * stride + D + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, s_mc[c]);
  __syncthreads();
  for (int c = d; c < nch; c += D) s_mc[c] = expf(s_mc[c] - M);  // rescale factor of chunk c
  __syncthreads();
  if (d == 0) {
    float L = 0.0f;
    for (int c = 0; c < nch; ++c) L = fmaf(s_f[c], s_mc[c], L);
    s_L = L;
  }
  float O = 0.0f;
#pragma unroll
  for (int u = 0; u < kMergePre; ++u)
    if (u < nch) O = fmaf(pre[u], s_mc[u], O);
  int c = kMergePre;
  for (; c + 8 <= nch; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = base[(c + u) * stride + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) O = fmaf(v[u], s_mc[c + u], O);
  }
  for (; c < nch; ++c) O = fmaf(base[c * stride + d], s_mc[c], O);
  __syncthreads();
  out[(b * H + h) * D + d] = O / s_L;
}

struct AttnGrid {
  int ch, nch;
};

// Largest chunk the LDS score array allows for H heads (a multiple of 4; below
// 4 the shape is unsupported).
int64_t attn_chunk_cap(int64_t H) {
  int64_t cap = (kAttnLdsFloats - 2 * H) / (H + 1);
  if (cap > kAttnMaxChunk) cap = kAttnMaxChunk;
  return cap / 4 * 4;
}

// Positions per chunk: about kAttnTargetWgs workgroups over the batch (at least
// S * B / kAttnTargetWgs positions, so at most ceil(kAttnTargetWgs / B) chunks), a multiple of 4,
// with the chunk's scores (CH * (H + 1) + 2H floats) within kAttnLdsFloats and
// at most kAttnMergeMax chunks; nch = 0 marks a shape beyond those limits.
AttnGrid attn_grid(int64_t B, int64_t S, int64_t H) {
  int64_t ch = (S * B + kAttnTargetWgs - 1) / kAttnTargetWgs;
  const int64_t min_ch = (S + kAttnMergeMax - 1) / kAttnMergeMax;
  if (ch < min_ch) ch = min_ch;
  int64_t cap = attn_chunk_cap(H);
  const int64_t s4 = (S + 3) / 4 * 4;
  if (cap > s4) cap = s4;
  ch = (ch + 3) / 4 * 4;
  if (ch > cap) ch = cap;
  if (ch < 4) ch = 4;
  AttnGrid g;
  g.ch = static_cast<int>(ch);
  const int64_t nch = (S + ch - 1) / ch;
  g.nch = (nch <= kAttnMergeMax && cap >= 4) ? static_cast<int>(nch) : 0;
  return g;
}

}  // namespace

bool attn_decode3_supported(int64_t B, int64_t S, int64_t H) { return attn_grid(B, S, H).nch > 0; }

// Chunk count bound over every attended length S in [1, S_cap]: a chunk that no
// cap shortens holds at least S * B / kAttnTargetWgs positions
// (ceil(kAttnTargetWgs / B) chunks at most); one the LDS cap shortens holds attn_chunk_cap(H) positions
// (ceil(S_cap / cap) chunks at most); one capped at the rounded length S is the
// only chunk.
int64_t attn_decode3_max_chunks(int64_t B, int64_t S_cap, int64_t H) {
  const int64_t by_batch = (kAttnTargetWgs + B - 1) / B;
  const int64_t cap = attn_chunk_cap(H);
  const int64_t by_cap = cap >= 4 ? (S_cap + cap - 1) / cap : 0;
  return by_batch > by_cap ? by_batch : by_cap;
}

size_t attn_decode3_workspace_bound(int64_t B, int64_t S_cap, int64_t H, int64_t D) {
  return static_cast<size_t>(B) * attn_decode3_max_chunks(B, S_cap, H) * H * (D + 4) * sizeof(float);
}

size_t attn_decode3_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  const AttnGrid g = attn_grid(B, S, H);
  return static_cast<size_t>(B) * g.nch * H * (D + 4) * sizeof(float);
}

hipError_t launch_attn_decode3(const float* q, const uint8_t* kp3, const float* ks3, const uint8_t* kp4,
                               const float* ks4, const uint8_t* vp3, const float* vs3, const uint8_t* vp4,
                               const float* vs4, const int32_t* slot_of, int64_t n_special, int64_t B, int64_t S,
                               int64_t H, int64_t D, float* out, void* ws, hipStream_t s) {
  return launch_attn_decode3_strided(q, H * D, kp3, ks3, kp4, ks4, vp3, vs3, vp4, vs4, slot_of, n_special, B, S, S, H,
                                     D, out, ws, s);
}

hipError_t launch_attn_decode3_strided(const float* q, int64_t q_stride, const uint8_t* kp3, const float* ks3,
                                       const uint8_t* kp4, const float* ks4, const uint8_t* vp3, const float* vs3,
                                       const uint8_t* vp4, const float* vs4, const int32_t* slot_of,
                                       int64_t n_special, int64_t B, int64_t S, int64_t S_cap, int64_t H, int64_t D,
                                       float* out, void* ws, hipStream_t s) {
  const AttnGrid g = attn_grid(B, S, H);
  float* part = static_cast<float*>(ws);
  const dim3 grid1(static_cast<unsigned>(g.nch * B));
  const size_t lds = (kAttnRedFloats + static_cast<size_t>(g.ch) * (H + 1) + 2 * H) * sizeof(float);
  const dim3 grid2(static_cast<unsigned>(B * H));
  if (D == 64) {
    hipLaunchKernelGGL(k_attn_chunk<64>, grid1, dim3(kAttnThreads), lds, s, q, kp3, ks3, kp4, ks4, vp3, vs3, vp4, vs4,
                       slot_of, n_special, B, S, S_cap, H, q_stride, g.ch, g.nch, part);
    hipLaunchKernelGGL(k_attn_merge<64>, grid2, dim3(64), 0, s, part, B, H, g.nch, out);
  } else {
    hipLaunchKernelGGL(k_attn_chunk<128>, grid1, dim3(kAttnThreads), lds, s, q, kp3, ks3, kp4, ks4, vp3, vs3, vp4,
                       vs4, slot_of, n_special, B, S, S_cap, H, q_stride, g.ch, g.nch, part);
    hipLaunchKernelGGL(k_attn_merge<128>, grid2, dim3(128), 0, s, part, B, H, g.nch, out);
  }
  return hipGetLastError();
}

}  // namespace bw
