// One BitNet a4.8 decoder layer for a single new token per sequence, chained
// from the library's kernels on one stream.
//
// BitNet a4.8 abstract: 4-bit activations (INT4/FP4) for the inputs of the
// attention and feed-forward layers, sparsified then 8-bit intermediate
// states, 3-bit KV cache; toshoseti review, «Метод»: 4 bits for the q/k/v and
// gate/up inputs, top-k (50 %) for the out_proj input, ReLU^2 gate for the
// down_proj input; «Эксперименты»: bos/eos kept at 4 bits in the KV cache.
// The pages give no layer formula; the plainest composition is used, with no
// normalization and no rotary embedding (neither is described):
//   c, s   = INT4(x)                         y_qkv = W_qkv (c, s)
//   append k = y_qkv[HD:2HD], v = y_qkv[2HD:3HD] at position pos (3-bit codes)
//   a      = attention(q = y_qkv[0:HD], cache positions 0..pos)
//   x1     = x + W_o SparseA8(a, top-k HD/2)
//   c, s   = INT4(x1)                        g = W_gate (c, s), u = W_up (c, s)
//   x_out  = x1 + W_down SparseA8(relu(g)^2 * u, top-k F/2)
// Launches: quantizer, q/k/v GEMV, KV append, attention (2), top-k INT8,
// out_proj GEMV with the residual added in its epilogue, quantizer, one
// gate/up GEMV writing g and u as two [B][F] arrays, ReLU^2 top-k INT8, down
// GEMV with the residual added in its epilogue.  For one or two sequences the
// quantizers run inside the q/k/v and gate/up GEMV launches (9 launches).
#include <mutex>

#include "bw_internal.h"

namespace bw {

// Workspace of the allocation-free decoder-layer entry point: one array per
// GPU, held from library load until the process ends.  Host code never uses
// this name as an address (on the host it is only a stand-in for the symbol);
// the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[kBlockScratchBytes];

namespace {

constexpr int kAppendThreads = 256;  // four waves, one (batch, head) vector each

__device__ __forceinline__ float wave_absmax(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Write the 3-bit codes (and, at a special position, the 4-bit slot) of the
// new token's K and V vectors at position pos, exactly as the cache packer
// defines them: a' = max(max|v|, 1e-5); 3-bit q = clamp(rne(fl(v * fl(3/a'))),
// -4, 3) with s3 = fl(a'/3), stored as fields u = q + 4, byte i of the three
// words of a 32-code group holding codes 8i .. 8i+7; 4-bit
// q = clamp(rne(fl(v * fl(7/a'))), -8, 7) with s4 = fl(a'/7), even d in the
// low nibble.  One wave per vector; lane l < D/8 holds d = 8l .. 8l+7 and
// writes byte l % 4 of the three words of group l / 4, as the packer's lanes
// do.  blockIdx.y selects K (0) or V (1).
template <int D>
__global__ __launch_bounds__(kAppendThreads) void k_kv_append3(
    const float* __restrict__ y_qkv, int64_t row_stride, int64_t B, int64_t H, int64_t pos, int64_t S_cap,
    const int32_t* __restrict__ slot_of, int64_t n_special, uint8_t* __restrict__ kp3, float* __restrict__ ks3,
    uint8_t* __restrict__ kp4, float* __restrict__ ks4, uint8_t* __restrict__ vp3, float* __restrict__ vs3,
    uint8_t* __restrict__ vp4, float* __restrict__ vs4) {
  constexpr int LPV = D / 8;  // lanes holding the vector
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer, ties to even
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kAppendThreads / 64) + (threadIdx.x >> 6);
  if (wid >= B * H) return;  // whole wave leaves together
  const bool is_v = blockIdx.y == 1;
  const int64_t b = wid / H;
  const int64_t h = wid - b * H;
  const int64_t hd = H * D;
  const float* __restrict__ src = y_qkv + b * row_stride + (is_v ? 2 * hd : hd) + h * D;
  uint8_t* __restrict__ p3 = is_v ? vp3 : kp3;
  float* __restrict__ s3 = is_v ? vs3 : ks3;
  uint8_t* __restrict__ p4 = is_v ? vp4 : kp4;
  float* __restrict__ s4 = is_v ? vs4 : ks4;

  const bool mine = lane < LPV;
  const int l = mine ? lane : 0;
  const float4 xa = *reinterpret_cast<const float4*>(src + 8 * l);
  const float4 xb = *reinterpret_cast<const float4*>(src + 8 * l + 4);
  const float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
  const float ap = fmaxf(wave_absmax(mine ? a : 0.0f), 1e-5f);
  const int64_t vec = (b * S_cap + pos) * H + h;

  // |x| <= a' keeps |x * fl(3/a')| < 3.5 (and |x * fl(7/a')| < 7.5): the clamps never act
  const float inv3 = __fdiv_rn(3.0f, ap);
  uint32_t f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (__float_as_uint(__fmul_rn(x[i], inv3) + kMagic) & 7u) ^ 4u;
  if (mine) {
    uint8_t* out = p3 + vec * (3 * D / 8) + 12 * (l >> 2) + (l & 3);
    out[0] = static_cast<uint8_t>(f[0] | (f[1] << 3) | ((f[6] & 3u) << 6));
    out[4] = static_cast<uint8_t>(f[2] | (f[3] << 3) | ((f[6] >> 2) << 6) | ((f[7] & 1u) << 7));
    out[8] = static_cast<uint8_t>(f[4] | (f[5] << 3) | ((f[7] >> 1) << 6));
  }
  if (lane == 0) s3[vec] = __fdiv_rn(ap, 3.0f);

  // 4-bit slot of a special position
  const int32_t slot = slot_of[b * S_cap + pos];
  if (slot >= 0 && slot < n_special) {
    const float inv7 = __fdiv_rn(7.0f, ap);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (__float_as_uint(__fmul_rn(x[i], inv7) + kMagic) & 0xFu) << (4 * i);
    const int64_t sv = static_cast<int64_t>(slot) * H + h;
    if (mine) reinterpret_cast<uint32_t*>(p4 + sv * (D / 2))[l] = w;
    if (lane == 0) s4[sv] = __fdiv_rn(ap, 7.0f);
  }
}

struct BlockWs {
  uint8_t* c4;
  float* sx4;
  float* y_qkv;
  float* att;
  void* attn_ws;
  int8_t* c8;
  float* s8;
  float* x1;
  float* y_gu;  // g [B][F], then u [B][F]
  int8_t* c8d;
  float* s8d;
  size_t bytes;
};

BlockWs block_ws(void* base, int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F) {
  const int64_t hd = H * D;
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    uint8_t* r = p ? p + off : nullptr;
    off += (n + 255) & ~static_cast<size_t>(255);
    return r;
  };
  BlockWs w;
  w.c4 = take(static_cast<size_t>(B) * hd / 2);
  w.sx4 = reinterpret_cast<float*>(take(4 * B));
  w.y_qkv = reinterpret_cast<float*>(take(4 * static_cast<size_t>(B) * 3 * hd));
  w.att = reinterpret_cast<float*>(take(4 * static_cast<size_t>(B) * hd));
  w.attn_ws = take(attn_decode3_workspace_bound(B, S_cap, H, D));
  w.c8 = reinterpret_cast<int8_t*>(take(static_cast<size_t>(B) * hd));
  w.s8 = reinterpret_cast<float*>(take(4 * B));
  w.x1 = reinterpret_cast<float*>(take(4 * static_cast<size_t>(B) * hd));
  w.y_gu = reinterpret_cast<float*>(take(8 * static_cast<size_t>(B) * F));
  w.c8d = reinterpret_cast<int8_t*>(take(static_cast<size_t>(B) * F));
  w.s8d = reinterpret_cast<float*>(take(4 * B));
  w.bytes = off;
  return w;
}

#define BW_TRY(expr)                  \
  do {                                \
    const hipError_t e_ = (expr);     \
    if (e_ != hipSuccess) return e_;  \
  } while (0)

}  // namespace

size_t block_decode_workspace_bytes(int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F) {
  return block_ws(nullptr, B, S_cap, H, D, F).bytes;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t block_scratch(void** ptr) {
  int dev = -1;
  BW_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    BW_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));  // with device dev current
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_block_decode(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                               const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                               const uint8_t* w_gu, const float* b_gu, const uint8_t* w_down, const float* b_down,
                               uint8_t* kp3, float* ks3, uint8_t* kp4, float* ks4, uint8_t* vp3, float* vs3,
                               uint8_t* vp4, float* vs4, const int32_t* slot_of, int64_t n_special, int64_t S_cap,
                               int64_t pos, void* ws, hipStream_t s) {
  const int64_t hd = H * D;
  const BlockWs w = block_ws(ws, B, S_cap, H, D, F);
  // attention input side: q/k/v projection and KV append
  const bool fused = gemv_quant_supported(B, hd);  // quantizer inside the GEMV launch
  if (fused) {
    BW_TRY(launch_gemv_quant(x, false, 0, B, hd, w_qkv, b_qkv, 3 * hd, w.y_qkv, w.c4, w.sx4, nullptr, nullptr, 3 * hd,
                             s));
  } else {
    BW_TRY(launch_quantize_act4(x, false, B, hd, 0, w.c4, w.sx4, s));
    BW_TRY(launch_bitlinear(0, w.c4, w.sx4, B, hd, w_qkv, b_qkv, 3 * hd, w.y_qkv, nullptr, s));
  }
  const dim3 agrid(static_cast<unsigned>((B * H + kAppendThreads / 64 - 1) / (kAppendThreads / 64)), 2);
  if (D == 64) {
    hipLaunchKernelGGL(k_kv_append3<64>, agrid, dim3(kAppendThreads), 0, s, w.y_qkv, 3 * hd, B, H, pos, S_cap,
                       slot_of, n_special, kp3, ks3, kp4, ks4, vp3, vs3, vp4, vs4);
  } else {
    hipLaunchKernelGGL(k_kv_append3<128>, agrid, dim3(kAppendThreads), 0, s, w.y_qkv, 3 * hd, B, H, pos, S_cap,
                       slot_of, n_special, kp3, ks3, kp4, ks4, vp3, vs3, vp4, vs4);
  }
  BW_TRY(hipGetLastError());
  BW_TRY(launch_attn_decode3_strided(w.y_qkv, 3 * hd, kp3, ks3, kp4, ks4, vp3, vs3, vp4, vs4, slot_of, n_special,
                                     B, pos + 1, S_cap, H, D, w.att, w.attn_ws, s));
  // out_proj on the top-k 50 % INT8 codes, residual
  BW_TRY(launch_sparse_a8(w.att, nullptr, false, B, hd, hd / 2, w.c8, w.s8, nullptr, s));
  BW_TRY(launch_gemv_ex(2, w.c8, w.s8, B, hd, w_o, b_o, hd, w.x1, nullptr, x, hd, s));
  // feed-forward: gate and up on INT4 codes, ReLU^2 * up top-k 50 % INT8, down_proj, residual
  if (fused) {
    BW_TRY(launch_gemv_quant(w.x1, false, 0, B, hd, w_gu, b_gu, 2 * F, w.y_gu, w.c4, w.sx4, nullptr, nullptr, F, s));
  } else {
    BW_TRY(launch_quantize_act4(w.x1, false, B, hd, 0, w.c4, w.sx4, s));
    BW_TRY(launch_gemv_ex(0, w.c4, w.sx4, B, hd, w_gu, b_gu, 2 * F, w.y_gu, nullptr, nullptr, F, s));
  }
  BW_TRY(launch_sparse_a8(w.y_gu, w.y_gu + B * F, false, B, F, F / 2, w.c8d, w.s8d, nullptr, s));
  BW_TRY(launch_gemv_ex(2, w.c8d, w.s8d, B, F, w_down, b_down, hd, x_out, nullptr, w.x1, hd, s));
  return hipSuccess;
}

}  // namespace bw
