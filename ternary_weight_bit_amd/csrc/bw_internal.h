// Host-side launchers behind the C ABI of libbw (include/bw.h).  Each returns
// the HIP error of its launches; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bw {

// Byte size of the scratch words bw_pack_ternary needs in its workspace.
constexpr size_t kPackWorkspaceBytes = 8192;

hipError_t launch_quantize_act4(const void* x, bool bf16, int64_t M, int64_t K, int fmt,
                                uint8_t* codes, float* scales, hipStream_t s);

hipError_t launch_pack_ternary(const void* W, bool bf16, int64_t N, int64_t K, int role,
                               uint8_t* packed, float* beta, void* ws, hipStream_t s);

// Largest token count served by the weight-streaming GEMV.
constexpr int64_t kGemvMaxM = 16;

// mode: 0 = INT4 codes, 1 = e2m1 codes, 2 = INT8 codes
hipError_t launch_gemv(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                       const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                       hipStream_t s);
// GEMV with an optional residual (y[m][n] = resid[m][n] + product, resid in
// the [M][N] layout) and column planes: column n goes to plane n / split, a
// row-major [M][split] array at y + (n / split) * M * split (split = N: [M][N]).
hipError_t launch_gemv_ex(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                          const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                          const float* resid, int64_t split, hipStream_t s);
// 4-bit quantizer and GEMV in one launch (every workgroup quantizes the token
// rows itself; workgroup 0 also stores codes and scales): M <= 2, K <= 8192.
constexpr int64_t kGemvQuantMaxM = 2;
constexpr int64_t kGemvQuantMaxK = 8192;
bool gemv_quant_supported(int64_t M, int64_t K);
hipError_t launch_gemv_quant(const void* x, bool bf16, int fmt, int64_t M, int64_t K, const uint8_t* w_packed,
                             const float* beta, int64_t N, float* y, uint8_t* codes, float* scales, void* acc_dbg,
                             const float* resid, int64_t split, hipStream_t s);
hipError_t launch_gemm(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                       const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                       hipStream_t s);
// Prefill GEMM with operands loaded straight into LDS; launch_gemm uses it
// whenever gemm_lds_supported holds (K % 128 == 0, operands below 2 GiB).
bool gemm_lds_supported(int mode, int64_t M, int64_t K, int64_t N);  // includes tiles < 2^30
int64_t gemm_lds_tiles(int64_t M, int64_t N);                          // grid tiles of one product
hipError_t launch_gemm_lds(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                           const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                           hipStream_t s);
// Several products over the same activation codes in one launch: product g
// takes tiles [tile_end[g-1], tile_end[g]) of one grid, with its own weights,
// beta, N and y, so the tiles of all of them share the CUs in one schedule.
constexpr int kMaxGroups = 4;
struct GemmGroups {
  const uint8_t* w[kMaxGroups];
  const float* beta[kMaxGroups];
  float* y[kMaxGroups];
  void* acc_dbg[kMaxGroups];
  int64_t N[kMaxGroups];
  int tile_end[kMaxGroups];
  int n;
};
// Every product of `g` must satisfy gemm_lds_supported and their tiles must
// sum below 2^31; the caller fills w, beta, y, acc_dbg, N and n (tile_end is
// filled here).
hipError_t launch_gemm_lds_grouped(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                                   GemmGroups g, hipStream_t s);
hipError_t launch_bitlinear(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                            const uint8_t* w_packed, const float* beta, int64_t N, float* y,
                            void* acc_dbg, hipStream_t s);

// Single-token gather product over K-major weights; the workspace holds the
// int32 partial sums [segments][M][N] of its first launch.
constexpr int64_t kGatherMaxM = 16;
size_t gather_a8_workspace_bytes(int64_t M, int64_t K, int64_t N);
hipError_t launch_gather_a8(const int8_t* codes, const float* sx, int64_t M, int64_t K,
                            const uint8_t* w_kmajor, const float* beta, int64_t N, float* y,
                            int32_t* acc_dbg, void* ws, hipStream_t s);

hipError_t launch_sparse_a8(const void* g, const void* u, bool bf16, int64_t M, int64_t K,
                            int64_t k_keep, int8_t* codes, float* scales, uint32_t* mask,
                            hipStream_t s);

// Single-token attention over the 3-bit KV cache: chunks of positions x batches,
// then a merge; the workspace holds each (chunk, head)'s partial sums.
constexpr int kAttnMaxChunk = 4096;     // positions per chunk
constexpr int64_t kAttnLdsFloats = 16384;  // chunk scores + per-head max/sum in LDS
constexpr int64_t kAttnMaxH = 1024;
bool attn_decode3_supported(int64_t B, int64_t S, int64_t H);  // S within the chunk x merge limits
size_t attn_decode3_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D);
// Workspace that covers every attended length S in [1, S_cap] (the decoder
// layer attends over 0..pos of a cache of S_cap positions).
size_t attn_decode3_workspace_bound(int64_t B, int64_t S_cap, int64_t H, int64_t D);
hipError_t launch_attn_decode3(const float* q, const uint8_t* kp3, const float* ks3, const uint8_t* kp4,
                               const float* ks4, const uint8_t* vp3, const float* vs3, const uint8_t* vp4,
                               const float* vs4, const int32_t* slot_of, int64_t n_special, int64_t B, int64_t S,
                               int64_t H, int64_t D, float* out, void* ws, hipStream_t s);
// Same, attending over positions [0, S) of a cache allocated with S_cap
// positions per sequence, q rows q_stride floats apart.
hipError_t launch_attn_decode3_strided(const float* q, int64_t q_stride, const uint8_t* kp3, const float* ks3,
                                       const uint8_t* kp4, const float* ks4, const uint8_t* vp3, const float* vs3,
                                       const uint8_t* vp4, const float* vs4, const int32_t* slot_of,
                                       int64_t n_special, int64_t B, int64_t S, int64_t S_cap, int64_t H, int64_t D,
                                       float* out, void* ws, hipStream_t s);

// One decoder layer for one new token per sequence (block.hip).
size_t block_decode_workspace_bytes(int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F);
// Static per-device workspace of the allocation-free variant: its size, and its
// device address on the current device (looked up once per device).
constexpr size_t kBlockScratchBytes = size_t(16) << 20;
hipError_t block_scratch(void** ptr);
hipError_t launch_block_decode(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                               const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                               const uint8_t* w_gu, const float* b_gu, const uint8_t* w_down, const float* b_down,
                               uint8_t* kp3, float* ks3, uint8_t* kp4, float* ks4, uint8_t* vp3, float* vs3,
                               uint8_t* vp4, float* vs4, const int32_t* slot_of, int64_t n_special, int64_t S_cap,
                               int64_t pos, void* ws, hipStream_t s);

// Streaming read of `bytes` bytes (measurement): sink[4b + q] = XOR of the
// 32-bit words of 4 KB quarter q of 16 KB block b.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);

hipError_t launch_kv_pack3(const void* kv, bool bf16, int64_t B, int64_t S, int64_t H, int64_t D,
                           const int32_t* slot_of, int64_t n_special, uint8_t* p3, float* s3,
                           uint8_t* p4, float* s4, hipStream_t s);

hipError_t launch_kv_unpack3(const uint8_t* p3, const float* s3, const uint8_t* p4, const float* s4,
                             const int32_t* slot_of, int64_t B, int64_t S, int64_t H, int64_t D,
                             int64_t n_special, bool out_bf16, void* out, hipStream_t s);

}  // namespace bw
