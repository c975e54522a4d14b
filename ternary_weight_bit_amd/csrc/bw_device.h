// Device-side helpers shared by the gfx950 kernels of libbw.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bw {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Raw buffer resources: a load whose byte offset (the vector offset) lies at or
// past the resource size returns zeros without touching memory.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;  // above every resource size used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kRsrcWord3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void bload12(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[3]) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
  w[0] = v[0];
  w[1] = v[1];
  w[2] = v[2];
}

__device__ __forceinline__ float bload_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 consecutive elements starting at element index `e` (e % 8 == 0) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t e, float (&v)[8]) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + e + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* __restrict__ base, int64_t e) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[e]) << 16);
  } else {
    return static_cast<const float*>(base)[e];
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix over the 64 lanes with DPP moves (no LDS round trips):
// Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4, 8), then the
// row totals are carried across rows (row_bcast 15 into rows 1 and 3,
// row_bcast 31 into rows 2 and 3).  Lanes without a source add the identity.
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/ = 0) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Same scheme for the maximum of non-negative values (identity 0).
__device__ __forceinline__ uint32_t wave_incl_umax(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return v;
}

// Value of lane `l` (wave-uniform l) of v.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Max over a 256-thread block; every thread gets the result.  `red` holds >= 4 floats.
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Correctly-rounded fp32 operations kept as single roundings.
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }

}  // namespace bw
