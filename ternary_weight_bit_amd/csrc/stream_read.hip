// Streaming-read measurement kernel: reads a buffer once, in the access
// pattern of the decode GEMV's weight stream, so that the GEMV's time can be
// set against the time the same bytes take to read on this part.
//
// One workgroup (4 waves) per 16 KB block; wave w reads the block's 4 KB
// quarter w with four 1 KB wave loads (16 bytes per lane), all issued before
// the first is used, XORs its 32-bit words across the wave with DPP moves and
// writes sink[4 * block + w] (no LDS, no barrier: each wave ends on its own,
// as the GEMV's waves end on their data).  A bytes % 16384 tail reads zeros
// past the end.
#include "bw_device.h"
#include "bw_internal.h"

namespace bw {
namespace {

// XOR over the 64 lanes (DPP row shifts, then the row results carried across
// rows); lane 63 ends with the total.
__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false));
  return v;
}

__global__ __launch_bounds__(256) void k_stream_read(const uint8_t* __restrict__ src, int64_t bytes,
                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t blk = blockIdx.x;
  const int64_t lim = (bytes - blk * 16384 < 16384) ? bytes - blk * 16384 : 16384;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + blk * 16384), 0,
                                                                     static_cast<int>(lim), kRsrcWord3);
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t off = static_cast<uint32_t>(wave * 4096 + u * 1024 + lane * 16);
    const auto q = __builtin_amdgcn_raw_buffer_load_b128(r, off < lim ? off : kOutOfRange, 0, 0);
    v[u] = make_uint4(q[0], q[1], q[2], q[3]);
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  x = wave_xor(x);
  if (lane == 63) sink[4 * blk + wave] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((bytes + 16383) / 16384));
  hipLaunchKernelGGL(k_stream_read, grid, dim3(256), 0, s, static_cast<const uint8_t*>(src), bytes, sink);
  return hipGetLastError();
}

}  // namespace bw
