// Dispatch of the BitLinear contraction: decode shapes (M <= 16 tokens) go to
// the weight-streaming GEMV, larger batches to the MFMA-tiled GEMM.
#include "bw_internal.h"

namespace bw {

hipError_t launch_bitlinear(int mode, const void* codes, const float* sx, int64_t M, int64_t K,
                            const uint8_t* w_packed, const float* beta, int64_t N, float* y,
                            void* acc_dbg, hipStream_t s) {
  if (M <= kGemvMaxM) return launch_gemv(mode, codes, sx, M, K, w_packed, beta, N, y, acc_dbg, s);
  return launch_gemm(mode, codes, sx, M, K, w_packed, beta, N, y, acc_dbg, s);
}

}  // namespace bw
