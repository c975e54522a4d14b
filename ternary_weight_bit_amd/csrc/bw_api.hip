// C ABI of libbw: host-side argument validation and dispatch to the gfx950
// kernels.  Every check runs before anything is enqueued, so a non-OK status
// leaves the outputs untouched.  See include/bw.h for the contract.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/bw.h"
#include "bw_internal.h"

namespace {

thread_local char g_err[512] = "";

bw_status fail(bw_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bw_status ok() {
  g_err[0] = '\0';
  return BW_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bw_status hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(BW_ERR_HIP, "%s: HIP error %d (%s)", where, static_cast<int>(e), hipGetErrorString(e));
  return ok();
}

#define BW_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

constexpr int64_t kMaxK = 131072;
constexpr int64_t kMaxKSparse = 16384;

bool valid_fmt(bw_act4_fmt f) { return f == BW_ACT_INT4 || f == BW_ACT_FP4_E2M1 || f == BW_ACT_INT4_E2M3; }

// Kernel mode of a 4-bit format: 0 = INT4 nibbles, 1 = e2m1, 3 = INT4 as e2m3 fields.
int mode_of(bw_act4_fmt f) { return f == BW_ACT_INT4 ? 0 : f == BW_ACT_FP4_E2M1 ? 1 : 3; }

}  // namespace

extern "C" {

int bw_abi_version(void) { return BW_ABI_VERSION; }
int bw_pack_layout_version(void) { return BW_PACK_LAYOUT_VERSION; }
const char* bw_last_error(void) { return g_err; }

size_t bw_ternary_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 4;
}

size_t bw_pack_ternary_workspace_bytes(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return bw::kPackWorkspaceBytes;
}

bw_status bw_pack_ternary(const void* W, bw_dtype w_dtype, int64_t N, int64_t K, bw_weight_role role,
                          uint8_t* w_packed, float* beta, void* workspace, size_t workspace_bytes,
                          void* stream) {
  BW_REQUIRE(W && w_packed && beta && workspace, BW_ERR_NULL, "bw_pack_ternary: NULL pointer");
  BW_REQUIRE(w_dtype == BW_F32 || w_dtype == BW_BF16, BW_ERR_DTYPE, "bw_pack_ternary: bad dtype %d", (int)w_dtype);
  BW_REQUIRE(role == BW_ROLE_A4 || role == BW_ROLE_A8 || role == BW_ROLE_A8_KMAJOR, BW_ERR_DTYPE,
             "bw_pack_ternary: bad role %d", (int)role);
  BW_REQUIRE(N >= 1 && K >= 1 && N % 16 == 0 && K % 64 == 0, BW_ERR_SHAPE,
             "bw_pack_ternary: need N %% 16 == 0 and K %% 64 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  BW_REQUIRE(N <= (int64_t(1) << 40) / K, BW_ERR_SHAPE, "bw_pack_ternary: N*K must be below 2^40");
  BW_REQUIRE(!misaligned(W) && !misaligned(w_packed) && !misaligned(beta) && !misaligned(workspace),
             BW_ERR_ALIGN, "bw_pack_ternary: device pointers must be 16-byte aligned");
  BW_REQUIRE(workspace_bytes >= bw::kPackWorkspaceBytes, BW_ERR_ARG,
             "bw_pack_ternary: workspace needs %zu bytes, got %zu", bw::kPackWorkspaceBytes, workspace_bytes);
  return hip_status(bw::launch_pack_ternary(W, w_dtype == BW_BF16, N, K, role, w_packed, beta, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "bw_pack_ternary");
}

bw_status bw_quantize(const void* x, bw_dtype x_dtype, int64_t M, int64_t K, bw_act4_fmt fmt, uint8_t* codes,
                      float* scales, void* stream) {
  BW_REQUIRE(x_dtype == BW_F32 || x_dtype == BW_BF16, BW_ERR_DTYPE, "bw_quantize: bad dtype %d", (int)x_dtype);
  BW_REQUIRE(valid_fmt(fmt), BW_ERR_DTYPE, "bw_quantize: bad format %d", (int)fmt);
  BW_REQUIRE(M >= 0 && K >= 64 && K % 64 == 0 && K <= kMaxK, BW_ERR_SHAPE,
             "bw_quantize: need M >= 0, K %% 64 == 0, 64 <= K <= %lld (M=%lld K=%lld)", (long long)kMaxK,
             (long long)M, (long long)K);
  if (M == 0) return ok();
  BW_REQUIRE(x && codes && scales, BW_ERR_NULL, "bw_quantize: NULL pointer");
  BW_REQUIRE(!misaligned(x) && !misaligned(codes) && !misaligned(scales), BW_ERR_ALIGN,
             "bw_quantize: device pointers must be 16-byte aligned");
  return hip_status(bw::launch_quantize_act4(x, x_dtype == BW_BF16, M, K, static_cast<int>(fmt), codes, scales,
                                             static_cast<hipStream_t>(stream)),
                    "bw_quantize");
}

static bw_status check_gemm(const char* who, const void* codes, const float* sx, int64_t M, int64_t K,
                            const uint8_t* w, const float* beta, int64_t N, const float* y, const void* acc) {
  BW_REQUIRE(M >= 0 && K >= 64 && K % 64 == 0 && K <= kMaxK && N >= 16 && N % 16 == 0, BW_ERR_SHAPE,
             "%s: need M >= 0, K %% 64 == 0, 64 <= K <= %lld, N %% 16 == 0, N >= 16 (M=%lld K=%lld N=%lld)", who,
             (long long)kMaxK, (long long)M, (long long)K, (long long)N);
  if (M == 0) return ok();
  BW_REQUIRE(codes && sx && w && beta && y, BW_ERR_NULL, "%s: NULL pointer", who);
  BW_REQUIRE(!misaligned(codes) && !misaligned(sx) && !misaligned(w) && !misaligned(beta) && !misaligned(y) &&
                 !misaligned(acc),
             BW_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
  return ok();
}

// e2m3 fields are read by the decode GEMV (M <= 16) and the LDS GEMM; the
// shape must fit the LDS GEMM's 32-bit offsets (it also bounds the GEMV's).
static bw_status check_e2m3(const char* who, int64_t M, int64_t K, int64_t N) {
  BW_REQUIRE(bw::gemm_lds_supported(3, M, K, N), BW_ERR_UNSUPPORTED,
             "%s: BW_ACT_INT4_E2M3 needs M*3K/4 and N*K/4 below 2^31 bytes (M=%lld K=%lld N=%lld)", who,
             (long long)M, (long long)K, (long long)N);
  return ok();
}

// One product: decode shapes (M <= 16) go to the GEMV in every format; larger
// batches of e2m3 fields to the LDS GEMM, the other formats through the GEMM
// dispatch.
static hipError_t launch_a4(int mode, const void* codes, const float* sx, int64_t M, int64_t K, const uint8_t* w,
                            const float* beta, int64_t N, float* y, void* acc, hipStream_t s) {
  if (mode == 3 && M > bw::kGemvMaxM) return bw::launch_gemm_lds(mode, codes, sx, M, K, w, beta, N, y, acc, s);
  return bw::launch_bitlinear(mode, codes, sx, M, K, w, beta, N, y, acc, s);
}

bw_status bw_bitlinear_a4(const uint8_t* codes, const float* x_scales, int64_t M, int64_t K, bw_act4_fmt fmt,
                          const uint8_t* w_packed, const float* beta, int64_t N, float* y, void* acc_dbg,
                          void* stream) {
  BW_REQUIRE(valid_fmt(fmt), BW_ERR_DTYPE, "bw_bitlinear_a4: bad format %d", (int)fmt);
  bw_status st = check_gemm("bw_bitlinear_a4", codes, x_scales, M, K, w_packed, beta, N, y, acc_dbg);
  if (st != BW_OK || M == 0) return st;
  if (fmt == BW_ACT_INT4_E2M3 && (st = check_e2m3("bw_bitlinear_a4", M, K, N)) != BW_OK) return st;
  return hip_status(launch_a4(mode_of(fmt), codes, x_scales, M, K, w_packed, beta, N, y, acc_dbg,
                              static_cast<hipStream_t>(stream)),
                    "bw_bitlinear_a4");
}

// Products over one set of codes: a single grouped launch of the LDS GEMM
// when every product takes it at this M, else one launch per product.
static bw_status bitlinear_grouped(const char* who, int mode, const void* codes, const float* x_scales, int64_t M,
                                   int64_t K, int n, const uint8_t* const* w, const float* const* beta,
                                   const int64_t* N, float* const* y, void* const* acc, hipStream_t s) {
  BW_REQUIRE(n >= 1 && n <= bw::kMaxGroups, BW_ERR_ARG, "%s: need 1 <= n_groups <= %d (n_groups=%d)", who,
             bw::kMaxGroups, n);
  BW_REQUIRE(w && beta && N && y, BW_ERR_NULL, "%s: NULL host array", who);
  for (int g = 0; g < n; ++g) {
    bw_status st = check_gemm(who, codes, x_scales, M, K, w[g], beta[g], N[g], y[g], acc ? acc[g] : nullptr);
    if (st != BW_OK) return st;
  }
  if (M == 0) return ok();
  if (mode == 3) {
    int64_t tiles = 0;
    for (int g = 0; g < n; ++g) {
      bw_status st = check_e2m3(who, M, K, N[g]);
      if (st != BW_OK) return st;
      tiles += bw::gemm_lds_tiles(M, N[g]);
    }
    BW_REQUIRE(tiles < (int64_t{1} << 31), BW_ERR_UNSUPPORTED, "%s: %lld tiles in one launch", who, (long long)tiles);
  }
  bool grouped = M > bw::kGemvMaxM;
  int64_t tiles = 0;
  for (int g = 0; g < n && grouped; ++g) {
    grouped = bw::gemm_lds_supported(mode, M, K, N[g]);
    tiles += grouped ? bw::gemm_lds_tiles(M, N[g]) : 0;
  }
  grouped = grouped && tiles < (int64_t{1} << 31);
  if (grouped) {
    bw::GemmGroups G{};
    G.n = n;
    for (int g = 0; g < n; ++g) {
      G.w[g] = w[g];
      G.beta[g] = beta[g];
      G.y[g] = y[g];
      G.acc_dbg[g] = acc ? acc[g] : nullptr;
      G.N[g] = N[g];
    }
    return hip_status(bw::launch_gemm_lds_grouped(mode, codes, x_scales, M, K, G, s), who);
  }
  for (int g = 0; g < n; ++g) {
    bw_status st = hip_status(
        launch_a4(mode, codes, x_scales, M, K, w[g], beta[g], N[g], y[g], acc ? acc[g] : nullptr, s), who);
    if (st != BW_OK) return st;
  }
  return ok();
}

bw_status bw_bitlinear_a4_grouped(const uint8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                  bw_act4_fmt fmt, int n_groups, const uint8_t* const* w_packed,
                                  const float* const* beta, const int64_t* N, float* const* y,
                                  void* const* acc_dbg, void* stream) {
  BW_REQUIRE(valid_fmt(fmt), BW_ERR_DTYPE, "bw_bitlinear_a4_grouped: bad format %d", (int)fmt);
  return bitlinear_grouped("bw_bitlinear_a4_grouped", mode_of(fmt), codes, x_scales, M, K, n_groups, w_packed, beta,
                           N, y, acc_dbg, static_cast<hipStream_t>(stream));
}

bw_status bw_quantize_bitlinear_a4(const void* x, bw_dtype x_dtype, int64_t M, int64_t K, bw_act4_fmt fmt,
                                   const uint8_t* w_packed, const float* beta, int64_t N, uint8_t* codes,
                                   float* scales, float* y, void* acc_dbg, void* stream) {
  BW_REQUIRE(x_dtype == BW_F32 || x_dtype == BW_BF16, BW_ERR_DTYPE, "bw_quantize_bitlinear_a4: bad dtype %d",
             (int)x_dtype);
  BW_REQUIRE(valid_fmt(fmt), BW_ERR_DTYPE, "bw_quantize_bitlinear_a4: bad format %d", (int)fmt);
  bw_status st = check_gemm("bw_quantize_bitlinear_a4", codes, scales, M, K, w_packed, beta, N, y, acc_dbg);
  if (st != BW_OK || M == 0) return st;
  if (fmt == BW_ACT_INT4_E2M3 && (st = check_e2m3("bw_quantize_bitlinear_a4", M, K, N)) != BW_OK) return st;
  BW_REQUIRE(x, BW_ERR_NULL, "bw_quantize_bitlinear_a4: NULL pointer");
  BW_REQUIRE(!misaligned(x), BW_ERR_ALIGN, "bw_quantize_bitlinear_a4: device pointers must be 16-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = x_dtype == BW_BF16;
  const int f = static_cast<int>(fmt);  // quantizer format
  if (fmt != BW_ACT_INT4_E2M3 && bw::gemv_quant_supported(M, K)) {
    return hip_status(bw::launch_gemv_quant(x, bf16, f, M, K, w_packed, beta, N, y, codes, scales, acc_dbg, nullptr,
                                            N, s),
                      "bw_quantize_bitlinear_a4");
  }
  st = hip_status(bw::launch_quantize_act4(x, bf16, M, K, f, codes, scales, s), "bw_quantize_bitlinear_a4");
  if (st != BW_OK) return st;
  return hip_status(launch_a4(mode_of(fmt), codes, scales, M, K, w_packed, beta, N, y, acc_dbg, s),
                    "bw_quantize_bitlinear_a4");
}

bw_status bw_quantize_sparse_a8(const void* gate_or_x, const void* up, bw_dtype dtype, int64_t M, int64_t K,
                                int64_t k_keep, int8_t* codes, float* scales, uint32_t* mask_dbg, void* stream) {
  BW_REQUIRE(dtype == BW_F32 || dtype == BW_BF16, BW_ERR_DTYPE, "bw_quantize_sparse_a8: bad dtype %d", (int)dtype);
  BW_REQUIRE(M >= 0 && K >= 64 && K % 64 == 0 && K <= kMaxKSparse, BW_ERR_SHAPE,
             "bw_quantize_sparse_a8: need M >= 0, K %% 64 == 0, 64 <= K <= %lld (M=%lld K=%lld)",
             (long long)kMaxKSparse, (long long)M, (long long)K);
  BW_REQUIRE(k_keep >= 1 && k_keep <= K, BW_ERR_ARG, "bw_quantize_sparse_a8: need 1 <= k_keep <= K (k_keep=%lld)",
             (long long)k_keep);
  if (M == 0) return ok();
  BW_REQUIRE(gate_or_x && codes && scales, BW_ERR_NULL, "bw_quantize_sparse_a8: NULL pointer");
  BW_REQUIRE(!misaligned(gate_or_x) && !misaligned(up) && !misaligned(codes) && !misaligned(scales) &&
                 !misaligned(mask_dbg),
             BW_ERR_ALIGN, "bw_quantize_sparse_a8: device pointers must be 16-byte aligned");
  return hip_status(bw::launch_sparse_a8(gate_or_x, up, dtype == BW_BF16, M, K, k_keep, codes, scales, mask_dbg,
                                         static_cast<hipStream_t>(stream)),
                    "bw_quantize_sparse_a8");
}

bw_status bw_bitlinear_sparse_a8(const int8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                 const uint8_t* w_packed, const float* beta, int64_t N, float* y, int32_t* acc_dbg,
                                 void* stream) {
  bw_status st = check_gemm("bw_bitlinear_sparse_a8", codes, x_scales, M, K, w_packed, beta, N, y, acc_dbg);
  if (st != BW_OK || M == 0) return st;
  return hip_status(bw::launch_bitlinear(2, codes, x_scales, M, K, w_packed, beta, N, y, acc_dbg,
                                         static_cast<hipStream_t>(stream)),
                    "bw_bitlinear_sparse_a8");
}

bw_status bw_bitlinear_sparse_a8_grouped(const int8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                         int n_groups, const uint8_t* const* w_packed,
                                         const float* const* beta, const int64_t* N, float* const* y,
                                         int32_t* const* acc_dbg, void* stream) {
  void* acc[bw::kMaxGroups] = {};
  if (acc_dbg && n_groups >= 1 && n_groups <= bw::kMaxGroups)
    for (int g = 0; g < n_groups; ++g) acc[g] = acc_dbg[g];
  return bitlinear_grouped("bw_bitlinear_sparse_a8_grouped", 2, codes, x_scales, M, K, n_groups, w_packed, beta, N,
                           y, acc_dbg ? acc : nullptr, static_cast<hipStream_t>(stream));
}

size_t bw_bitlinear_sparse_a8_gather_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K < 64 || K % 64 != 0 || N <= 0 || M > bw::kGatherMaxM) return 0;
  return bw::gather_a8_workspace_bytes(M, K, N);
}

bw_status bw_bitlinear_sparse_a8_gather(const int8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                        const uint8_t* w_kmajor, const float* beta, int64_t N, float* y,
                                        int32_t* acc_dbg, void* workspace, size_t workspace_bytes, void* stream) {
  bw_status st = check_gemm("bw_bitlinear_sparse_a8_gather", codes, x_scales, M, K, w_kmajor, beta, N, y, acc_dbg);
  if (st != BW_OK || M == 0) return st;
  BW_REQUIRE(M <= bw::kGatherMaxM, BW_ERR_SHAPE, "bw_bitlinear_sparse_a8_gather: need M <= %lld (M=%lld)",
             (long long)bw::kGatherMaxM, (long long)M);
  BW_REQUIRE(N <= (int64_t(1) << 33) / K, BW_ERR_SHAPE,
             "bw_bitlinear_sparse_a8_gather: the packed weights must stay below 2^31 bytes (N=%lld K=%lld)",
             (long long)N, (long long)K);
  BW_REQUIRE(workspace, BW_ERR_NULL, "bw_bitlinear_sparse_a8_gather: NULL workspace");
  BW_REQUIRE(!misaligned(workspace), BW_ERR_ALIGN, "bw_bitlinear_sparse_a8_gather: workspace must be 16-byte aligned");
  const size_t need = bw::gather_a8_workspace_bytes(M, K, N);
  BW_REQUIRE(workspace_bytes >= need, BW_ERR_ARG, "bw_bitlinear_sparse_a8_gather: workspace needs %zu bytes, got %zu",
             need, workspace_bytes);
  return hip_status(bw::launch_gather_a8(codes, x_scales, M, K, w_kmajor, beta, N, y, acc_dbg, workspace,
                                         static_cast<hipStream_t>(stream)),
                    "bw_bitlinear_sparse_a8_gather");
}

static bw_status check_kv(const char* who, int64_t B, int64_t S, int64_t H, int64_t D, int64_t n_special) {
  BW_REQUIRE(B >= 0 && S >= 0 && H >= 1 && n_special >= 0, BW_ERR_SHAPE,
             "%s: need B, S >= 0, H >= 1, n_special >= 0", who);
  BW_REQUIRE(D == 32 || D == 64 || D == 128 || D == 256 || D == 512, BW_ERR_SHAPE,
             "%s: head_dim must be 32, 64, 128, 256 or 512 (D=%lld)", who, (long long)D);
  BW_REQUIRE(B == 0 || S == 0 || (B <= (int64_t(1) << 40) / S / H / D), BW_ERR_SHAPE, "%s: tensor too large", who);
  return ok();
}

bw_status bw_kv_pack3(const void* kv, bw_dtype dtype, int64_t B, int64_t S, int64_t H, int64_t D,
                      const int32_t* slot_of, int64_t n_special, uint8_t* p3, float* s3, uint8_t* p4, float* s4,
                      void* stream) {
  BW_REQUIRE(dtype == BW_F32 || dtype == BW_BF16, BW_ERR_DTYPE, "bw_kv_pack3: bad dtype %d", (int)dtype);
  bw_status st = check_kv("bw_kv_pack3", B, S, H, D, n_special);
  if (st != BW_OK) return st;
  if (B == 0 || S == 0) return ok();
  BW_REQUIRE(kv && slot_of && p3 && s3, BW_ERR_NULL, "bw_kv_pack3: NULL pointer");
  BW_REQUIRE(n_special == 0 || (p4 && s4), BW_ERR_NULL, "bw_kv_pack3: p4/s4 required when n_special > 0");
  BW_REQUIRE(!misaligned(kv) && !misaligned(slot_of) && !misaligned(p3) && !misaligned(s3) && !misaligned(p4) &&
                 !misaligned(s4),
             BW_ERR_ALIGN, "bw_kv_pack3: device pointers must be 16-byte aligned");
  return hip_status(bw::launch_kv_pack3(kv, dtype == BW_BF16, B, S, H, D, slot_of, n_special, p3, s3, p4, s4,
                                        static_cast<hipStream_t>(stream)),
                    "bw_kv_pack3");
}

bw_status bw_kv_unpack3(const uint8_t* p3, const float* s3, const uint8_t* p4, const float* s4,
                        const int32_t* slot_of, int64_t B, int64_t S, int64_t H, int64_t D, int64_t n_special,
                        bw_dtype out_dtype, void* out, void* stream) {
  BW_REQUIRE(out_dtype == BW_F32 || out_dtype == BW_BF16, BW_ERR_DTYPE, "bw_kv_unpack3: bad dtype %d",
             (int)out_dtype);
  bw_status st = check_kv("bw_kv_unpack3", B, S, H, D, n_special);
  if (st != BW_OK) return st;
  if (B == 0 || S == 0) return ok();
  BW_REQUIRE(p3 && s3 && slot_of && out, BW_ERR_NULL, "bw_kv_unpack3: NULL pointer");
  BW_REQUIRE(n_special == 0 || (p4 && s4), BW_ERR_NULL, "bw_kv_unpack3: p4/s4 required when n_special > 0");
  BW_REQUIRE(!misaligned(p3) && !misaligned(s3) && !misaligned(p4) && !misaligned(s4) && !misaligned(slot_of) &&
                 !misaligned(out),
             BW_ERR_ALIGN, "bw_kv_unpack3: device pointers must be 16-byte aligned");
  return hip_status(bw::launch_kv_unpack3(p3, s3, p4, s4, slot_of, B, S, H, D, n_special, out_dtype == BW_BF16,
                                          out, static_cast<hipStream_t>(stream)),
                    "bw_kv_unpack3");
}

size_t bw_attn_decode_kv3_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (B <= 0 || S <= 0 || H <= 0 || H > bw::kAttnMaxH || (D != 64 && D != 128)) return 0;
  if (!bw::attn_decode3_supported(B, S, H)) return 0;
  return bw::attn_decode3_workspace_bytes(B, S, H, D);
}

bw_status bw_attn_decode_kv3(const float* q, const uint8_t* k_p3, const float* k_s3, const uint8_t* k_p4,
                             const float* k_s4, const uint8_t* v_p3, const float* v_s3, const uint8_t* v_p4,
                             const float* v_s4, const int32_t* slot_of, int64_t n_special, int64_t B, int64_t S,
                             int64_t H, int64_t D, float* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  BW_REQUIRE(B >= 0 && H >= 1 && H <= bw::kAttnMaxH && n_special >= 0 && S >= 1, BW_ERR_SHAPE,
             "bw_attn_decode_kv3: need B >= 0, S >= 1, 1 <= H <= %lld, n_special >= 0 (B=%lld S=%lld H=%lld)",
             (long long)bw::kAttnMaxH, (long long)B, (long long)S, (long long)H);
  BW_REQUIRE(D == 64 || D == 128, BW_ERR_SHAPE, "bw_attn_decode_kv3: head_dim must be 64 or 128 (D=%lld)",
             (long long)D);
  BW_REQUIRE(B <= (int64_t(1) << 40) / S / H / D && B * H <= (int64_t(1) << 31) - 1, BW_ERR_SHAPE,
             "bw_attn_decode_kv3: tensor too large");
  if (B == 0) return ok();
  BW_REQUIRE(bw::attn_decode3_supported(B, S, H), BW_ERR_SHAPE,
             "bw_attn_decode_kv3: S=%lld with H=%lld exceeds the chunk limits", (long long)S, (long long)H);
  BW_REQUIRE(q && k_p3 && k_s3 && v_p3 && v_s3 && slot_of && out && workspace, BW_ERR_NULL,
             "bw_attn_decode_kv3: NULL pointer");
  BW_REQUIRE(n_special == 0 || (k_p4 && k_s4 && v_p4 && v_s4), BW_ERR_NULL,
             "bw_attn_decode_kv3: 4-bit slabs required when n_special > 0");
  BW_REQUIRE(!misaligned(q) && !misaligned(k_p3) && !misaligned(k_s3) && !misaligned(k_p4) && !misaligned(k_s4) &&
                 !misaligned(v_p3) && !misaligned(v_s3) && !misaligned(v_p4) && !misaligned(v_s4) &&
                 !misaligned(slot_of) && !misaligned(out) && !misaligned(workspace),
             BW_ERR_ALIGN, "bw_attn_decode_kv3: device pointers must be 16-byte aligned");
  const size_t need = bw::attn_decode3_workspace_bytes(B, S, H, D);
  BW_REQUIRE(workspace_bytes >= need, BW_ERR_ARG, "bw_attn_decode_kv3: workspace needs %zu bytes, got %zu", need,
             workspace_bytes);
  return hip_status(bw::launch_attn_decode3(q, k_p3, k_s3, k_p4, k_s4, v_p3, v_s3, v_p4, v_s4, slot_of, n_special, B,
                                            S, H, D, out, workspace, static_cast<hipStream_t>(stream)),
                    "bw_attn_decode_kv3");
}

static bool block_shape_ok(int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F) {
  const int64_t hd = H * D;
  return B >= 1 && B <= bw::kGemvMaxM && H >= 1 && H <= bw::kAttnMaxH && (D == 64 || D == 128) && hd % 64 == 0 &&
         hd <= kMaxKSparse && F >= 64 && F % 64 == 0 && F <= kMaxKSparse && S_cap >= 1 &&
         B <= (int64_t(1) << 40) / S_cap / hd && bw::attn_decode3_supported(B, S_cap, H);
}

size_t bw_block_decode_workspace_bytes(int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F) {
  if (!block_shape_ok(B, S_cap, H, D, F)) return 0;
  return bw::block_decode_workspace_bytes(B, S_cap, H, D, F);
}

static bw_status check_block(const char* who, const float* x, float* x_out, int64_t B, int64_t H, int64_t D,
                             int64_t F, const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o,
                             const float* b_o, const uint8_t* w_gate_up, const float* b_gate_up,
                             const uint8_t* w_down, const float* b_down, uint8_t* k_p3, float* k_s3, uint8_t* k_p4,
                             float* k_s4, uint8_t* v_p3, float* v_s3, uint8_t* v_p4, float* v_s4,
                             const int32_t* slot_of, int64_t n_special, int64_t S_cap, int64_t pos) {
  BW_REQUIRE(block_shape_ok(B, S_cap, H, D, F), BW_ERR_SHAPE,
             "%s: need 1 <= B <= %lld, D = 64 or 128, H*D %% 64 == 0 and <= %lld, F %% 64 == 0 and "
             "<= %lld, S_cap within the attention limits (B=%lld H=%lld D=%lld F=%lld S_cap=%lld)",
             who, (long long)bw::kGemvMaxM, (long long)kMaxKSparse, (long long)kMaxKSparse, (long long)B,
             (long long)H, (long long)D, (long long)F, (long long)S_cap);
  BW_REQUIRE(pos >= 0 && pos < S_cap && n_special >= 0, BW_ERR_ARG,
             "%s: need 0 <= pos < S_cap and n_special >= 0 (pos=%lld)", who, (long long)pos);
  BW_REQUIRE(x && x_out && w_qkv && b_qkv && w_o && b_o && w_gate_up && b_gate_up && w_down && b_down && k_p3 &&
                 k_s3 && v_p3 && v_s3 && slot_of,
             BW_ERR_NULL, "%s: NULL pointer", who);
  BW_REQUIRE(n_special == 0 || (k_p4 && k_s4 && v_p4 && v_s4), BW_ERR_NULL,
             "%s: 4-bit slabs required when n_special > 0", who);
  const void* ptrs[] = {x, x_out, w_qkv, b_qkv, w_o, b_o, w_gate_up, b_gate_up, w_down, b_down, k_p3, k_s3, k_p4,
                        k_s4, v_p3, v_s3, v_p4, v_s4, slot_of};
  for (const void* p : ptrs) BW_REQUIRE(!misaligned(p), BW_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
  // the attention region is sized for every attended length up to S_cap; the
  // launch at this position must fit in it
  BW_REQUIRE(bw::attn_decode3_workspace_bytes(B, pos + 1, H, D) <= bw::attn_decode3_workspace_bound(B, S_cap, H, D),
             BW_ERR_UNSUPPORTED, "%s: attention workspace at pos=%lld exceeds its region", who, (long long)pos);
  return ok();
}

bw_status bw_block_decode(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                          const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                          const uint8_t* w_gate_up, const float* b_gate_up, const uint8_t* w_down,
                          const float* b_down, uint8_t* k_p3, float* k_s3, uint8_t* k_p4, float* k_s4,
                          uint8_t* v_p3, float* v_s3, uint8_t* v_p4, float* v_s4, const int32_t* slot_of,
                          int64_t n_special, int64_t S_cap, int64_t pos, void* workspace, size_t workspace_bytes,
                          void* stream) {
  bw_status st = check_block("bw_block_decode", x, x_out, B, H, D, F, w_qkv, b_qkv, w_o, b_o, w_gate_up, b_gate_up,
                             w_down, b_down, k_p3, k_s3, k_p4, k_s4, v_p3, v_s3, v_p4, v_s4, slot_of, n_special,
                             S_cap, pos);
  if (st != BW_OK) return st;
  BW_REQUIRE(workspace, BW_ERR_NULL, "bw_block_decode: NULL workspace");
  BW_REQUIRE(!misaligned(workspace), BW_ERR_ALIGN, "bw_block_decode: device pointers must be 16-byte aligned");
  const size_t need = bw::block_decode_workspace_bytes(B, S_cap, H, D, F);
  BW_REQUIRE(workspace_bytes >= need, BW_ERR_ARG, "bw_block_decode: workspace needs %zu bytes, got %zu", need,
             workspace_bytes);
  return hip_status(bw::launch_block_decode(x, x_out, B, H, D, F, w_qkv, b_qkv, w_o, b_o, w_gate_up, b_gate_up, w_down,
                                            b_down, k_p3, k_s3, k_p4, k_s4, v_p3, v_s3, v_p4, v_s4, slot_of,
                                            n_special, S_cap, pos, workspace, static_cast<hipStream_t>(stream)),
                    "bw_block_decode");
}

bw_status bw_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  BW_REQUIRE(bytes >= 0 && bytes % 16 == 0 && bytes < (int64_t(1) << 40), BW_ERR_SHAPE,
             "bw_stream_read: need 0 <= bytes < 2^40 and bytes %% 16 == 0 (bytes=%lld)", (long long)bytes);
  if (bytes == 0) return ok();
  BW_REQUIRE(src && sink, BW_ERR_NULL, "bw_stream_read: NULL pointer");
  BW_REQUIRE(!misaligned(src) && !misaligned(sink), BW_ERR_ALIGN, "bw_stream_read: device pointers must be 16-byte aligned");
  return hip_status(bw::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)), "bw_stream_read");
}

size_t bw_block_decode_noalloc_max_bytes(void) { return bw::kBlockScratchBytes; }

bw_status bw_block_decode_noalloc(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                                  const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                                  const uint8_t* w_gate_up, const float* b_gate_up, const uint8_t* w_down,
                                  const float* b_down, uint8_t* k_p3, float* k_s3, uint8_t* k_p4, float* k_s4,
                                  uint8_t* v_p3, float* v_s3, uint8_t* v_p4, float* v_s4, const int32_t* slot_of,
                                  int64_t n_special, int64_t S_cap, int64_t pos, void* stream) {
  bw_status st = check_block("bw_block_decode_noalloc", x, x_out, B, H, D, F, w_qkv, b_qkv, w_o, b_o, w_gate_up,
                             b_gate_up, w_down, b_down, k_p3, k_s3, k_p4, k_s4, v_p3, v_s3, v_p4, v_s4, slot_of,
                             n_special, S_cap, pos);
  if (st != BW_OK) return st;
  const size_t need = bw::block_decode_workspace_bytes(B, S_cap, H, D, F);
  BW_REQUIRE(need <= bw::kBlockScratchBytes, BW_ERR_UNSUPPORTED,
             "bw_block_decode_noalloc: this shape needs %zu bytes of workspace, above the %zu-byte static scratch "
             "(use bw_block_decode with a caller workspace)",
             need, bw::kBlockScratchBytes);
  void* ws = nullptr;
  st = hip_status(bw::block_scratch(&ws), "bw_block_decode_noalloc (scratch address)");
  if (st != BW_OK) return st;
  return hip_status(bw::launch_block_decode(x, x_out, B, H, D, F, w_qkv, b_qkv, w_o, b_o, w_gate_up, b_gate_up, w_down,
                                            b_down, k_p3, k_s3, k_p4, k_s4, v_p3, v_s3, v_p4, v_s4, slot_of,
                                            n_special, S_cap, pos, ws, static_cast<hipStream_t>(stream)),
                    "bw_block_decode_noalloc");
}

}  // extern "C"
