/*
 * bw.h -- C ABI of the BitNet a4.8 hybrid-quantized BitLinear library for
 * AMD MI355X (gfx950).  Library: ternary_weight_bit_amd/libbw.so.
 *
 * What the calls compute is stated on the BitNet a4.8 pages:
 *   - "BitNet a4.8: 4-bit Activations for 1-bit LLMs", abstract (arXiv
 *     2411.04965v1): ternary-weight layers take 4-bit activations at the
 *     inputs of attention and FFN (INT4/FP4 kernels) and sparsified, then
 *     8-bit, intermediate states; the model supports a 3-bit KV cache;
 *   - toshoseti review of the paper, «Метод»: 4-bit activations for the
 *     q/k/v/gate/up inputs only, top-k sparsification (50 %) of the out
 *     projection input, ReLU^2 in place of swish in the FFN gate, FP4 as the
 *     wide-range alternative to INT4; opening lines: ternary weights,
 *     absmax INT8 activations (b1.58); «Эксперименты»: 3-bit KV caches with
 *     bos/eos tokens kept at 4 bits.
 * The pages give no formula; the exact arithmetic each call follows is stated
 * in its comment below.
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *     and owns every buffer; the library allocates nothing and keeps no
 *     device state, except the one static workspace array per GPU that
 *     bw_block_decode_noalloc uses.  Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     on it and return without waiting.
 *   - Arguments are validated on the host before anything is launched.  A
 *     status other than BW_OK means nothing was enqueued and the outputs are
 *     untouched; bw_last_error() (host, per thread) then holds a message.
 *     A HIP launch failure returns BW_ERR_HIP.  No C++ exception crosses
 *     this interface.
 *   - M == 0 (or B*S == 0) is a valid empty call: BW_OK, nothing launched.
 *   - Arithmetic: IEEE fp32 with round-half-to-even, one correctly-rounded
 *     operation at a time (no fused multiply-add) wherever a float decides a
 *     code; a' = max(absmax, 1e-5).
 *   - Calls that overlap on one stream-ordered buffer race; calls on
 *     different buffers are independent.
 */
#ifndef BW_H_
#define BW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BW_ABI_VERSION 2
#define BW_PACK_LAYOUT_VERSION 2

typedef enum {
  BW_OK = 0,
  BW_ERR_NULL = 1,        /* a required pointer is NULL */
  BW_ERR_SHAPE = 2,       /* a size breaks the shape rules of the call */
  BW_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  BW_ERR_DTYPE = 4,       /* unknown dtype / format / role enum */
  BW_ERR_ARG = 5,         /* other bad argument (k_keep, workspace size, ...) */
  BW_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  BW_ERR_UNSUPPORTED = 7  /* valid request this build does not implement */
} bw_status;

typedef enum { BW_F32 = 0, BW_BF16 = 1 } bw_dtype;

typedef enum {
  BW_ACT_INT4 = 0,      /* two's-complement 4-bit integers, absmax scale a'/7 */
  BW_ACT_FP4_E2M1 = 1,  /* e2m1 floats (magnitudes 0,.5,1,1.5,2,3,4,6), scale a'/6 */
  BW_ACT_INT4_E2M3 = 2  /* the values and scales of BW_ACT_INT4, each value stored as a
                           6-bit e2m3 field (the operand of the fp6 matrix cores) */
} bw_act4_fmt;

/* Which activations a packed weight meets; selects the within-word order of
 * the 2-bit codes (both orders are 2 bits per weight, same tile structure). */
typedef enum {
  BW_ROLE_A4 = 0,        /* q/k/v/gate/up: meets 4-bit activations (bw_bitlinear_a4) */
  BW_ROLE_A8 = 1,        /* out_proj/down_proj: meets 8-bit codes (bw_bitlinear_sparse_a8) */
  BW_ROLE_A8_KMAJOR = 2  /* out_proj/down_proj, K-major rows for bw_bitlinear_sparse_a8_gather */
} bw_weight_role;

/* host */ int bw_abi_version(void);
/* Version of the stored formats (packed ternary weights and the 3-bit KV
 * slab); data written under another version must be packed again. */
/* host */ int bw_pack_layout_version(void);
/* host: message for the last non-OK status returned on this thread ("" if none) */
const char* bw_last_error(void);

/* ------------------------------------------------------------------------ *
 * Ternary weights (offline, once per weight tensor).
 * Source: toshoseti review, opening lines -- BitNet b1.58 (whose weights
 * BitNet a4.8 keeps) uses ternary {-1, 0, +1} weights.
 *
 * Computes, for one tensor W[N][K] (nn.Linear out x in, row-major):
 *   beta  = fp32( fp64(sum |w|) / (N*K) ), with the sum over all N*K
 *           magnitudes formed exactly and rounded once to fp64;
 *   beta' = max(beta, 1e-5);
 *   t     = sign(w) * [2|w| > beta']   (RoundClip(w/beta', -1, 1), ties to 0)
 * and writes t packed at 2 bits per weight, codes 00 = 0, 01 = +1, 11 = -1:
 *   tiles of 16 output channels x 64 inputs, 256 bytes each, at byte offset
 *   (nb*(K/64) + kb)*256; inside a tile channel c owns bytes [16c, 16c+16) as
 *   four little-endian uint32 words, word j covering inputs 64kb+16j+(0..15);
 *   code slot i (bits 2i..2i+1) holds input offset
 *     BW_ROLE_A4: (i odd ? 8 : 0) + i/2
 *     BW_ROLE_A8: 4*(i%4) + i/4
 * BW_ROLE_A8_KMAJOR instead stores one contiguous run per input: input k
 *   owns bytes [k*N/4, (k+1)*N/4); little-endian uint32 word g of the run
 *   holds outputs 16g + i (i = 0..15) at bits 2i..2i+1 with code t + 1
 *   (00 = -1, 01 = 0, 10 = +1; 11 is never written).
 * beta[N] (fp32) receives beta' in every entry, so the packed bytes and beta
 * arrays of separately-scaled tensors (fused q/k/v, gate/up) concatenate
 * along N.
 *
 * Shapes: N % 16 == 0, K % 64 == 0, N, K >= 1, N*K < 2^40.  W dtype BW_F32
 * or BW_BF16.  Non-finite weights are not supported.
 * workspace: device, >= bw_pack_ternary_workspace_bytes(N, K) bytes; its
 * contents on entry are ignored (the call clears what it uses).
 * ------------------------------------------------------------------------ */
/* host */ size_t bw_ternary_packed_bytes(int64_t N, int64_t K);
/* host */ size_t bw_pack_ternary_workspace_bytes(int64_t N, int64_t K);
bw_status bw_pack_ternary(const void* W, bw_dtype w_dtype, int64_t N, int64_t K,
                          bw_weight_role role, uint8_t* w_packed, float* beta,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * 4-bit activation quantizer (inputs of q/k/v/gate/up).
 * Source: BitNet a4.8 abstract (4-bit activations for the attention and FFN
 * inputs, INT4/FP4 kernels); toshoseti review «Метод» (only q/k/v/gate/up
 * get 4 bits; FP4 considered for its wider range).
 *
 * Per token (row) m of x[M][K]: a' = max(max_k |x|, 1e-5);
 *   BW_ACT_INT4:     inv = fl(7/a'), s = fl(a'/7), q = clamp(rne(fl(x*inv)), -8, 7)
 *   BW_ACT_FP4_E2M1: inv = fl(6/a'), s = fl(a'/6), t = fl(x*inv) rounded to the
 *                    nearest e2m1 magnitude (ties to the even code, saturate
 *                    at 6), sign bit copied from t.
 * codes[M][K/2] (uint8): two codes per byte, even k in the low nibble.
 * BW_ACT_INT4_E2M3: the same q and s as BW_ACT_INT4; codes[M][3K/4] (uint8)
 *   hold per value the field f = (q < 0) << 5 | |q| (e2m3: sign bit, 2-bit
 *   exponent, 3-bit mantissa with bias 1, so f reads as q/8 exactly for
 *   |q| <= 15).  Per 64 values (48 bytes): let S0, S1 be the 24-byte
 *   little-endian bit streams of the fields of values 0..31 and 32..63
 *   (value j at bits 6j..6j+5); the bytes are S0[0:16], S1[0:16], S0[16:24],
 *   S1[16:24].
 * scales[M] (fp32): s.
 * Shapes: K % 64 == 0, K <= 131072.  x dtype BW_F32 or BW_BF16.
 * ------------------------------------------------------------------------ */
bw_status bw_quantize(const void* x, bw_dtype x_dtype, int64_t M, int64_t K, bw_act4_fmt fmt,
                      uint8_t* codes, float* scales, void* stream);

/* ------------------------------------------------------------------------ *
 * W1.58A4 BitLinear: 4-bit activation codes x ternary weights.
 * Source: BitNet a4.8 abstract (ternary layers on 4-bit activations, run by
 * INT4/FP4 kernels).
 *
 *   acc[m][n] = sum_k v(codes[m][k]) * t[n][k]   (v = integer code, or the
 *               e2m1 value; exact: int32, resp. fp32 multiples of 1/2)
 *   y[m][n]   = fl( fl(acc * x_scales[m]) * beta[n] )
 * codes/x_scales: as written by bw_quantize with the same fmt.  w_packed:
 * BW_ROLE_A4 layout of t[N][K].  y: fp32 [M][N] row-major.
 * acc_dbg: NULL, or [M][N] receiving acc (int32 for BW_ACT_INT4 and
 * BW_ACT_INT4_E2M3, fp32 for BW_ACT_FP4_E2M1), for exactness checks.
 * BW_ACT_INT4_E2M3 gives the same acc and y as BW_ACT_INT4 on the same
 * values (bit for bit) from the fp6 x fp4 matrix instruction, at any M (the
 * weight-streaming GEMV up to 16 tokens, the LDS GEMM above); it
 * returns BW_ERR_UNSUPPORTED when M*3K/4 or N*K/4 reaches 2^31 bytes.
 * Shapes: K % 64 == 0, K <= 131072, N % 16 == 0.
 * ------------------------------------------------------------------------ */
bw_status bw_bitlinear_a4(const uint8_t* codes, const float* x_scales, int64_t M, int64_t K,
                          bw_act4_fmt fmt, const uint8_t* w_packed, const float* beta,
                          int64_t N, float* y, void* acc_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * Several W1.58A4 BitLinear products over the same 4-bit codes in one call.
 * Source: as bw_bitlinear_a4 (BitNet a4.8 abstract: ternary layers on 4-bit
 * activations); the projections that read one activation (q/k/v, or gate
 * and up) share its codes.
 * For g < n_groups, y[g] receives exactly bw_bitlinear_a4(codes, x_scales,
 * M, K, fmt, w_packed[g], beta[g], N[g]) (bit for bit), and acc_dbg[g] its
 * accumulators.  With M > 16 tokens and K % 128 == 0 all products run as one
 * launch whose grid holds the tiles of every product, so one product's tiles
 * fill the CUs another's leave idle; otherwise one launch per product.
 * w_packed, beta, N, y: HOST arrays of n_groups entries (device pointers of
 * the same kinds as bw_bitlinear_a4's, and sizes).  acc_dbg: NULL, or a host
 * array of n_groups entries, each NULL or as bw_bitlinear_a4's.  The host
 * arrays are read during the call only.
 * Shapes: 1 <= n_groups <= 4; every product as bw_bitlinear_a4.
 * ------------------------------------------------------------------------ */
bw_status bw_bitlinear_a4_grouped(const uint8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                  bw_act4_fmt fmt, int n_groups, const uint8_t* const* w_packed,
                                  const float* const* beta, const int64_t* N, float* const* y,
                                  void* const* acc_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * 4-bit quantizer and W1.58A4 BitLinear in one call.
 * Source: as bw_quantize and bw_bitlinear_a4 (BitNet a4.8 abstract: 4-bit
 * activations for the attention and FFN inputs, INT4/FP4 kernels).
 * Computes exactly bw_quantize(x) followed by bw_bitlinear_a4 on its codes:
 * writes codes and scales[M] (bw_quantize's bytes) and y[M][N]
 * (bw_bitlinear_a4's values).  For one or two tokens (M <= 2, K <= 8192) and
 * BW_ACT_INT4 or BW_ACT_FP4_E2M1 it is one launch in which every workgroup
 * quantizes the tokens itself; otherwise the two launches of the separate
 * calls.
 * acc_dbg: as bw_bitlinear_a4.
 * Shapes: K % 64 == 0, K <= 131072, N % 16 == 0.  x dtype BW_F32 or BW_BF16.
 * ------------------------------------------------------------------------ */
bw_status bw_quantize_bitlinear_a4(const void* x, bw_dtype x_dtype, int64_t M, int64_t K, bw_act4_fmt fmt,
                                   const uint8_t* w_packed, const float* beta, int64_t N, uint8_t* codes,
                                   float* scales, float* y, void* acc_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * Sparsified 8-bit activations (inputs of out_proj and down_proj).
 * Source: BitNet a4.8 abstract (intermediate states sparsified, then 8-bit);
 * toshoseti review «Метод» (top-k at 50 % for the out projection input;
 * ReLU^2 gate to sparsify the down projection input); 9pt.com article,
 * methodology (low-magnitude entries are the ones dropped); toshoseti
 * review, opening lines (absmax INT8).
 *
 * Per token m: h = up ? fl(fl(r*r) * up) with r = max(gate, 0) : x;
 * survivors = the k_keep entries first in the order (|h| descending, index
 * ascending); a' = max(max |h| over survivors, 1e-5); inv = fl(127/a');
 * codes = clamp(rne(fl(h*inv)), -128, 127) for survivors, 0 otherwise;
 * scales[m] = fl(a'/127).
 * up: NULL selects the plain-input front end (out_proj).  k_keep = K turns
 * the sparsifier off (the b1.58 INT8 path).
 * codes: int8 [M][K].  mask_dbg: NULL, or uint32 [M][K/32] with bit i of
 * word w set when entry 32w+i survives.
 * Shapes: K % 64 == 0, K <= 16384, 1 <= k_keep <= K.  dtype BW_F32 or BW_BF16
 * (gate and up share it).
 * ------------------------------------------------------------------------ */
bw_status bw_quantize_sparse_a8(const void* gate_or_x, const void* up, bw_dtype dtype,
                                int64_t M, int64_t K, int64_t k_keep, int8_t* codes,
                                float* scales, uint32_t* mask_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * W1.58A8 BitLinear on the sparsified INT8 codes.
 * Source: as bw_quantize_sparse_a8 (8-bit codes feeding ternary layers).
 *   acc[m][n] = sum_k codes[m][k] * t[n][k]  (int32, exact)
 *   y[m][n]   = fl( fl(acc * x_scales[m]) * beta[n] )
 * w_packed: BW_ROLE_A8 layout.  acc_dbg: NULL or int32 [M][N].
 * Shapes: K % 64 == 0, K <= 131072, N % 16 == 0.
 * ------------------------------------------------------------------------ */
bw_status bw_bitlinear_sparse_a8(const int8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                 const uint8_t* w_packed, const float* beta, int64_t N, float* y,
                                 int32_t* acc_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * Several W1.58A8 BitLinear products over the same INT8 codes in one call.
 * Source: as bw_bitlinear_sparse_a8.  The b1.58 path (absmax INT8 of every
 * entry, toshoseti review, opening lines) feeds q/k/v and gate/up from one
 * set of codes the same way the 4-bit path does.
 * For g < n_groups, y[g] receives exactly bw_bitlinear_sparse_a8(codes,
 * x_scales, M, K, w_packed[g], beta[g], N[g]); launches as
 * bw_bitlinear_a4_grouped.  Host arrays and acc_dbg as there (int32 [M][N]).
 * Shapes: 1 <= n_groups <= 4; every product as bw_bitlinear_sparse_a8.
 * ------------------------------------------------------------------------ */
bw_status bw_bitlinear_sparse_a8_grouped(const int8_t* codes, const float* x_scales, int64_t M, int64_t K,
                                         int n_groups, const uint8_t* const* w_packed,
                                         const float* const* beta, const int64_t* N, float* const* y,
                                         int32_t* const* acc_dbg, void* stream);

/* ------------------------------------------------------------------------ *
 * W1.58A8 product that reads only the weight rows of nonzero codes.
 * Source: BitNet a4.8 abstract (only 55 % of the parameters are active, the
 * sparsified inputs of out_proj/down_proj being mostly zeros); toshoseti
 * review, «Метод» (the top-k pattern is random, so a tiled weight layout
 * cannot skip it).  Computes exactly what bw_bitlinear_sparse_a8 computes,
 *   acc[m][n] = sum_k codes[m][k] * t[n][k]  (int32, exact)
 *   y[m][n]   = fl( fl(acc * x_scales[m]) * beta[n] )
 * but each token reads from the BW_ROLE_A8_KMAJOR weights only the rows k
 * with codes[m][k] != 0: at 50 % sparsity half of the weight bytes.  Tokens
 * are independent, so it saves bytes only at M = 1 (single-token decode);
 * larger M re-reads the weights once per token.
 * w_kmajor: BW_ROLE_A8_KMAJOR layout.  acc_dbg: NULL or int32 [M][N].
 * workspace: device, >= bw_bitlinear_sparse_a8_gather_workspace_bytes(M, K, N)
 *   bytes (int32 partial sums, a few hundred KB at decode shapes); contents
 *   on entry are ignored.  Calls sharing one workspace must be stream-ordered.
 * Shapes: K % 64 == 0, K <= 131072, N % 16 == 0, 1 <= M <= 16,
 *   N*K/4 <= 2^31.  workspace_bytes() returns 0 for shapes outside these.
 * ------------------------------------------------------------------------ */
/* host */ size_t bw_bitlinear_sparse_a8_gather_workspace_bytes(int64_t M, int64_t K, int64_t N);
bw_status bw_bitlinear_sparse_a8_gather(const int8_t* codes, const float* x_scales, int64_t M,
                                        int64_t K, const uint8_t* w_kmajor, const float* beta,
                                        int64_t N, float* y, int32_t* acc_dbg, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * 3-bit KV cache with 4-bit special tokens.
 * Source: toshoseti review «Эксперименты» (3-bit KV caches; bos/eos tokens
 * kept at 4 bits); BitNet a4.8 abstract (3-bit KV cache).
 *
 * kv: [B][S][H][D] (BW_F32 or BW_BF16).  Per vector v = kv[b][s][h][:]:
 *   a' = max(max |v|, 1e-5);
 *   3-bit: s3 = fl(a'/3), q = clamp(rne(fl(v*fl(3/a'))), -4, 3) (always written);
 *   if 0 <= slot_of[b][s] < n_special (a special token): also
 *          s4 = fl(a'/7), q4 = clamp(rne(fl(v*fl(7/a'))), -8, 7) into that slot.
 * p3: uint8 [B][S][H][3*D/8]; per group of 32 codes three little-endian
 *     uint32 words W0, W1, W2 of fields u = q + 4 (0..7); byte i of the three
 *     words holds codes 8i..8i+7 (u0..u7):  W0 = u0 | u1<<3 | (u6&3)<<6,
 *     W1 = u2 | u3<<3 | (u6>>2)<<6 | (u7&1)<<7,  W2 = u4 | u5<<3 | (u7>>1)<<6.
 *     s3: fp32 [B][S][H].
 * p4: uint8 [n_special][H][D/2], even d in the low nibble.  s4: fp32
 *     [n_special][H].  Slots no position names are left untouched.
 * slot_of: int32 [B][S]; values outside [0, n_special) mark ordinary tokens.
 *     Two positions naming one slot race.
 * unpack: out[b][s][h][d] = fl(q * s) from the side slot for special tokens,
 *     from the 3-bit slab otherwise; BW_BF16 output is that fp32 value
 *     rounded half-to-even.
 * Shapes: D in {32, 64, 128, 256, 512}; n_special >= 0 (p4/s4 may be NULL
 * when n_special == 0).
 * ------------------------------------------------------------------------ */
bw_status bw_kv_pack3(const void* kv, bw_dtype dtype, int64_t B, int64_t S, int64_t H, int64_t D,
                      const int32_t* slot_of, int64_t n_special, uint8_t* p3, float* s3,
                      uint8_t* p4, float* s4, void* stream);
bw_status bw_kv_unpack3(const uint8_t* p3, const float* s3, const uint8_t* p4, const float* s4,
                        const int32_t* slot_of, int64_t B, int64_t S, int64_t H, int64_t D,
                        int64_t n_special, bw_dtype out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------ *
 * Single-token attention over the 3-bit KV cache.
 * Source: BitNet a4.8 abstract (3-bit KV cache); toshoseti review,
 * «Эксперименты» (bos/eos kept at 4 bits); 9pt.com article, methodology (the
 * 3-bit cache as part of faster, leaner inference).  The pages give no
 * attention formula; this is standard scaled dot-product attention of one
 * query per (batch, head) over all S cached positions:
 *   k_s, v_s = dequantized vectors as bw_kv_unpack3 defines them (code *
 *              scale; the 4-bit side-slab codes where 0 <= slot_of[b][s] <
 *              n_special);
 *   z_s = (q . k_s) / sqrt(D);  p = softmax_s(z);  out = sum_s p_s v_s.
 * fp32 arithmetic throughout (dot products, exp, sums), so results differ
 * from an exact evaluation by rounding only.
 * q: fp32 [B][H][D].  K and V: p3/s3/p4/s4 slabs as written by bw_kv_pack3
 * for each tensor with the same slot_of.  out: fp32 [B][H][D].
 * workspace: device, >= bw_attn_decode_kv3_workspace_bytes(B, S, H, D) bytes
 *   (per-chunk partial sums; about 2 MB for 8 x 4096 x 32 x 128); contents
 *   on entry are ignored.  Calls sharing a workspace must be stream-ordered.
 * Shapes: D = 64 or 128, S >= 1, 1 <= H <= 1024.  k_p4/k_s4/v_p4/v_s4 may be
 * NULL when n_special == 0.
 * ------------------------------------------------------------------------ */
/* host */ size_t bw_attn_decode_kv3_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D);
bw_status bw_attn_decode_kv3(const float* q, const uint8_t* k_p3, const float* k_s3, const uint8_t* k_p4,
                             const float* k_s4, const uint8_t* v_p3, const float* v_s3, const uint8_t* v_p4,
                             const float* v_s4, const int32_t* slot_of, int64_t n_special, int64_t B,
                             int64_t S, int64_t H, int64_t D, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * One decoder layer for one new token per sequence (decode step).
 * Source: BitNet a4.8 abstract (4-bit inputs of attention and FFN, sparsified
 * 8-bit intermediate states, 3-bit KV cache); toshoseti review, «Метод»
 * (INT4 for q/k/v/gate/up inputs, top-k 50 % for the out_proj input, ReLU^2
 * gate for down_proj) and «Эксперименты» (bos/eos at 4 bits).  The pages give
 * no layer formula; the composition, without normalization or rotary
 * embedding (neither is described), is, with HD = H*D:
 *   y_qkv = bitlinear_a4(quantize(x, INT4), W_qkv)            [B][3HD]
 *   append k = y_qkv[:, HD:2HD], v = y_qkv[:, 2HD:3HD] at position pos of the
 *          3-bit cache (the codec of bw_kv_pack3; the 4-bit slot if special)
 *   a     = attention of q = y_qkv[:, 0:HD] over positions 0..pos (as
 *           bw_attn_decode_kv3)
 *   x1    = x + bitlinear_sparse_a8(quantize_sparse_a8(a, k_keep = HD/2), W_o)
 *   g, u  = bitlinear_a4(quantize(x1, INT4), W_gate), (..., W_up)
 *   x_out = x1 + bitlinear_sparse_a8(quantize_sparse_a8(g, up = u,
 *           k_keep = F/2), W_down)
 * with every intermediate in fp32 exactly as the separate calls produce it.
 * x, x_out: fp32 [B][HD] (distinct buffers).  Weights packed by
 * bw_pack_ternary: W_qkv [3HD][HD] and W_gate_up [2F][HD] (gate rows, then
 * up rows) in the BW_ROLE_A4 layout; W_o [HD][HD] and W_down [HD][F] in
 * BW_ROLE_A8; b_* the matching beta arrays.  Cache: k_/v_ p3, s3 [B][S_cap]
 * [H][...] and p4, s4 [n_special][H][...] as bw_kv_pack3 writes them, with
 * slot_of [B][S_cap]; position pos of every sequence is overwritten.
 * workspace: >= bw_block_decode_workspace_bytes(B, S_cap, H, D, F) bytes;
 * contents on entry are ignored.
 * Shapes: 1 <= B <= 16, D = 64 or 128, HD % 64 == 0, HD <= 16384,
 * F % 64 == 0, F <= 16384, 0 <= pos < S_cap.
 * ------------------------------------------------------------------------ */
/* host */ size_t bw_block_decode_workspace_bytes(int64_t B, int64_t S_cap, int64_t H, int64_t D, int64_t F);
bw_status bw_block_decode(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                          const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                          const uint8_t* w_gate_up, const float* b_gate_up, const uint8_t* w_down,
                          const float* b_down, uint8_t* k_p3, float* k_s3, uint8_t* k_p4, float* k_s4,
                          uint8_t* v_p3, float* v_s3, uint8_t* v_p4, float* v_s4, const int32_t* slot_of,
                          int64_t n_special, int64_t S_cap, int64_t pos, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Streaming read (measurement aid, not a step of the method).
 * Reads src[0, bytes) once in the access pattern of the decode GEMV's weight
 * stream (one 256-thread workgroup per 16 KB block, each wave reading a 4 KB
 * quarter with 16-byte loads, all of a lane's loads in flight before the
 * first is used) and writes sink[4b + q] = XOR of the little-endian 32-bit
 * words of quarter q of block b (a partial block reads zeros past `bytes`).
 * Timing it beside bw_bitlinear_a4 on the same weight bytes gives the read
 * ceiling of that launch shape.
 * sink: device uint32 [4 * ceil(bytes / 16384)].  Shapes: bytes % 16 == 0.
 * ------------------------------------------------------------------------ */
bw_status bw_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------ *
 * Decoder layer without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 * Computes exactly what bw_block_decode computes, with the same arguments
 * except the workspace, which is a static device array of
 * bw_block_decode_noalloc_max_bytes() bytes (16 MiB) that the library holds on
 * every GPU it runs on until the process ends.  The array of the current
 * device (hipGetDevice) is used; `stream` must belong to that device.  The
 * call allocates and frees nothing; its first call on a device looks up the
 * array's device address there.
 * A shape whose workspace (bw_block_decode_workspace_bytes) exceeds the array
 * is rejected with BW_ERR_UNSUPPORTED before anything is launched (7B shapes:
 * about 7 MB at 16 sequences).
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents (nothing in it has to start at zero): calls that overlap on one GPU
 * (on different streams, or from host threads without ordering) race; the
 * caller serializes them.
 * ------------------------------------------------------------------------ */
/* host */ size_t bw_block_decode_noalloc_max_bytes(void);
bw_status bw_block_decode_noalloc(const float* x, float* x_out, int64_t B, int64_t H, int64_t D, int64_t F,
                                  const uint8_t* w_qkv, const float* b_qkv, const uint8_t* w_o, const float* b_o,
                                  const uint8_t* w_gate_up, const float* b_gate_up, const uint8_t* w_down,
                                  const float* b_down, uint8_t* k_p3, float* k_s3, uint8_t* k_p4, float* k_s4,
                                  uint8_t* v_p3, float* v_s3, uint8_t* v_p4, float* v_s4,
                                  const int32_t* slot_of, int64_t n_special, int64_t S_cap, int64_t pos,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BW_H_ */
