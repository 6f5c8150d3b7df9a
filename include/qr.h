/*
 * qr.h - C ABI of libquarot_hip.so: QuaRot's online Hadamard rotation fused
 * with INT4 quantization, the W4A4 GEMM, and the head-wise K/V rotation with
 * 4-bit cache quantization, as HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (QuaRot: Outlier-Free 4-Bit Inference in Rotated
 * LLMs, arXiv 2404.00456; "QuaRot paper" below is its text, "QuaRot blog" is
 * "QuaRot: Rotating Away the Outliers That Make 4-Bit LLMs Impossible"):
 *   - randomized Hadamard H diag(s), Kronecker H_{2^n} (x) H_m for widths that
 *     are not powers of two: QuaRot paper, background on Hadamard matrices;
 *   - online Hadamard before the down projection, in fp32: QuaRot paper, FFN
 *     paragraph and the FP16-vs-FP32 Hadamard study (Table 10);
 *   - per-token symmetric INT4 (scale = max|x| / 7, round to nearest) and the
 *     INT32-accumulating 4-bit GEMM with row x column scale dequantization:
 *     QuaRot paper, activation-quantization and performance paragraphs;
 *   - post-RoPE head-wise rotation of queries and keys, asymmetric group-128
 *     KV quantization with Init/Append routines: QuaRot paper, keys/queries
 *     paragraph, implementation paragraph, attention-routines paragraph;
 *   - the Decode routine, flash-style attention of the FP16 query over the
 *     dequantized cache: QuaRot paper, attention paragraph and attention
 *     routines;
 *   - RMSNorm without scale in fp32 before the QKV/gate/up quantizer, and the
 *     Hadamard-heads block before the O projection's quantizer: QuaRot paper,
 *     method section, activation-quantization paragraph, attention-block
 *     paragraph (Figure 6).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; it launches on `stream` and
 *     returns.  Results are ready when the stream reaches that point.
 *   - Arguments are validated on the host before any launch; on error nothing
 *     is launched and the status says why.  Empty work (T == 0, N == 0,
 *     S_new == 0) returns QR_OK without launching.  A kernel fault surfaces at
 *     the caller's next synchronization, not here.
 *   - Packed INT4: byte j of a row holds element 2j in its low nibble and
 *     element 2j+1 in its high nibble.  Symmetric codes are two's-complement
 *     nibbles in [-8, 7]; asymmetric (KV) codes are unsigned nibbles in [0, 15].
 *   - fp16 is IEEE binary16, fp32 is IEEE binary32; all rounding is
 *     round-half-to-even.  Entry points are thread-safe (no global state is
 *     written).
 *   - Supported rotation widths d: 2^n for 3 <= n <= 13, 2^n * 28 for
 *     1 <= n <= 10 and 2^n * 172 for 1 <= n <= 6 (H_28: Paley's second construction over
 *     GF(13); H_172: Williamson's construction of order 4 * 43).  Use
 *     qr_hadamard_factor() to query.
 */
#ifndef QR_H_
#define QR_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QR_ABI_VERSION 1

typedef enum {
  QR_OK = 0,
  QR_ERR_NULL = 1,        /* a required pointer is NULL */
  QR_ERR_SHAPE = 2,       /* negative size, inconsistent sizes, out-of-range position */
  QR_ERR_UNSUPPORTED = 3, /* width/group/head size the kernels do not implement */
  QR_ERR_ALIGN = 4,       /* pointer or stride not aligned as required */
  QR_ERR_LAUNCH = 5,      /* the kernel launch itself failed */
  QR_ERR_ARG = 6,         /* a scalar argument is out of range (clip ratio, enum) */
  QR_ERR_SCRATCH = 7      /* the call needs more scratch than the library's static buffer
                             holds (qr_kv_decode_attention_noalloc only) */
} qr_status;

typedef enum {
  QR_ROT_NONE = 0,         /* quantize only */
  QR_ROT_HADAMARD = 1,     /* rotate by H_d diag(s) / sqrt(d), then quantize */
  QR_ROT_HADAMARD_F16 = 2  /* the same rotation with the transform's additions in fp16
                              (qr_hadamard_quant only; d = 28672 and 11008) */
} qr_rot;

/* Library ABI version (QR_ABI_VERSION of the build). */
int qr_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* qr_status_str(int status);

/* Host-only query: d = 2^(*log2_pow2) * (*m) as the kernels factor it.
 * Returns QR_ERR_UNSUPPORTED (outputs untouched) if d is not a supported
 * width; QR_ERR_NULL if an output pointer is NULL. */
qr_status qr_hadamard_factor(int32_t d, int32_t* log2_pow2, int32_t* m);

/*
 * Fused online Hadamard rotation + per-token symmetric INT4 quantization.
 *
 *   x_f16      [T, ld_x] fp16, row t holds x_t in its first d entries.
 *   rot        QR_ROT_HADAMARD: z = H_d (s * x) in fp32, y = z / sqrt(d);
 *              QR_ROT_NONE: y = z = x.
 *   signs      [d] int8, each +1 or -1 (the randomized Hadamard's s), or NULL
 *              for all +1.  Ignored when rot == QR_ROT_NONE.
 *   clip_ratio in [1/1024, 1].  Per row: a = max_i |y_i|,
 *              scale = fp16(clip_ratio * a / 7), q_i = clamp(rne(y_i / scale), -8, 7),
 *              q = 0 when scale == 0 (an overflowing scale is +Inf and gives q = 0).
 *   q_u8       [T, d/2] packed codes (output, row-major, contiguous).
 *   scale_f16  [T] fp16 scales (output).
 *   z_dbg      NULL, or [T, d] fp32 (output): the transform output z before the
 *              1/sqrt(d) factor (x itself for QR_ROT_NONE).
 *
 * The exact fp32 recipe the kernel implements, per row (c = the fp32 nearest
 * to 1/sqrt(d), or 1 for QR_ROT_NONE; every step rounds to fp32):
 *   a_z = max|z|; a = a_z * c; s_h = fp16(fp32(clip * a) / 7);
 *   m = c * (1 / s_h)  (m = 0 if s_h == 0);
 *   q_i = clamp(round_half_even(exact z_i * m), -8, 7).
 * The order of the fp32 additions inside z is not specified.
 *
 * QR_ROT_HADAMARD_F16 (QuaRot paper, appendix on the FP16 Hadamard
 * transformation, Table 10: running the online transform in fp16 leaves
 * accuracy unchanged).  Supported for the down-projection widths
 * d = 28672 = 1024 * 28 (Llama-2-70B) and d = 11008 = 64 * 172 (Llama-2-7B);
 * other widths return QR_ERR_UNSUPPORTED.  The dense H_m products (H_4 (x)
 * H_28 for 28672, H_172 for 11008) of the fp16 inputs accumulate in fp32 as
 * before; their conversion to fp16 and each remaining butterfly stage (8 for
 * 28672, 6 for 11008) round to fp16 (nearest even), on values scaled by 2^-e
 * (e = 7 for 28672, 8 for 11008, so that the dense stage's sums stay in the
 * fp16 range).  z_dbg returns that fp16 result times 2^e, and the
 * quantization is the recipe above applied to it, bit for bit.  With R
 * roundings (9 for 28672, 7 for 11008) the error per row obeys
 *   ||z_dbg - z||_2 <= R * 2^-11 * ||z||_2 + 2^(e-25) * S * sqrt(d),
 *   S = sum over j = 0 .. R-1 of 2^(j/2)  (S < 53 for R = 9, < 25 for R = 7):
 * each rounding is relative 2^-11 of a vector whose norm the remaining
 * stages, sqrt(2) times orthogonal each, carry to ||z||; the second term
 * covers fp16 subnormals (absolute error 2^-25 before the factor 2^e, grown
 * by sqrt(2) per remaining stage).  Rows whose |z| / 2^e exceeds the fp16
 * range (65504) overflow to an infinite scale: the mean |x| of a row must
 * stay below about 290 (28672) or 1500 (11008).
 *
 * Requirements: T >= 0; d supported; ld_x >= d and ld_x % 8 == 0; x_f16
 * 16-byte aligned; q_u8 and signs 4-byte aligned; z_dbg 16-byte aligned if
 * given.
 */
qr_status qr_hadamard_quant(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, qr_rot rot,
                            const int8_t* signs, float clip_ratio, void* q_u8, void* scale_f16,
                            float* z_dbg, hipStream_t stream);

/*
 * Rotation only (for example post-RoPE queries, whose rotation cancels against
 * the rotated keys in q.k):  y = H_d (s * x) / sqrt(d), computed as
 * fp32(z * c) with z and c as in qr_hadamard_quant, written as fp32
 * (y_is_f32 != 0) or rounded to fp16.
 *   x_f16 [T, ld_x] fp16; signs [d] int8 or NULL; y [T, d] contiguous.
 * Requirements as qr_hadamard_quant (y 16-byte aligned, signs 4-byte aligned).
 */
qr_status qr_hadamard(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, const int8_t* signs,
                      void* y, int32_t y_is_f32, hipStream_t stream);

/*
 * RMSNorm without its scale, in fp32, fused with per-token symmetric INT4
 * quantization: the input quantizer of the QKV, gate and up projections
 * (QuaRot paper, method section: the RMSNorm scale diag(alpha) is absorbed
 * into the next weights; activation-quantization paragraph: RMSNorm without
 * scaling stays in FP32 and its output is quantized per token).
 *   x_f16      [T, ld_x] fp16, row t holds x_t in its first d entries.
 *   eps        in [0, 1]: r = 1 / sqrt(sum_i x_i^2 / d + eps), y = x * r.
 *   clip_ratio in [1/1024, 1]; scale and codes as in qr_hadamard_quant with
 *              y in place of the rotated row.
 *   q_u8       [T, d/2] packed codes (output); scale_f16 [T] fp16 (output).
 *   r_dbg      NULL, or [T] fp32 (output): r per row.
 * fp32 recipe, per row: ss = sum of the exact squares x_i^2 (fp32 additions
 * in an unspecified order); t = fp32(fp32(ss / d) + eps);
 * r = fp32(1 / fp32(sqrt(t))), or 0 when t == 0; then the qr_hadamard_quant
 * recipe with z = x and c = r: a = max|x| * r; s_h = fp16(fp32(clip * a) / 7);
 * m = r * (1 / s_h) (0 if s_h == 0); q_i = clamp(rne(exact x_i * m), -8, 7).
 * Requirements: T >= 0; d % 8 == 0, 8 <= d <= 16384; ld_x >= d,
 * ld_x % 8 == 0; x_f16 16-byte aligned; q_u8 4-byte aligned.
 */
qr_status qr_rmsnorm_quant(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, float eps,
                           float clip_ratio, void* q_u8, void* scale_f16, float* r_dbg,
                           hipStream_t stream);

/*
 * Hadamard heads fused with per-token symmetric INT4 quantization: the input
 * quantizer of the O projection (QuaRot paper, attention-block paragraph:
 * with (I (x) H_dh) fused into W_v and W_out offline, the forward pass applies
 * Z <- Z (H_nh (x) I) to the attention output; Figure 6).  Per row, with
 * element i = h * head_dim + j:
 *   z[h, j] = sum_h' H_nh[h, h'] x[h', j]   (Sylvester H_nh, entries +-1),
 *   y = z / sqrt(n_heads), then scale and codes as in qr_hadamard_quant.
 *   x_f16      [T, ld_x] fp16, d = n_heads * head_dim.
 *   q_u8       [T, d/2] packed codes (output); scale_f16 [T] fp16 (output).
 *   z_dbg      NULL, or [T, d] fp32 (output): z before the 1/sqrt(n_heads).
 * fp32 recipe: the qr_hadamard_quant recipe with c = fp32(1/sqrt(n_heads)); the
 * order of the additions inside z is not specified.
 * Requirements: T >= 0; n_heads and head_dim powers of two with
 * 2 <= n_heads <= 64 and 4J <= head_dim <= 64J, J = max(2, min(8, 128 / n_heads))
 * (n_heads = 64: head_dim 8 .. 128; 32: 16 .. 256; <= 16: 32 .. 512);
 * ld_x >= d, ld_x % 8 == 0; x_f16 16-byte aligned; q_u8 4-byte aligned; z_dbg
 * 16-byte aligned if given.
 */
qr_status qr_hadamard_heads_quant(const void* x_f16, int64_t T, int32_t n_heads, int32_t head_dim,
                                  int64_t ld_x, float clip_ratio, void* q_u8, void* scale_f16,
                                  float* z_dbg, hipStream_t stream);

/*
 * W4A4 GEMM with fused dequantization epilogue:
 *   acc[t, n] = sum_k A[t, k] W[n, k]   (int32, exact)
 *   Y[t, n]   = fp16(fp32(fp32(acc) * a_scale[t]) * w_scale[n])
 *   a_q        [T, K/2] packed signed INT4 (row-major, contiguous).
 *   a_scale    [T] fp16 token scales.
 *   w_q        [N, K/2] packed signed INT4 (row-major, contiguous: one output
 *              channel per row, the layout qr_hadamard_quant writes when run
 *              on W with T := N).
 *   w_scale    [N] fp16 channel scales.
 *   y_f16      [T, N] fp16 output (contiguous).
 *   acc_dbg    NULL, or [T, N] int32 (output): the exact accumulators.
 * Requirements: T, N >= 0; K > 0, K % 64 == 0, K <= 131008; a_q and w_q
 * 16-byte aligned; y_f16 and acc_dbg 4-byte aligned.
 */
qr_status qr_w4a4_gemm(const void* a_q, const void* a_scale_f16, int64_t T, const void* w_q,
                       const void* w_scale_f16, int64_t N, int64_t K, void* y_f16,
                       int32_t* acc_dbg, hipStream_t stream);

/*
 * b-bit variants (QuaRot paper: round-to-nearest 6- and 8-bit weights and
 * activations are lossless, Table 9).  Codes are symmetric b-bit integers,
 * 2 <= bits <= 8, stored one per byte (int8, two's complement):
 *   scale = fp16(clip * max|y| / qmax), qmax = 2^(bits-1) - 1,
 *   q = clamp(rne(y / scale), -2^(bits-1), qmax), q = 0 if scale == 0,
 * with the fp32 recipe of the INT4 entry points and 7 replaced by qmax.
 *   qr_hadamard_quant_i8: as qr_hadamard_quant (QR_ROT_NONE or
 *     QR_ROT_HADAMARD, the same widths), q_i8 [T, d]; every width runs the
 *     LDS-staged kernel (one workgroup per row).
 *   qr_rmsnorm_quant_i8, qr_hadamard_heads_quant_i8: as their INT4 versions,
 *     q_i8 [T, d].
 * Requirements as the INT4 versions, with q_i8 8-byte aligned.
 */
qr_status qr_hadamard_quant_i8(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, qr_rot rot,
                               const int8_t* signs, float clip_ratio, int32_t bits, void* q_i8,
                               void* scale_f16, float* z_dbg, hipStream_t stream);
qr_status qr_rmsnorm_quant_i8(const void* x_f16, int64_t T, int32_t d, int64_t ld_x, float eps,
                              float clip_ratio, int32_t bits, void* q_i8, void* scale_f16,
                              float* r_dbg, hipStream_t stream);
qr_status qr_hadamard_heads_quant_i8(const void* x_f16, int64_t T, int32_t n_heads,
                                     int32_t head_dim, int64_t ld_x, float clip_ratio,
                                     int32_t bits, void* q_i8, void* scale_f16, float* z_dbg,
                                     hipStream_t stream);

/*
 * Group-wise scales (QuaRot paper: group-wise quantization with different group
 * sizes, one of its studied variants).  As qr_hadamard_quant, but the row is
 * cut into groups of `group` consecutive elements and each group gets its own
 * scale, with the same fp32 recipe applied per group:
 *   scale_f16  [T, d / group] fp16 (output, row-major);
 *   q_u8       [T, d/2] packed INT4 codes, as qr_hadamard_quant.
 * group: a power of two with 8 <= group <= 512 dividing d.  Every width runs the
 * LDS-staged kernel (one workgroup per row).  qr_w4a4_gemm_groups consumes these.
 */
qr_status qr_hadamard_quant_groups(const void* x_f16, int64_t T, int32_t d, int64_t ld_x,
                                   qr_rot rot, const int8_t* signs, float clip_ratio,
                                   int32_t group, void* q_u8, void* scale_f16, float* z_dbg,
                                   hipStream_t stream);

/*
 * W4A4 GEMM with group-wise scales on both operands (the outputs of
 * qr_hadamard_quant_groups for the activations and for the weights, T := N):
 *   acc_g[t, n] = sum over k in group g of A[t, k] W[n, k]   (int32, exact),
 *   f = 0;  for g = 0, 1, ...:  f = fp32(f + fp32(fp32(fp32(acc_g) * a_scale[t, g])
 *                                                * w_scale[n, g])),
 *   Y[t, n] = fp16(f).
 *   a_scale [T, K/group], w_scale [N, K/group] fp16 (row-major); codes as
 *   qr_w4a4_gemm.  group: a power of two, 64 <= group <= 512, dividing K.
 * Requirements as qr_w4a4_gemm (no accumulator output).
 */
qr_status qr_w4a4_gemm_groups(const void* a_q, const void* a_scale_f16, int64_t T, const void* w_q,
                              const void* w_scale_f16, int64_t N, int64_t K, int32_t group,
                              void* y_f16, hipStream_t stream);

/*
 * GEMM on codes stored one per byte (b <= 8 bits, for example the outputs of
 * the _i8 quantizers above), with the epilogue of qr_w4a4_gemm:
 *   acc[t, n] = sum_k A[t, k] W[n, k]   (int32, exact: |acc| <= 2^14 K < 2^31),
 *   Y[t, n]   = fp16(fp32(fp32(acc) * a_scale[t]) * w_scale[n]); fp32(acc)
 *               rounds to nearest even once |acc| > 2^24.
 *   a_q [T, K] int8, w_q [N, K] int8 (row-major, contiguous); a_scale [T],
 *   w_scale [N] fp16; y_f16 [T, N] fp16; acc_dbg NULL or [T, N] int32.
 * Requirements: T, N >= 0; K > 0, K % 16 == 0, K <= 131008; a_q and w_q
 * 16-byte aligned; y_f16 and acc_dbg 4-byte aligned.
 */
qr_status qr_w8a8_gemm(const void* a_q, const void* a_scale_f16, int64_t T, const void* w_q,
                       const void* w_scale_f16, int64_t N, int64_t K, void* y_f16,
                       int32_t* acc_dbg, hipStream_t stream);

/*
 * Head-wise rotation + asymmetric 4-bit group quantization of new K or V
 * tokens, written into a packed cache (Init: start_pos = 0, S_new = prompt
 * length; Append: S_new = 1 at the next position).
 *   kv_f16      [B, S_new, H, Dh] fp16; token (b, s) starts at element
 *               (b * S_new + s) * ld_token, head h at + h * Dh.
 *   rot         QR_ROT_HADAMARD: y = H_Dh (s * x) / sqrt(Dh) per head (keys);
 *               QR_ROT_NONE: y = x (values, whose rotation is fused offline).
 *   signs       [Dh] int8 +-1 or NULL (all +1).
 *   group       group size G dividing Dh (G even, G >= 8).
 *   clip_ratio  in [1/1024, 1].  Per group: mx = clip * max y, mn = clip * min y,
 *               scale = fp16((mx - mn) / 15), min = fp16(mn),
 *               q = clamp(rne((y - min) / scale), 0, 15), q = 0 if scale == 0.
 *               fp32 recipe: y = fp32(z * c); s_h = fp16(fp32(mx_c - mn_c) / 15);
 *               m_h = fp16(mn_c); q = clamp(rne(exact fp32(y - m_h) * fp32(1/s_h)), 0, 15).
 *   cache_q     [B, H, S_max, Dh/2] uint8 packed unsigned codes.
 *   cache_meta  [B, H, S_max, Dh/G, 2] fp16 (scale, min) pairs.
 *   start_pos   first cache position written; positions start_pos ..
 *               start_pos + S_new - 1 are overwritten, nothing else is touched.
 *   z_dbg       NULL, or [B, S_new, H, Dh] fp32: z before the 1/sqrt(Dh) factor.
 * Requirements: B, H >= 1, S_new >= 0; Dh a power of two, 8 <= Dh <= 256;
 * ld_token >= H * Dh, ld_token % 8 == 0; 0 <= start_pos and
 * start_pos + S_new <= S_max; kv_f16 16-byte aligned; cache_q, cache_meta and
 * signs 4-byte aligned.
 */
qr_status qr_kv_rotate_quant(const void* kv_f16, int32_t B, int32_t S_new, int32_t H, int32_t Dh,
                             int64_t ld_token, qr_rot rot, const int8_t* signs, int32_t group,
                             float clip_ratio, void* cache_q, void* cache_meta, int32_t S_max,
                             int32_t start_pos, float* z_dbg, hipStream_t stream);

/*
 * qr_kv_rotate_quant with b-bit codes, 2 <= bits <= 4 (QuaRot paper, KV
 * bit-width study, Table 6): 15 becomes L = 2^bits - 1 in the formulas above
 * (scale = fp16((mx - mn) / L), q = clamp(rne((y - min) / scale), 0, L)).  The
 * codes keep the 4-bit cache layout, so qr_kv_decode_attention reads a cache
 * of any of these widths unchanged.  bits = 4 is qr_kv_rotate_quant.
 * Requirements as qr_kv_rotate_quant; bits outside [2, 4] is QR_ERR_ARG.
 */
qr_status qr_kv_rotate_quant_bits(const void* kv_f16, int32_t B, int32_t S_new, int32_t H,
                                  int32_t Dh, int64_t ld_token, qr_rot rot, const int8_t* signs,
                                  int32_t group, float clip_ratio, int32_t bits, void* cache_q,
                                  void* cache_meta, int32_t S_max, int32_t start_pos,
                                  float* z_dbg, hipStream_t stream);

/*
 * Decode routine (QuaRot paper, attention routines Init / Append / Decode):
 * attention of one new query per sequence over the 4-bit K/V cache that
 * qr_kv_rotate_quant wrote, for grouped-query heads.  For batch b, query head
 * hq and its KV head h = hq / (Hq / Hkv), over cache positions j = 0 .. L-1:
 *   k_j = code * scale + min, v_j likewise (the cache's (scale, min) pair),
 *   s_j = softmax_scale * (q[b, hq] . k_j),   out[b, hq] = sum_j softmax(s)_j v_j.
 * The query must carry the same head-wise rotation as the cached keys (for
 * example qr_hadamard on the post-RoPE queries with the keys' signs); values
 * are used as cached.
 *   q_f16        [B, Hq, Dh] fp16, contiguous.
 *   k_cache_q, v_cache_q        [B, Hkv, S_max, Dh/2] uint8 packed codes.
 *   k_cache_meta, v_cache_meta  [B, Hkv, S_max, Dh/group, 2] fp16 (scale, min).
 *   L            positions used, 1 <= L <= S_max (the same for every sequence).
 *   out_f16      [B, Hq, Dh] fp16 (output, contiguous).
 *   workspace    caller-owned device scratch of at least
 *                qr_kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L) bytes: fp32
 *                partial results of the split over positions; its contents on
 *                entry do not matter and are overwritten.  Calls that overlap on
 *                one workspace race.  When that size is 0 (B * Hkv large enough
 *                that one workgroup per KV head fills the GPU) workspace may be
 *                NULL.
 * Arithmetic: q . k_j is formed in fp32 from exact fp16 operands (codes are
 * exact; scale and min are applied in fp32), softmax in fp32 with exp2; the
 * weights times the value scale enter the value product as fp16 (the pages'
 * FP16 dot product), min terms in fp32; the output is rounded once to fp16.
 * Requirements: Dh = 128, group = 128, Hq % Hkv == 0, Hq / Hkv <= 16,
 * softmax_scale > 0; q_f16, k_cache_q and v_cache_q 16-byte aligned, the
 * metadata and the workspace 4-byte aligned.  B == 0 returns QR_OK.
 */
int64_t qr_kv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dh, int32_t L);

qr_status qr_kv_decode_attention(const void* q_f16, int32_t B, int32_t Hq, int32_t Hkv, int32_t Dh,
                                 const void* k_cache_q, const void* k_cache_meta,
                                 const void* v_cache_q, const void* v_cache_meta, int32_t S_max,
                                 int32_t L, int32_t group, float softmax_scale, void* out_f16,
                                 void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * qr_kv_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same computation, arguments, requirements
 * and errors as qr_kv_decode_attention, and bit-identical output.  The split
 * records live in a static device array of QR_KV_DECODE_SCRATCH_BYTES bytes
 * that the library holds on each GPU it runs on until the process ends; its
 * device address is looked up on the first call on each device (with that
 * device current).  The call allocates and frees nothing.
 *   Size limit: a call whose qr_kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L)
 *   exceeds QR_KV_DECODE_SCRATCH_BYTES returns QR_ERR_SCRATCH and launches
 *   nothing (the limit covers every shape whose B * Hkv divides 256 or is at
 *   least 256, for any L and Hq / Hkv <= 16).
 *   Concurrency: every call on one GPU shares that GPU's array, so calls that
 *   overlap on one GPU (on different streams, or from several host threads
 *   without ordering) race.  No scratch content has to start at zero.
 *   The array's address could not be obtained: QR_ERR_LAUNCH.
 */
#define QR_KV_DECODE_SCRATCH_BYTES ((int64_t)4 << 20)

qr_status qr_kv_decode_attention_noalloc(const void* q_f16, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t Dh, const void* k_cache_q,
                                         const void* k_cache_meta, const void* v_cache_q,
                                         const void* v_cache_meta, int32_t S_max, int32_t L,
                                         int32_t group, float softmax_scale, void* out_f16,
                                         hipStream_t stream);

/*
 * Measurement support, not a step of the method: the rate the int8 matrix
 * cores that qr_w4a4_gemm runs on sustain with no memory traffic.  grid
 * workgroups of 256 threads each run iters iterations of four independent
 * chains of v_mfma_i32_32x32x32_i8 (4 x 65536 int ops per wavefront and
 * iteration) on register-held fragments:
 *   fragments_i8  [64, 16] int8 (input): lane l's A fragment is row l; its
 *                 B fragment in chain j is row (l + 7 + 16 j) mod 64.  Each
 *                 fragment is the lane's 16 bytes of the 32 x 32 x 32 operand
 *                 (rows l mod 32; the lanes l < 32 and l >= 32 hold the two
 *                 16-element halves of k).
 *   checksum_i32  [grid * 256] int32 (output): per thread, the sum, modulo
 *                 2^32, of its 4 x 16 accumulator values.  Over the 64 lanes
 *                 of a wavefront this sums to iters * sum_j sum_{h, e}
 *                 (sum_{l in half h} A_l[e]) (sum_{l in half h} B_{j,l}[e]).
 *   clocks_u64    NULL, or [grid, 4] uint64 (output): per workgroup, the
 *                 shader clock counter before and after wavefront 0's loop,
 *                 then the 100 MHz constant counter before and after it.
 * Requirements: grid >= 1 and iters >= 1 (else QR_ERR_SHAPE); fragments 16-,
 * checksum 4- and clocks 8-byte aligned.
 */
qr_status qr_calibrate_mfma_i8(const void* fragments_i8, int32_t grid, int32_t iters,
                               int32_t* checksum_i32, uint64_t* clocks_u64, hipStream_t stream);

/*
 * Measurement support, not a step of the method: a plain stream with the
 * rotate+quant kernels' traffic mix (16 bytes read for every 4 written), the
 * practical HBM ceiling those kernels are measured against.
 *   src      [n16] 16-byte chunks (input), read once, non-temporally.
 *   dst_u32  [n16] uint32 (output): dst[i] = XOR of the four dwords of chunk i,
 *            written once, non-temporally.
 * grid workgroups of 256 threads stride over the chunks, two in flight per
 * thread.  Requirements: n16 >= 0 (0 launches nothing) and grid >= 1 (else
 * QR_ERR_SHAPE); src 16-byte and dst 4-byte aligned.
 */
qr_status qr_calibrate_stream(const void* src, int64_t n16, void* dst_u32, int32_t grid,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QR_H_ */
