/*
 * bgt.h -- C ABI of libbgt: the fine-grained W4A8 integer-scale linear layer
 * Y = X.W on AMD MI355X (gfx950), its two controls (float-scale W4A8,
 * zero-point W8A8), and two variants of the same epilogue: fine-grained W8A8
 * with integer scales and the grouped (mixture-of-experts) W4A8 GEMM.
 *
 * Pages cited:
 *   [IS] "Integer Scale: A Free Lunch for Faster Fine-grained Quantization of
 *        LLMs" summary page (dignews.cc).
 *   [QB] "探秘Transformer系列之（34）--- 量化基礎" (rzrgm.cn blog).
 *   [QN] "Quantization" notes (zsc0tt.pages.dev).
 *   [EX] "extreme quantization LLMs" page (apxml.com).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless
 *     marked [host]. Matrices are row-major; sizes are element counts.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. Work is enqueued asynchronously on it unless stated otherwise.
 *   - Ownership: the caller owns every buffer. The library allocates no
 *     device memory and keeps no state between calls; calls on different
 *     streams are independent. Outputs must not alias inputs.
 *   - Errors: arguments are validated on the host before any HIP call; a
 *     failed validation returns a negative status and writes nothing. A HIP
 *     launch or copy failure returns BGT_ERR_HIP (outputs then unspecified).
 *   - Shapes: group size is 128 along K; K % 128 == 0; N % 16 == 0; M >= 1.
 *     Pointers passed to the GEMMs and the packer must be 16-byte aligned.
 *   - Rounding: round() is half away from zero; x/s is an IEEE binary32
 *     division (the int8 mapping of [QB] §2.2 rounds "四舍五入").
 */
#ifndef BGT_H
#define BGT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BGT_OK                     0
#define BGT_WARN_ACC_MAY_OVERFLOW  1   /* pack: worst-case |A| = 128*127*q_max * G *
                                          max(iscale) reaches 2^31 (q_max 7 or 127)     */
#define BGT_ERR_NULL              -1   /* a required pointer is NULL                    */
#define BGT_ERR_SHAPE             -2   /* a size is out of range or not a multiple     */
#define BGT_ERR_ALIGN             -3   /* a pointer or leading dimension is misaligned */
#define BGT_ERR_ALPHA             -4   /* amplifier not a power of two in [1, 2^30]     */
#define BGT_ERR_MODE              -5   /* unknown mode, element type or scale width    */
#define BGT_ERR_HIP               -6   /* a HIP call failed                             */
#define BGT_ERR_RANGE             -7   /* an integer scale does not fit its element     */

/* Element types of activations (x) and outputs (y) in the _ex entry points
 * and bgt_w4a8_linear_is: IEEE binary32, IEEE binary16, bfloat16. Every
 * computation is in fp32 / int32; an fp16 or bf16 x is widened exactly, an
 * fp16 or bf16 y is the fp32 result rounded once, to nearest even. */
#define BGT_F32   0
#define BGT_F16   1
#define BGT_BF16  2

/* Quantization modes of bgt_quantize_act. */
#define BGT_QUANT_SYM_I8   0
#define BGT_QUANT_ASYM_U8  1

#define BGT_GROUP 128

/*
 * bgt_quantize_act -- per-row dynamic quantization (one scale per token).
 *
 * SYM_I8 ([QN] Symmetric Quantization; [QB] §2.2 absmax onto [-127,127];
 * per-token granularity of [QB] §2.3.3; computed at run time, the dynamic
 * quantization of [QB] §2.4.1):
 *     a_i = max_k |x_ik|,  s_i = a_i / 127,
 *     q_ik = clip(round(x_ik / s_i), -127, 127)      (s_i = 0 -> q_ik = 0).
 * ASYM_U8 ([QN] Asymmetric Quantization with q in [0,255]; [QB] §2.2.1 eq. 1):
 *     s_i = (max_k x_ik - min_k x_ik) / 255,
 *     z_i = clip(round(0 - min_k x_ik / s_i), 0, 255),
 *     q_ik = clip(round(x_ik / s_i) + z_i, 0, 255)   (s_i = 0 -> z_i = 0, q = 0),
 *     rowsum_i = sum_k q_ik.
 * Applied to W^T (N x K) this is the per-channel weight quantization of the
 * W8A8 control ([QN] Per-Channel Quantization): rowsum is then colsum_w.
 * ASYM precondition: the range is the row's raw min and max (no forced zero),
 * so a row represents its values only when min <= 0 <= max. For a row of one
 * sign z clips to 0 or 255 and the codes saturate; the result is still the
 * formula above (no status reports it), and bgt_w8a8_gemm_zp on such rows is
 * the formula's value, not X.W.
 *
 *   x       rows x cols float32, leading dimension ld >= cols (elements).
 *   q       rows x cols int8 (SYM) or uint8 (ASYM), dense (leading dim cols).
 *   scale   [rows] float32.
 *   zero    [rows] int32, ASYM only (ignored for SYM, may be NULL).
 *   rowsum  [rows] int32, optional (NULL = not written); SYM gives sum of int8 codes.
 * Requirements: rows >= 1, 1 <= cols <= 2^24, ld >= cols. Inputs must be
 * finite. x, q 16-byte aligned and ld % 4 == 0 and cols % 16 == 0 take the
 * vector path; other shapes are accepted and run a scalar path.
 */
int bgt_quantize_act(const float* x, int64_t rows, int64_t cols, int64_t ld, int mode,
                     void* q, float* scale, int32_t* zero, int32_t* rowsum, void* stream);

/* bgt_quantize_act with x of element type x_type (BGT_F32, BGT_F16 or BGT_BF16;
 * the activations of the [IS] page's models are FP16). fp16 / bf16 values are
 * widened to fp32 exactly; everything else is bgt_quantize_act. The vector
 * path needs x 16-byte aligned, ld % 4 == 0 and cols % 16 == 0. Unknown
 * x_type: BGT_ERR_MODE. */
int bgt_quantize_act_ex(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld,
                        int mode, void* q, float* scale, int32_t* zero, int32_t* rowsum,
                        void* stream);

/*
 * bgt_pack_weights_int4 -- offline group-wise int4 weight quantization,
 * nibble packing and integer scales.
 *
 * Per column j and group l (rows 128l .. 128l+127) of W (K x N) ([IS] 方法
 * Fig. 3(a): weights split into groups quantized independently; [QB] §2.3.3
 * per-group scales):
 *     s_lj = max |w| / 7,   q_kj = clip(round(w_kj / s_lj), -7, 7)   (s = 0 -> q = 0),
 *     fscale[l][j] = s_lj,  iscale[l][j] = round(s_lj * alpha)      ([IS] Fig. 3(c)).
 * alpha > 0 must be a power of two in [1, 2^30] ([IS] Table 1 uses 1024).
 * alpha == 0 runs the amplifier search of [IS] 方法: the smallest 2^n, n >= 0,
 * with (min over positive s_lj) * 2^n >= 1; all-zero matrices give 1.
 * The amplifier used is written to *alpha_out [host].
 *
 * Packed layout (two's-complement nibbles, two codes per byte as [EX] "data
 * packing" describes), N*K/2 bytes. With G = K/128:
 *     t = j/16, c = j%16, l = k/128, r = k%128,
 *     h = r/64, s = (r%64)/16, e = r%16, lane = 16*s + c,
 *     byte(k, j) = ((t*G + l)*64 + lane)*16 + 8*h + 4*(e/8) + (e%4),
 *     the code sits in the low nibble when (e%8) < 4, else in the high nibble.
 * So each (16-column tile, group) pair is one contiguous 1 KiB block; within
 * it, 16 bytes per lane of a 64-wide wavefront.
 *
 *   w        K x N float32 (finite).
 *   packed   N*K/2 bytes.  fscale, iscale: (K/128) x N, float32 / int32.
 * Returns BGT_ERR_RANGE if some iscale would reach 2^23 (the GEMMs multiply
 * integer scales in 24-bit signed lanes), BGT_WARN_ACC_MAY_OVERFLOW when the
 * worst-case accumulator 113792 * G * max(iscale) (|q_x| <= 127, |q_w| <= 7,
 * 128 products per group) reaches 2^31 (the GEMM still wraps mod 2^32).
 * Synchronous: returns after the work on `stream` has finished.
 */
int bgt_pack_weights_int4(const float* w, int64_t K, int64_t N, int64_t group, int alpha,
                          uint8_t* packed, float* fscale, int32_t* iscale, int* alpha_out,
                          void* stream);

/*
 * bgt_w4a8_gemm_is -- W4A8 GEMM with the Integer Scale epilogue ([IS] 方法,
 * Fig. 3(c); the grouped output of 動機 3.1):
 *     p_ilj  = sum_{k in group l} qx[i][k] * q_w[k][j]          (int32)
 *     A_ij   = sum_l p_ilj * iscale[l][j]                        (int32, mod 2^32)
 *     y_ij   = ((float)A_ij * sx[i]) * (1/alpha)                 (one int->float per output)
 * so the I32->F32 conversion happens once per output instead of once per
 * group ([IS] 動機 3.2, Fig. 2).
 *
 *   qx      M x K int8 (codes of bgt_quantize_act SYM), sx [M] float32.
 *   packed  the layout of bgt_pack_weights_int4; iscale (K/128) x N int32 with
 *           every entry in [0, 2^23), 16-byte aligned.
 *   alpha   power of two in [1, 2^30], the one the integer scales were made with.
 *   y       M x N float32.
 *   acc_out optional M x N int32 (NULL = not written): A_ij itself.
 * Requirements: 1 <= M <= 65536, N % 16 == 0, 16 <= N <= 2^24,
 * K % 128 == 0, 128 <= K <= 65536.
 */
int bgt_w4a8_gemm_is(const int8_t* qx, const float* sx, const uint8_t* packed,
                     const int32_t* iscale, int alpha, int64_t M, int64_t N, int64_t K,
                     float* y, int32_t* acc_out, void* stream);

/*
 * bgt_w4a8_gemm_is_noalloc -- bgt_w4a8_gemm_is for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, requirements and
 * results, computed by the same kernels, and no hipMalloc / hipFree or other
 * allocating call. Where the GEMM splits K (see bgt_w4a8_workspace_bytes) it
 * keeps the split sums in a static device array of 32 MiB instead of the
 * library's workspace; each GPU holds its own copy from the library's load
 * until the process ends. On a 256-CU device every valid shape fits (a split
 * launch writes at most one 256 x 128 int32 tile per CU); a shape needing
 * more returns BGT_ERR_SHAPE, and BGT_ERR_HIP if the array's address cannot
 * be obtained. Nothing carries over between calls (every split sum read is
 * first written by the same call), but all calls on one GPU share the array:
 * calls that overlap on one GPU (several streams or threads) race.
 */
int bgt_w4a8_gemm_is_noalloc(const int8_t* qx, const float* sx, const uint8_t* packed,
                             const int32_t* iscale, int alpha, int64_t M, int64_t N, int64_t K,
                             float* y, int32_t* acc_out, void* stream);

/*
 * bgt_repack_int4_canonical -- accept int4 weights in the canonical layout.
 * The pages allow any packing of sub-byte codes into standard bytes (the
 * apxml extreme-quantization page, 实现与评估考量, "data packing"); the
 * canonical layout read here is the plain one: the codes of W^T with K
 * contiguous per output column, two per byte, even k in the low nibble,
 *     canonical byte (j*K + k)/2, nibble k % 2 (0 = low), 4-bit two's complement,
 * for the K x N codes q_kj. The call rewrites them into the kernel-native
 * layout of bgt_pack_weights_int4 (the codes themselves are unchanged), so
 * weights quantized elsewhere can be fed to the GEMMs with the caller's own
 * scales. Asynchronous on `stream`.
 *
 *   canonical  N*K/2 bytes (device, caller-owned, read only).
 *   packed     N*K/2 bytes (device, caller-owned): the native layout.
 * Requirements: K % 128 == 0, 128 <= K <= 65536, N % 16 == 0, 16 <= N <= 2^24;
 * both pointers non-NULL (BGT_ERR_NULL) and 16-byte aligned (BGT_ERR_ALIGN).
 * Nothing is written on a rejected call.
 */
int bgt_repack_int4_canonical(const uint8_t* canonical, int64_t K, int64_t N, uint8_t* packed,
                              void* stream);

/*
 * bgt_narrow_iscale -- store integer scales in narrower elements ([IS] 方法:
 * the amplified scales of Fig. 4(a) fit 16-bit integers at alpha = 2^10, most
 * of them 8 bits). out[i] = iscale[i] as uint8 (width 1) or uint16 (width 2);
 * the values, and so every GEMM result, are unchanged. Decode-regime GEMMs
 * stream the scales with the weights, so 1-byte scales cut their bytes by
 * 3*G*N (2.1 MB of 48 MB for K=4096, N=22016).
 *
 *   iscale  count int32 values (device), e.g. the (K/128) x N output of
 *           bgt_pack_weights_int4.
 *   out     count * width bytes (device).
 * Requirements: width 1 or 2 (else BGT_ERR_MODE), 1 <= count <= 2^36, both
 * pointers 16-byte aligned. Returns BGT_ERR_RANGE, writing nothing, if some
 * value is negative or does not fit the element (> 255 or > 65535).
 * Blocking: iscale is copied to the host and checked before the narrowing is
 * enqueued on `stream`.
 */
int bgt_narrow_iscale(const int32_t* iscale, int64_t count, int width, void* out, void* stream);

/*
 * bgt_w4a8_gemm_is_narrow -- bgt_w4a8_gemm_is with the integer scales stored
 * in elements of `width` bytes: 1 (uint8), 2 (uint16) or 4 (int32, the same
 * call as bgt_w4a8_gemm_is). Same formulas, arguments and requirements;
 * iscale must be 16-byte aligned. Results are bit-identical to the int32 call
 * on the same scale values. Unknown width: BGT_ERR_MODE.
 */
int bgt_w4a8_gemm_is_narrow(const int8_t* qx, const float* sx, const uint8_t* packed,
                            const void* iscale, int width, int alpha, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* acc_out, void* stream);

/* bgt_w4a8_gemm_is_narrow with y of element type y_type (BGT_F32, BGT_F16 or
 * BGT_BF16): y_ij is the fp32 value of bgt_w4a8_gemm_is rounded once to the
 * type (round to nearest even). acc_out is unchanged (int32). */
int bgt_w4a8_gemm_is_ex(const int8_t* qx, const float* sx, const uint8_t* packed,
                        const void* iscale, int width, int alpha, int64_t M, int64_t N, int64_t K,
                        void* y, int y_type, int32_t* acc_out, void* stream);

/*
 * bgt_w4a8_linear_is -- the whole decode-time linear layer from fp32
 * activations: per-token quantization of x exactly as bgt_quantize_act SYM
 * computes it (codes into qx, scales into sx), then bgt_w4a8_gemm_is_narrow
 * on those codes. For M <= 4 with K/128 = 16, 32, 86 or 112, x 16-byte aligned
 * and ldx % 4 == 0 this is one launch: every workgroup of the decode kernel
 * quantizes the rows itself while its weight stream is in flight, so the
 * separate quantizer launch disappears (the fusion of the quantization into
 * the GEMM that [QB] §2.4.1 dynamic quantization invites); otherwise it is the
 * quantizer followed by the GEMM. qx, sx and y are bit-identical either way.
 *
 *   x       M x K of element type x_type (BGT_F32, BGT_F16, BGT_BF16; finite),
 *           leading dimension ldx >= K (elements).
 *   packed, iscale, width, alpha: as bgt_w4a8_gemm_is_narrow.
 *   qx      M x K int8 (dense), sx [M] float32: written (the quantized activations).
 *   y       M x N of element type y_type (fp32 result rounded once).
 * Requirements: those of bgt_w4a8_gemm_is_narrow; qx 16-byte aligned.
 */
int bgt_w4a8_linear_is(const void* x, int x_type, int64_t ldx, const uint8_t* packed,
                       const void* iscale, int width, int alpha, int64_t M, int64_t N, int64_t K,
                       int8_t* qx, float* sx, void* y, int y_type, void* stream);

/* Diagnostics: 1 when bgt_w4a8_linear_is runs as one launch for these
 * arguments (M, K, x, ldx), 0 when it runs the quantizer and the GEMM. */
int bgt_w4a8_linear_fused(int64_t M, int64_t K, const void* x, int64_t ldx);

/*
 * bgt_w4a8_gemm_fs -- the float-scale control ([IS] 方法 Fig. 3(b)): every
 * group's integer result is converted to float and scaled by its float scale,
 * groups in ascending order, one fused multiply-add each:
 *     acc = 0;  for l = 0..G-1: acc = fma((float)p_ilj, fscale[l][j], acc);
 *     y_ij = acc * sx[i].
 * Same arguments and requirements as bgt_w4a8_gemm_is, with fscale
 * (K/128) x N float32 in place of iscale and alpha.
 */
int bgt_w4a8_gemm_fs(const int8_t* qx, const float* sx, const uint8_t* packed,
                     const float* fscale, int64_t M, int64_t N, int64_t K, float* y,
                     void* stream);

/* bgt_w4a8_gemm_fs with y of element type y_type (fp32 result rounded once). */
int bgt_w4a8_gemm_fs_ex(const int8_t* qx, const float* sx, const uint8_t* packed,
                        const float* fscale, int64_t M, int64_t N, int64_t K, void* y, int y_type,
                        void* stream);

/*
 * bgt_w8a8_gemm_zp -- the asymmetric W8A8 control through the zero-point
 * expansion of [QN] 矩阵乘法中的量化计算 (output requantization left out):
 *     A_mn = sum_k qw[n][k] qx[m][k] - zw[n] rowsum_x[m] - zx[m] colsum_w[n]
 *            + K zw[n] zx[m]                                    (int32, exact)
 *     y_mn = (float)A_mn * (sx[m] * sw[n])
 * the per-token x per-channel outer product of scales of [QB] §2.3.3.
 *
 *   qx M x K uint8, sx/zx/rowsum_x [M]  (bgt_quantize_act ASYM on X)
 *   qw N x K uint8, sw/zw/colsum_w [N]  (bgt_quantize_act ASYM on W^T)
 *   y  M x N float32; acc_out optional M x N int32.
 * Requirements: 1 <= M <= 65536, N % 16 == 0, 16 <= N <= 2^24,
 * K % 128 == 0, 128 <= K <= 32768 (so |A| <= K*255^2 < 2^31).
 * Rows of X and of W^T whose range does not contain 0 saturate in the
 * quantizer (see bgt_quantize_act): y is then the expansion's value for the
 * saturated codes.
 */
int bgt_w8a8_gemm_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                     const int32_t* rowsum_x, const uint8_t* qw, const float* sw,
                     const int32_t* zw, const int32_t* colsum_w, int64_t M, int64_t N,
                     int64_t K, float* y, int32_t* acc_out, void* stream);

/*
 * bgt_w4a8_moe_gemm_is -- grouped (mixture-of-experts) W4A8 GEMM with the
 * Integer Scale epilogue: the layer of [IS] 5.3 (the integer-scale W4A8
 * scheme applied to Mixtral 8x7B), where each token is routed to a few of E
 * experts and every expert is its own fine-grained W4A8 linear layer.
 * The R routed (token, expert) slots are sorted by expert; for every slot r
 * of expert e (expert_offsets[e] <= r < expert_offsets[e+1]):
 *     y[r][j] = the integer-scale output of bgt_w4a8_gemm_is for activation
 *               row slot_token[r] of (qx, sx) and expert e's weights.
 *
 *   qx, sx          T x K int8 codes and [T] scales of the tokens (bgt_quantize_act SYM).
 *   expert_offsets  [E+1] int32 on the device: 0 = offs[0] <= ... <= offs[E] = R.
 *   slot_token      [R] int32 on the device, each in [0, T); a token appears at
 *                   most once per expert (so no expert has more than T slots).
 *   packed          E x (N*K/2) bytes: expert e's bgt_pack_weights_int4 layout
 *                   at byte e*N*K/2.
 *   iscale          E x (K/128) x N elements of `width` bytes (1, 2, 4), all
 *                   made with the one amplifier alpha; values in [0, 2^23).
 *   y               R x N of element type y_type, row r = slot r.
 *   acc_out         optional R x N int32 (the integer accumulators).
 * Routing outside these rules cannot make the kernels read or write outside
 * the buffers (offsets are clamped to [0, R], tokens to [0, T), at most T
 * rows per expert, rounded up to a multiple of 16, are computed on the
 * grouped decode path), but gives unspecified rows of y. Requirements:
 * 1 <= T <= 65536, N and K as bgt_w4a8_gemm_is, 1 <= E <= 256,
 * 1 <= R <= min(T*E, 2^24); qx, packed, iscale, y, acc_out 16-byte aligned.
 * Kernels: with K/128 in {16, 32, 112}, a weight-streaming grouped decode
 * kernel for T <= 64 and, up to T = 1024, whenever the mean expert (R/E
 * slots) needs at most two row passes of 64 slots (three of 32 at
 * K/128 = 112); experts
 * without slots read no weights there. Otherwise one tiled launch over the
 * experts' 256-row tiles.
 */
int bgt_w4a8_moe_gemm_is(const int8_t* qx, const float* sx, int64_t T,
                         const int32_t* expert_offsets, const int32_t* slot_token, int64_t E,
                         int64_t R, const uint8_t* packed, const void* iscale, int width,
                         int alpha, int64_t N, int64_t K, void* y, int y_type, int32_t* acc_out,
                         void* stream);

/* Diagnostics: name of the kernel bgt_w4a8_moe_gemm_is launches for T tokens,
 * E experts and R slots ("invalid shape" outside the entry point's limits). */
const char* bgt_w4a8_moe_kernel_name(int64_t T, int64_t E, int64_t R, int64_t K);

/*
 * bgt_pack_weights_int8 -- offline group-wise int8 weight quantization for the
 * fine-grained W8A8 layer of the [IS] page's LLaMA-3 scheme (5.4: 8-bit
 * weights for the down projection, groups of 128), with integer scales.
 * Per column j and group l, the closed forms of bgt_pack_weights_int4 at
 * q_max = 127:
 *     s_lj = max |w| / 127,   q_kj = clip(round(w_kj / s_lj), -127, 127)   (s = 0 -> q = 0),
 *     fscale[l][j] = s_lj,    iscale[l][j] = round(s_lj * alpha).
 * alpha as in bgt_pack_weights_int4 (0 = the amplifier search). The scales
 * are q_max ratio 127/7 smaller than the int4 ones, so the same alpha gives
 * integer scales about 18 times smaller.
 *
 * Int8 fragment layout, N*K bytes. With G = K/128:
 *     t = j/16, c = j%16, l = k/128, r = k%128,
 *     h = r/64, s = (r%64)/16, e = r%16,
 *     byte(k, j) = (((t*G + l)*2 + h)*64 + 16*s + c)*16 + e.
 * Each (16-column tile, group) pair is one contiguous 2 KiB block of two
 * 1 KiB halves (64 k each); within a half, 16 bytes per lane of a 64-wide
 * wavefront.
 *
 *   w       K x N float32 (finite).
 *   qw      N*K bytes, 16-byte aligned.  fscale, iscale: (K/128) x N.
 * Returns BGT_ERR_RANGE if some iscale would reach 2^23,
 * BGT_WARN_ACC_MAY_OVERFLOW when the worst-case accumulator
 * 2064512 * G * max(iscale) (|q_x|, |q_w| <= 127, 128 products per group)
 * reaches 2^31. Synchronous.
 */
int bgt_pack_weights_int8(const float* w, int64_t K, int64_t N, int64_t group, int alpha,
                          int8_t* qw, float* fscale, int32_t* iscale, int* alpha_out,
                          void* stream);

/*
 * bgt_w8a8_gemm_is -- fine-grained W8A8 GEMM with the Integer Scale epilogue
 * ([IS] 5.4 LLaMA-3 scheme; epilogue of 方法 Fig. 3(c)):
 *     p_ilj  = sum_{k in group l} qx[i][k] * q_w[k][j]          (int32, |p| < 2^23)
 *     A_ij   = sum_l p_ilj * iscale[l][j]                        (int32, mod 2^32)
 *     y_ij   = ((float)A_ij * sx[i]) * (1/alpha).
 *
 *   qx      M x K int8 (bgt_quantize_act SYM), sx [M] float32.
 *   qw      the int8 fragment layout of bgt_pack_weights_int8.
 *   iscale  (K/128) x N, elements of `width` bytes (1: uint8, 2: uint16,
 *           4: int32), every value in [0, 2^23); 16-byte aligned.
 *   alpha   power of two in [1, 2^30], the one the integer scales were made with.
 *   y       M x N of element type y_type (fp32 result rounded once).
 *   acc_out optional M x N int32 (NULL = not written): A_ij itself.
 * Requirements: as bgt_w4a8_gemm_is; qx, qw, iscale, y, acc_out 16-byte aligned.
 * The groups split into S parts whose int32 sums meet in the library's
 * split-K workspace (the buffer described at bgt_w4a8_workspace_bytes:
 * S*M*N*4 bytes, allocated on first need, never during graph capture, where
 * the GEMM then runs unsplit) in two cases: for M > 64 with few 256 x 128
 * tiles (they fill at most half of the CUs), and for 16 < M <= 64 with N/16
 * even, where a workgroup takes two 16-column tiles over one part (S doubles
 * to at most 8 while the workgroups fit the CUs and every part keeps at least
 * 16 groups).
 */
int bgt_w8a8_gemm_is(const int8_t* qx, const float* sx, const int8_t* qw, const void* iscale,
                     int width, int alpha, int64_t M, int64_t N, int64_t K, void* y, int y_type,
                     int32_t* acc_out, void* stream);

/* Diagnostics: name of the kernel bgt_w8a8_gemm_is launches for this shape. */
const char* bgt_w8a8_is_kernel_name(int64_t M, int64_t N, int64_t K);

/* Human-readable text of a status code (static storage). */
const char* bgt_status_string(int status);

/* ABI version of this header (major*100 + minor): 101 adds the narrow
 * integer-scale entry points, 102 the fused linear layer, 103 fp16 / bf16
 * activation and output types, 104 the fine-grained W8A8 integer-scale GEMM,
 * 105 the grouped (mixture-of-experts) W4A8 integer-scale GEMM, 106 the
 * expert count and slot count in bgt_w4a8_moe_kernel_name, 107 the canonical
 * int4 layout (bgt_repack_int4_canonical), 108 bgt_set_prefill_kernel and
 * bgt_w4a8_workspace_bytes, 109 bgt_w4a8_gemm_is_noalloc. */
int bgt_abi_version(void);

/* Diagnostics: name of the GEMM kernel that bgt_w4a8_gemm_is (float_scale = 0)
 * or bgt_w4a8_gemm_fs (float_scale = 1) launches for this shape, as it
 * appears in profiler traces (static storage; "invalid shape" if rejected). */
const char* bgt_w4a8_kernel_name(int64_t M, int64_t N, int64_t K, int float_scale);

/* Tuning / testing control (no page defines it): which tile kernel the dense
 * W4A8 GEMMs (integer and float scale) take for M > 64. Both compute the same
 * bits; they differ only in speed.
 *   BGT_PREFILL_AUTO  (default) the 256 x 256 tile kernel when its launch takes
 *                     few enough rounds of one workgroup per CU (5 * its
 *                     rounds <= 3 * the 256 x 128 kernel's), else 256 x 128;
 *   BGT_PREFILL_WIDE  always the 256 x 256 tile kernel;
 *   BGT_PREFILL_TILED always the 256 x 128 tile kernel.
 * The grouped GEMM (bgt_w4a8_moe_gemm_is) past its decode range takes the
 * 256 x 256 kernel over the experts' row tiles when K/128 <= 32 (AUTO) or
 * under BGT_PREFILL_WIDE, in both cases only when T*K < 2^31; otherwise, and
 * under BGT_PREFILL_TILED, the 256 x 128 kernel.
 * Process-wide; takes effect for GEMMs launched after the call (set it before
 * capturing a graph). Returns BGT_OK, or BGT_ERR_MODE for another value. */

#define BGT_PREFILL_AUTO 0
#define BGT_PREFILL_WIDE 1
#define BGT_PREFILL_TILED 2
int bgt_set_prefill_kernel(int mode);

/* Device workspace the integer-scale W4A8 GEMMs (bgt_w4a8_gemm_is, _narrow,
 * _ex) use for this shape, in bytes: 0 for most shapes; S*M*N*4 when the
 * 256 x 128 tile kernel splits K into S parts (M > 64 with few tiles: the
 * tiles fill at most half of the CUs, at least 4 groups per part), whose
 * int32 sums are then added (exact mod 2^32) by a second kernel. The library
 * keeps one such buffer per device, allocated on first need and reused; a
 * GEMM launched while its stream is being captured into a graph does not
 * allocate and runs unsplit unless the buffer is already large enough.
 * Calls that overlap on one device (several streams) share the buffer and
 * race. Negative: the status of an invalid shape. */
int64_t bgt_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* BGT_H */
