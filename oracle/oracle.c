/*
 * oracle.c -- plain, slow CPU oracle for the fine-grained quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the
 * bench's CPU-baseline leg may load this library. It shares no code, header,
 * table or helper with the HIP path (bit_gemm_token_amd/csrc); the two meet
 * only through the seeded float32 inputs of synth/.
 *
 * Built with: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, so every float operation below is the single IEEE
 * binary32 operation written; x86-64 evaluates float in SSE, no excess
 * precision). Integer sums are int64; OpenMP only splits independent rows or
 * outputs, never a sum.
 *
 * Pages cited (the method's sources):
 *   [QB] "探秘Transformer系列之（34）--- 量化基礎" (rzrgm.cn blog): §1.4 accumulation
 *        types, §2.2 absmax mapping to [-127,127], §2.2.1 eqs. (1),(2), the
 *        per-token x per-channel outer-product dequantization (§2.3.3 granularity).
 *   [QN] "Quantization" notes (zsc0tt.pages.dev): 量化公式, Asymmetric / Symmetric
 *        Quantization, Per-Channel, 矩阵乘法中的量化计算 (zero-point expansion).
 *   [IS] "Integer Scale: A Free Lunch for Faster Fine-grained Quantization of
 *        LLMs" summary page (dignews.cc): 動機 3.1-3.2, 方法 (Fig. 3 a/b/c, the
 *        amplifier search code, default amplifier), 實驗 5.1 Table 1, 5.4
 *        (LLaMA-3 scheme: fine-grained W8A8 for the down projection).
 *   [EX] "extreme quantization LLMs" (apxml.com): data packing of sub-byte codes.
 *
 * Readings where the pages are silent or garbled: round() is C roundf (half away from zero, the "四舍五入" of
 * [QB] §2.2); x/s is a true IEEE division; a zero range gives scale 0 and
 * codes 0; the amplifier search starts at 2^0 and returns 1 when the smallest
 * scale is already >= 1; int4 codes are clipped to [-7,7] (qmax = 2^(b-1)-1
 * as [QN] Symmetric Quantization gives for int8).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

static int clampi(long v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : (int)v); }

/* ------------------------------------------------------------------------
 * O1. Per-token dynamic symmetric int8 quantization of activations.
 * [QN] Symmetric Quantization: alpha = max(|x_min|,|x_max|), q_max = 127,
 * s = alpha / q_max, z = 0, q = clip(round(x/s), -q_max, q_max).
 * [QB] §2.3.3: per-token = one scale per row of the activation matrix;
 * [QB] dynamic quantization: the scale is computed at run time from the row.
 * ---------------------------------------------------------------------- */
EXPORT void orc_quant_sym_i8(const float* x, int64_t rows, int64_t cols, int64_t ld,
                             int8_t* q, float* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float* xr = x + i * ld;
        float a = 0.0f;                                 /* max |x| over the row */
        for (int64_t k = 0; k < cols; ++k) {
            float v = fabsf(xr[k]);
            if (v > a) a = v;
        }
        float si = a / 127.0f;
        s[i] = si;
        for (int64_t k = 0; k < cols; ++k) {
            int code = 0;
            if (si != 0.0f) {
                float r = roundf(xr[k] / si);
                code = clampi((long)r, -127, 127);
            }
            q[i * cols + k] = (int8_t)code;
        }
    }
}

/* ------------------------------------------------------------------------
 * O5 (first half). Per-row asymmetric uint8 quantization.
 * [QN] Asymmetric Quantization with q_min = 0, q_max = 255 (the [0,255] range
 * of [QB] §2.2 affine quantization): s = (x_max - x_min)/(q_max - q_min),
 * z = clip(round(q_min - x_min/s), q_min, q_max),
 * q = clip(round(x/s) + z, q_min, q_max). Also returns sum_k q (row sum),
 * the activation-side term of the zero-point expansion.
 * ---------------------------------------------------------------------- */
EXPORT void orc_quant_asym_u8(const float* x, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* q, float* s, int32_t* z, int32_t* rowsum)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float* xr = x + i * ld;
        float mn = xr[0], mx = xr[0];
        for (int64_t k = 1; k < cols; ++k) {
            if (xr[k] < mn) mn = xr[k];
            if (xr[k] > mx) mx = xr[k];
        }
        float si = (mx - mn) / 255.0f;
        int zi = 0;
        if (si != 0.0f) {
            float zf = roundf(0.0f - mn / si);
            zi = clampi((long)zf, 0, 255);
        }
        long sum = 0;
        for (int64_t k = 0; k < cols; ++k) {
            int code = 0;
            if (si != 0.0f) {
                float r = roundf(xr[k] / si);
                code = clampi((long)r + zi, 0, 255);
            }
            q[i * cols + k] = (uint8_t)code;
            sum += code;
        }
        s[i] = si;
        z[i] = zi;
        rowsum[i] = (int32_t)sum;
    }
}

/* ------------------------------------------------------------------------
 * O2. Group-wise symmetric int4 weight quantization, g rows of K per group.
 * [IS] 方法 Fig. 3(a): W (K x N) is split into groups quantized
 * independently; s_ij is the scale of weight group g_ij. [QB] §2.3.3 per-group:
 * K consecutive rows of a weight column share one scale. Closed forms as O1
 * with q_max = 7.
 * w: K x N row-major. codes: K x N row-major int8. fscale: (K/g) x N.
 * ---------------------------------------------------------------------- */
static void group_quant_sym(const float* w, int64_t K, int64_t N, int64_t g, int qmax,
                            int8_t* codes, float* fscale)
{
    const int64_t G = K / g;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t l = 0; l < G; ++l) {
            float a = 0.0f;
            for (int64_t r = 0; r < g; ++r) {
                float v = fabsf(w[(l * g + r) * N + j]);
                if (v > a) a = v;
            }
            float sl = a / (float)qmax;
            fscale[l * N + j] = sl;
            for (int64_t r = 0; r < g; ++r) {
                int code = 0;
                if (sl != 0.0f) {
                    float t = roundf(w[(l * g + r) * N + j] / sl);
                    code = clampi((long)t, -qmax, qmax);
                }
                codes[(l * g + r) * N + j] = (int8_t)code;
            }
        }
    }
}

EXPORT void orc_group_quant_int4(const float* w, int64_t K, int64_t N, int64_t g,
                                 int8_t* codes, float* fscale)
{
    group_quant_sym(w, K, N, g, 7, codes, fscale);
}

/* O2 with q_max = 127: group-wise symmetric int8 weights, the fine-grained
 * W8A8 of the [IS] page's LLaMA-3 recipe (5.4 LLaMA-3 量化方案: 8-bit weights
 * for the down projection, groups of 128); same closed forms as O1. */
EXPORT void orc_group_quant_int8(const float* w, int64_t K, int64_t N, int64_t g,
                                 int8_t* codes, float* fscale)
{
    group_quant_sym(w, K, N, g, 127, codes, fscale);
}

/* ------------------------------------------------------------------------
 * O2 step 4. The amplifier search of [IS] 方法: starting from 2^0, keep
 * doubling until the smallest group scale times the amplifier is >= 1.
 * Zero scales (all-zero groups) are ignored; if there is no positive scale,
 * or the smallest one is already >= 1, the amplifier is 1.
 * Returns the exponent n (alpha = 2^n); -1 if n would exceed max_log2.
 * ---------------------------------------------------------------------- */
EXPORT int orc_amplifier_log2(const float* fscale, int64_t count, int max_log2)
{
    float smin = INFINITY;
    for (int64_t i = 0; i < count; ++i)
        if (fscale[i] > 0.0f && fscale[i] < smin) smin = fscale[i];
    if (!(smin < INFINITY)) return 0;
    int n = 0;
    double amplified = (double)smin;      /* smin * 2^n, exact in double */
    while (amplified < 1.0) {
        amplified *= 2.0;
        ++n;
        if (n > max_log2) return -1;
    }
    return n;
}

/* O2 step 5. Integer scales round(s * alpha) ([IS] 方法 Fig. 3(c)). */
EXPORT void orc_integer_scales(const float* fscale, int64_t count, int alpha, int32_t* iscale)
{
    for (int64_t i = 0; i < count; ++i) {
        float amplified = fscale[i] * (float)alpha;   /* exact: alpha is 2^n */
        iscale[i] = (int32_t)roundf(amplified);
    }
}

/* ------------------------------------------------------------------------
 * Narrow storage of integer scales ([IS] 方法, Fig. 4(a): at alpha = 2^10
 * the amplified scales fit 16-bit integers, most of them 8 bits). The values
 * are unchanged; only the element width differs. width 1: uint8, width 2:
 * uint16. Returns the number of values that do not fit the element (negative
 * or too large); when that number is not zero, nothing is written. Returns -1
 * for an unknown width.
 * ---------------------------------------------------------------------- */
EXPORT int64_t orc_narrow_iscale(const int32_t* iscale, int64_t count, int width, void* out)
{
    if (width != 1 && width != 2) return -1;
    const int64_t top = width == 1 ? 255 : 65535;
    int64_t bad = 0;
    for (int64_t i = 0; i < count; ++i)
        if (iscale[i] < 0 || iscale[i] > top) ++bad;
    if (bad) return bad;
    for (int64_t i = 0; i < count; ++i) {
        if (width == 1) ((uint8_t*)out)[i] = (uint8_t)iscale[i];
        else ((uint16_t*)out)[i] = (uint16_t)iscale[i];
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * fp32 -> bfloat16, round to nearest, ties to even (the bfloat16 format keeps
 * the sign, the 8 exponent bits and the top 7 fraction bits of binary32).
 * Written from that definition: the dropped 16 bits decide the rounding; a
 * NaN stays a (quiet) NaN. Used for the fp16 / bf16 output types, where the
 * output is the fp32 result rounded once.
 * ---------------------------------------------------------------------- */
EXPORT void orc_f32_to_bf16(const float* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        memcpy(&b, &in[i], 4);
        if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) {   /* NaN */
            out[i] = (uint16_t)((b >> 16) | 0x0040u);
            continue;
        }
        const uint32_t keep = b >> 16, drop = b & 0xFFFFu;
        uint32_t r = keep;
        if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) r = keep + 1u;
        out[i] = (uint16_t)r;
    }
}

/* ------------------------------------------------------------------------
 * Weight MSE between the integer-scale and the float-scale dequantized
 * weights ([IS] 方法, Fig. 4(c): "weight MSE between integer and float
 * scales under different amplifiers"). With codes q (K x N), float scales s
 * and integer scales S = round(s * alpha) of group l:
 *     w_fs = q * s,   w_is = q * S / alpha,
 *     MSE  = (1 / (K N)) * sum_{k,j} (w_is - w_fs)^2        (double).
 * Also returns, through the pointers (each may be NULL), the largest integer
 * scale and the number of integer scales above 255 (those that need more
 * than 8 bits; Fig. 4(a)).
 * ---------------------------------------------------------------------- */
EXPORT double orc_weight_mse_is_fs(const int8_t* codes, const float* fscale,
                                   const int32_t* iscale, int alpha, int64_t K, int64_t N,
                                   int64_t g, int32_t* max_iscale, int64_t* above_8bit)
{
    const int64_t G = K / g;
    double sum = 0.0;
    int32_t mx = 0;
    int64_t wide = 0;
    for (int64_t l = 0; l < G; ++l)
        for (int64_t j = 0; j < N; ++j) {
            const int32_t S = iscale[l * N + j];
            if (S > mx) mx = S;
            if (S > 255) ++wide;
            const double d = (double)S / (double)alpha - (double)fscale[l * N + j];
            double q2 = 0.0;
            for (int64_t r = 0; r < g; ++r) {
                const double q = (double)codes[(l * g + r) * N + j];
                q2 += q * q;
            }
            sum += q2 * d * d;
        }
    if (max_iscale) *max_iscale = mx;
    if (above_8bit) *above_8bit = wide;
    return sum / ((double)K * (double)N);
}

/* ------------------------------------------------------------------------
 * Packed int4 layout ([EX] "data packing": two 4-bit codes per byte). The
 * index map is the one the library header declares; it is restated here
 * from that declaration, independently of the kernels:
 *   t = j/16, c = j%16; l = k/128, r = k%128;
 *   h = r/64, s = (r%64)/16, e = r%16; lane = 16*s + c;
 *   byte = ((t*G + l)*64 + lane)*16 + 8*h + 4*(e/8) + (e%4);
 *   nibble = low 4 bits if (e%8) < 4, else high 4 bits;
 *   a code is stored as 4-bit two's complement.
 * codes: K x N row-major; packed: N*K/2 bytes.
 * ---------------------------------------------------------------------- */
static int64_t packed_byte(int64_t k, int64_t j, int64_t G, int* high)
{
    int64_t t = j / 16, c = j % 16, l = k / 128, r = k % 128;
    int64_t h = r / 64, s = (r % 64) / 16, e = r % 16;
    int64_t lane = 16 * s + c;
    *high = (e % 8) >= 4;
    return ((t * G + l) * 64 + lane) * 16 + 8 * h + 4 * (e / 8) + (e % 4);
}

EXPORT void orc_pack_int4(const int8_t* codes, int64_t K, int64_t N, uint8_t* packed)
{
    const int64_t G = K / 128;
    memset(packed, 0, (size_t)(N * K / 2));
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            int high;
            int64_t b = packed_byte(k, j, G, &high);
            uint8_t nib = (uint8_t)(codes[k * N + j] & 0xF);
            packed[b] |= high ? (uint8_t)(nib << 4) : nib;
        }
}

EXPORT void orc_unpack_int4(const uint8_t* packed, int64_t K, int64_t N, int8_t* codes)
{
    const int64_t G = K / 128;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            int high;
            int64_t b = packed_byte(k, j, G, &high);
            int nib = high ? (packed[b] >> 4) & 0xF : packed[b] & 0xF;
            codes[k * N + j] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
}

/* Canonical int4 layout (the "data packing" of the apxml extreme-quantization
 * page, 实现与评估考量: several low-bit codes stored in one standard byte; the
 * order is this library's reading): the codes of W^T, K contiguous per output
 * column, two per byte, even k in the low nibble:
 *     byte(k, j) = (j*K + k) / 2,   nibble = k % 2 (0 = low),
 * 4-bit two's complement. */
EXPORT void orc_pack_int4_canonical(const int8_t* codes, int64_t K, int64_t N, uint8_t* out)
{
    memset(out, 0, (size_t)(N * K / 2));
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t b = (j * K + k) / 2;
            const uint8_t nib = (uint8_t)(codes[k * N + j] & 0xF);
            out[b] |= (k % 2) ? (uint8_t)(nib << 4) : nib;
        }
}

EXPORT void orc_unpack_int4_canonical(const uint8_t* in, int64_t K, int64_t N, int8_t* codes)
{
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t byte = in[(j * K + k) / 2];
            const int nib = (k % 2) ? (byte >> 4) & 0xF : byte & 0xF;
            codes[k * N + j] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
}

/* Int8 fragment layout of the fine-grained W8A8 weights (the byte formula
 * stated with bgt_pack_weights_int8): for t = j/16, c = j%16, l = k/128,
 * r = k%128, h = r/64, s = (r%64)/16, e = r%16,
 *     byte(k, j) = (((t*G + l)*2 + h)*64 + 16*s + c)*16 + e.
 * A pure permutation of the N*K codes; the inverse reads them back. */
static int64_t layout8_byte(int64_t k, int64_t j, int64_t G)
{
    int64_t t = j / 16, c = j % 16, l = k / 128, r = k % 128;
    int64_t h = r / 64, s = (r % 64) / 16, e = r % 16;
    return (((t * G + l) * 2 + h) * 64 + 16 * s + c) * 16 + e;
}

EXPORT void orc_layout_int8(const int8_t* codes, int64_t K, int64_t N, int8_t* out)
{
    const int64_t G = K / 128;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) out[layout8_byte(k, j, G)] = codes[k * N + j];
}

EXPORT void orc_unlayout_int8(const int8_t* in, int64_t K, int64_t N, int8_t* codes)
{
    const int64_t G = K / 128;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) codes[k * N + j] = in[layout8_byte(k, j, G)];
}

/* ------------------------------------------------------------------------
 * O3. W4A8 GEMM with the Integer Scale epilogue ([IS] 方法, Fig. 3(c)).
 *   p[i][l][j] = sum_{k in group l} qx[i][k] * qw[k][j]       (int64)
 *   A[i][j]    = sum_l p[i][l][j] * iscale[l][j]               (int64)
 *   y[i][j]    = ((float)(int32)A[i][j] * sx[i]) * (1/alpha)
 * The accumulator of [QB] §1.4 is int32: A outside int32 is counted in the
 * return value (overflow flag); y then uses A reduced mod 2^32, which is what
 * any int32 wrap-around accumulation gives.
 * Only the listed rows x cols are computed (all of them when rows/cols NULL).
 * Outputs A_out, y_out: nrows x ncols, row-major, in list order.
 * ---------------------------------------------------------------------- */
static int32_t wrap32(int64_t v) { return (int32_t)(uint32_t)(uint64_t)v; }

EXPORT int64_t orc_w4a8_gemm_is(const int8_t* qx, const float* sx, const int8_t* qw,
                                const int32_t* iscale, int alpha,
                                int64_t M, int64_t N, int64_t K, int64_t g,
                                const int64_t* rows, int64_t nrows,
                                const int64_t* cols, int64_t ncols,
                                int64_t* A_out, float* y_out)
{
    const int64_t G = K / g;
    const float inv_alpha = 1.0f / (float)alpha;   /* exact: alpha is 2^n */
    int64_t overflow = 0;
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    #pragma omp parallel for schedule(dynamic, 1) reduction(+:overflow)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows ? rows[ii] : ii;
        for (int64_t jj = 0; jj < ncols; ++jj) {
            int64_t j = cols ? cols[jj] : jj;
            int64_t A = 0;
            for (int64_t l = 0; l < G; ++l) {
                int64_t p = 0;
                for (int64_t r = 0; r < g; ++r) {
                    int64_t k = l * g + r;
                    p += (int64_t)qx[i * K + k] * (int64_t)qw[k * N + j];
                }
                A += p * (int64_t)iscale[l * N + j];
            }
            if (A < INT32_MIN || A > INT32_MAX) ++overflow;
            float af = (float)wrap32(A);
            float t = af * sx[i];
            if (A_out) A_out[ii * ncols + jj] = A;
            if (y_out) y_out[ii * ncols + jj] = t * inv_alpha;
        }
    }
    return overflow;
}

/* ------------------------------------------------------------------------
 * O4. W4A8 GEMM with the float-scale epilogue ([IS] 方法, Fig. 3(b), and
 * 動機 3.2): every group's integer result is converted to float and
 * multiplied by its float scale; groups are taken in ascending order with one
 * fused multiply-add each, then the activation scale is applied.
 *   acc = 0; for l: acc = fmaf((float)p[i][l][j], fscale[l][j], acc)
 *   y = acc * sx[i]
 * ---------------------------------------------------------------------- */
EXPORT void orc_w4a8_gemm_fs(const int8_t* qx, const float* sx, const int8_t* qw,
                             const float* fscale, int64_t M, int64_t N, int64_t K, int64_t g,
                             const int64_t* rows, int64_t nrows,
                             const int64_t* cols, int64_t ncols, float* y_out)
{
    const int64_t G = K / g;
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t i = rows ? rows[ii] : ii;
        for (int64_t jj = 0; jj < ncols; ++jj) {
            int64_t j = cols ? cols[jj] : jj;
            float acc = 0.0f;
            for (int64_t l = 0; l < G; ++l) {
                int64_t p = 0;
                for (int64_t r = 0; r < g; ++r) {
                    int64_t k = l * g + r;
                    p += (int64_t)qx[i * K + k] * (int64_t)qw[k * N + j];
                }
                acc = fmaf((float)p, fscale[l * N + j], acc);
            }
            y_out[ii * ncols + jj] = acc * sx[i];
        }
    }
}

/* ------------------------------------------------------------------------
 * O5 (second half). Asymmetric W8A8 GEMM through the zero-point expansion of
 * [QN] 矩阵乘法中的量化计算:
 *   (q_W - Z_W)(q_X - Z_X) = q_W q_X - Z_W q_X - Z_X q_W + Z_W Z_X,
 * summed over k: A = sum_k qw qx - zw*rowsum_x - zx*colsum_w + K*zw*zx.
 * The output requantization (S_Y, Z_Y) is not applied: Y stays float, and the
 * float factor is the per-token x per-channel scale product of [QB] §2.3.3
 * (outer product of the scale vectors, applied elementwise):
 *   y = (float)A * (sx[m] * sw[n]).
 * qx: M x K uint8; qw: N x K uint8 (per-channel codes, one row per output).
 * ---------------------------------------------------------------------- */
EXPORT int64_t orc_w8a8_gemm_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                                const int32_t* rowsum_x,
                                const uint8_t* qw, const float* sw, const int32_t* zw,
                                const int32_t* colsum_w, int64_t M, int64_t N, int64_t K,
                                const int64_t* rows, int64_t nrows,
                                const int64_t* cols, int64_t ncols,
                                int64_t* A_out, float* y_out)
{
    int64_t overflow = 0;
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    #pragma omp parallel for schedule(dynamic, 1) reduction(+:overflow)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        int64_t m = rows ? rows[ii] : ii;
        for (int64_t jj = 0; jj < ncols; ++jj) {
            int64_t n = cols ? cols[jj] : jj;
            int64_t dot = 0;
            for (int64_t k = 0; k < K; ++k)
                dot += (int64_t)qw[n * K + k] * (int64_t)qx[m * K + k];
            int64_t A = dot - (int64_t)zw[n] * rowsum_x[m] - (int64_t)zx[m] * colsum_w[n]
                        + K * (int64_t)zw[n] * (int64_t)zx[m];
            if (A < INT32_MIN || A > INT32_MAX) ++overflow;
            float scale = sx[m] * sw[n];
            if (A_out) A_out[ii * ncols + jj] = A;
            if (y_out) y_out[ii * ncols + jj] = (float)wrap32(A) * scale;
        }
    }
    return overflow;
}
