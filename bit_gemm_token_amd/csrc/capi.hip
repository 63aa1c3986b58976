// capi.hip -- the extern "C" entry points of libbgt (see include/bgt.h).
//
// Every argument is validated on the host before the first HIP call, so a
// rejected call touches neither the device nor any output. Kernels are
// enqueued on the caller's stream; nothing is allocated on the device.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bgt.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_alpha(int a) { return a >= 1 && a <= (1 << 30) && (a & (a - 1)) == 0; }

bool valid_type(int t) { return t == BGT_F32 || t == BGT_F16 || t == BGT_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? BGT_OK : BGT_ERR_HIP; }

int check_gemm_shape(int64_t M, int64_t N, int64_t K, int64_t kmax) {
  if (M < 1 || M > 65536) return BGT_ERR_SHAPE;
  if (N < 16 || N > (1 << 24) || N % 16 != 0) return BGT_ERR_SHAPE;
  if (K < BGT_GROUP || K > kmax || K % BGT_GROUP != 0) return BGT_ERR_SHAPE;
  return BGT_OK;
}

// Amplifier search of the Integer Scale page (方法): the smallest 2^n, n >= 0,
// with smin * 2^n >= 1. With smin = m * 2^e, m in [0.5, 1): n = max(0, 1 - e).
int searched_alpha_log2(float smin) {
  if (!(smin > 0.0f) || isinf(smin) || smin >= 1.0f) return 0;
  int e = 0;
  frexpf(smin, &e);
  return 1 - e;
}

}  // namespace

extern "C" {

int bgt_abi_version(void) { return 109; }

int bgt_w4a8_linear_fused(int64_t M, int64_t K, const void* x, int64_t ldx) {
  return bgt::w4a8_linear_fused(M, K, x, ldx) ? 1 : 0;
}

const char* bgt_w4a8_kernel_name(int64_t M, int64_t N, int64_t K, int float_scale) {
  if (check_gemm_shape(M, N, K, 65536) != BGT_OK) return "invalid shape";
  return bgt::w4a8_kernel_name(M, N, K, float_scale != 0);
}

int64_t bgt_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  return (int64_t)bgt::w4a8_split_bytes(M, N, K, false);
}

int bgt_set_prefill_kernel(int mode) {
  return bgt::set_prefill_kernel(mode) == 0 ? BGT_OK : BGT_ERR_MODE;
}

const char* bgt_status_string(int status) {
  switch (status) {
    case BGT_OK: return "ok";
    case BGT_WARN_ACC_MAY_OVERFLOW: return "warning: worst-case accumulator may exceed int32";
    case BGT_ERR_NULL: return "error: required pointer is NULL";
    case BGT_ERR_SHAPE: return "error: size out of range or not a required multiple";
    case BGT_ERR_ALIGN: return "error: pointer or leading dimension misaligned";
    case BGT_ERR_ALPHA: return "error: amplifier must be a power of two in [1, 2^30]";
    case BGT_ERR_MODE: return "error: unknown quantization mode, element type, scale width or kernel choice";
    case BGT_ERR_HIP: return "error: HIP call failed";
    case BGT_ERR_RANGE: return "error: integer scale out of range (pack: >= 2^23; narrow: above the element type)";
    default: return "unknown status";
  }
}

int bgt_quantize_act(const float* x, int64_t rows, int64_t cols, int64_t ld, int mode, void* q,
                     float* scale, int32_t* zero, int32_t* rowsum, void* stream) {
  return bgt_quantize_act_ex(x, BGT_F32, rows, cols, ld, mode, q, scale, zero, rowsum, stream);
}

int bgt_quantize_act_ex(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld,
                        int mode, void* q, float* scale, int32_t* zero, int32_t* rowsum,
                        void* stream) {
  if (mode != BGT_QUANT_SYM_I8 && mode != BGT_QUANT_ASYM_U8) return BGT_ERR_MODE;
  if (!valid_type(x_type)) return BGT_ERR_MODE;
  if (!x || !q || !scale) return BGT_ERR_NULL;
  if (mode == BGT_QUANT_ASYM_U8 && !zero) return BGT_ERR_NULL;
  if (rows < 1 || rows > 0x7FFFFFFF || cols < 1 || cols > (1 << 24) || ld < cols)
    return BGT_ERR_SHAPE;
  return hip_status(bgt::launch_quant_rows(x, x_type, rows, cols, ld, mode == BGT_QUANT_ASYM_U8, q,
                                           scale, zero, rowsum, static_cast<hipStream_t>(stream)));
}

namespace {

// Shared by the int4 and int8 packers: group quantization into `codes`, then
// the amplifier (given or searched), the range check and the integer scales.
// pmax: the largest |p| of one group with these codes (128 * 127 * q_max).
int pack_weights(bool int8_codes, double pmax, const float* w, int64_t K, int64_t N,
                 int64_t group, int alpha, void* codes, float* fscale, int32_t* iscale,
                 int* alpha_out, void* stream) {
  if (!w || !codes || !fscale || !iscale || !alpha_out) return BGT_ERR_NULL;
  if (group != BGT_GROUP) return BGT_ERR_SHAPE;
  if (K < BGT_GROUP || K > 65536 || K % BGT_GROUP != 0) return BGT_ERR_SHAPE;
  if (N < 16 || N > (1 << 24) || N % 16 != 0) return BGT_ERR_SHAPE;
  if (alpha != 0 && !pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(codes)) return BGT_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t G = K / BGT_GROUP;

  hipError_t e = bgt::launch_group_quant_pack(int8_codes, w, K, N, codes, fscale, iscale, s);
  if (e != hipSuccess) return BGT_ERR_HIP;
  uint32_t bits[2];
  e = hipMemcpyAsync(bits, iscale, sizeof(bits), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return BGT_ERR_HIP;
  float smin, smax;
  memcpy(&smin, &bits[0], 4);
  memcpy(&smax, &bits[1], 4);

  int a = alpha;
  if (a == 0) {
    const int n = searched_alpha_log2(smin);
    if (n > 30) return BGT_ERR_ALPHA;
    a = 1 << n;
  }
  *alpha_out = a;
  const double top = roundf(smax * (float)a);     // largest integer scale
  if (!(top < 8388608.0)) return BGT_ERR_RANGE;   // 2^23

  e = bgt::launch_integer_scales(fscale, G * N, a, iscale, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return BGT_ERR_HIP;
  if (pmax * (double)G * top >= 2147483648.0) return BGT_WARN_ACC_MAY_OVERFLOW;
  return BGT_OK;
}

}  // namespace

int bgt_pack_weights_int4(const float* w, int64_t K, int64_t N, int64_t group, int alpha,
                          uint8_t* packed, float* fscale, int32_t* iscale, int* alpha_out,
                          void* stream) {
  // |p| <= 128 * 127 * 7 = 113792 per group with the packer's codes
  return pack_weights(false, 113792.0, w, K, N, group, alpha, packed, fscale, iscale, alpha_out,
                      stream);
}

int bgt_pack_weights_int8(const float* w, int64_t K, int64_t N, int64_t group, int alpha,
                          int8_t* qw, float* fscale, int32_t* iscale, int* alpha_out,
                          void* stream) {
  // |p| <= 128 * 127 * 127 = 2064512 per group
  return pack_weights(true, 2064512.0, w, K, N, group, alpha, qw, fscale, iscale, alpha_out,
                      stream);
}

int bgt_w4a8_gemm_is(const int8_t* qx, const float* sx, const uint8_t* packed,
                     const int32_t* iscale, int alpha, int64_t M, int64_t N, int64_t K, float* y,
                     int32_t* acc_out, void* stream) {
  return bgt_w4a8_gemm_is_narrow(qx, sx, packed, iscale, 4, alpha, M, N, K, y, acc_out, stream);
}

int bgt_w4a8_gemm_is_narrow(const int8_t* qx, const float* sx, const uint8_t* packed,
                            const void* iscale, int width, int alpha, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* acc_out, void* stream) {
  return bgt_w4a8_gemm_is_ex(qx, sx, packed, iscale, width, alpha, M, N, K, y, BGT_F32, acc_out,
                             stream);
}

int bgt_w4a8_gemm_is_ex(const int8_t* qx, const float* sx, const uint8_t* packed,
                        const void* iscale, int width, int alpha, int64_t M, int64_t N, int64_t K,
                        void* y, int y_type, int32_t* acc_out, void* stream) {
  if (!qx || !sx || !packed || !iscale || !y) return BGT_ERR_NULL;
  if (width != 1 && width != 2 && width != 4) return BGT_ERR_MODE;
  if (!valid_type(y_type)) return BGT_ERR_MODE;
  int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  if (!pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(qx) || !aligned16(packed) || !aligned16(iscale) || !aligned16(y) ||
      (acc_out && !aligned16(acc_out)))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w4a8(false, qx, sx, packed, iscale, width, nullptr, alpha, M, N,
                                     K, bgt::OutY{y, y_type}, acc_out,
                                     static_cast<hipStream_t>(stream)));
}

int bgt_w4a8_gemm_is_noalloc(const int8_t* qx, const float* sx, const uint8_t* packed,
                             const int32_t* iscale, int alpha, int64_t M, int64_t N, int64_t K,
                             float* y, int32_t* acc_out, void* stream) {
  if (!qx || !sx || !packed || !iscale || !y) return BGT_ERR_NULL;
  int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  if (!pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(qx) || !aligned16(packed) || !aligned16(iscale) || !aligned16(y) ||
      (acc_out && !aligned16(acc_out)))
    return BGT_ERR_ALIGN;
  size_t cap = 0;
  int32_t* ws = bgt::noalloc_scratch(&cap);
  if (bgt::w4a8_split_bytes(M, N, K, false) > cap) return BGT_ERR_SHAPE;
  if (ws == nullptr) return BGT_ERR_HIP;
  return hip_status(bgt::launch_w4a8(false, qx, sx, packed, iscale, 4, nullptr, alpha, M, N, K,
                                     bgt::OutY{y, BGT_F32}, acc_out,
                                     static_cast<hipStream_t>(stream), ws));
}

int bgt_w4a8_linear_is(const void* x, int x_type, int64_t ldx, const uint8_t* packed,
                       const void* iscale, int width, int alpha, int64_t M, int64_t N, int64_t K,
                       int8_t* qx, float* sx, void* y, int y_type, void* stream) {
  if (!x || !packed || !iscale || !qx || !sx || !y) return BGT_ERR_NULL;
  if (width != 1 && width != 2 && width != 4) return BGT_ERR_MODE;
  if (!valid_type(x_type) || !valid_type(y_type)) return BGT_ERR_MODE;
  int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  if (ldx < K) return BGT_ERR_SHAPE;
  if (!pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(packed) || !aligned16(iscale) || !aligned16(qx) || !aligned16(y))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w4a8_linear(x, x_type, ldx, packed, iscale, width, alpha, M, N, K,
                                            qx, sx, bgt::OutY{y, y_type},
                                            static_cast<hipStream_t>(stream)));
}

int bgt_w4a8_gemm_fs(const int8_t* qx, const float* sx, const uint8_t* packed,
                     const float* fscale, int64_t M, int64_t N, int64_t K, float* y,
                     void* stream) {
  return bgt_w4a8_gemm_fs_ex(qx, sx, packed, fscale, M, N, K, y, BGT_F32, stream);
}

int bgt_w4a8_gemm_fs_ex(const int8_t* qx, const float* sx, const uint8_t* packed,
                        const float* fscale, int64_t M, int64_t N, int64_t K, void* y, int y_type,
                        void* stream) {
  if (!qx || !sx || !packed || !fscale || !y) return BGT_ERR_NULL;
  if (!valid_type(y_type)) return BGT_ERR_MODE;
  int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  if (!aligned16(qx) || !aligned16(packed) || !aligned16(fscale) || !aligned16(y))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w4a8(true, qx, sx, packed, nullptr, 4, fscale, 1, M, N, K,
                                     bgt::OutY{y, y_type}, nullptr,
                                     static_cast<hipStream_t>(stream)));
}

int bgt_repack_int4_canonical(const uint8_t* canonical, int64_t K, int64_t N, uint8_t* packed,
                              void* stream) {
  if (!canonical || !packed) return BGT_ERR_NULL;
  if (K < BGT_GROUP || K > 65536 || K % BGT_GROUP != 0) return BGT_ERR_SHAPE;
  if (N < 16 || N > (1 << 24) || N % 16 != 0) return BGT_ERR_SHAPE;
  if (!aligned16(canonical) || !aligned16(packed)) return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_repack_canonical(canonical, K, N, packed,
                                                 static_cast<hipStream_t>(stream)));
}

int bgt_narrow_iscale(const int32_t* iscale, int64_t count, int width, void* out, void* stream) {
  if (!iscale || !out) return BGT_ERR_NULL;
  if (width != 1 && width != 2) return BGT_ERR_MODE;
  if (count < 1 || count > ((int64_t)1 << 36)) return BGT_ERR_SHAPE;
  if (!aligned16(iscale) || !aligned16(out)) return BGT_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // range check on the host (an offline step): every value in [0, 2^(8*width)),
  // read back in chunks of at most 4 Mi values
  const int32_t top = width == 1 ? 255 : 65535;
  const int64_t chunk = std::min<int64_t>(count, (int64_t)1 << 22);
  std::vector<int32_t> h((size_t)chunk);
  for (int64_t i0 = 0; i0 < count; i0 += chunk) {
    const int64_t n = std::min<int64_t>(chunk, count - i0);
    hipError_t e = hipMemcpyAsync(h.data(), iscale + i0, (size_t)n * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return BGT_ERR_HIP;
    for (int64_t k = 0; k < n; ++k)
      if (h[(size_t)k] < 0 || h[(size_t)k] > top) return BGT_ERR_RANGE;
  }
  return hip_status(bgt::launch_narrow_scales(iscale, count, width, out, s));
}

int bgt_w4a8_moe_gemm_is(const int8_t* qx, const float* sx, int64_t T,
                         const int32_t* expert_offsets, const int32_t* slot_token, int64_t E,
                         int64_t R, const uint8_t* packed, const void* iscale, int width,
                         int alpha, int64_t N, int64_t K, void* y, int y_type, int32_t* acc_out,
                         void* stream) {
  if (!qx || !sx || !expert_offsets || !slot_token || !packed || !iscale || !y)
    return BGT_ERR_NULL;
  if (width != 1 && width != 2 && width != 4) return BGT_ERR_MODE;
  if (!valid_type(y_type)) return BGT_ERR_MODE;
  int st = check_gemm_shape(T, N, K, 65536);
  if (st != BGT_OK) return st;
  if (E < 1 || E > 256 || R < 1 || R > T * E || R > (1 << 24)) return BGT_ERR_SHAPE;
  if (!pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(qx) || !aligned16(packed) || !aligned16(iscale) || !aligned16(y) ||
      (acc_out && !aligned16(acc_out)))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w4a8_moe(qx, sx, T, expert_offsets, slot_token, E, R, packed,
                                         iscale, width, alpha, N, K, bgt::OutY{y, y_type},
                                         acc_out, static_cast<hipStream_t>(stream)));
}

const char* bgt_w4a8_moe_kernel_name(int64_t T, int64_t E, int64_t R, int64_t K) {
  if (T < 1 || T > 65536 || K < BGT_GROUP || K > 65536 || K % BGT_GROUP != 0 || E < 1 ||
      E > 256 || R < 1 || R > T * E || R > (int64_t{1} << 24))
    return "invalid shape";
  return bgt::w4a8_moe_kernel_name(T, E, R, K);
}

int bgt_w8a8_gemm_is(const int8_t* qx, const float* sx, const int8_t* qw, const void* iscale,
                     int width, int alpha, int64_t M, int64_t N, int64_t K, void* y, int y_type,
                     int32_t* acc_out, void* stream) {
  if (!qx || !sx || !qw || !iscale || !y) return BGT_ERR_NULL;
  if (width != 1 && width != 2 && width != 4) return BGT_ERR_MODE;
  if (!valid_type(y_type)) return BGT_ERR_MODE;
  int st = check_gemm_shape(M, N, K, 65536);
  if (st != BGT_OK) return st;
  if (!pow2_alpha(alpha)) return BGT_ERR_ALPHA;
  if (!aligned16(qx) || !aligned16(qw) || !aligned16(iscale) || !aligned16(y) ||
      (acc_out && !aligned16(acc_out)))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w8a8_is(qx, sx, qw, iscale, width, alpha, M, N, K,
                                        bgt::OutY{y, y_type}, acc_out,
                                        static_cast<hipStream_t>(stream)));
}

const char* bgt_w8a8_is_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (check_gemm_shape(M, N, K, 65536) != BGT_OK) return "invalid shape";
  return bgt::w8a8_is_kernel_name(M, N, K);
}

int bgt_w8a8_gemm_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                     const int32_t* rowsum_x, const uint8_t* qw, const float* sw,
                     const int32_t* zw, const int32_t* colsum_w, int64_t M, int64_t N, int64_t K,
                     float* y, int32_t* acc_out, void* stream) {
  if (!qx || !sx || !zx || !rowsum_x || !qw || !sw || !zw || !colsum_w || !y) return BGT_ERR_NULL;
  int st = check_gemm_shape(M, N, K, 32768);
  if (st != BGT_OK) return st;
  if (!aligned16(qx) || !aligned16(qw) || !aligned16(y) || (acc_out && !aligned16(acc_out)))
    return BGT_ERR_ALIGN;
  return hip_status(bgt::launch_w8a8_zp(qx, sx, zx, rowsum_x, qw, sw, zw, colsum_w, M, N, K, y,
                                        acc_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
