// launch.h -- internal launchers of libbgt (host side). Arguments are already
// validated by the C ABI layer (capi.hip) when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace bgt {

// x: rows x cols activations of element type x_type (kF32, kF16, kBF16)
hipError_t launch_quant_rows(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld,
                             bool asym, void* q, float* scale, int32_t* zero, int32_t* rowsum,
                             hipStream_t stream);

// Group quantization + packing (int4 nibbles, or int8 codes in the int8 fragment
// layout); also leaves min(positive s) and max(s) as float bits in iscale[0],
// iscale[1] (scratch until launch_integer_scales overwrites them).
hipError_t launch_group_quant_pack(bool int8_codes, const float* w, int64_t K, int64_t N,
                                   void* packed, float* fscale, int32_t* iscale,
                                   hipStream_t stream);

// canonical int4 layout (W^T, K contiguous, even k in the low nibble) ->
// kernel-native layout; K % 128 == 0, N % 16 == 0
hipError_t launch_repack_canonical(const uint8_t* canonical, int64_t K, int64_t N,
                                   uint8_t* packed, hipStream_t stream);

hipError_t launch_integer_scales(const float* fscale, int64_t count, int alpha, int32_t* iscale,
                                 hipStream_t stream);

// iscale holds (K/128) x N integer scales of iscale_bytes bytes each (4: int32,
// 2: uint16, 1: uint8); ignored (and fscale used) when float_scale is set.
// ws: split-K workspace of at least w4a8_split_bytes() bytes, or nullptr for
// the library's own (allocated on first need; unavailable while the stream is
// being captured, when the GEMM runs unsplit).
hipError_t launch_w4a8(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                       const void* iscale, int iscale_bytes, const float* fscale, int alpha,
                       int64_t M, int64_t N, int64_t K, OutY y, int32_t* acc_out,
                       hipStream_t stream, int32_t* ws = nullptr);

// CUs of the current device (256 when it cannot be queried)
int device_cus();

// the library's split-K workspace on the current device, at least `bytes`
// (allocated or grown on first need, never while `stream` is being captured);
// nullptr if unavailable
int32_t* split_workspace(size_t bytes, hipStream_t stream);

// adds `splits` M x N int32 parts (exact mod 2^32) and converts each output
// once: y = ((float)sum * sx[i]) * inv_alpha; y and acc_out rows ldn apart
void launch_split_reduce(const int32_t* part, int splits, int M, int N, int ldn, const float* sx,
                         float inv_alpha, OutY y, int32_t* acc_out, hipStream_t stream);

// bytes of split-K workspace a W4A8 GEMM of this shape uses (0: none)
size_t w4a8_split_bytes(int64_t M, int64_t N, int64_t K, bool float_scale);

// the no-allocation scratch on the current device (nullptr if its address
// cannot be obtained) and its size in bytes
int32_t* noalloc_scratch(size_t* capacity);

// the large-M W4A8 GEMM (256 x 256 tiles) over N columns whose scales, y and
// acc_out rows are ldn elements apart; inv_alpha = 1/alpha (exact)
void launch_w4a8_wide(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                      const void* iscale, int iscale_bytes, const float* fscale, float inv_alpha,
                      int M, int N, int K, int ldn, OutY y, int32_t* acc_out, hipStream_t stream);
// the same kernel over the experts' row tiles of a grouped GEMM (integer
// scale; rows of y and acc_out are slots; requires T*K < 2^31)
void launch_w4a8_wide_grouped(const int8_t* qx, const float* sx, const uint8_t* packed,
                              const void* iscale, int iscale_bytes, float inv_alpha, int N, int K,
                              const Route& rt, OutY y, int32_t* acc_out, hipStream_t stream);

// per-token quantization of x (M x K of element type x_type, leading dimension
// ldx) into q_out /
// s_out, then the integer-scale GEMM into y; one launch when
// w4a8_linear_fused() holds (M <= 4, K/128 in {16, 32, 86, 112}, x 16-byte aligned,
// ldx % 4 == 0), else the quantizer and the GEMM.
bool w4a8_linear_fused(int64_t M, int64_t K, const void* x, int64_t ldx);
hipError_t launch_w4a8_linear(const void* x, int x_type, int64_t ldx, const uint8_t* packed,
                              const void* iscale, int iscale_bytes, int alpha, int64_t M,
                              int64_t N, int64_t K, int8_t* q_out, float* s_out, OutY y,
                              hipStream_t stream);

// narrow (K/128) x N integer scales to 2-byte or 1-byte elements (values must fit)
hipError_t launch_narrow_scales(const int32_t* in, int64_t count, int out_bytes, void* out,
                                hipStream_t stream);

// name of the kernel a W4A8 GEMM of this shape dispatches to (diagnostics)
const char* w4a8_kernel_name(int64_t M, int64_t N, int64_t K, bool float_scale);

// large-M W4A8 kernel choice: automatic, or forced to the 256 x 256 / 256 x 128
// tile kernel; returns 0, or -1 for an unknown mode
enum PrefillKernel { kPrefillAuto = 0, kPrefillWide = 1, kPrefillTiled = 2 };
int set_prefill_kernel(int mode);

// grouped (mixture-of-experts) W4A8 integer-scale GEMM: E experts' packed
// weights and scales back to back; slots sorted by expert (offs: E+1 offsets,
// tok: the activation row of each of the R slots); y has R rows
hipError_t launch_w4a8_moe(const int8_t* qx, const float* sx, int64_t T, const int32_t* offs,
                           const int32_t* tok, int64_t E, int64_t R, const uint8_t* packed,
                           const void* iscale, int iscale_bytes, int alpha, int64_t N, int64_t K,
                           OutY y, int32_t* acc_out, hipStream_t stream);
const char* w4a8_moe_kernel_name(int64_t T, int64_t E, int64_t R, int64_t K);

// fine-grained W8A8 with the integer-scale epilogue; qw in the int8 fragment
// layout of bgt_pack_weights_int8, iscale of iscale_bytes bytes per element
hipError_t launch_w8a8_is(const int8_t* qx, const float* sx, const int8_t* qw, const void* iscale,
                          int iscale_bytes, int alpha, int64_t M, int64_t N, int64_t K, OutY y,
                          int32_t* acc_out, hipStream_t stream);
const char* w8a8_is_kernel_name(int64_t M, int64_t N, int64_t K);

hipError_t launch_w8a8_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                          const int32_t* rowsum_x, const uint8_t* qw, const float* sw,
                          const int32_t* zw, const int32_t* colsum_w, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc_out, hipStream_t stream);

}  // namespace bgt
