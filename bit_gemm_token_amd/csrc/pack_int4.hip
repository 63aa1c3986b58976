// pack_int4.hip -- offline group-wise weight quantization and packing (gfx950):
// int4 codes for the W4A8 GEMMs and int8 codes for the fine-grained W8A8 one.
//
// Per column j and group l of 128 rows of W (K x N row-major), following the
// Integer Scale page (方法, Fig. 3(a): weights split into groups quantized
// independently) with the symmetric closed forms of the "Quantization" notes
// page at q_max = 7 (int4) or 127 (int8; the down-projection recipe of the
// Integer Scale page, 5.4):
//     s = max|w| / q_max,  q = clip(round(w / s), -q_max, q_max),  fscale = s,
// then the integer scales round(s * alpha) of Fig. 3(c).
//
// One thread per (column, group): the 128 values of its group are a strided
// column walk, coalesced across the 256 threads of a workgroup (consecutive
// columns). The thread builds the group's codes in registers and writes them
// with 16-byte stores into the lane slots of the (16-column tile, group)
// block of the device layout (int4: one 1 KiB block, four stores; int8: two
// 1 KiB halves, eight stores).
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace bgt {

constexpr int kPThreads = 256;

// packed word index (0..15) and bit offset of code r (0..127) within a
// column's 64-byte slice of a group block; see the layout in bgt.h
__device__ __forceinline__ void code_slot(int r, int& word, int& shift) {
  const int h = r / 64, s = (r % 64) / 16, e = r % 16;
  word = 4 * s + 2 * h + e / 8;
  shift = 8 * (e % 4) + 4 * ((e % 8) >= 4);
}

template <bool W8>
__global__ __launch_bounds__(kPThreads) void k_group_quant_pack(
    const float* __restrict__ w, int64_t K, int64_t N, uint4* __restrict__ packed,
    float* __restrict__ fscale, int32_t* __restrict__ minmax) {
  constexpr float kQmax = W8 ? 127.0f : 7.0f;
  constexpr int kQ = W8 ? 127 : 7;
  const int64_t j = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
  const int64_t l = blockIdx.y;
  const int64_t G = K / kGroup;
  float s = 0.0f;
  const bool active = j < N;
  if (active) {
    const float* col = w + (l * kGroup) * N + j;
    float v[kGroup];
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      v[r] = col[(int64_t)r * N];
      a = fmaxf(a, fabsf(v[r]));
    }
    s = a / kQmax;
    const int64_t t = j / 16, c = j % 16;
    if constexpr (W8) {
      // half h, slot sl = (r % 64) / 16: lane 16*sl + c holds codes r = 64h + 16sl .. +15
      uint4* blk = packed + (t * G + l) * 128 + c;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int code = 0;
          if (s != 0.0f) code = clamp_int((int)round_away(v[16 * q + e] / s), -kQ, kQ);
          wd[e / 4] |= ((uint32_t)code & 0xFFu) << (8 * (e % 4));
        }
        blk[(q / 4) * 64 + 16 * (q % 4)] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    } else {
      uint32_t words[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) words[i] = 0u;
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        int code = 0;
        if (s != 0.0f) code = clamp_int((int)round_away(v[r] / s), -kQ, kQ);
        int word, shift;
        code_slot(r, word, shift);
        words[word] |= ((uint32_t)code & 0xFu) << shift;
      }
      uint4* blk = packed + (t * G + l) * 64 + c;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        blk[16 * sl] = make_uint4(words[4 * sl], words[4 * sl + 1], words[4 * sl + 2], words[4 * sl + 3]);
    }
    fscale[l * N + j] = s;
  }
  // min over positive scales and max over all scales, as ordered float bits
  // (non-negative floats order like their bit patterns)
  const float pos = (active && s > 0.0f) ? s : INFINITY;
  const float mn = wave_min(pos);
  const float mx = wave_max(active ? s : 0.0f);
  if ((threadIdx.x % kWave) == 0) {
    atomicMin(&minmax[0], (int32_t)__float_as_uint(mn));
    atomicMax(&minmax[1], (int32_t)__float_as_uint(mx));
  }
}

__global__ void k_init_minmax(int32_t* minmax) {
  minmax[0] = (int32_t)__float_as_uint(INFINITY);
  minmax[1] = 0;
}

__global__ __launch_bounds__(kPThreads) void k_integer_scales(
    const float* __restrict__ fscale, int64_t count, float alpha, int32_t* __restrict__ iscale) {
  const int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
  if (i < count) iscale[i] = (int32_t)round_away(fscale[i] * alpha);   // exact product: alpha = 2^n
}

hipError_t launch_group_quant_pack(bool int8_codes, const float* w, int64_t K, int64_t N,
                                   void* packed, float* fscale, int32_t* iscale,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(k_init_minmax, dim3(1), dim3(1), 0, stream, iscale);
  dim3 grid((unsigned)((N + kPThreads - 1) / kPThreads), (unsigned)(K / kGroup));
  uint4* out = static_cast<uint4*>(packed);
  if (int8_codes)
    hipLaunchKernelGGL(k_group_quant_pack<true>, grid, dim3(kPThreads), 0, stream, w, K, N, out,
                       fscale, iscale);
  else
    hipLaunchKernelGGL(k_group_quant_pack<false>, grid, dim3(kPThreads), 0, stream, w, K, N, out,
                       fscale, iscale);
  return hipGetLastError();
}

hipError_t launch_integer_scales(const float* fscale, int64_t count, int alpha, int32_t* iscale,
                                 hipStream_t stream) {
  dim3 grid((unsigned)((count + kPThreads - 1) / kPThreads));
  hipLaunchKernelGGL(k_integer_scales, grid, dim3(kPThreads), 0, stream, fscale, count,
                     (float)alpha, iscale);
  return hipGetLastError();
}

// Narrow storage of integer scales: the same values in 2-byte or 1-byte
// unsigned elements (the caller has checked that every value fits).
template <typename T>
__global__ __launch_bounds__(kPThreads) void k_narrow_scales(
    const int32_t* __restrict__ in, int64_t count, T* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
  if (i < count) out[i] = (T)in[i];
}

hipError_t launch_narrow_scales(const int32_t* in, int64_t count, int out_bytes, void* out,
                                hipStream_t stream) {
  dim3 grid((unsigned)((count + kPThreads - 1) / kPThreads));
  if (out_bytes == 2)
    hipLaunchKernelGGL(k_narrow_scales<uint16_t>, grid, dim3(kPThreads), 0, stream, in, count,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(k_narrow_scales<uint8_t>, grid, dim3(kPThreads), 0, stream, in, count,
                       static_cast<uint8_t*>(out));
  return hipGetLastError();
}

// Canonical -> kernel-native int4 layout. The canonical layout holds W^T with K
// contiguous, two codes per byte, even k in the low nibble: the 16 codes
// k0 .. k0+15 of column j (k0 a multiple of 16) are the 8 bytes at (j*K +
// k0)/2, nibble i = code k0+i. A native 16-byte chunk (tile t, group g, lane
// 16s + c) holds column 16t + c: bytes 0..7 the codes 128g + 16s + e, bytes
// 8..15 the codes 128g + 64 + 16s + e (e = 0..15), each dword's byte b
// carrying e_b (low nibble) and e_{b+4} (high nibble). One thread per native
// chunk: two 8-byte canonical reads, and per 8 codes a perfect shuffle of the
// nibbles (e0 e1 .. e7 -> e0 e4 e1 e5 e2 e6 e3 e7).
__device__ __forceinline__ uint32_t nibble_shuffle(uint32_t x) {
  x = (x & 0xFF0000FFu) | ((x & 0x00FF0000u) >> 8) | ((x & 0x0000FF00u) << 8);
  return (x & 0xF00FF00Fu) | ((x & 0x0F000F00u) >> 4) | ((x & 0x00F000F0u) << 4);
}

__global__ __launch_bounds__(256) void k_repack_canonical(const uint2* __restrict__ canonical,
                                                          int64_t K, int64_t N,
                                                          uint4* __restrict__ packed) {
  const int64_t G = K / kGroup;
  const int64_t chunks = N * K / 32;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = q / (64 * G), g = (q / 64) % G;
    const int lane = (int)(q % 64), s4 = lane / 16, c = lane % 16;
    const int64_t j = 16 * t + c;
    const int64_t k0 = kGroup * g + 16 * s4;
    const uint2 a = canonical[(j * K + k0) / 16];          // codes k0 .. k0+15 (h = 0)
    const uint2 b = canonical[(j * K + k0 + 64) / 16];     // codes k0+64 .. k0+79 (h = 1)
    packed[q] = make_uint4(nibble_shuffle(a.x), nibble_shuffle(a.y), nibble_shuffle(b.x),
                           nibble_shuffle(b.y));
  }
}

hipError_t launch_repack_canonical(const uint8_t* canonical, int64_t K, int64_t N,
                                   uint8_t* packed, hipStream_t stream) {
  const int64_t chunks = N * K / 32;
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 65536);
  hipLaunchKernelGGL(k_repack_canonical, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint2*>(canonical), K, N,
                     reinterpret_cast<uint4*>(packed));
  return hipGetLastError();
}

}  // namespace bgt
