// quant_act.hip -- per-token dynamic quantization of activations (gfx950).
//
// SYM_I8 follows the symmetric formulas of the "Quantization" notes page
// (Symmetric Quantization: alpha = max|x|, s = alpha/127, q = clip(round(x/s),
// -127, 127)) at the per-token granularity of the "量化基礎" page (§2.3.3 量化粒度:
// one scale per activation row). ASYM_U8 follows the same page's Asymmetric
// Quantization with q in [0, 255] and also produces the row sum of the codes,
// the activation-side term of its zero-point expansion.
//
// One 1024-thread workgroup per row. The row is read once with 16-byte loads,
// all of a thread's loads issued before the first is used (one round trip to
// memory), and kept in registers (up to kVecPerThread float4 per thread); the row
// statistic is a wave64 shuffle reduction followed by a 16-wave LDS step; the
// codes are written as packed 4-byte words (one word per float4), so both
// the read and the write of a row are fully coalesced.
#include "device_common.h"
#include "launch.h"

namespace bgt {

constexpr int kQThreads = 1024;
constexpr int kQWaves = kQThreads / kWave;
// float4 slots per thread held in registers: 1 for rows up to 4096 elements, 4
// (rows up to 16384) beyond; longer rows stream their rest a second time. With
// 1024 threads the per-thread work after the row statistic (the quotient and
// rounding of each element) is a quarter of a 256-thread row's
constexpr int kVecShort = 1, kVecLong = 4;

template <bool ASYM>
struct RowStat {
  float a;   // SYM: max |x|;  ASYM: max x
  float b;   // ASYM: min x
};

template <bool ASYM>
__device__ __forceinline__ void block_reduce(RowStat<ASYM>& st, float* lds) {
  float a = wave_max(st.a);
  float b = ASYM ? wave_min(st.b) : 0.0f;
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) { lds[w] = a; if (ASYM) lds[kQWaves + w] = b; }
  __syncthreads();
  a = lds[0];
  b = ASYM ? lds[kQWaves] : 0.0f;
#pragma unroll
  for (int i = 1; i < kQWaves; ++i) {
    a = fmaxf(a, lds[i]);
    if (ASYM) b = fminf(b, lds[kQWaves + i]);
  }
  st.a = a;
  st.b = b;
}

__device__ __forceinline__ int block_sum(int v, int* lds) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();                       // lds may still be read from the previous reduce
  if (l == 0) lds[w] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < kQWaves; ++i) s += lds[i];
  return s;
}

// code of one element; s and z are the row's scale and zero point
template <bool ASYM>
__device__ __forceinline__ int quant_code(float x, float s, int z) {
  if (s == 0.0f) return 0;
  float r = round_away(x / s);               // IEEE division, then round half away
  if (ASYM) return clamp_int((int)r + z, 0, 255);
  return clamp_int((int)r, -127, 127);
}

// The same code with x / s as Markstein's corrected quotient (P. Markstein,
// IBM J. Res. Dev. 1990): with r = 1/s correctly rounded, q0 = x*r,
// e = fma(-q0, s, x) is exact and fma(e, r, q0) is x / s correctly rounded,
// as long as s, r and the residual stay normal (the caller keeps s within
// [2^-100, 2^100]; |x| <= 255 s here). Three operations instead of the
// division's scale / reciprocal / refine / fixup sequence.
template <bool ASYM>
__device__ __forceinline__ int quant_code_rcp(float x, float s, float r, int z) {
  const float q0 = x * r;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
  const float c = round_away(q);
  if (ASYM) return clamp_int((int)c + z, 0, 255);
  return clamp_int((int)c, -127, 127);
}

// Vector path: cols % 16 == 0, ld % 4 == 0, x and q 16-byte aligned.
template <bool ASYM, int IT, int kVecPerThread>
__global__ __launch_bounds__(kQThreads) void k_quant_rows_vec(
    const void* __restrict__ x, int64_t cols, int64_t ld, uint8_t* __restrict__ q,
    float* __restrict__ scale, int32_t* __restrict__ zero, int32_t* __restrict__ rowsum) {
  __shared__ float lds[2 * kQWaves];
  const int64_t row = blockIdx.x;
  const int64_t xr = row * ld / 4;                   // row start, in 4-element units
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * cols);
  const int64_t nvec = cols / 4;
  const int t = threadIdx.x;

  // every slot of the row is requested before any is used (one round trip to
  // memory, not one per slot): slot u exists for the whole workgroup when
  // u*kQThreads < nvec (a uniform branch); a thread past the row's end in its last
  // slot loads the row's last vector (in bounds) and leaves it out below
  float4 cache[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    if ((int64_t)u * kQThreads < nvec) {
      const int64_t v = t + (int64_t)u * kQThreads;
      cache[u] = load_x4<IT>(x, xr + (v < nvec ? v : nvec - 1));
    }
  }
  RowStat<ASYM> st{ASYM ? -INFINITY : 0.0f, ASYM ? INFINITY : 0.0f};
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t v = t + (int64_t)u * kQThreads;
    if (v < nvec) {
      const float4 f = cache[u];
      if (ASYM) {
        st.a = fmaxf(st.a, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
        st.b = fminf(st.b, fminf(fminf(f.x, f.y), fminf(f.z, f.w)));
      } else {
        st.a = fmaxf(st.a, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
      }
    }
  }
  for (int64_t v = t + (int64_t)kVecPerThread * kQThreads; v < nvec; v += kQThreads) {
    float4 f = load_x4<IT>(x, xr + v);
    if (ASYM) {
      st.a = fmaxf(st.a, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
      st.b = fminf(st.b, fminf(fminf(f.x, f.y), fminf(f.z, f.w)));
    } else {
      st.a = fmaxf(st.a, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
  }
  block_reduce<ASYM>(st, lds);

  float s;
  int z = 0;
  if (ASYM) {
    s = (st.a - st.b) / 255.0f;
    if (s != 0.0f) z = clamp_int((int)round_away(0.0f - st.b / s), 0, 255);
  } else {
    s = st.a / 127.0f;
  }

  int sum = 0;
  // row-uniform: the corrected quotient where s keeps it exact, else the division
  const bool rcp = s >= 0x1.0p-100f && s <= 0x1.0p100f;
  const float rs = rcp ? 1.0f / s : 0.0f;
  auto emit = [&](int64_t v, float4 f) {
    int c0, c1, c2, c3;
    if (rcp) {
      c0 = quant_code_rcp<ASYM>(f.x, s, rs, z);
      c1 = quant_code_rcp<ASYM>(f.y, s, rs, z);
      c2 = quant_code_rcp<ASYM>(f.z, s, rs, z);
      c3 = quant_code_rcp<ASYM>(f.w, s, rs, z);
    } else {
      c0 = quant_code<ASYM>(f.x, s, z);
      c1 = quant_code<ASYM>(f.y, s, z);
      c2 = quant_code<ASYM>(f.z, s, z);
      c3 = quant_code<ASYM>(f.w, s, z);
    }
    sum += c0 + c1 + c2 + c3;
    qr[v] = (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) |
            ((uint32_t)(c2 & 0xFF) << 16) | ((uint32_t)(c3 & 0xFF) << 24);
  };
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t v = t + (int64_t)u * kQThreads;
    if (v < nvec) emit(v, cache[u]);
  }
  for (int64_t v = t + (int64_t)kVecPerThread * kQThreads; v < nvec; v += kQThreads) emit(v, load_x4<IT>(x, xr + v));

  if (rowsum != nullptr || ASYM) {
    const int total = block_sum(sum, reinterpret_cast<int*>(lds));
    if (t == 0) {
      if (rowsum) rowsum[row] = total;
    }
  }
  if (t == 0) {
    scale[row] = s;
    if (ASYM) zero[row] = z;
  }
}

// Scalar path: any cols, any ld, any alignment.
template <bool ASYM, int IT>
__global__ __launch_bounds__(kQThreads) void k_quant_rows_scalar(
    const void* __restrict__ x, int64_t cols, int64_t ld, uint8_t* __restrict__ q,
    float* __restrict__ scale, int32_t* __restrict__ zero, int32_t* __restrict__ rowsum) {
  __shared__ float lds[2 * kQWaves];
  const int64_t row = blockIdx.x;
  const int64_t xr = row * ld;
  uint8_t* qr = q + row * cols;
  const int t = threadIdx.x;
  RowStat<ASYM> st{ASYM ? -INFINITY : 0.0f, ASYM ? INFINITY : 0.0f};
  for (int64_t k = t; k < cols; k += kQThreads) {
    const float f = load_x1<IT>(x, xr + k);
    if (ASYM) { st.a = fmaxf(st.a, f); st.b = fminf(st.b, f); }
    else st.a = fmaxf(st.a, fabsf(f));
  }
  block_reduce<ASYM>(st, lds);
  float s;
  int z = 0;
  if (ASYM) {
    s = (st.a - st.b) / 255.0f;
    if (s != 0.0f) z = clamp_int((int)round_away(0.0f - st.b / s), 0, 255);
  } else {
    s = st.a / 127.0f;
  }
  int sum = 0;
  for (int64_t k = t; k < cols; k += kQThreads) {
    const int c = quant_code<ASYM>(load_x1<IT>(x, xr + k), s, z);
    sum += c;
    qr[k] = (uint8_t)(c & 0xFF);
  }
  if (rowsum != nullptr || ASYM) {
    const int total = block_sum(sum, reinterpret_cast<int*>(lds));
    if (t == 0 && rowsum) rowsum[row] = total;
  }
  if (t == 0) {
    scale[row] = s;
    if (ASYM) zero[row] = z;
  }
}

template <int IT>
static void launch_quant_rows_t(bool vec, bool asym, dim3 grid, dim3 block, hipStream_t stream,
                                const void* x, int64_t cols, int64_t ld, uint8_t* qb, float* scale,
                                int32_t* zero, int32_t* rowsum) {
  if (vec) {
    const bool shortrow = cols <= 4 * kQThreads * kVecShort;
    if (asym && shortrow) hipLaunchKernelGGL((k_quant_rows_vec<true, IT, kVecShort>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
    else if (asym) hipLaunchKernelGGL((k_quant_rows_vec<true, IT, kVecLong>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
    else if (shortrow) hipLaunchKernelGGL((k_quant_rows_vec<false, IT, kVecShort>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
    else hipLaunchKernelGGL((k_quant_rows_vec<false, IT, kVecLong>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
  } else {
    if (asym) hipLaunchKernelGGL((k_quant_rows_scalar<true, IT>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
    else hipLaunchKernelGGL((k_quant_rows_scalar<false, IT>), grid, block, 0, stream, x, cols, ld, qb, scale, zero, rowsum);
  }
}

hipError_t launch_quant_rows(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ld,
                             bool asym, void* q, float* scale, int32_t* zero, int32_t* rowsum,
                             hipStream_t stream) {
  // vector path: 4-element loads (16 bytes fp32, 8 bytes fp16 / bf16) and
  // packed 4-byte code stores
  const bool vec = (cols % 16 == 0) && (ld % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(q) % 16 == 0);
  dim3 grid((unsigned)rows), block(kQThreads);
  uint8_t* qb = static_cast<uint8_t*>(q);
  if (x_type == kF16) launch_quant_rows_t<kF16>(vec, asym, grid, block, stream, x, cols, ld, qb, scale, zero, rowsum);
  else if (x_type == kBF16) launch_quant_rows_t<kBF16>(vec, asym, grid, block, stream, x, cols, ld, qb, scale, zero, rowsum);
  else launch_quant_rows_t<kF32>(vec, asym, grid, block, stream, x, cols, ld, qb, scale, zero, rowsum);
  return hipGetLastError();
}

}  // namespace bgt
