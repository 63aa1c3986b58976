// device_common.h -- helpers shared by the gfx950 kernels of libbgt (internal).
//
// Wave64 reductions, the half-away-from-zero rounding the quantizers use, the
// int4 -> int8 unpacks of the packed weight layout, and MFMA operand types.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bgt {

// Element types of activations and outputs (the BGT_F32 / BGT_F16 / BGT_BF16
// codes of the C ABI).
constexpr int kF32 = 0, kF16 = 1, kBF16 = 2;

// Four consecutive activation elements of element type IT as stored (16 bytes
// of fp32, 8 of fp16 / bf16), and widened to fp32 (exact for fp16 and bf16).
template <int IT> struct XRaw { using T = uint2; };
template <> struct XRaw<kF32> { using T = float4; };

template <int IT>
__device__ __forceinline__ float4 widen_x4(const typename XRaw<IT>::T& u) {
  if constexpr (IT == kF32) {
    return u;
  } else if constexpr (IT == kF16) {
    const __half2 a = *reinterpret_cast<const __half2*>(&u.x);
    const __half2 b = *reinterpret_cast<const __half2*>(&u.y);
    return make_float4(__low2float(a), __high2float(a), __low2float(b), __high2float(b));
  } else {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
  }
}

// x[4*i .. 4*i+3] widened to fp32: one 16-byte (fp32) or 8-byte load.
template <int IT>
__device__ __forceinline__ float4 load_x4(const void* x, int64_t i) {
  return widen_x4<IT>(reinterpret_cast<const typename XRaw<IT>::T*>(x)[i]);
}
template <int IT>
__device__ __forceinline__ float load_x1(const void* x, int64_t i) {
  if constexpr (IT == kF32) return static_cast<const float*>(x)[i];
  else if constexpr (IT == kF16) return __half2float(static_cast<const __half*>(x)[i]);
  else return __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16);
}

// The output matrix y and its element type. Values are computed in fp32 and
// rounded once to the stored type (fp16, bf16: round to nearest even).
struct OutY {
  void* p;
  int type;
  // the same output from column c on (row stride unchanged)
  OutY cols(int64_t c) const {
    return OutY{static_cast<char*>(p) + c * (type == kF32 ? 4 : 2), type};
  }
  __device__ __forceinline__ void put(int64_t o, float v) const {
    if (type == kF32) static_cast<float*>(p)[o] = v;
    else if (type == kF16) static_cast<__half*>(p)[o] = __float2half(v);
    else static_cast<__hip_bfloat16*>(p)[o] = __float2bfloat16(v);
  }
  // the same, as a non-temporal store (output written once, not re-read)
  __device__ __forceinline__ void put_nt(int64_t o, float v) const {
    if (type == kF32) {
      __builtin_nontemporal_store(v, static_cast<float*>(p) + o);
    } else {
      const __half h = __float2half(v);
      const __hip_bfloat16 b = __float2bfloat16(v);
      const uint16_t bits = type == kF16 ? *reinterpret_cast<const uint16_t*>(&h)
                                         : *reinterpret_cast<const uint16_t*>(&b);
      __builtin_nontemporal_store(bits, static_cast<uint16_t*>(p) + o);
    }
  }
};

// Expert routing of a grouped (mixture-of-experts) GEMM. The routed slots are
// sorted by expert: the slots of expert e are offs[e] .. offs[e+1]-1; slot r
// multiplies activation row tok[r] with expert e's weights and writes output
// row r. Expert e's packed weights and scales start wstride bytes and sstride
// elements after expert e-1's. Kernels clamp offsets to [0, R] and token
// indices to [0, T-1], so malformed routing cannot reach outside the buffers.
struct Route {
  const int32_t* offs;
  const int32_t* tok;
  int E, T, R;
  int64_t wstride, sstride;
};

__device__ __forceinline__ int clamp_route(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kGroup = 128;

// ----------------------------------------------------------------- rounding
// round() of the pages: half away from zero (C roundf). llvm.round lowers to
// trunc + |x - trunc(x)| >= 0.5 correction, exact for every float.
__device__ __forceinline__ float round_away(float v) { return __builtin_roundf(v); }

__device__ __forceinline__ int clamp_int(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ----------------------------------------------------------- int4 unpacking
// A 32-bit word of the packed layout holds 8 consecutive codes e0..e7 of one
// column: byte b carries e_b in its low nibble and e_{b+4} in its high nibble.
//
// unpack_x16: nibble moved to the high half of each byte, i.e. each int8 is
// 16 * code (exact for codes in [-8, 7]). Two ops per four codes; the x16 is
// divided out of the int32 dot product afterwards (an exact shift).
__device__ __forceinline__ void unpack_x16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = (w << 4) & 0xF0F0F0F0u;   // bytes: 16*e0, 16*e1, 16*e2, 16*e3
  hi = w & 0xF0F0F0F0u;          // bytes: 16*e4, 16*e5, 16*e6, 16*e7
}

// unpack_i8: true int8 codes (sign-extended nibbles). Per byte, with u the
// unsigned nibble, ((u ^ 8) + 0x78) ^ 0x80 == u - 16*(u >= 8); no carry crosses
// a byte because (u ^ 8) + 0x78 <= 0x87.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t u) {
  return ((u ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ void unpack_i8(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = sext_nibbles(w & 0x0F0F0F0Fu);
  hi = sext_nibbles((w >> 4) & 0x0F0F0F0Fu);
}

// ----------------------------------------------------------- memory helpers
template <typename T>
__device__ __forceinline__ T load_nt(const T* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint4 load_u4_nt(const uint4* p) {
  // streamed once per launch: non-temporal so it does not evict reused data
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(q));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ v4i load_v4i(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}

// ------------------------------------------------------ integer epilogue
// 24-bit signed multiply-add: exact mod 2^32 while |p| < 2^23 and
// 0 <= iscale < 2^23 (guaranteed: a group's |p| is at most 128*127*8 with int4
// weights and 128*127*127 with int8 weights; iscale range checked at pack)
__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }

// Marks a register value as rewritten here, so the compiler cannot re-associate
// accumulations across this point (re-associating a group's multiply-adds with
// the next group's keeps every product of a group live and exhausts the
// register file). Emits no instruction.
template <typename T>
__device__ __forceinline__ void opaque_reg(T& v) { asm volatile("" : "+v"(v)); }

// ------------------------------------------------------- waits, barriers
// compile-time integer (selects an LDS stage array by index)
template <int N_> struct IC { static constexpr int value = N_; };

// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] and [15:14],
// expcnt[6:4] = 7 meaning "don't wait", lgkmcnt[11:8]).
template <int VM>
__device__ __forceinline__ void wait_vm_lds0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt vmcnt(VM) only (lgkmcnt field at its maximum: no LDS wait).
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) only (vmcnt field at its maximum: no memory wait).
__device__ __forceinline__ void wait_lds0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// Workgroup barrier for the LDS ring: the caller has already waited for its
// own LDS stores (lgkmcnt) and LDS-DMA loads (vmcnt); a plain s_barrier then
// suffices, with no fence that would also drain the loads still in flight.
__device__ __forceinline__ void lds_barrier() { __builtin_amdgcn_s_barrier(); }

// Grouped tile order of the tiled GEMMs: tiles go in groups of 4 row tiles per
// column tile, so the tiles resident on one XCD share activation rows and
// weight columns in its L2.
__device__ __forceinline__ void tile_grouped(int t, int ntm, int ntn, int& tm, int& tn) {
  constexpr int GM = 4;
  const int group = t / (GM * ntn);
  const int first = group * GM;
  const int gsz = ntm - first < GM ? ntm - first : GM;
  const int in = t - group * GM * ntn;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Tile order of the tiled GEMMs: workgroup ids are dealt round-robin to the 8
// XCDs, so consecutive ids of one XCD are remapped to consecutive tiles (when
// the tile count is a multiple of 8), then taken in grouped order.
__device__ __forceinline__ void tile_of(int pid, int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);   // XCD-contiguous
  tile_grouped(pid, ntm, ntn, tm, tn);
}

// Row tiles of bm slots of expert i of a grouped GEMM (0 past the last expert).
__device__ __forceinline__ int expert_row_tiles(const Route& rt, int i, int bm) {
  if (i >= rt.E) return 0;
  const int lo = clamp_route(rt.offs[i], 0, rt.R);
  const int hi = clamp_route(rt.offs[i + 1], lo, rt.R);
  return (hi - lo + bm - 1) / bm;
}

// Tile of workgroup pid in a grouped (mixture-of-experts) tiled GEMM. The
// routing's row tiles (expert i has ceil(rows_i / bm), experts in order) times
// ntn column tiles are dealt so that each XCD (pid % 8) takes an equal
// contiguous run of them in grouped order; the launch's grid is only an upper
// bound on that count (the host does not read the routing), and its spare
// workgroups, which return false here, are spread over the XCDs instead of
// filling the last ones. The wave reads the offsets 64 experts per load and
// sums and scans them with lane shuffles. On true: the tile's expert e, its
// first slot a and slot count rows, its row tile tm within the expert and
// column tile tn (all wave-uniform).
__device__ __forceinline__ bool grouped_tile(int pid, int bm, int ntn, const Route& rt, int& e,
                                             int& a, int& rows, int& tm, int& tn) {
  const int lane = threadIdx.x % kWave;
  int rtiles = 0;
  for (int base = 0; base < rt.E; base += kWave) rtiles += wave_sum(expert_row_tiles(rt, base + lane, bm));
  rtiles = __builtin_amdgcn_readfirstlane(rtiles);
  const int real = rtiles * ntn;
  const int x = pid & 7, j = pid >> 3, q = real >> 3, rem = real & 7;
  if (j >= q + (x < rem ? 1 : 0)) return false;
  int gtm;
  tile_grouped(x * q + (x < rem ? x : rem) + j, rtiles, ntn, gtm, tn);
  for (int base = 0; base < rt.E; base += kWave) {
    const int nt = expert_row_tiles(rt, base + lane, bm);
    int incl = nt;                                   // inclusive prefix over the lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int excl = incl - nt;
    const unsigned long long hit = __ballot(gtm >= excl && gtm < incl);
    if (hit != 0ull) {
      const int l = (int)__builtin_ctzll(hit);
      e = __builtin_amdgcn_readfirstlane(base + l);
      tm = __builtin_amdgcn_readfirstlane(gtm - __shfl(excl, l, kWave));
      a = clamp_route(rt.offs[e], 0, rt.R);
      rows = clamp_route(rt.offs[e + 1], a, rt.R) - a;
      return true;
    }
    gtm -= __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
  }
  return false;
}

}  // namespace bgt
