// gemm.hip -- fine-grained W4A8 GEMMs (integer-scale and float-scale epilogues)
// and the asymmetric W8A8 zero-point control, for gfx950.
//
// The method (Integer Scale page, 方法, Fig. 3): X (M x K) and W (K x N) are
// split into groups of 128 along K; each group's int8 x int4 dot products give
// an int32 partial p_ilj; the integer-scale epilogue (Fig. 3(c)) accumulates
// A_ij = sum_l p_ilj * round(s_lj * alpha) in integers and converts once,
// y_ij = ((float)A_ij * s_i) / alpha; the float-scale control (Fig. 3(b))
// converts every group: acc = fma((float)p_ilj, s_lj, acc), y = acc * s_i.
//
// Contractions run on the int8 matrix cores:
//   v_mfma_i32_16x16x64_i8 (skinny kernel): A 16 x 64, B 64 x 16 per wave;
//     lane L supplies A row L%16 / B column L%16, bytes 16*(L/16).. of the
//     64-wide K slice; result lane L, register r holds C[4*(L/16) + r][L%16].
//   v_mfma_i32_32x32x32_i8 (tiled kernel): lane L supplies row/column L%32,
//     bytes 16*(L/32).. of the 32-wide K slice; result lane L, register r
//     holds C[8*(r/4) + 4*(L/32) + r%4][L%32].
// The K order inside one MFMA does not matter as long as A and B use the same
// one (it is a dot product), which is what lets the packed weight layout put
// each lane's 16 bytes next to each other.
#include "device_common.h"
#include "launch.h"

namespace bgt {

// 24-bit signed multiply-add: exact mod 2^32 while |p| < 2^23 and
// 0 <= iscale < 2^23 (guaranteed: |p| <= 128*127*8, iscale range checked at pack)
__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }

// =====================================================================
// Skinny kernel (small M): one workgroup per 16-column tile; its KS waves
// split the groups; each wave streams its share of the tile's packed 1 KiB
// group blocks with 16-byte non-temporal loads (a whole wave reads one
// contiguous KiB), unpacks in registers and runs 2 MFMAs per group and row
// block. Integer partial sums of the waves meet in LDS (exact, any order).
// The float-scale control keeps its ascending fma chain in one wave (KS = 1).
// =====================================================================
template <int MR, int KS, bool FS>
__global__ __launch_bounds__(kWave * KS) void k_w4a8_skinny(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint4* __restrict__ packed, const int32_t* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int CH = (MR <= 2) ? 8 : 4;   // group blocks in flight per batch
  const int G = K / kGroup;
  const int t = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = lane % 16, s4 = lane / 16;
  const int j = t * 16 + c;
  const int gb = (G * wave) / KS, ge = (G * (wave + 1)) / KS;

  const int8_t* arow[MR];
  bool avalid[MR];
#pragma unroll
  for (int rb = 0; rb < MR; ++rb) {
    const int i = rb * 16 + c;
    avalid[rb] = i < M;
    arow[rb] = qx + (int64_t)(i < M ? i : M - 1) * K + 16 * s4;
  }

  int acc[MR][4];
  float facc[MR][4];
#pragma unroll
  for (int rb = 0; rb < MR; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[rb][r] = 0; facc[rb][r] = 0.0f; }

  const uint4* bp = packed + (int64_t)t * G * 64 + lane;
  for (int g0 = gb; g0 < ge; g0 += CH) {
    uint4 bw[CH];
    int isc[CH];
    float fsc[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int l = g0 + u;
      if (l < ge) {
        bw[u] = load_u4_nt(bp + (int64_t)l * 64);
        if (FS) fsc[u] = fscale[(int64_t)l * N + j];
        else isc[u] = iscale[(int64_t)l * N + j];
      } else {
        bw[u] = make_uint4(0, 0, 0, 0);
        isc[u] = 0;
        fsc[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int l = g0 + u;
      if (l < ge) {
        uint32_t x0, x1, x2, x3, x4, x5, x6, x7;
        unpack_x16(bw[u].x, x0, x1);
        unpack_x16(bw[u].y, x2, x3);
        unpack_x16(bw[u].z, x4, x5);
        unpack_x16(bw[u].w, x6, x7);
        const v4i b0 = {(int)x0, (int)x1, (int)x2, (int)x3};
        const v4i b1 = {(int)x4, (int)x5, (int)x6, (int)x7};
#pragma unroll
        for (int rb = 0; rb < MR; ++rb) {
          v4i a0 = load_v4i(arow[rb] + (int64_t)l * kGroup);
          v4i a1 = load_v4i(arow[rb] + (int64_t)l * kGroup + 64);
          if (!avalid[rb]) { a0 = v4i{0, 0, 0, 0}; a1 = v4i{0, 0, 0, 0}; }
          v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pv = p[r] >> 4;          // B codes entered the MFMA as 16*q
            if (FS) facc[rb][r] = __builtin_fmaf((float)pv, fsc[u], facc[rb][r]);
            else acc[rb][r] = mad24(pv, isc[u], acc[rb][r]);
          }
        }
      }
    }
  }

  if (!FS && KS > 1) {
    __shared__ int red[(KS > 1 ? KS - 1 : 1) * MR * 4 * kWave];
    if (wave > 0) {
#pragma unroll
      for (int rb = 0; rb < MR; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(((wave - 1) * MR + rb) * 4 + r) * kWave + lane] = acc[rb][r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < KS; ++w)
#pragma unroll
      for (int rb = 0; rb < MR; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rb][r] += red[(((w - 1) * MR + rb) * 4 + r) * kWave + lane];
  }

#pragma unroll
  for (int rb = 0; rb < MR; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rb * 16 + 4 * s4 + r;
      if (i < M) {
        const int64_t o = (int64_t)i * N + j;
        if (FS) {
          y[o] = facc[rb][r] * sx[i];
        } else {
          const float t0 = (float)acc[rb][r] * sx[i];
          y[o] = t0 * inv_alpha;
          if (acc_out) acc_out[o] = acc[rb][r];
        }
      }
    }
}

// =====================================================================
// Tiled kernel (larger M): a BM x BN output tile per 256-thread workgroup,
// 2 x 2 waves, each wave TM x TN blocks of 32 x 32. One K step is one group
// of 128. A (int8 rows) and B are staged in LDS as [row or column][128 bytes]
// with a 16-byte pad (conflict-free 16-byte reads of 8 consecutive lanes).
// The next group's A and B are loaded into registers while the current one
// is multiplied. For W4, B is unpacked once per workgroup into true int8 in
// LDS; for the W8A8 control the uint8 codes of both operands are re-centred
// by 128 (x ^ 0x80) so the signed MFMA sees the same differences q - z.
// =====================================================================
enum class Epi { IS, FS, ZP };

constexpr int kLdsRow = 144;   // 128 bytes of K + 16 pad

template <int TM, int TN, Epi E>
__global__ __launch_bounds__(256, 2) void k_gemm_tiled(
    const uint8_t* __restrict__ xa,          // A codes: M x K (int8 for W4, uint8 for ZP)
    const float* __restrict__ sx,
    const uint8_t* __restrict__ wb,          // W4: packed layout; ZP: qw N x K uint8
    const int32_t* __restrict__ iscale, const float* __restrict__ fscale,
    const int32_t* __restrict__ zx, const int32_t* __restrict__ rowsum_x,
    const float* __restrict__ sw, const int32_t* __restrict__ zw,
    const int32_t* __restrict__ colsum_w, float inv_alpha, int M, int N, int K,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int BM = 2 * TM * 32, BN = 2 * TN * 32;
  constexpr bool W4 = (E != Epi::ZP);
  constexpr int A_CH = BM * 8 / 256;                       // 16-byte chunks per thread
  constexpr int B_CH = W4 ? (BN * 4 / 256) : (BN * 8 / 256);
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");
  __shared__ __align__(16) uint8_t As[BM * kLdsRow];
  __shared__ __align__(16) uint8_t Bs[BN * kLdsRow];

  const int G = K / kGroup;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int ntiles = N / 16;

  uint4 ra[A_CH], rbuf[B_CH];
  auto load_group = [&](int l) {
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
      const int q = tid + 256 * u, row = q / 8, k16 = q % 8;
      const int gi = m0 + row;
      const uint4* src = reinterpret_cast<const uint4*>(
          xa + (int64_t)(gi < M ? gi : M - 1) * K + (int64_t)l * kGroup + 16 * k16);
      ra[u] = (gi < M) ? *src : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < B_CH; ++u) {
      const int q = tid + 256 * u;
      if (W4) {
        const int tl = q / 64, lb = q % 64, tg = n0 / 16 + tl;
        const uint4* src = reinterpret_cast<const uint4*>(wb) +
                           ((int64_t)(tg < ntiles ? tg : ntiles - 1) * G + l) * 64 + lb;
        rbuf[u] = (tg < ntiles) ? load_u4_nt(src) : make_uint4(0, 0, 0, 0);
      } else {
        const int col = q / 8, k16 = q % 8, gj = n0 + col;
        const uint4* src = reinterpret_cast<const uint4*>(
            wb + (int64_t)(gj < N ? gj : N - 1) * K + (int64_t)l * kGroup + 16 * k16);
        rbuf[u] = (gj < N) ? *src : make_uint4(0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u);
      }
    }
  };
  auto store_group = [&]() {
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
      const int q = tid + 256 * u, row = q / 8, k16 = q % 8;
      uint4 v = ra[u];
      if (!W4) { v.x ^= 0x80808080u; v.y ^= 0x80808080u; v.z ^= 0x80808080u; v.w ^= 0x80808080u; }
      *reinterpret_cast<uint4*>(As + row * kLdsRow + 16 * k16) = v;
    }
#pragma unroll
    for (int u = 0; u < B_CH; ++u) {
      const int q = tid + 256 * u;
      if (W4) {
        const int tl = q / 64, lb = q % 64, s = lb / 16, cc = lb % 16;
        uint32_t l0, h0, l1, h1, l2, h2, l3, h3;
        unpack_i8(rbuf[u].x, l0, h0);
        unpack_i8(rbuf[u].y, l1, h1);
        unpack_i8(rbuf[u].z, l2, h2);
        unpack_i8(rbuf[u].w, l3, h3);
        uint8_t* dst = Bs + (tl * 16 + cc) * kLdsRow + 16 * s;
        *reinterpret_cast<uint4*>(dst) = make_uint4(l0, h0, l1, h1);        // k = 16s + 0..15
        *reinterpret_cast<uint4*>(dst + 64) = make_uint4(l2, h2, l3, h3);   // k = 64 + 16s + 0..15
      } else {
        const int col = q / 8, k16 = q % 8;
        uint4 v = rbuf[u];
        v.x ^= 0x80808080u; v.y ^= 0x80808080u; v.z ^= 0x80808080u; v.w ^= 0x80808080u;
        *reinterpret_cast<uint4*>(Bs + col * kLdsRow + 16 * k16) = v;
      }
    }
  };

  // per-lane accumulators
  int acc[TM][TN][16];
  float facc[TM][TN][16];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[a][b][r] = 0; facc[a][b][r] = 0.0f; }

  const int lr = lane % 32, hf = lane / 32;
  int colj[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) colj[b] = n0 + wn * (TN * 32) + b * 32 + lr;

  int isc[TN], iscn[TN];
  float fsc[TN], fscn[TN];
  auto load_scales = [&](int l, int* is, float* fs) {
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int jj = colj[b] < N ? colj[b] : N - 1;
      if (E == Epi::IS) is[b] = iscale[(int64_t)l * N + jj];
      if (E == Epi::FS) fs[b] = fscale[(int64_t)l * N + jj];
    }
  };

  load_group(0);
  if (E != Epi::ZP) load_scales(0, isc, fsc);
  for (int l = 0; l < G; ++l) {
    __syncthreads();
    store_group();
    __syncthreads();
    if (l + 1 < G) {
      load_group(l + 1);
      if (E != Epi::ZP) load_scales(l + 1, iscn, fscn);
    }
    v16i p[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        if (E == Epi::ZP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) p[a][b][r] = acc[a][b][r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) p[a][b][r] = 0;
        }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4i av[TM], bv[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        av[a] = *reinterpret_cast<const v4i*>(As + (wm * TM * 32 + a * 32 + lr) * kLdsRow + 64 * hf + 16 * m);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bv[b] = *reinterpret_cast<const v4i*>(Bs + (wn * TN * 32 + b * 32 + lr) * kLdsRow + 64 * hf + 16 * m);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          p[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[a], bv[b], p[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (E == Epi::IS) acc[a][b][r] = mad24(p[a][b][r], isc[b], acc[a][b][r]);
          else if (E == Epi::FS) facc[a][b][r] = __builtin_fmaf((float)p[a][b][r], fsc[b], facc[a][b][r]);
          else acc[a][b][r] = p[a][b][r];
        }
    if (E != Epi::ZP) {
#pragma unroll
      for (int b = 0; b < TN; ++b) { isc[b] = iscn[b]; fsc[b] = fscn[b]; }
    }
  }

  // epilogue: one conversion per output
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int j = colj[b];
      if (j >= N) continue;
      int32_t zwj = 0, cwj = 0;
      float swj = 0.0f;
      if (E == Epi::ZP) { zwj = zw[j] - 128; cwj = colsum_w[j] - 128 * K; swj = sw[j]; }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * (TM * 32) + a * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (i >= M) continue;
        const int64_t o = (int64_t)i * N + j;
        if (E == Epi::IS) {
          const float t0 = (float)acc[a][b][r] * sx[i];
          y[o] = t0 * inv_alpha;
          if (acc_out) acc_out[o] = acc[a][b][r];
        } else if (E == Epi::FS) {
          y[o] = facc[a][b][r] * sx[i];
        } else {
          // acc = sum (qw-128)(qx-128); expand (qw - zw)(qx - zx) with the re-centred
          // codes and zero points (same differences), all exact mod 2^32
          const int32_t zxi = zx[i] - 128, rxi = rowsum_x[i] - 128 * K;
          const int32_t A = acc[a][b][r] - zwj * rxi - zxi * cwj + K * zwj * zxi;
          const float sc = sx[i] * swj;
          y[o] = (float)A * sc;
          if (acc_out) acc_out[o] = A;
        }
      }
    }
}

// ------------------------------------------------------------------ launchers
template <int MR, bool FS>
static void launch_skinny(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const int32_t* iscale, const float* fscale, float inv_alpha, int M,
                          int N, int K, float* y, int32_t* acc_out, hipStream_t stream) {
  constexpr int KS = FS ? 1 : 4;
  dim3 grid(N / 16), block(kWave * KS);
  hipLaunchKernelGGL((k_w4a8_skinny<MR, KS, FS>), grid, block, 0, stream, qx, sx,
                     reinterpret_cast<const uint4*>(packed), iscale, fscale, inv_alpha, M, N, K, y,
                     acc_out);
}

hipError_t launch_w4a8(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                       const int32_t* iscale, const float* fscale, int alpha, int64_t M64,
                       int64_t N64, int64_t K64, float* y, int32_t* acc_out, hipStream_t stream) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  const float inv_alpha = 1.0f / (float)alpha;   // exact: alpha = 2^n
  if (M <= 64) {
    const int mr = (M + 15) / 16;
    if (float_scale) {
      switch (mr) {
        case 1: launch_skinny<1, true>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        case 2: launch_skinny<2, true>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        case 3: launch_skinny<3, true>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        default: launch_skinny<4, true>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
      }
    } else {
      switch (mr) {
        case 1: launch_skinny<1, false>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        case 2: launch_skinny<2, false>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        case 3: launch_skinny<3, false>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
        default: launch_skinny<4, false>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
      }
    }
  } else {
    constexpr int TM = 2, TN = 2, BM = 2 * TM * 32, BN = 2 * TN * 32;
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
    const uint8_t* xa = reinterpret_cast<const uint8_t*>(qx);
    if (float_scale)
      hipLaunchKernelGGL((k_gemm_tiled<TM, TN, Epi::FS>), grid, block, 0, stream, xa, sx, packed,
                         nullptr, fscale, nullptr, nullptr, nullptr, nullptr, nullptr, inv_alpha,
                         M, N, K, y, nullptr);
    else
      hipLaunchKernelGGL((k_gemm_tiled<TM, TN, Epi::IS>), grid, block, 0, stream, xa, sx, packed,
                         iscale, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, inv_alpha,
                         M, N, K, y, acc_out);
  }
  return hipGetLastError();
}

hipError_t launch_w8a8_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                          const int32_t* rowsum_x, const uint8_t* qw, const float* sw,
                          const int32_t* zw, const int32_t* colsum_w, int64_t M64, int64_t N64,
                          int64_t K64, float* y, int32_t* acc_out, hipStream_t stream) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  constexpr int TM = 1, TN = 1, BM = 64, BN = 64;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
  hipLaunchKernelGGL((k_gemm_tiled<TM, TN, Epi::ZP>), grid, block, 0, stream, qx, sx, qw,
                     nullptr, nullptr, zx, rowsum_x, sw, zw, colsum_w, 1.0f, M, N, K, y, acc_out);
  return hipGetLastError();
}

}  // namespace bgt
