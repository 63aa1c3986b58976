// gemm_w8is.hip -- fine-grained W8A8 GEMM with the integer-scale epilogue (gfx950).
//
// The Integer Scale page (5.4, the LLaMA-3 scheme) keeps the down projection
// at 8-bit weights, fine-grained: per-token int8 activations, group-wise (128)
// symmetric int8 weights, and the same integer-scale epilogue as the W4A8
// layer (方法, Fig. 3(c)):
//     p_ilj = sum_{k in group l} qx[i][k] * qw[k][j]      (|p| <= 128*127*127 < 2^23)
//     A_ij  = sum_l p_ilj * iscale[l][j]                   (int32, mod 2^32)
//     y_ij  = ((float)A_ij * sx[i]) * (1/alpha).
//
// Weights are in the int8 fragment layout (bgt_pack_weights_int8): each
// (16-column tile, group) pair is 2 KiB, two 1 KiB halves of 64 k, lane L of a
// half holding column L%16 and the 16 codes k = 16*(L/16) .. +15 of the half,
// i.e. one B operand of v_mfma_i32_16x16x64_i8 per half, read with one
// contiguous 16-byte load per lane.
//
// Three kernels:
//   split (M <= 64, weight streaming): one workgroup per 16-column tile, its
//     KS waves split the groups; each wave keeps D groups of weights, their
//     activation fragments and scales in flight in registers, runs two MFMAs
//     per group and row block and applies the group's integer scale with a
//     24-bit multiply-add. The waves' int32 sums (exact, any order) meet in LDS.
//     For M > 16 a workgroup takes two column tiles over one part of the
//     groups instead (each activation fragment serves both tiles, halving the
//     activation reads that dominate there); the parts' sums are added by the
//     reduction kernel.
//   tiled (M > 64): 64 x 64 output tiles, 8 waves, nine LDS-copy stages of one
//     group (activations row-major with XOR-swizzled 16-byte chunks, weights
//     straight from the fragment layout, the group's 64 scales), eight in
//     flight; waves 0-3 and 4-7 take the two 64-k halves of a group on a 2 x 2
//     arrangement of 32 x 32 blocks (v_mfma_i32_32x32x32_i8), apply the
//     group's scale to their half's partial and meet once at the end.
//   wide (large M): 256 x 128 tiles, 8 waves of 64 x 64, three copy stages;
//     3x the ops per copied byte of the 64 x 64 tile, chosen when its rounds
//     of workgroups move fewer copy bytes.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bgt {

// =====================================================================
// Split kernel
// =====================================================================
constexpr int kSplitMaxWaves = 16;
constexpr int kSplitCTWaves = 8;                   // waves of a workgroup of several column tiles
constexpr int split_max_waves(int mr) { return mr == 4 ? 8 : kSplitMaxWaves; }
constexpr int split_bound(int mr, int ct) { return ct > 1 ? kSplitCTWaves : split_max_waves(mr); }

// CT > 1 (M > 16): a workgroup covers CT adjacent column tiles over one of
// `splits` parts of the groups, and each wave applies every activation
// fragment it loads to all CT tiles, so the activation rows are read CT
// times less often; workgroup b takes tiles CT*(b / splits) .. + CT - 1 and
// part b % splits (splits divides 8, so each XCD's workgroups share one
// part's rows in their L2). The part's int32 sums go to part[s] (M x N, exact
// mod 2^32) for the reduction kernel, which adds the parts and converts.
template <int MR, int D, int CT, typename ST>
__global__ __launch_bounds__(split_bound(MR, CT) * 64) void k_w8is_split(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const uint4* __restrict__ qw,
    const ST* __restrict__ iscale, float inv_alpha, int M, int N, int K, OutY y,
    int32_t* __restrict__ acc_out, int splits, int32_t* __restrict__ part) {
  __shared__ int32_t red[split_max_waves(MR) * MR * 4 * 64];
  const int G = K / kGroup;
  const int KS = blockDim.x / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int c = lane % 16, s4 = lane / 16;
  const int sp = CT > 1 ? (int)blockIdx.x % splits : 0;
  const int t = CT > 1 ? ((int)blockIdx.x / splits) * CT : (int)blockIdx.x;
  const int gb = CT > 1 ? sp * G / splits : 0, gw = CT > 1 ? (sp + 1) * G / splits - gb : G;
  const int g0 = gb + wave * gw / KS, g1 = gb + (wave + 1) * gw / KS;   // this wave's groups

  const uint4* wsrc = qw + (int64_t)t * G * 128 + lane;       // + 128 G ct + 128 g + 64 h
  const ST* ssrc = iscale + 16 * t + c;                       // + 16 ct + N g
  // activation fragments: row 16 rb + c, bytes 16 s4 .. of each 64-k half;
  // rows past M are zero
  const int8_t* xsrc[MR];
  bool xrow[MR];
#pragma unroll
  for (int rb = 0; rb < MR; ++rb) {
    xrow[rb] = 16 * rb + c < M;
    xsrc[rb] = qx + (int64_t)(xrow[rb] ? 16 * rb + c : 0) * K + 16 * s4;
  }

  uint4 wb[D][CT][2];
  v4i xb[D][MR][2];
  int32_t sb[D][CT];
  auto fetch = [&](int j, int g) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      wb[j][ct][0] = load_u4_nt(wsrc + ((int64_t)ct * G + g) * 128);
      wb[j][ct][1] = load_u4_nt(wsrc + ((int64_t)ct * G + g) * 128 + 64);
      sb[j][ct] = (int32_t)ssrc[(int64_t)g * N + 16 * ct];
    }
#pragma unroll
    for (int rb = 0; rb < MR; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        xb[j][rb][h] = v4i{0, 0, 0, 0};
        if (xrow[rb]) xb[j][rb][h] = load_v4i(xsrc[rb] + 128 * g + 64 * h);
      }
  };

  int acc[CT][MR][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rb = 0; rb < MR; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ct][rb][r] = 0;

#pragma unroll
  for (int j = 0; j < D; ++j)
    if (g0 + j < g1) fetch(j, g0 + j);
#pragma unroll 1
  for (int g = g0; g < g1; g += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (g + j < g1) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          int32_t sc = sb[j][ct];
          if (sizeof(ST) < 4) opaque_reg(sc);          // keep the 24-bit multiply-adds as written
          const v4i b0 = {(int)wb[j][ct][0].x, (int)wb[j][ct][0].y, (int)wb[j][ct][0].z,
                          (int)wb[j][ct][0].w};
          const v4i b1 = {(int)wb[j][ct][1].x, (int)wb[j][ct][1].y, (int)wb[j][ct][1].z,
                          (int)wb[j][ct][1].w};
#pragma unroll
          for (int rb = 0; rb < MR; ++rb) {
            v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j][rb][0], b0, v4i{0, 0, 0, 0}, 0, 0, 0);
            p = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j][rb][1], b1, p, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ct][rb][r] = mad24(p[r], sc, acc[ct][rb][r]);
          }
        }
        if (g + j + D < g1) fetch(j, g + j + D);
      }
    }
  }

  // the waves' sums meet in LDS, one column tile at a time:
  // red[wave][rb*4 + r][lane]; then thread e < MR*256 adds element
  // (rb*4 + r, lane) over the waves (wrapping adds)
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if (ct > 0) __syncthreads();                     // the previous tile's sums are read
#pragma unroll
    for (int rb = 0; rb < MR; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * MR * 4 + rb * 4 + r) * 64 + lane] = acc[ct][rb][r];
    __syncthreads();
    for (int e = threadIdx.x; e < MR * 4 * 64; e += blockDim.x) {
      const int i4 = e / 64, ln = e % 64;
      const int row = 16 * (i4 / 4) + 4 * (ln / 16) + i4 % 4;
      if (row >= M) continue;
      uint32_t a = 0u;
      for (int w = 0; w < KS; ++w) a += (uint32_t)red[(w * MR * 4 + i4) * 64 + ln];
      const int32_t A = (int32_t)a;
      const int64_t o = (int64_t)row * N + 16 * (t + ct) + ln % 16;
      if constexpr (CT > 1) {
        part[(int64_t)sp * M * N + o] = A;
      } else {
        const float t0 = (float)A * sx[row];
        y.put(o, t0 * inv_alpha);
        if (acc_out) acc_out[o] = A;
      }
    }
  }
}

// =====================================================================
// Tiled kernel
// =====================================================================
constexpr int kW8isWaves = 8;

template <int GC, typename ST>
__global__ __launch_bounds__(kW8isWaves * 64) void k_w8is_tiled(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const int8_t* __restrict__ qw,
    const ST* __restrict__ iscale, float inv_alpha, int M, int N, int K, OutY y,
    int32_t* __restrict__ acc_out) {
  // GC > 0: K / 128 fixed at compile time and the step loop unrolls completely
  constexpr int NST = 9, BM = 64, BN = 64;
  constexpr int SB = sizeof(ST);
  constexpr int AB = (BM + BN) * 128;                 // operand bytes of a stage
  constexpr int STG = AB + 256;                       // + the group's 64 scales (<= 256 B)
  constexpr int LOADS = 3;                            // copies per stage per wave: 2 operand KiB + scales
  __shared__ __align__(16) int8_t S0[STG];
  __shared__ __align__(16) int8_t S1[STG];
  __shared__ __align__(16) int8_t S2[STG];
  __shared__ __align__(16) int8_t S3[STG];
  __shared__ __align__(16) int8_t S4[STG];
  __shared__ __align__(16) int8_t S5[STG];
  __shared__ __align__(16) int8_t S6[STG];
  __shared__ __align__(16) int8_t S7[STG];
  __shared__ __align__(16) int8_t S8[STG];
  auto stage = [&](auto ic) -> int8_t* {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 0) return S0;
    else if constexpr (i == 1) return S1;
    else if constexpr (i == 2) return S2;
    else if constexpr (i == 3) return S3;
    else if constexpr (i == 4) return S4;
    else if constexpr (i == 5) return S5;
    else if constexpr (i == 6) return S6;
    else if constexpr (i == 7) return S7;
    else return S8;
  };
  const int G = GC > 0 ? GC : K / kGroup;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int kh = wave / 4, wm = (wave % 4) / 2, wn = wave % 2;
  const int lr = lane % 32, hf = lane / 32;
  const int ntn = (N + BN - 1) / BN;
  const int n0 = (blockIdx.x % ntn) * BN, m0 = (blockIdx.x / ntn) * BM;
  const int T = N / 16;

  // operand copies: the 16 KiB blocks of a stage are spread over the waves, two
  // each. Block b < 8: activation rows 8b .. 8b+7, lane L fills row 8b + L/8,
  // chunk slot L%8 with the row's chunk (L%8) ^ ((row/2) % 8) (rows past M
  // re-read the last row). Block b >= 8: half (b-8)%2 of weight tile
  // n0/16 + (b-8)/2 (tiles past N re-read the last tile), copied as it is.
  const int8_t* src[2];
  int dst[2];
  int64_t gstep[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int b = wave * 2 + u;
    if (b < 8) {
      const int r8 = 8 * b + lane / 8;
      const int ck = 16 * ((lane % 8) ^ ((r8 >> 1) & 7));
      src[u] = qx + (int64_t)(m0 + r8 < M ? m0 + r8 : M - 1) * K + ck;
      gstep[u] = kGroup;
    } else {
      const int bb = b - 8, tl = n0 / 16 + bb / 2 < T ? n0 / 16 + bb / 2 : T - 1;
      src[u] = qw + ((int64_t)tl * G * 2 + bb % 2) * 1024 + lane * 16;
      gstep[u] = 2048;
    }
    dst[u] = b * 1024;
  }
  // scale copy: dword d = 2*SB*wave + lane (lane < 2*SB) of the group's 64*SB
  // scale bytes; dwords past N re-read the row's last dword
  const bool scopy = lane < 2 * SB;
  const int sd = 2 * SB * wave + lane;
  const int scol = n0 + sd * (4 / SB) < N ? n0 + sd * (4 / SB) : N - 4 / SB;
  const int8_t* ssrc = reinterpret_cast<const int8_t*>(iscale) + (int64_t)scol * SB;
  auto issue = [&](int g, int8_t* S) {
    const int gc = g < G ? g : G - 1;                 // past the end: a surplus copy, never read
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[u] + (int64_t)gc * gstep[u]),
          (__attribute__((address_space(3))) void*)(S + dst[u]), 16, 0, 0);
    if (scopy)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(ssrc + (int64_t)gc * N * SB),
          (__attribute__((address_space(3))) void*)(S + AB + 8 * SB * wave), 4, 0, 0);
  };

  // fragments: A row ra, B column 32 wn + lr (tile 2 wn + lr/16, lane slot
  // 16 m + lr%16 of half hf); the k chunk of MFMA m is 4 hf + m for both
  const int ra = wm * 32 + lr;
  constexpr int boff = BM * 128;                      // weight half-blocks follow the rows
  const int bcol = ((2 * wn + lr / 16) * 2 + hf) * 1024 + (lr % 16) * 16;
  const int scol_l = (32 * wn + lr) * SB;
  v16i acc = v16i{0};
  v16i pp = v16i{0};
  int32_t spp = 0;
  // step l: MFMAs of group l into p; then the previous group's partial times
  // its scale (its MFMAs have finished under this group's)
  auto compute = [&](const int8_t* S, bool apply_prev) {
    v4i av[2], bv[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * kh + mm;
      av[mm] = *reinterpret_cast<const v4i*>(S + ra * 128 + 16 * ((4 * hf + m) ^ ((ra >> 1) & 7)));
      bv[mm] = *reinterpret_cast<const v4i*>(S + boff + bcol + 256 * m);
    }
    int32_t sc = (int32_t)*reinterpret_cast<const ST*>(S + AB + scol_l);
    v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0], bv[0], v16i{0}, 0, 0, 0);
    p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[1], bv[1], p, 0, 0, 0);
    if (apply_prev) {
      opaque_reg(spp);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = mad24(pp[r], spp, acc[r]);
      opaque_reg(acc);                               // one group at a time: no partials kept live
    }
    pp = p;
    spp = sc;
  };
  auto step = [&](int l, auto j) {
    constexpr int J = decltype(j)::value;
    wait_vm_lds0<(NST - 2) * LOADS>();
    lds_barrier();
    issue(l + NST - 1, stage(IC<(J + NST - 1) % NST>{}));
    compute(stage(IC<J>{}), l > 0);
  };
  issue(0, S0);
  issue(1, S1);
  issue(2, S2);
  issue(3, S3);
  issue(4, S4);
  issue(5, S5);
  issue(6, S6);
  issue(7, S7);
  auto steps = [&](int l) {
    step(l + 0, IC<0>{});
    if (l + 1 >= G) return false;
    step(l + 1, IC<1>{});
    if (l + 2 >= G) return false;
    step(l + 2, IC<2>{});
    if (l + 3 >= G) return false;
    step(l + 3, IC<3>{});
    if (l + 4 >= G) return false;
    step(l + 4, IC<4>{});
    if (l + 5 >= G) return false;
    step(l + 5, IC<5>{});
    if (l + 6 >= G) return false;
    step(l + 6, IC<6>{});
    if (l + 7 >= G) return false;
    step(l + 7, IC<7>{});
    if (l + 8 >= G) return false;
    step(l + 8, IC<8>{});
    return true;
  };
  if constexpr (GC > 0) {
#pragma unroll
    for (int l = 0; l < G; l += NST) if (!steps(l)) break;
  } else {
#pragma unroll 1
    for (int l = 0; l < G; l += NST) if (!steps(l)) break;
  }
  opaque_reg(spp);
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = mad24(pp[r], spp, acc[r]);

  // the two k halves meet: waves 4-7 park their sums in stage 0, waves 0-3 add
  wait_vm_lds0<0>();
  lds_barrier();
  int32_t* R = reinterpret_cast<int32_t*>(S0);
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) R[((wave % 4) * 16 + r) * 64 + lane] = acc[r];
  }
  wait_lds0();
  lds_barrier();
  if (kh == 1) return;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    acc[r] = (int32_t)((uint32_t)acc[r] + (uint32_t)R[((wave % 4) * 16 + r) * 64 + lane]);

  const int j = n0 + wn * 32 + lr;
  if (j >= N) return;
  float sxr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = m0 + wm * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
    sxr[r] = sx[i < M ? i : M - 1];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = m0 + wm * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
    if (i >= M) continue;
    const int64_t o = (int64_t)i * N + j;
    const float t0 = (float)acc[r] * sxr[r];
    y.put(o, t0 * inv_alpha);
    if (acc_out) acc_out[o] = acc[r];
  }
}

// =====================================================================
// Wide tiled kernel (large M): 256 x 128 output tiles, 8 waves of 64 x 64
// (2 x 2 blocks of 32 x 32, v_mfma_i32_32x32x32_i8 over the whole group).
// Three LDS-copy stages of one group, two in flight: 256 activation rows
// (XOR-swizzled 16-byte chunks), the 8 weight tiles' 2 KiB fragment blocks as
// stored, and the group's 128 scales: seven copies per wave per stage. Per
// group each wave runs its four blocks in turn (four MFMAs each, into a fresh
// accumulator) and scales block k-1's partial with its column's integer
// scale under block k's MFMAs.
// =====================================================================
template <int GC, typename ST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_w8is_wide(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const int8_t* __restrict__ qw,
    const ST* __restrict__ iscale, float inv_alpha, int M, int N, int K, OutY y,
    int32_t* __restrict__ acc_out, int splits, int32_t* __restrict__ part) {
  constexpr int NW = 8, WN = 2, BM = 256, BN = 128;
  constexpr int SB = sizeof(ST);
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int AB = A_BYTES + B_BYTES, STG = AB + 512;
  constexpr int A_CP = BM / 8 / NW;                   // 1 KiB activation copies per wave (4)
  constexpr int B_CP = B_BYTES / 1024 / NW;           // 1 KiB weight copies per wave (2)
  constexpr int LOADS = A_CP + B_CP + 1;              // + the scale copy
  __shared__ __align__(16) int8_t S0[STG];
  __shared__ __align__(16) int8_t S1[STG];
  __shared__ __align__(16) int8_t S2[STG];
  auto stage = [&](auto ic) -> int8_t* {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 0) return S0;
    else if constexpr (i == 1) return S1;
    else return S2;
  };
  // split K (GC == 0 launches only): workgroup id = ks * tiles + tile; split
  // ks runs groups g0 .. g0+G-1 = [ks*GT/splits, (ks+1)*GT/splits) and leaves
  // its integer-scaled int32 sums in part[ks] (M x N) for the reduction
  const int GT = K / kGroup;
  const int ntiles = (int)gridDim.x / splits;
  const int ks = (int)blockIdx.x / ntiles, tb = (int)blockIdx.x - ks * ntiles;
  const int g0 = (int)((int64_t)ks * GT / splits);
  const int G = GC > 0 ? GC : (int)((int64_t)(ks + 1) * GT / splits) - g0;
  const int T = N / 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, hf = lane / 32;
  int tm, tn;
  tile_of(tb, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // activation copy i of this wave: block b = NW*i + wave (rows 8b .. 8b+7),
  // lane L fills row 8b + L/8, slot L%8 with chunk (L%8) ^ ((row/2) % 8)
  // (32-bit offsets from the tile's first row)
  const int8_t* abase = qx + (int64_t)m0 * K;
  int aoff[A_CP];
#pragma unroll
  for (int i = 0; i < A_CP; ++i) {
    const int r = 8 * (NW * i + wave) + lane / 8;
    const int rr = m0 + r < M ? r : M - 1 - m0;
    aoff[i] = rr * K + 16 * ((lane % 8) ^ ((r >> 1) & 7));
  }
  // weight copy u: half-block q = 2*wave + u = (tile q/2 of the 8, half q%2)
  const int8_t* bsrc[B_CP];
#pragma unroll
  for (int u = 0; u < B_CP; ++u) {
    const int q = B_CP * wave + u;
    const int tl = n0 / 16 + q / 2 < T ? n0 / 16 + q / 2 : T - 1;
    bsrc[u] = qw + ((int64_t)tl * GT * 2 + q % 2) * 1024 + lane * 16;
  }
  // scale copy: dword d = 4*SB*wave + lane (lane < 4*SB) of the group's 128*SB
  // bytes; dwords past N re-read the row's last dword
  const bool scopy = lane < 4 * SB;
  const int sd = 4 * SB * wave + lane;
  const int scol = n0 + sd * (4 / SB) < N ? n0 + sd * (4 / SB) : N - 4 / SB;
  const int8_t* ssrc = reinterpret_cast<const int8_t*>(iscale) + (int64_t)scol * SB;
  auto issue = [&](int g, int8_t* S) {
    const int gc = (g < G ? g : G - 1) + g0;          // past the end: surplus copies, never read
#pragma unroll
    for (int i = 0; i < A_CP; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(abase + aoff[i] + (int64_t)gc * kGroup),
          (__attribute__((address_space(3))) void*)(S + (NW * i + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < B_CP; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bsrc[u] + (int64_t)gc * 2048),
          (__attribute__((address_space(3))) void*)(S + A_BYTES + (B_CP * wave + u) * 1024), 16, 0, 0);
    if (scopy)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(ssrc + (int64_t)gc * N * SB),
          (__attribute__((address_space(3))) void*)(S + AB + 16 * SB * wave), 4, 0, 0);
  };

  // fragments of block (a, b): A row wm*64 + 32a + lr, B column wn*64 + 32b + lr
  // (tile col/16, lane slot 16m + col%16 of half hf); MFMA m takes k chunk 4hf + m
  v4i av[2][4], bv[2][4];
  int32_t sc[2];
  auto read_frags = [&](const int8_t* S) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int ra = wm * 64 + 32 * a + lr;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        av[a][m] = *reinterpret_cast<const v4i*>(S + ra * 128 + 16 * ((4 * hf + m) ^ ((ra >> 1) & 7)));
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int cl = wn * 64 + 32 * b + lr;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        bv[b][m] = *reinterpret_cast<const v4i*>(S + A_BYTES + ((cl / 16 * 2 + hf) * 64 + 16 * m + cl % 16) * 16);
      sc[b] = (int32_t)*reinterpret_cast<const ST*>(S + AB + cl * SB);
    }
  };

  v16i acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = v16i{0};
  v16i pp = v16i{0};
  int32_t spp = 0;
  // block k of the group: its MFMA chain, then the previous block's partial
  // times its scale (block 3 of the previous group for k = 0)
  auto block = [&](auto kk, bool apply) {
    constexpr int k = decltype(kk)::value, kp = (k + 3) % 4;
    v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[k / 2][0], bv[k % 2][0], v16i{0}, 0, 0, 0);
#pragma unroll
    for (int m = 1; m < 4; ++m)
      p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[k / 2][m], bv[k % 2][m], p, 0, 0, 0);
    if (apply) {
      opaque_reg(spp);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[kp][r] = mad24(pp[r], spp, acc[kp][r]);
      opaque_reg(acc[kp]);
    }
    pp = p;
    spp = sc[k % 2];
  };
  auto step = [&](int l, auto j) {
    constexpr int J = decltype(j)::value;
    wait_vm_lds0<LOADS>();                            // group l landed (l+1 may be in flight)
    lds_barrier();                                    // ... in every wave; stage of l-1 free
    issue(l + 2, stage(IC<(J + 2) % 3>{}));
    read_frags(stage(IC<J>{}));
    block(IC<0>{}, l > 0);
    block(IC<1>{}, true);
    block(IC<2>{}, true);
    block(IC<3>{}, true);
  };
  issue(0, S0);
  issue(1, S1);
  auto steps = [&](int l) {
    step(l + 0, IC<0>{});
    if (l + 1 >= G) return false;
    step(l + 1, IC<1>{});
    if (l + 2 >= G) return false;
    step(l + 2, IC<2>{});
    return true;
  };
  if constexpr (GC > 0) {
#pragma unroll
    for (int l = 0; l < G; l += 3) if (!steps(l)) break;
  } else {
#pragma unroll 1
    for (int l = 0; l < G; l += 3) if (!steps(l)) break;
  }
  opaque_reg(spp);
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[3][r] = mad24(pp[r], spp, acc[3][r]);
  wait_vm_lds0<0>();                                  // surplus copies of the last steps

  if (part != nullptr) {                              // split K: this split's sums
    int32_t* pp2 = part + (int64_t)ks * M * N;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int a = k / 2, b = k % 2;
      const int j = n0 + wn * 64 + 32 * b + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 64 + 32 * a + 8 * (r / 4) + 4 * hf + (r % 4);
        if (i < M && j < N) pp2[(int64_t)i * N + j] = acc[k][r];
      }
    }
    return;
  }

  // one conversion per output; the lane's 32 token scales first
  float srow[2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * 64 + 32 * a + 8 * (r / 4) + 4 * hf + (r % 4);
      srow[a][r] = sx[i < M ? i : M - 1];
    }
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int a = k / 2, b = k % 2;
    const int j = n0 + wn * 64 + 32 * b + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * 64 + 32 * a + 8 * (r / 4) + 4 * hf + (r % 4);
      if (!full && (i >= M || j >= N)) continue;
      const int64_t o = (int64_t)i * N + j;
      const float t0 = (float)acc[k][r] * srow[a][r];
      y.put(o, t0 * inv_alpha);
      if (acc_out) acc_out[o] = acc[k][r];
    }
  }
}

// ------------------------------------------------------------------ launchers
// waves per split workgroup: about 4096 waves over the chip (16 per CU), at
// least two groups per wave, at most 16 (8 for four row blocks: LDS)
static int split_waves(int64_t N, int64_t K, int mr) {
  const int64_t T = N / 16, G = K / kGroup;
  int ks = 1;
  const int cap = split_max_waves(mr);
  while (ks < cap && T * ks < 4096 && 2 * (2 * ks) <= G) ks *= 2;
  return ks;
}

// M in 17..64: kSplitCT column tiles per split workgroup, whose groups split
// into S parts when that pays: S doubles (to at most 8) while the workgroups
// still fit the CUs and every part keeps at least two groups for each of its
// eight waves. 1: the one-tile launch, no parts.
constexpr int kSplitCT = 2;
static int w8is_split_parts(int M, int N, int K) {
  if (M <= 16 || (N / 16) % kSplitCT != 0) return 1;
  const int64_t cus = device_cus(), wg = N / 16 / kSplitCT;
  const int G = K / kGroup;
  int s = 1;
  while (s < 8 && wg * 2 * s <= cus && G / (2 * s) >= 2 * kSplitCTWaves) s *= 2;
  return s;
}

// M > 64: the 256 x 128 tile copies 3x the bytes of a 64 x 64 tile per group
// for 8x the work; with one workgroup per CU (LDS), pick the tile whose rounds
// of 256 workgroups move fewer bytes in total. When the 256 x 128 tiles fill
// at most half of the CUs, their groups split into S parts instead (S doubles
// while tiles * 2S fits the CUs, at least 8 groups per part), the parts'
// int32 sums added by a second kernel (exact mod 2^32), and that tile is taken.
static int w8is_splits(int M, int N, int K) {
  const int64_t wide = ((M + 255) / 256) * (int64_t)((N + 127) / 128), cus = device_cus();
  const int G = K / kGroup;
  int s = 1;
  while (wide * s * 2 <= cus && s * 2 * 8 <= G) s *= 2;
  return s;
}

static bool w8is_use_wide(int M, int N, int K) {
  if (w8is_splits(M, N, K) > 1) return true;
  const int64_t small = ((M + 63) / 64) * (int64_t)((N + 63) / 64);
  const int64_t wide = ((M + 255) / 256) * (int64_t)((N + 127) / 128);
  return ((wide + 255) / 256) * 97 < ((small + 255) / 256) * 32;
}

template <typename ST>
static void launch_w8is_t(const int8_t* qx, const float* sx, const int8_t* qw, const ST* iscale,
                          float inv_alpha, int M, int N, int K, OutY y, int32_t* acc_out,
                          hipStream_t stream) {
  if (M <= 64) {
    const int mr = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const uint4* w = reinterpret_cast<const uint4*>(qw);
    int splits = w8is_split_parts(M, N, K);
    int32_t* part = nullptr;
    if (splits > 1) {
      part = split_workspace((size_t)splits * M * N * sizeof(int32_t), stream);
      if (part == nullptr) splits = 1;
    }
    if (splits > 1) {
      dim3 grid((unsigned)(N / 16 / kSplitCT * splits)), block(kSplitCTWaves * kWave);
      if (mr == 2)
        hipLaunchKernelGGL((k_w8is_split<2, 3, kSplitCT, ST>), grid, block, 0, stream, qx, sx, w,
                           iscale, inv_alpha, M, N, K, y, acc_out, splits, part);
      else
        hipLaunchKernelGGL((k_w8is_split<4, 2, kSplitCT, ST>), grid, block, 0, stream, qx, sx, w,
                           iscale, inv_alpha, M, N, K, y, acc_out, splits, part);
      launch_split_reduce(part, splits, M, N, N, sx, inv_alpha, y, acc_out, stream);
      return;
    }
    const int ks = split_waves(N, K, mr);
    dim3 grid((unsigned)(N / 16)), block((unsigned)(ks * kWave));
    if (mr == 1)
      hipLaunchKernelGGL((k_w8is_split<1, 4, 1, ST>), grid, block, 0, stream, qx, sx, w, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    else if (mr == 2)
      hipLaunchKernelGGL((k_w8is_split<2, 3, 1, ST>), grid, block, 0, stream, qx, sx, w, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    else
      hipLaunchKernelGGL((k_w8is_split<4, 2, 1, ST>), grid, block, 0, stream, qx, sx, w, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    return;
  }
  const int G = K / kGroup;
  if (w8is_use_wide(M, N, K)) {
    const int tiles = ((M + 255) / 256) * ((N + 127) / 128);
    int splits = w8is_splits(M, N, K);
    int32_t* part = nullptr;
    if (splits > 1) {
      part = split_workspace((size_t)splits * M * N * sizeof(int32_t), stream);
      if (part == nullptr) splits = 1;
    }
    if (splits > 1) {
      hipLaunchKernelGGL((k_w8is_wide<0, ST>), dim3((unsigned)(tiles * splits)), dim3(512), 0,
                         stream, qx, sx, qw, iscale, inv_alpha, M, N, K, y, acc_out, splits, part);
      launch_split_reduce(part, splits, M, N, N, sx, inv_alpha, y, acc_out, stream);
      return;
    }
    dim3 grid((unsigned)tiles), block(512);
    if (G == 112)
      hipLaunchKernelGGL((k_w8is_wide<112, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    else if (G == 32)
      hipLaunchKernelGGL((k_w8is_wide<32, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    else
      hipLaunchKernelGGL((k_w8is_wide<0, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                         inv_alpha, M, N, K, y, acc_out, 1, nullptr);
    return;
  }
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  dim3 grid((unsigned)tiles), block(kW8isWaves * 64);
  if (G == 112)
    hipLaunchKernelGGL((k_w8is_tiled<112, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                       inv_alpha, M, N, K, y, acc_out);
  else if (G == 32)
    hipLaunchKernelGGL((k_w8is_tiled<32, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                       inv_alpha, M, N, K, y, acc_out);
  else
    hipLaunchKernelGGL((k_w8is_tiled<0, ST>), grid, block, 0, stream, qx, sx, qw, iscale,
                       inv_alpha, M, N, K, y, acc_out);
}

hipError_t launch_w8a8_is(const int8_t* qx, const float* sx, const int8_t* qw, const void* iscale,
                          int iscale_bytes, int alpha, int64_t M, int64_t N, int64_t K, OutY y,
                          int32_t* acc_out, hipStream_t stream) {
  const float inv_alpha = 1.0f / (float)alpha;        // exact: alpha is 2^n
  const int m = (int)M, n = (int)N, k = (int)K;
  if (iscale_bytes == 1)
    launch_w8is_t(qx, sx, qw, static_cast<const uint8_t*>(iscale), inv_alpha, m, n, k, y, acc_out,
                  stream);
  else if (iscale_bytes == 2)
    launch_w8is_t(qx, sx, qw, static_cast<const uint16_t*>(iscale), inv_alpha, m, n, k, y, acc_out,
                  stream);
  else
    launch_w8is_t(qx, sx, qw, static_cast<const int32_t*>(iscale), inv_alpha, m, n, k, y, acc_out,
                  stream);
  return hipGetLastError();
}

const char* w8a8_is_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M <= 64) return "k_w8is_split";
  return w8is_use_wide((int)M, (int)N, (int)K) ? "k_w8is_wide" : "k_w8is_tiled";
}

}  // namespace bgt
