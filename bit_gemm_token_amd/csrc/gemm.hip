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
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "device_common.h"
#include "launch.h"

namespace bgt {

// =====================================================================
// Skinny kernel (small M): one workgroup per 16-column tile; its KS waves
// split the groups; each wave streams its share of the tile's packed 1 KiB
// group blocks with 16-byte non-temporal loads (a whole wave reads one
// contiguous KiB), unpacks in registers and runs 2 MFMAs per group and row
// block. Integer partial sums of the waves meet in LDS (exact, any order).
// The float-scale control keeps its ascending fma chain in one wave (KS = 1).
// =====================================================================
template <int MR, int KS, bool FS, typename ST>
__global__ __launch_bounds__(kWave * KS) void k_w4a8_skinny(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint4* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K,
    OutY y, int32_t* __restrict__ acc_out) {
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
        else {
          isc[u] = (int)iscale[(int64_t)l * N + j];
          if (sizeof(ST) < 4) opaque_reg(isc[u]);   // keep the 24-bit multiply-adds as written
        }
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
          y.put(o, facc[rb][r] * sx[i]);
        } else {
          const float t0 = (float)acc[rb][r] * sx[i];
          y.put(o, t0 * inv_alpha);
          if (acc_out) acc_out[o] = acc[rb][r];
        }
      }
    }
}

// =====================================================================
// Streaming kernel (small M, the memory-bound decode regime).
// Persistent workgroups of KS loader waves plus one finisher wave.
//   Loader wave w owns groups [w*GPW, (w+1)*GPW) for the whole launch and
//   keeps their activation fragments in registers (loaded once), so the only
//   per-tile traffic is the packed weights and their scales. The workgroup
//   walks column tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...; two
//   register sets ping-pong so the next tile's blocks are in flight while the
//   current one is contracted. Loader waves issue loads only, all of them
//   unconditional (indices clamped, unused data ignored), so their waits
//   count exactly the loads still needed.
//   The finisher wave does every global store: it adds the loaders' partial
//   results from LDS, converts once and writes y (stores and loads never
//   share a wave's memory counter, so stores cannot stall the prefetch).
// Exchange through LDS, two copies (tile parity), one barrier per tile:
//   integer scale: per-wave int32 partial sums, added in any order (exact);
//   float scale:   the per-group int32 results and scales, so the finisher can
//                  run the ascending fma chain of Fig. 3(b) per output.
// A copy is rewritten two tiles later, after the finisher has passed the
// intermediate barrier, i.e. after it finished reading that copy.
// =====================================================================
template <int MR, int GPW, bool FS, int MAXT, int WPE, typename ST>
__global__ __launch_bounds__(MAXT) __attribute__((amdgpu_waves_per_eu(WPE))) void k_w4a8_stream(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint4* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K,
    OutY y, int32_t* __restrict__ acc_out) {
  extern __shared__ int lds[];
  constexpr int NR = MR * 4;                       // accumulator registers per lane
  const int G = K / kGroup, T = N / 16;
  const int KS = blockDim.x / kWave - 1;           // loader waves
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int lane = threadIdx.x % kWave;
  const int c = lane % 16, s4 = lane / 16;
  // one exchange copy: IS = KS x NR x 64 ints; FS = G x NR x 64 ints + G x 16 floats
  const int area = FS ? (G * NR * kWave + G * 16) : (KS * NR * kWave);
  const int P = gridDim.x;

  if (wave == KS) {
    // ------------------------------------------------------------- finisher
    float srow[NR];
#pragma unroll
    for (int idx = 0; idx < NR; ++idx) {
      const int i = (idx / 4) * 16 + 4 * s4 + (idx % 4);
      srow[idx] = sx[i < M ? i : M - 1];
    }
    int it = 0;
    for (int t = blockIdx.x; t < T; t += P, ++it) {
      __syncthreads();
      const int* xa = lds + (it & 1) * area;
      const int j = t * 16 + c;
#pragma unroll
      for (int idx = 0; idx < NR; ++idx) {
        const int i = (idx / 4) * 16 + 4 * s4 + (idx % 4);
        if (FS) {
          const float* fb = reinterpret_cast<const float*>(xa + G * NR * kWave);
          float a = 0.0f;
          for (int l = 0; l < G; ++l)
            a = __builtin_fmaf((float)xa[(l * NR + idx) * kWave + lane], fb[l * 16 + c], a);
          if (i < M) y.put((int64_t)i * N + j, a * srow[idx]);
        } else {
          int sum = 0;
          for (int w = 0; w < KS; ++w) sum += xa[(w * NR + idx) * kWave + lane];
          if (i < M) {
            const float t0 = (float)sum * srow[idx];
            y.put((int64_t)i * N + j, t0 * inv_alpha);
            if (acc_out) acc_out[(int64_t)i * N + j] = sum;
          }
        }
      }
    }
    return;
  }

  // --------------------------------------------------------------- loaders
  const int gb = wave * GPW;
  bool gvalid[GPW];
  int gcl[GPW];
#pragma unroll
  for (int u = 0; u < GPW; ++u) {
    gvalid[u] = gb + u < G;
    gcl[u] = gb + u < G ? gb + u : G - 1;
  }
  v4i a0[GPW][MR], a1[GPW][MR];
#pragma unroll
  for (int u = 0; u < GPW; ++u)
#pragma unroll
    for (int rb = 0; rb < MR; ++rb) {
      const int i = rb * 16 + c;
      const int8_t* src = qx + (int64_t)(i < M ? i : M - 1) * K + (int64_t)gcl[u] * kGroup + 16 * s4;
      a0[u][rb] = load_v4i(src);
      a1[u][rb] = load_v4i(src + 64);
    }
  // rows beyond M contribute zero (their outputs are never stored; zeroing keeps
  // the accumulators of valid rows independent of clamped duplicates anyway)
  const bool rvalid0 = c < M;

  auto issue = [&](int t, uint4* b, int* is, float* fs) {
    const int tc = t < T ? t : T - 1;
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      b[u] = load_u4_nt(packed + ((int64_t)tc * G + gcl[u]) * 64 + lane);
      if (FS) fs[u] = fscale[(int64_t)gcl[u] * N + tc * 16 + c];
      else {
        is[u] = (int)iscale[(int64_t)gcl[u] * N + tc * 16 + c];
        if (sizeof(ST) < 4) opaque_reg(is[u]);     // keep the 24-bit multiply-adds as written
      }
    }
  };
  auto contract = [&](int it, const uint4* b, const int* is, const float* fs) {
    int* xa = lds + (it & 1) * area;
    int acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0;
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      if (!gvalid[u]) continue;                     // wave-uniform
      uint32_t x0, x1, x2, x3, x4, x5, x6, x7;
      unpack_x16(b[u].x, x0, x1);
      unpack_x16(b[u].y, x2, x3);
      unpack_x16(b[u].z, x4, x5);
      unpack_x16(b[u].w, x6, x7);
      const v4i b0 = {(int)x0, (int)x1, (int)x2, (int)x3};
      const v4i b1 = {(int)x4, (int)x5, (int)x6, (int)x7};
#pragma unroll
      for (int rb = 0; rb < MR; ++rb) {
        const bool rv = rb == 0 ? rvalid0 : (rb * 16 + c < M);
        const v4i z = {0, 0, 0, 0};
        v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(rv ? a0[u][rb] : z, b0, z, 0, 0, 0);
        p = __builtin_amdgcn_mfma_i32_16x16x64_i8(rv ? a1[u][rb] : z, b1, p, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pv = p[r] >> 4;        // B codes entered the MFMA as 16*q
          if (FS) xa[(gb + u) * NR * kWave + (rb * 4 + r) * kWave + lane] = pv;
          else acc[rb * 4 + r] = mad24(pv, is[u], acc[rb * 4 + r]);
        }
      }
      if (FS && s4 == 0) reinterpret_cast<float*>(xa + G * NR * kWave)[(gb + u) * 16 + c] = fs[u];
    }
    if (!FS) {
#pragma unroll
      for (int r = 0; r < NR; ++r) xa[(wave * NR + r) * kWave + lane] = acc[r];
    }
    __syncthreads();
  };

  uint4 bA[GPW], bB[GPW];
  int iA[GPW], iB[GPW];
  float fA[GPW], fB[GPW];
  int t = blockIdx.x, it = 0;
  issue(t, bA, iA, fA);
  while (t < T) {
    issue(t + P, bB, iB, fB);
    contract(it, bA, iA, fA);
    ++it;
    t += P;
    if (t >= T) break;
    issue(t + P, bA, iA, fA);
    contract(it, bB, iB, fB);
    ++it;
    t += P;
  }
}

// =====================================================================
// Prefill kernel (large M, compute-bound): BM x BN output tile per
// workgroup of WM x WN waves (two waves per SIMD), each wave 2 x 2 blocks of
// 32 x 32 (v_mfma_i32_32x32x32_i8). One K step is one group of 128.
//   A: the waves copy the BM x 128 int8 tile straight into LDS
//      (global_load_lds_dwordx4: lane L of an instruction fills bytes
//      16L..16L+15 of a 1 KiB block = 8 rows); rows are stored unpadded with
//      their 16-byte chunks XOR-swizzled by (row / 2) % 8: a row spans 32 of
//      the 64 banks (rows of one parity share them), so within any 16
//      consecutive rows each (parity, chunk) pair is distinct and a 16-lane
//      read phase of an MFMA operand fetch is conflict-free. The group's scales follow.
//   B: each lane copies one 16-byte packed int4 chunk into LDS, later
//      unpacks that same chunk to true int8 and writes it to the unpacked B
//      stage ([column][128 k], padded rows).
// Pipeline: three A/packed stages and two unpacked B stages. Step l runs the
// MFMAs of group l in four blocks; between blocks 1 and 2 the waves unpack
// group l+1, meet at a barrier and request group l+3. The operand fragments
// of group l+1 are read from LDS under the MFMAs of blocks 2, 3 of step l and
// blocks 0, 1 of step l+1, and each block's scale epilogue runs under the
// next block's MFMAs.
// Integer-scale epilogue per group: acc += p * iscale (24-bit multiply-add,
// exact mod 2^32); float-scale control: acc = fma((float)p, fscale, acc).
// Workgroups are mapped so consecutive tiles of one XCD (WG id % 8) share
// weight columns and activation rows in that XCD's L2.
// =====================================================================
constexpr int kBRow = 144;   // LDS bytes per unpacked B column: 128 + 16 pad


// 16-byte LDS read of data that this lane's own LDS copy wrote, after the
// caller's s_waitcnt on vmcnt. Written as one asm block that waits for its
// own result, so the compiler does not add a wait for every copy in flight
// (it cannot tell the copy stages apart and would drain them all).
__device__ __forceinline__ uint4 lds_read_own_copy(const uint4* p) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const uint32_t a = lds_addr(p);
  u4v v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a));
  return make_uint4(v.x, v.y, v.z, v.w);
}


template <int WM, int WN, int TMW, int TNW, bool FS, typename ST, bool GR = false>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_w4a8_prefill(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint4* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K, int ldn,
    OutY y, int32_t* __restrict__ acc_out, Route rt, int splits, int32_t* __restrict__ part) {
  static_assert(TMW == 2 && TNW == 2, "four 32 x 32 blocks per wave");
  constexpr int NW = WM * WN, NT = NW * 64;
  constexpr int BM = WM * TMW * 32, BN = WN * TNW * 32, NB = TMW * TNW;
  constexpr int A_INSTR = BM / (8 * NW);            // 1 KiB (8-row) blocks per wave per group
  constexpr int B_CH = BN * 4 / NT;                 // packed 16-byte chunks per thread per group
  constexpr int LOADS = A_INSTR + 1 + B_CH;         // LDS copies per group per wave
  static_assert(A_INSTR >= 1 && B_CH >= 1 && BN <= NT, "tile too small for the workgroup");
  static_assert(BN % 64 == 0 && NW >= BN / 64, "scales: one 64-column slice per wave");
  constexpr int A_BYTES = BM * 128, STAGE = A_BYTES + BN * 4;
  __shared__ __align__(16) int8_t SA0[STAGE];
  __shared__ __align__(16) int8_t SA1[STAGE];
  __shared__ __align__(16) int8_t SA2[STAGE];
  __shared__ __align__(16) int8_t SB0[BN * kBRow];
  __shared__ __align__(16) int8_t SB1[BN * kBRow];
  __shared__ __align__(16) uint4 SP0[BN * 4];
  __shared__ __align__(16) uint4 SP1[BN * 4];
  __shared__ __align__(16) uint4 SP2[BN * 4];

  // split K (integer scale only): workgroup id = ks * tiles + tile; split ks
  // runs groups g0 .. g0+G-1 = [ks*GT/splits, (ks+1)*GT/splits) and leaves its
  // integer-scaled int32 sums in part[ks] (M x N) for k_split_reduce
  const int GT = K / kGroup, T = N / 16;
  const int ntiles = (int)gridDim.x / splits;
  const int ks = (int)blockIdx.x / ntiles, tb = (int)blockIdx.x - ks * ntiles;
  const int g0 = (int)((int64_t)ks * GT / splits);
  const int G = (int)((int64_t)(ks + 1) * GT / splits) - g0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, hf = lane / 32;
  int tm, tn;
  // grouped GEMM: the grid covers ceil(R/BM) + E row tiles, an upper bound on
  // the sum over experts of ceil(rows/BM); the experts' row tiles (experts in
  // order) are dealt evenly over the XCDs and the spare workgroups exit
  int r0 = 0;
  if constexpr (GR) {
    int e, a, rows;
    if (!grouped_tile(tb, BM, (N + BN - 1) / BN, rt, e, a, rows, tm, tn)) return;
    M = rows;
    r0 = a;
    packed += e * rt.wstride / 16;
    if (FS) fscale += e * rt.sstride;
    else iscale += e * rt.sstride;
  } else {
    tile_of(tb, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- copies of one group (a group index past the end is clamped to the
  // last group: those copies land in a free stage and are never read, and
  // they keep the number of copies per step fixed for the wait counts)
  // A: lane L of block b fills row 8b + L/8, chunk slot L%8, with the row's
  // global chunk (L%8) ^ ((row / 2) % 8), row = 8b + L/8.
  // (grouped: the slot's activation row, as a 64-bit offset from X)
  using AO = typename std::conditional<GR, int64_t, int>::type;
  const int8_t* abase = GR ? qx : qx + (int64_t)m0 * K;
  AO aoff[A_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    const int r = 8 * (i * NW + wave) + lane / 8;
    const int rr = m0 + r < M ? r : M - 1 - m0;
    const AO ro = GR ? (AO)clamp_route(rt.tok[r0 + m0 + rr], 0, rt.T - 1) * K : (AO)rr * K;
    aoff[i] = ro + 16 * ((lane % 8) ^ ((r >> 1) & 7));
  }
  // scales: wave w copies the 64-column slice w % (BN/64) into a 256-byte
  // slot (several waves write the same slice with the same values); each lane
  // copies 4 bytes = CPL scale elements. With narrow elements (CPL > 1) the
  // lanes past the slice, and any lane past N, copy clamped in-bounds columns
  // into the unused rest of the slot.
  using SL = typename std::conditional<FS, int32_t, ST>::type;   // scale element as stored
  constexpr int SB = sizeof(SL), CPL = 4 / SB;
  static_assert(SB == 1 || SB == 2 || SB == 4, "scale element of 1, 2 or 4 bytes");
  const char* ssrc = FS ? reinterpret_cast<const char*>(fscale) : reinterpret_cast<const char*>(iscale);
  const int sslot = wave % (BN / 64);
  const int scol = n0 + sslot * 64 + lane * CPL;
  const int soff = scol <= N - CPL ? scol : N - CPL;
  // B: chunk q = tid + NT*u of the tile's packed group block
  const uint4* bsrc[B_CH];
#pragma unroll
  for (int u = 0; u < B_CH; ++u) {
    const int q = tid + NT * u, tl = q / 64, lb = q % 64;
    const int tg = n0 / 16 + tl < T ? n0 / 16 + tl : T - 1;
    bsrc[u] = packed + (int64_t)tg * GT * 64 + lb;
  }
  auto issue_group = [&](int g, int8_t* SA, uint4* SP) {
    const int gc = (g < G ? g : G - 1) + g0;
    const int8_t* base = abase + (int64_t)gc * kGroup;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(base + aoff[i]),
          (__attribute__((address_space(3))) void*)(SA + (i * NW + wave) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(ssrc + ((int64_t)gc * ldn + soff) * SB),
        (__attribute__((address_space(3))) void*)(SA + A_BYTES + sslot * 256), 4, 0, 0);
#pragma unroll
    for (int u = 0; u < B_CH; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bsrc[u] + (int64_t)gc * 64),
          (__attribute__((address_space(3))) void*)(SP + (u * NW + wave) * 64), 16, 0, 0);
  };
  // unpack this lane's own packed chunk(s) into the int8 B stage
  auto store_b = [&](const uint4* SP, int8_t* SB) {
#pragma unroll
    for (int u = 0; u < B_CH; ++u) {
      const int q = tid + NT * u, tl = q / 64, lb = q % 64, s = lb / 16, cc = lb % 16;
      const uint4 w = lds_read_own_copy(SP + q);
      uint32_t l0, h0, l1, h1, l2, h2, l3, h3;
      unpack_i8(w.x, l0, h0);
      unpack_i8(w.y, l1, h1);
      unpack_i8(w.z, l2, h2);
      unpack_i8(w.w, l3, h3);
      int8_t* dst = SB + (tl * 16 + cc) * kBRow + 16 * s;
      *reinterpret_cast<uint4*>(dst) = make_uint4(l0, h0, l1, h1);        // k = 16s + 0..15
      *reinterpret_cast<uint4*>(dst + 64) = make_uint4(l2, h2, l3, h3);   // k = 64 + 16s + 0..15
    }
  };

  // ---- operand fragments (32 rows or columns, K order 64*hf + 16*m + e)
  v4i av[TMW][4], bv[TNW][4];
  int32_t scb[TNW], scn[TNW], spc = 0;
  auto read_av = [&](int a, const int8_t* SA) {
    const int row = wm * (TMW * 32) + a * 32 + lr;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      av[a][m] = *reinterpret_cast<const v4i*>(SA + row * 128 + 16 * ((4 * hf + m) ^ ((row >> 1) & 7)));
  };
  auto read_bv = [&](int b, const int8_t* SB) {
    const int cl = wn * (TNW * 32) + b * 32 + lr;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      bv[b][m] = *reinterpret_cast<const v4i*>(SB + cl * kBRow + 64 * hf + 16 * m);
  };
  auto read_sc = [&](const int8_t* SA, int32_t (&sc)[TNW]) {
    // one aligned dword read per scale; narrow elements are shifted out of it
    const uint32_t* S = reinterpret_cast<const uint32_t*>(SA + A_BYTES);
#pragma unroll
    for (int b = 0; b < TNW; ++b) {
      const int col = wn * (TNW * 32) + b * 32 + lr;           // column within the tile
      const int byte = (col / 64) * 256 + (col % 64) * SB;      // slot col/64
      const uint32_t w = S[byte / 4];
      sc[b] = SB == 4 ? (int32_t)w : (int32_t)((w >> (8 * (byte % 4))) & ((1u << (8 * SB)) - 1u));
      // hide the narrow value range: with it the compiler rewrites the 24-bit
      // multiply-adds and re-associates them across groups (register blow-up)
      if (SB != 4) opaque_reg(sc[b]);
    }
  };

  int acc[NB][16];
  float facc[NB][16];
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc[k][r] = 0; facc[k][r] = 0.0f; }

  // block k: MFMA chain over the group's 128 k while the VALU applies the
  // scale to block k-1's partials (1 MFMA : 4 VALU); `pre` issues LDS reads
  // of fragments needed later. The last block's partials carry into the next
  // step (pc[1]).
  v16i pc[2] = {v16i{0}, v16i{0}};
  auto epilogue = [&](auto kk, const v16i& p, int32_t sc) {
    constexpr int k = decltype(kk)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (FS) facc[k][r] = __builtin_fmaf((float)p[r], __int_as_float(sc), facc[k][r]);
      else acc[k][r] = mad24(p[r], sc, acc[k][r]);
    }
  };
  auto block = [&](auto kk, const v4i (&a)[4], const v4i (&b)[4], int32_t sc_prev, auto pre) {
    constexpr int k = decltype(kk)::value;
    constexpr int kp = (k + NB - 1) % NB;
    v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], v16i{0}, 0, 0, 0);
#pragma unroll
    for (int m = 1; m < 4; ++m) p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[m], b[m], p, 0, 0, 0);
    epilogue(IC<kp>{}, pc[(k + 1) % 2], sc_prev);
    pc[k % 2] = p;
    pre();
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);     // LDS reads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
      if (i < 3) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- step l; L6 = l mod 6 fixes the stages at compile time: A/packed
  // stage l % 3, unpacked B stage l % 2.
  auto step = [&](int l, auto l6) {
    constexpr int L6 = decltype(l6)::value;
    constexpr int s0 = L6 % 3, s1 = (L6 + 1) % 3, b1 = (L6 + 1) % 2, b0 = L6 % 2;
    int8_t* A0 = s0 == 0 ? SA0 : (s0 == 1 ? SA1 : SA2);
    int8_t* A1 = s1 == 0 ? SA0 : (s1 == 1 ? SA1 : SA2);
    uint4* P0 = s0 == 0 ? SP0 : (s0 == 1 ? SP1 : SP2);
    uint4* P1 = s1 == 0 ? SP0 : (s1 == 1 ? SP1 : SP2);
    int8_t* B0 = b0 == 0 ? SB0 : SB1;
    int8_t* B1 = b1 == 0 ? SB0 : SB1;
    block(IC<0>{}, av[0], bv[0], spc, [&] { read_bv(1, B0); });
    block(IC<1>{}, av[0], bv[1], scb[0], [&] { read_av(1, A0); });
    // group l+1: own copies landed (group l+2 may still be in flight), unpack
    // its B, all LDS traffic of this wave done, barrier; then request l+3
    // into the stage group l leaves
    wait_vm<LOADS>();
    store_b(P1, B1);
    wait_vm_lds0<LOADS>();
    lds_barrier();
    issue_group(l + 3, A0, P0);
    block(IC<2>{}, av[1], bv[0], scb[1], [&] { read_av(0, A1); read_sc(A1, scn); });
    block(IC<3>{}, av[1], bv[1], scb[0], [&] { read_bv(0, B1); });
    spc = scb[1];
#pragma unroll
    for (int b = 0; b < TNW; ++b) scb[b] = scn[b];
  };

  // ---- prologue: groups 0, 1, 2 requested; group 0 unpacked and its first
  // fragments read
  issue_group(0, SA0, SP0);
  issue_group(1, SA1, SP1);
  issue_group(2, SA2, SP2);
  wait_vm<2 * LOADS>();
  store_b(SP0, SB0);
  wait_vm_lds0<2 * LOADS>();
  lds_barrier();
  read_av(0, SA0);
  read_sc(SA0, scb);
  read_bv(0, SB0);

  for (int l = 0; l < G; l += 6) {
    step(l + 0, IC<0>{});
    if (l + 1 >= G) break;
    step(l + 1, IC<1>{});
    if (l + 2 >= G) break;
    step(l + 2, IC<2>{});
    if (l + 3 >= G) break;
    step(l + 3, IC<3>{});
    if (l + 4 >= G) break;
    step(l + 4, IC<4>{});
    if (l + 5 >= G) break;
    step(l + 5, IC<5>{});
  }
  epilogue(IC<NB - 1>{}, pc[(NB - 1) % 2], spc);
  wait_vm_lds0<0>();                                // surplus copies of the last steps

  if (!FS && part != nullptr) {                     // split K: this split's sums
    int32_t* pp = part + (int64_t)ks * M * N;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int a = k / TNW, b = k % TNW;
      const int j = n0 + wn * (TNW * 32) + b * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * (TMW * 32) + a * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (i < M && j < N) pp[(int64_t)i * N + j] = acc[k][r];
      }
    }
    return;
  }

  // ---- one conversion per output. The lane's 32 token scales are loaded
  // first (row indices clamped), so the stores below need no waits; full
  // tiles store without per-element predicates.
  float srow[TMW][16];
#pragma unroll
  for (int a = 0; a < TMW; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * (TMW * 32) + a * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
      const int ic = i < M ? i : M - 1;
      srow[a][r] = sx[GR ? clamp_route(rt.tok[r0 + ic], 0, rt.T - 1) : ic];
    }
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int a = k / TNW, b = k % TNW;
    const int j = n0 + wn * (TNW * 32) + b * 32 + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * (TMW * 32) + a * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
      if (!full && (i >= M || j >= N)) continue;
      const int64_t o = (int64_t)(r0 + i) * ldn + j;
      if (FS) {
        y.put_nt(o, facc[k][r] * srow[a][r]);
      } else {
        const float t0 = (float)acc[k][r] * srow[a][r];
        y.put_nt(o, t0 * inv_alpha);
        if (acc_out) __builtin_nontemporal_store(acc[k][r], acc_out + o);
      }
    }
  }
}

// Split-K reduction of the 256 x 128 tile kernel: out = sum of the splits'
// integer-scaled int32 sums (exact mod 2^32 in any order), then the one
// conversion per output as in the GEMM epilogue. Four consecutive outputs
// (one row: N is a multiple of 16) per thread.
__global__ __launch_bounds__(256) void k_split_reduce(const int32_t* __restrict__ part, int splits,
                                                      int64_t MN, int N, int ldn,
                                                      const float* __restrict__ sx,
                                                      float inv_alpha, OutY y,
                                                      int32_t* __restrict__ acc_out) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= MN) return;
  v4i a = *reinterpret_cast<const v4i*>(part + e);
  for (int k = 1; k < splits; ++k) a += *reinterpret_cast<const v4i*>(part + k * MN + e);
  const int64_t i = e / N, o = i * ldn + (e - i * N);   // part is M x N, y rows ldn apart
  const float si = sx[i];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float t0 = (float)a[r] * si;
    y.put(o + r, t0 * inv_alpha);
  }
  if (acc_out) *reinterpret_cast<v4i*>(acc_out + o) = a;
}

// =====================================================================
// Asymmetric W8A8 control through the zero-point expansion: 64 x 64 output
// tiles, 8 waves. Every load is an LDS copy (global_load_lds) of 1 KiB
// blocks (8 rows x 128 k, 16-byte chunks XOR-swizzled by (row/2) % 8 so the
// 32 x 32 x 32 fragment reads are conflict-free); nine copy stages of 128 k
// (A and B rows), eight in flight, each its own array so the compiler's wait
// counts stay per stage. Waves 0-3 and 4-7 take the two 64-k halves of a
// stage on the same 2 x 2 arrangement of 32 x 32 blocks; the halves meet
// once through LDS before the epilogue. uint8 codes enter the int8 MFMA
// re-centred by 128 (xor 0x80), and the epilogue expands with the re-centred
// zero points and row sums (the same differences), exact mod 2^32.
// =====================================================================
constexpr int kW8Waves = 8;                        // waves per W8A8 workgroup

template <int NST, int GC, int NW>
__global__ __launch_bounds__(NW * 64) void k_w8a8_zp(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, const int32_t* __restrict__ zx,
    const int32_t* __restrict__ rowsum_x, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, const int32_t* __restrict__ zw,
    const int32_t* __restrict__ colsum_w, int M, int N, int K, OutY y,
    int32_t* __restrict__ acc_out) {
  static_assert(NST == 9, "nine copy stages");
  static_assert(NW == 8 || NW == 16, "8 or 16 waves: 2 or 4 k slices of the 2 x 2 blocks");
  // GC > 0: K / 128 fixed at compile time, the step loop unrolls completely
  // (a loop header would make the compiler wait for every copy in flight)
  constexpr int BM = 64, BN = 64, STG = (BM + BN) * 128;
  constexpr int KSPL = NW / 4;                       // k slices of a stage
  constexpr int MPW = 4 / KSPL;                      // 32-k MFMA steps per wave per stage
  constexpr int LOADS = 16 / NW;                     // 1 KiB copies per stage per wave
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

  // copies: the 16 blocks of a stage (A rows 8b..8b+7 for b < 8, then B)
  // are spread over the waves, LOADS each; lane L of block b fills row
  // 8(b%8) + L/8, chunk slot L%8, with the row's global chunk
  // (L%8) ^ ((row/2) % 8); rows past M or N re-read the last row
  const uint8_t* src[LOADS];
  int dst[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int b = wave * LOADS + u, isb = b / 8, r8 = 8 * (b % 8) + lane / 8;
    const int ck = 16 * ((lane % 8) ^ ((r8 >> 1) & 7));
    src[u] = isb == 0 ? qx + (int64_t)(m0 + r8 < M ? m0 + r8 : M - 1) * K + ck
                      : qw + (int64_t)(n0 + r8 < N ? n0 + r8 : N - 1) * K + ck;
    dst[u] = isb * BM * 128 + (b % 8) * 1024;
  }
  auto issue = [&](int g, int8_t* S) {
    const int gc = g < G ? g : G - 1;              // past the end: a surplus copy, never read
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[u] + (int64_t)gc * kGroup),
          (__attribute__((address_space(3))) void*)(S + dst[u]), 16, 0, 0);
  };

  v16i acc = v16i{0};
  const int ra = wm * 32 + lr, rb = wn * 32 + lr;
  auto compute = [&](const int8_t* S) {
    v4i av[MPW], bv[MPW];
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm) {
      const int m = MPW * kh + mm;
      av[mm] = *reinterpret_cast<const v4i*>(S + ra * 128 + 16 * ((4 * hf + m) ^ ((ra >> 1) & 7)));
      bv[mm] = *reinterpret_cast<const v4i*>(S + BM * 128 + rb * 128 + 16 * ((4 * hf + m) ^ ((rb >> 1) & 7)));
    }
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm) {
      const v4i c80 = {(int)0x80808080, (int)0x80808080, (int)0x80808080, (int)0x80808080};
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mm] ^ c80, bv[mm] ^ c80, acc, 0, 0, 0);
    }
  };
  // step l (slot J = l % NST): stage l landed in every wave, then request
  // stage l + NST - 1 into the slot stage l - 1 used
  auto step = [&](int l, auto j) {
    constexpr int J = decltype(j)::value;
    wait_vm_lds0<(NST - 2) * LOADS>();
    lds_barrier();
    issue(l + NST - 1, stage(IC<(J + NST - 1) % NST>{}));
    compute(stage(IC<J>{}));
  };
  issue(0, S0);
  issue(1, S1);
  issue(2, S2);
  issue(3, S3);
  issue(4, S4);
  issue(5, S5);
  issue(6, S6);
  issue(7, S7);
#pragma unroll
  for (int l = 0; l < G; l += NST) {
    step(l + 0, IC<0>{});
    if (l + 1 >= G) break;
    step(l + 1, IC<1>{});
    if (l + 2 >= G) break;
    step(l + 2, IC<2>{});
    if (l + 3 >= G) break;
    step(l + 3, IC<3>{});
    if (l + 4 >= G) break;
    step(l + 4, IC<4>{});
    if (l + 5 >= G) break;
    step(l + 5, IC<5>{});
    if (l + 6 >= G) break;
    step(l + 6, IC<6>{});
    if (l + 7 >= G) break;
    step(l + 7, IC<7>{});
    if (l + 8 >= G) break;
    step(l + 8, IC<8>{});
  }
  // the k slices meet: slices 1..KSPL-1 park their sums in the (now free)
  // stages 0..KSPL-2, slice 0 adds them
  wait_vm_lds0<0>();
  lds_barrier();
  if (kh > 0) {
    int32_t* R = reinterpret_cast<int32_t*>(kh == 1 ? S0 : (kh == 2 ? S1 : S2));
#pragma unroll
    for (int r = 0; r < 16; ++r) R[((wave % 4) * 16 + r) * 64 + lane] = acc[r];
  }
  wait_lds0();
  lds_barrier();
  if (kh > 0) return;
#pragma unroll
  for (int q = 1; q < KSPL; ++q) {
    const int32_t* R = reinterpret_cast<const int32_t*>(q == 1 ? S0 : (q == 2 ? S1 : S2));
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += R[((wave % 4) * 16 + r) * 64 + lane];
  }

  const int j = n0 + rb;
  if (j >= N) return;
  // the lane's 16 rows' terms are loaded together first (rows past M clamped),
  // so the stores below wait for nothing
  const int32_t zwj = zw[j] - 128, cwj = colsum_w[j] - 128 * K;
  const float swj = sw[j];
  int32_t zxr[16], rxr[16];
  float sxr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = m0 + wm * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
    const int ic = i < M ? i : M - 1;
    zxr[r] = zx[ic];
    rxr[r] = rowsum_x[ic];
    sxr[r] = sx[ic];
  }
  // acc = sum (qw-128)(qx-128); expand (qw - zw)(qx - zx) with the re-centred
  // codes and zero points (same differences), all exact mod 2^32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = m0 + wm * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
    if (i >= M) continue;
    const int32_t zxi = zxr[r] - 128, rxi = rxr[r] - 128 * K;
    const int32_t A = acc[r] - zwj * rxi - zxi * cwj + K * zwj * zxi;
    const float sc = sxr[r] * swj;
    const int64_t o = (int64_t)i * N + j;
    y.put(o, (float)A * sc);
    if (acc_out) acc_out[o] = A;
  }
}

// =====================================================================
// Decode kernel (M <= 64, weight streaming): one wave owns one 16-column tile
// for all K and MR/RS of the MR 16-row blocks of X (RS waves share a tile, each
// streaming its weights), so no partial sums cross waves; a workgroup of W*RS
// waves serves W consecutive tiles.
//   X: the workgroup stages X (16*MR rows, clamped past M) in LDS in MFMA
//      fragment order, one K chunk of CG groups (at most 64 KiB) at a time,
//      double-buffered: fragment (g, rb, h) of a chunk = 1 KiB where lane L
//      holds row 16rb + L%16, k = 128g + 64h + 16(L/16) .. +15. The next
//      chunk's rows are loaded into registers under the current chunk's work;
//      the chunk's fragments are dealt round-robin to the W*RS waves.
//   W: each wave keeps D packed 1 KiB group blocks of its tile (16 bytes per
//      lane, non-temporal) and their D scales in flight, refilling one slot
//      per group; unpack by nibble-to-high-half (codes enter as 16*q), two
//      v_mfma_i32_16x16x64_i8 per group and row block, partial >> 4, then the
//      group's integer scale by v_mad_i32_i24 (float-scale control: the
//      ascending fma chain).
// Every load is a register load, so the compiler's wait counts stay exact.
// =====================================================================
// groups per staged X chunk: the largest divisor of G up to 32 (one row
// block; 16 on 2-wave workgroups, so a wave stages at most 16 fragments,
// unless the rows are quantized in the kernel and written to LDS directly)
// or 8 (more), so a chunk is at most 64 KiB, that is a multiple of the weight
// ring depth D; NW = the workgroup's waves
// the largest divisor of n up to d (groups in flight of a wave's n groups)
constexpr int ring_depth(int n, int d) {
  int r = d < n ? d : n;
  while (n % r != 0) --r;
  return r;
}

constexpr int decode_chunk_groups(int G, int MR, int D, int NW, bool FQ) {
  int c = MR == 1 ? (NW >= 4 || FQ ? 32 : 16) : 8;
  while (c > D && (G % c != 0 || c % D != 0)) --c;
  return c;
}

template <bool FS, int W, int D, int G, int MR, typename ST, bool FQ, int IT, bool GR = false,
          int GQ = G, int RS = 1, int KS = 1, bool CX = false>
__global__ __launch_bounds__(W * RS * KS * 64) void k_w4a8_decode(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint4* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N,
    OutY y, int32_t* __restrict__ acc_out,
    const void* __restrict__ xf, int ldx, int8_t* __restrict__ q_out, float* __restrict__ s_out,
    Route rt) {
  constexpr int NWV = W * RS * KS;                   // waves of the workgroup
  constexpr int CG = decode_chunk_groups(G, MR, D, NWV, FQ);  // groups per X chunk (<= 64 KiB)
  constexpr int NCH = G / CG;                        // chunks
  constexpr int CFR = CG * MR * 2;                   // 1 KiB fragments per chunk
  constexpr int MRW = MR / RS;                       // row blocks per wave
  constexpr int FPW = (CFR + NWV - 1) / NWV;         // fragments per wave per chunk (the last may be short)
  using SL = typename std::conditional<FS, int32_t, ST>::type;   // scale element as stored
  constexpr int SCW = W * 16;                        // scale columns of the workgroup
  constexpr int SEL = 16 / sizeof(SL);               // scale elements per 16-byte chunk
  constexpr int SCT = G * SCW / SEL;                 // 16-byte scale chunks of the workgroup
  constexpr int SCH = (SCT + NWV * 64 - 1) / (NWV * 64); // ... per thread
  static_assert(G % D == 0 && G % CG == 0, "shape of the pipeline");
  static_assert(SCW % SEL == 0, "scale staging");
  static_assert(!FQ || (MR == 1 && (NCH == 1 || CX) && !FS),
                "fused quantization: one row block, one chunk (or compact rows)");
  static_assert(!CX || FQ, "compact rows: quantized in the kernel");
  static_assert(!(GR && FQ), "grouped GEMM takes quantized activations");
  static_assert(RS >= 1 && MR % RS == 0 && (RS == 1 || (!FQ && !GR)), "row split: dense launches");
  static_assert(KS == 1 || (RS == 1 && MR == 1 && (NCH == 1 || CX) && !FS && !GR && G % KS == 0),
                "K split: one row block and one X chunk (or compact rows), integer scale");
  constexpr int GK = G / KS;                         // groups per wave
  constexpr int DK = ring_depth(GK, D);              // ... of them in flight
  constexpr int NBUF = NCH > 1 ? 2 : 1;
  // X in LDS: MFMA fragment order, one or two chunks; compact rows (CX): the
  // (at most four) quantized rows, row r at byte r*K, fragments gathered at
  // read time (rows past M read row M-1; their outputs are not stored)
  __shared__ __align__(16) int8_t sA[CX ? 4 * GQ * kGroup : NBUF * CFR * 1024];
  __shared__ __align__(16) SL sS[G * SCW];           // [group][column of the workgroup]
  __shared__ float sX[16 * MR];                      // token scales
  // G groups in the pipeline; the last G - GQ are padding (K = 128 GQ): their
  // loads repeat group GQ-1 and their staged scales are zero, so they add
  // exactly nothing (0 * p in the integer epilogue, fma(p, +0, acc) = acc)
  static_assert(GQ <= G && (GQ == G || CX || (!FQ && !GR)), "padded groups: dense launches only");
  constexpr int K = GQ * kGroup;
  auto gq = [](int g) { return GQ == G || g < GQ ? g : GQ - 1; };
  const int T = N / 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int c = lane % 16, s4 = lane / 16;
  // tile of the workgroup, row-block share, K share
  const int tw = wave % W, hr = (wave / W) % RS, ks = wave / (W * RS);
  const int t = blockIdx.x * W + tw;
  const bool tvalid = t < T;
  const int tc = tvalid ? t : T - 1;

  // grouped GEMM: this workgroup serves expert blockIdx.y, row pass
  // blockIdx.z: the expert's slots r0 .. r0+M-1 with r0 = first slot +
  // 16*MR*z (the 16*MR rows of a workgroup); an expert or a pass without
  // slots reads nothing
  int r0 = 0;
  if constexpr (GR) {
    const int e = blockIdx.y;
    const int ra = clamp_route(rt.offs[e], 0, rt.R);
    const int rb = clamp_route(rt.offs[e + 1], ra, rt.R);
    r0 = ra + (int)blockIdx.z * 16 * MR;
    if (r0 >= rb) return;
    M = rb - r0 < 16 * MR ? rb - r0 : 16 * MR;
    packed += e * rt.wstride / 16;
    if (FS) fscale += e * rt.sstride;
    else iscale += e * rt.sstride;
  }

  // ---- X chunk staging: this wave's fragments f = wave + NWV*i of chunk ch
  // (32-bit offsets from the X base; grouped: the rows of the expert's slots,
  // looked up once)
  int xo[GR ? FPW : 1];
  if constexpr (GR) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const int f = wave + NWV * i, rb = (f / 2) % MR;
      const int row = 16 * rb + c < M ? 16 * rb + c : M - 1;
      xo[i] = (CFR % NWV == 0 || f < CFR) ? clamp_route(rt.tok[r0 + row], 0, rt.T - 1) * K : 0;
    }
  }
  v4i xa[FPW];
  auto load_chunk = [&](int ch) {
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const int f = wave + NWV * i, gl = f / (2 * MR), rb = (f / 2) % MR, h = f % 2;
      const int row = 16 * rb + c < M ? 16 * rb + c : M - 1;
      const int ro = GR ? xo[GR ? i : 0] : row * K;
      if (CFR % NWV == 0 || f < CFR)                 // wave-uniform
        xa[i] = load_v4i(qx + (ro + 128 * gq(ch * CG + gl) + 64 * h + 16 * s4));
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      if (CFR % NWV == 0 || wave + NWV * i < CFR)
        *reinterpret_cast<v4i*>(sA + (buf * CFR + wave + NWV * i) * 1024 + lane * 16) = xa[i];
  };
  // fused quantization (FQ, M <= 4): the rows (element type IT, widened to
  // fp32), each thread XV groups of 4 of every row (the last one partial when
  // K/4 is not a multiple of the workgroup's threads: the groups past the
  // row's end count for nothing), requested before the scales and the weights
  constexpr int XV = FQ ? (K / 4 + NWV * 64 - 1) / (NWV * 64) : 1;
  constexpr bool XR = FQ && XV * NWV * 64 * 4 != K;
  auto xin = [&](int v) { return !XR || v < XV - 1 || (int)threadIdx.x + NWV * 64 * v < K / 4; };
  // (the rows are read as stored, every load unconditional, from the row
  // start past the row's end, and widened only after the weights are
  // requested: a load under a lane condition, or converted in its own block,
  // makes the compiler wait for it before the next, one round trip each)
  typename XRaw<IT>::T xr[4][XV];
  if constexpr (FQ) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < XV; ++v)
        if (i < M)
          xr[i][v] = reinterpret_cast<const typename XRaw<IT>::T*>(xf)[
              (int64_t)i * (ldx / 4) + (xin(v) ? threadIdx.x + NWV * 64 * v : 0)];
  } else {
    load_chunk(0);
  }
  // token scales of the (at most 64) rows, read back from LDS at the end;
  // requested before the weights so that storing them waits for no weight
  float sxi = 0.0f;
  if constexpr (!FQ) {
    const int ti = threadIdx.x < M ? threadIdx.x : M - 1;
    const int tr = GR ? clamp_route(rt.tok[r0 + ti], 0, rt.T - 1) : ti;
    if (threadIdx.x < 16 * MR) sxi = sx[tr];
  }
  // ---- the workgroup's scales for all groups, 16-byte chunks of SEL
  // elements (columns past N clamped; chunk q lands at byte 16q of sS)
  const SL* scl = FS ? reinterpret_cast<const SL*>(fscale) : reinterpret_cast<const SL*>(iscale);
  // (loads unconditional from an in-bounds group, the padding's zeros selected
  // afterwards, as for the rows above; chunks past SCT are never stored)
  v4i sv[SCH];
#pragma unroll
  for (int u = 0; u < SCH; ++u) {
    const int q = threadIdx.x + NWV * 64 * u, g = q / (SCW / SEL), c0 = (q % (SCW / SEL)) * SEL;
    const int col = blockIdx.x * SCW + c0 < N ? blockIdx.x * SCW + c0 : N - SEL;
    const int gl = g < GQ ? g : GQ - 1;
    sv[u] = load_v4i(reinterpret_cast<const int8_t*>(scl + ((int64_t)gl * N + col)));
  }
#pragma unroll
  for (int u = 0; u < SCH; ++u) {
    const int q = threadIdx.x + NWV * 64 * u, g = q / (SCW / SEL);
    if (GQ < G && g >= GQ) sv[u] = v4i{0, 0, 0, 0};
  }
  // ---- first D groups of the tile in flight (K split: of this wave's GK
  // groups from g0w, DK in flight)
  const uint4* wsrc = packed + (int64_t)tc * GQ * 64 + lane;
  const int g0w = ks * GK;
  uint4 wb[DK];
#pragma unroll
  for (int j = 0; j < DK; ++j) wb[j] = load_u4_nt(wsrc + (int64_t)gq(g0w + j) * 64);
  if constexpr (FQ) {
    // ---- per-token quantization of the rows, as the quantizer computes it:
    // a = max|x|, s = a / 127, q = clamp(round(x / s), -127, 127) (s = 0 -> 0).
    // x / s is Markstein's corrected quotient (P. Markstein, IBM J. Res. Dev.
    // 1990): with r = 1/s correctly rounded, q0 = x*r, e = fma(-q0, s, x)
    // (exact), fma(e, r, q0) is x / s correctly rounded while s, r and the
    // residual stay normal; rows with an extreme scale take the division.
    __shared__ float sAm[4 * NWV];
    float4 xv[4][XV];
    float am[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      am[i] = 0.0f;
      if (i < M)
#pragma unroll
        for (int v = 0; v < XV; ++v) {
          xv[i][v] = widen_x4<IT>(xr[i][v]);        // past the row's end: not counted, not stored
          const float a = fmaxf(fmaxf(fabsf(xv[i][v].x), fabsf(xv[i][v].y)),
                                fmaxf(fabsf(xv[i][v].z), fabsf(xv[i][v].w)));
          am[i] = fmaxf(am[i], xin(v) ? a : 0.0f);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)                 // the four rows' butterflies side by side
#pragma unroll
      for (int i = 0; i < 4; ++i) am[i] = fmaxf(am[i], __shfl_xor(am[i], o, kWave));
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) sAm[i * NWV + wave] = am[i];
    // rows M..15 of the fragment block are zero codes
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      if (!CX && c >= M && (CFR % NWV == 0 || wave + NWV * i < CFR))
        *reinterpret_cast<v4i*>(sA + (wave + NWV * i) * 1024 + lane * 16) = v4i{0, 0, 0, 0};
    wait_lds0();
    lds_barrier();
    // codes of one float4: MODE 0 all zero (s = 0), 1 corrected product, 2 division
    auto quant4 = [&](const float4& x, float sc, float r, auto mode) -> uint32_t {
      constexpr int MODE = decltype(mode)::value;
      if (MODE == 0) return 0u;
      auto one = [&](float e) -> uint32_t {
        float q;
        if (MODE == 1) {
          const float q0 = e * r;
          q = __builtin_fmaf(__builtin_fmaf(-q0, sc, e), r, q0);
        } else {
          q = e / sc;
        }
        return (uint32_t)clamp_int((int)round_away(q), -127, 127) & 0xFFu;
      };
      return one(x.x) | (one(x.y) << 8) | (one(x.z) << 16) | (one(x.w) << 24);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < M) {
        float a = sAm[i * NWV];
#pragma unroll
        for (int w = 1; w < NWV; ++w) a = fmaxf(a, sAm[i * NWV + w]);
        const float sc = a / 127.0f;
        const float r = 1.0f / sc;
        if (threadIdx.x == i) {
          sX[i] = sc;
          if (blockIdx.x == 0) s_out[i] = sc;
        }
        uint32_t word[XV];
        // row-uniform choice (the corrected product needs s, 1/s and the
        // residual to stay normal)
        if (sc == 0.0f) {
#pragma unroll
          for (int v = 0; v < XV; ++v) word[v] = quant4(xv[i][v], sc, r, IC<0>{});
        } else if (sc >= 0x1.0p-100f && sc <= 0x1.0p100f) {
#pragma unroll
          for (int v = 0; v < XV; ++v) word[v] = quant4(xv[i][v], sc, r, IC<1>{});
        } else {
#pragma unroll
          for (int v = 0; v < XV; ++v) word[v] = quant4(xv[i][v], sc, r, IC<2>{});
        }
#pragma unroll
        for (int v = 0; v < XV; ++v) {
          if (!xin(v)) continue;
          const int k = 4 * (threadIdx.x + NWV * 64 * v);
          // fragment (group g, half h) lane 16*(k%64/16) + row, byte k%16
          const int g = k / 128, h = (k % 128) / 64, sq = (k % 64) / 16;
          if (CX)
            *reinterpret_cast<uint32_t*>(sA + i * K + k) = word[v];
          else
            *reinterpret_cast<uint32_t*>(sA + (g * 2 + h) * 1024 + (16 * sq + i) * 16 + k % 16) = word[v];
          if (blockIdx.x == 0) *reinterpret_cast<uint32_t*>(q_out + (int64_t)i * K + k) = word[v];
        }
      }
    if (threadIdx.x >= M && threadIdx.x < 16) sX[threadIdx.x] = 0.0f;
  } else {
    store_chunk(0);
    if (threadIdx.x < 16 * MR) sX[threadIdx.x] = sxi;
  }
#pragma unroll
  for (int u = 0; u < SCH; ++u) {
    const int q = threadIdx.x + NWV * 64 * u;
    if (SCT % (NWV * 64) == 0 || q < SCT) *reinterpret_cast<v4i*>(sS + q * SEL) = sv[u];
  }
  if constexpr (NCH > 1 && !FQ) load_chunk(1);
  wait_lds0();
  lds_barrier();

  // this wave's row blocks: hr*MRW .. hr*MRW + MRW - 1
  int acc[MRW][4];
  float facc[MRW][4];
#pragma unroll
  for (int rb = 0; rb < MRW; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[rb][r] = 0; facc[rb][r] = 0.0f; }
  auto group = [&](int g, const uint4& w) {
    int32_t sc = (int32_t)sS[g * SCW + tw * 16 + c];
    if (sizeof(SL) < 4) opaque_reg(sc);              // keep the 24-bit multiply-adds as written
    const int8_t* base = CX ? sA + (c < M ? c : M - 1) * K + kGroup * gq(g) + 16 * s4
                            : sA + ((g / CG) % NBUF) * CFR * 1024 + (g % CG) * MR * 2048 +
                                  hr * MRW * 2048 + lane * 16;
    uint32_t x0, x1, x2, x3, x4, x5, x6, x7;
    unpack_x16(w.x, x0, x1);
    unpack_x16(w.y, x2, x3);
    unpack_x16(w.z, x4, x5);
    unpack_x16(w.w, x6, x7);
    const v4i b0 = {(int)x0, (int)x1, (int)x2, (int)x3};
    const v4i b1 = {(int)x4, (int)x5, (int)x6, (int)x7};
#pragma unroll
    for (int rb = 0; rb < MRW; ++rb) {
      const v4i a0 = *reinterpret_cast<const v4i*>(base + (CX ? 0 : rb * 2048));
      const v4i a1 = *reinterpret_cast<const v4i*>(base + (CX ? 64 : rb * 2048 + 1024));
      v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
      p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, p, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pv = p[r] >> 4;                    // exact: every product is 16 * q_x * q_w
        if (FS) facc[rb][r] = __builtin_fmaf((float)pv, __int_as_float(sc), facc[rb][r]);
        else acc[rb][r] = mad24(pv, sc, acc[rb][r]);
      }
    }
  };
  // chunk ch: groups ch*CG .. ch*CG+CG-1 (slot = group % D, D divides CG);
  // every chunk but the last refills each slot with group g + D, then hands
  // the staged rows of chunk ch+1 to LDS and requests those of ch+2
  static_assert(CG % D == 0, "ring slots repeat per chunk");
  auto chunk = [&](int ch, auto last) {
    constexpr bool LAST = decltype(last)::value;
#pragma unroll
    for (int gl = 0; gl < CG; ++gl) {
      const int g = ch * CG + gl;
      group(g, wb[gl % D]);
      if (!LAST || gl + D < CG) wb[gl % D] = load_u4_nt(wsrc + (int64_t)gq(g + D) * 64);
      __builtin_amdgcn_sched_barrier(0);             // keep each group's fragments short-lived
    }
    if (!LAST) {
      store_chunk((ch + 1) % NBUF);
      if (ch + 2 < NCH) load_chunk(ch + 2);
      wait_lds0();
      lds_barrier();
    }
  };
  if constexpr (KS > 1 || CX) {
    // this wave's GK groups from g0w, DK at a time (ring slot j)
#pragma unroll 1
    for (int gb = 0; gb < GK; gb += DK) {
#pragma unroll
      for (int j = 0; j < DK; ++j) {
        const int g = g0w + gb + j;
        group(g, wb[j]);
        if (GK > DK && gb + j + DK < GK) wb[j] = load_u4_nt(wsrc + (int64_t)gq(g + DK) * 64);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // K split: the other waves' int32 sums of the tile meet wave ks = 0's
    // in LDS (wrapping adds, exact in any order), which converts
    __shared__ int32_t sRed[(KS > 1 ? KS - 1 : 1) * W * 4 * kWave];
    if (KS > 1 && ks > 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) sRed[(((ks - 1) * W + tw) * 4 + r) * kWave + lane] = acc[0][r];
    if constexpr (KS > 1) {
      wait_lds0();
      lds_barrier();
    }
    if (ks > 0) return;
#pragma unroll
    for (int k = 1; k < KS; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[0][r] = (int32_t)((uint32_t)acc[0][r] +
                              (uint32_t)sRed[(((k - 1) * W + tw) * 4 + r) * kWave + lane]);
  } else {
#pragma unroll 1
    for (int ch = 0; ch < NCH - 1; ++ch) chunk(ch, std::false_type{});
    chunk(NCH - 1, std::true_type{});
  }

  // ---- one conversion per output
  if (tvalid) {
    const int j = t * 16 + c;
#pragma unroll
    for (int rb = 0; rb < MRW; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * (hr * MRW + rb) + 4 * s4 + r;
        if (i >= M) continue;
        const int64_t o = (int64_t)(r0 + i) * N + j;
        const float si = sX[i];
        if (FS) {
          y.put(o, facc[rb][r] * si);
        } else {
          const float t0 = (float)acc[rb][r] * si;
          y.put(o, t0 * inv_alpha);
          if (acc_out) acc_out[o] = acc[rb][r];
        }
      }
  }
}

// ------------------------------------------------------------------ launchers
template <int MR, bool FS, typename ST>
static void launch_skinny(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const ST* iscale, const float* fscale, float inv_alpha, int M,
                          int N, int K, OutY y, int32_t* acc_out, hipStream_t stream) {
  constexpr int KS = FS ? 1 : 4;
  dim3 grid(N / 16), block(kWave * KS);
  hipLaunchKernelGGL((k_w4a8_skinny<MR, KS, FS, ST>), grid, block, 0, stream, qx, sx,
                     reinterpret_cast<const uint4*>(packed), iscale, fscale, inv_alpha, M, N, K, y,
                     acc_out);
}

// Workgroups that fit on the device at once for kernel k (block threads,
// dyn_lds bytes), cached per (device, kernel, block, lds).
static int resident_blocks(const void* k, int block, size_t dyn_lds) {
  struct Entry { int dev; const void* k; int block; size_t lds; int n; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (const Entry& e : cache)
      if (e.dev == dev && e.k == k && e.block == block && e.lds == dyn_lds) return e.n;
  }
  int ncu = 0, occ = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, block, dyn_lds) != hipSuccess) return 0;
  const int n = (occ < 1 ? 1 : occ) * ncu;
  std::lock_guard<std::mutex> g(mu);
  cache.push_back({dev, k, block, dyn_lds, n});
  return n;
}

// Stream-kernel configuration per row-block count: groups per loader wave,
// block size bound and waves per SIMD (chosen so no variant spills).
template <int MR> struct StreamCfg;
template <> struct StreamCfg<1> { static constexpr int GPW = 4, MAXT = 576, WPE = 5; };
template <> struct StreamCfg<2> { static constexpr int GPW = 4, MAXT = 576, WPE = 3; };
template <> struct StreamCfg<3> { static constexpr int GPW = 3, MAXT = 768, WPE = 3; };
template <> struct StreamCfg<4> { static constexpr int GPW = 3, MAXT = 768, WPE = 3; };

constexpr size_t kLdsCap = 160 * 1024;             // gfx950 LDS per workgroup

static size_t stream_lds_bytes(int MR, int GPW, bool FS, int G) {
  const int NR = MR * 4, KS = (G + GPW - 1) / GPW;
  const size_t area = 4u * (FS ? (size_t)G * NR * kWave + (size_t)G * 16 : (size_t)KS * NR * kWave);
  return 2 * area;                                 // two copies, tile parity
}

enum class W4Path { Decode, Stream, Skinny, Tiled, Wide };
// wide_cols > 0 (wide path): the 256 x 256 tile kernel covers columns
// 0 .. wide_cols-1 and the 256 x 128 one the rest (see plan_w4a8)
struct W4Plan { W4Path path; int mr; int wide_cols = 0; };

// The kernel a W4A8 GEMM of this shape runs: small M streams the weights
// (decode kernel when K is a multiple of 16 groups and the X block fits LDS;
// else the stream kernel while its loader waves and exchange area fit a
// workgroup; else the skinny kernel); larger M takes the LDS-tiled MFMA kernel.
constexpr int kDecodeW = 8;                        // waves (tiles) per grouped decode workgroup
// dense decode: waves per workgroup from the tile count T = N/16, so that the
// T/W workgroups (one per CU, each streaming W tiles) spread over the 256 CUs
// (2-wave workgroups for one row block only: more would not fit the registers)
constexpr int decode_waves(int T, int mr) {
  return T <= 512 && mr == 1 ? 2 : (T <= 1024 ? 4 : (T <= 1536 ? 6 : 8));
}
// group blocks in flight per wave: fewer when each wave also holds several row blocks
constexpr int decode_depth(int mr) { return mr == 1 ? 16 : 8; }
// waves per 16-column tile: with four row blocks on 4- or 6-wave workgroups
// each tile's blocks are split over two waves, so a SIMD holds two or three
// waves of half the VALU work each (16 waves would leave too few registers)
constexpr int decode_row_split(int mr, int w) { return mr == 4 && w <= 6 ? 2 : 1; }
// waves per 16-column tile splitting K (integer scale, one row block, 16 or 32
// groups): workgroups of one or two tiles (N/16 <= 512 tiles) take 4 waves per
// tile, each streaming a quarter of the tile's groups, all of them in flight
// (one round trip to memory instead of two); their sums meet in LDS. Where
// that split applies and N/16 <= 256, the tiles go one per workgroup (4
// waves), so N = 4096 runs on 256 workgroups rather than 128 of two tiles. (On 4-wave workgroups
// a split in two measured no faster: 688 tiles already fill the CUs.)
constexpr int decode_k_split(int mr, int w, bool fs, int g, int gq) {
  return mr != 1 || fs || g != gq || (g != 16 && g != 32) || (w != 2 && w != 1) ? 1 : 4;
}

// K = 11008 (86 groups, run as 96 with the last ten masked) and K = 14336 (112)
// take the decode kernel for one row block on 2- or 4-wave workgroups, whose
// LDS holds their scales (with more row blocks the weight-split kernels win)
static bool decode_padded(int G, int N, int mr) {
  return (G == 86 || G == 112) && mr == 1 && decode_waves(N / 16, mr) <= 4;
}

// Large M (> 64): the 256 x 256 tile kernel or the 256 x 128 one. Both run
// one workgroup per CU (their LDS rings fill a CU), so a launch takes
// ceil(tiles / CUs) rounds; at K = 4096 a round costs about 80 us for the
// 256 x 256 tiles and about 48 us for the 256 x 128 ones (N = 22016, M = 256
// .. 4096): costs below are in units of 16 us, 5 and 3 per round. When the
// 256 x 256 tiles would leave a last, partial round, the wide launch keeps
// the whole column tiles that fill its full rounds and the 256 x 128 kernel
// takes the remaining columns in a second launch, if those fit one round.
// set_prefill_kernel() forces one kernel (benchmarks, tests; forcing the wide
// one keeps the split of the last round).
static std::atomic<int> g_prefill_kernel{0};        // PrefillKernel

int device_cus() {
  static std::atomic<int> cached{0};
  int n = cached.load();
  if (n > 0) return n;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 256;                                      // MI355X; planning without a device
  }
  cached.store(n);
  return n;
}

// columns of the wide launch when its last round goes to the 256 x 128
// kernel, else 0
static int wide_split_cols(int M, int N) {
  const int64_t cus = device_cus(), tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int64_t R = tm * tn / cus;                  // full rounds of 256 x 256 tiles
  if (R < 1 || tm * tn % cus == 0) return 0;
  const int64_t c1 = R * cus / tm;                  // whole column tiles in them
  if (c1 < 1 || c1 >= tn) return 0;
  const int64_t rest = tm * ((N - 256 * c1 + 127) / 128);
  return rest <= cus ? (int)(256 * c1) : 0;
}

static bool wide_tiles_win(int M, int N, int split_cols) {
  const int64_t cus = device_cus(), tm = (M + 255) / 256;
  const int64_t tw = tm * ((N + 255) / 256);
  const int64_t rt = (tm * ((N + 127) / 128) + cus - 1) / cus;
  const int64_t cw = split_cols > 0 ? 5 * (tw / cus) + 3 : 5 * ((tw + cus - 1) / cus);
  return cw <= 3 * rt;
}

int set_prefill_kernel(int mode) {
  if (mode < kPrefillAuto || mode > kPrefillTiled) return -1;
  g_prefill_kernel.store(mode);
  return 0;
}

static W4Plan plan_w4a8(int M, int N, int K, bool fs) {
  if (M > 64) {
    const int f = g_prefill_kernel.load();
    if (f == kPrefillTiled) return {W4Path::Tiled, 0};
    const int wc = wide_split_cols(M, N);
    if (f == kPrefillWide || wide_tiles_win(M, N, wc)) return {W4Path::Wide, 0, wc};
    return {W4Path::Tiled, 0};
  }
  const int mr = (M + 15) / 16, G = K / kGroup;
  if (G == 16 || G == 32 || decode_padded(G, N, mr)) return {W4Path::Decode, mr};
  int gpw = 0, maxt = 0;
  switch (mr) {
    case 1: gpw = StreamCfg<1>::GPW; maxt = StreamCfg<1>::MAXT; break;
    case 2: gpw = StreamCfg<2>::GPW; maxt = StreamCfg<2>::MAXT; break;
    case 3: gpw = StreamCfg<3>::GPW; maxt = StreamCfg<3>::MAXT; break;
    default: gpw = StreamCfg<4>::GPW; maxt = StreamCfg<4>::MAXT; break;
  }
  const int ks = (G + gpw - 1) / gpw;
  const bool fits = (ks + 1) * kWave <= maxt && stream_lds_bytes(mr, gpw, fs, G) <= kLdsCap;
  return {fits ? W4Path::Stream : W4Path::Skinny, mr};
}

template <int MR, bool FS, typename ST>
static bool launch_stream(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const ST* iscale, const float* fscale, float inv_alpha, int M,
                          int N, int K, OutY y, int32_t* acc_out, hipStream_t stream) {
  using C = StreamCfg<MR>;
  const int G = K / kGroup, T = N / 16;
  const int KS = (G + C::GPW - 1) / C::GPW;        // loader waves (+1 finisher)
  const size_t lds = stream_lds_bytes(MR, C::GPW, FS, G);
  auto kern = k_w4a8_stream<MR, C::GPW, FS, C::MAXT, C::WPE, ST>;
  const int pmax = resident_blocks(reinterpret_cast<const void*>(kern), (KS + 1) * kWave, lds);
  if (pmax < 1) return false;
  const int per = (T + pmax - 1) / pmax;          // tiles per workgroup
  const int grid = (T + per - 1) / per;
  hipLaunchKernelGGL(kern, dim3(grid), dim3((KS + 1) * kWave), lds, stream, qx, sx,
                     reinterpret_cast<const uint4*>(packed), iscale, fscale, inv_alpha, M, N, K,
                     y, acc_out);
  return true;
}

template <bool FS, typename ST>
static void launch_small_m(const W4Plan& plan, const int8_t* qx, const float* sx,
                           const uint8_t* packed, const ST* iscale, const float* fscale,
                           float inv_alpha, int M, int N, int K, OutY y, int32_t* acc_out,
                           hipStream_t stream) {
  bool done = false;
  if (plan.path == W4Path::Stream) {
    switch (plan.mr) {
      case 1: done = launch_stream<1, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
      case 2: done = launch_stream<2, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
      case 3: done = launch_stream<3, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
      default: done = launch_stream<4, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
    }
  }
  if (done) return;
  switch (plan.mr) {
    case 1: launch_skinny<1, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
    case 2: launch_skinny<2, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
    case 3: launch_skinny<3, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
    default: launch_skinny<4, FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream); break;
  }
}

const char* w4a8_kernel_name(int64_t M, int64_t N, int64_t K, bool float_scale) {
  static const char* names[2][3][4] = {
      {{"k_w4a8_stream<1,IS>", "k_w4a8_stream<2,IS>", "k_w4a8_stream<3,IS>", "k_w4a8_stream<4,IS>"},
       {"k_w4a8_skinny<1,4,IS>", "k_w4a8_skinny<2,4,IS>", "k_w4a8_skinny<3,4,IS>", "k_w4a8_skinny<4,4,IS>"},
       {"k_w4a8_prefill<4,2,2,2,IS>", "", "", ""}},
      {{"k_w4a8_stream<1,FS>", "k_w4a8_stream<2,FS>", "k_w4a8_stream<3,FS>", "k_w4a8_stream<4,FS>"},
       {"k_w4a8_skinny<1,1,FS>", "k_w4a8_skinny<2,1,FS>", "k_w4a8_skinny<3,1,FS>", "k_w4a8_skinny<4,1,FS>"},
       {"k_w4a8_prefill<4,2,2,2,FS>", "", "", ""}}};
  const W4Plan p = plan_w4a8((int)M, (int)N, (int)K, float_scale);
  const int fs = float_scale ? 1 : 0;
  if (p.path == W4Path::Wide) return float_scale ? "k_w4a8_wide<FS>" : "k_w4a8_wide<IS>";
  if (p.path == W4Path::Tiled) return names[fs][2][0];
  if (p.path == W4Path::Decode) return float_scale ? "k_w4a8_decode<FS>" : "k_w4a8_decode<IS>";
  return names[fs][p.path == W4Path::Stream ? 0 : 1][p.mr - 1];
}

template <bool FS, int G, int GQ, int W, int MRMAX, typename ST>
static void launch_decode_w(int mr, hipStream_t stream, const int8_t* qx, const float* sx,
                            const uint4* pk, const ST* iscale, const float* fscale,
                            float inv_alpha, int M, int N, OutY y, int32_t* acc_out) {
  const void* nx = nullptr;
  int8_t* nq = nullptr;
  float* ns = nullptr;
  const dim3 grid((N / 16 + W - 1) / W);
#define BGT_DECODE(MRR)                                                                           \
  hipLaunchKernelGGL((k_w4a8_decode<FS, W, decode_depth(MRR), G, MRR, ST, false, kF32, false, GQ, \
                                    decode_row_split(MRR, W),                                     \
                                    decode_k_split(MRR, W, FS, G, GQ)>),                          \
                     grid,                                                                        \
                     dim3(W * decode_row_split(MRR, W) * decode_k_split(MRR, W, FS, G, GQ) * kWave), \
                     0, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out, nx, 0, nq, \
                     ns, Route{})
  if constexpr (MRMAX == 1) {
    BGT_DECODE(1);
  } else {
    switch (mr) {
      case 1: BGT_DECODE(1); break;
      case 2: BGT_DECODE(2); break;
      case 3: BGT_DECODE(3); break;
      default: BGT_DECODE(4); break;
    }
  }
#undef BGT_DECODE
}

template <bool FS, int G, int GQ, typename ST>
static void launch_decode(int mr, hipStream_t stream, const int8_t* qx, const float* sx,
                          const uint4* pk, const ST* iscale, const float* fscale, float inv_alpha,
                          int M, int N, OutY y, int32_t* acc_out) {
  const int w = decode_waves(N / 16, mr);
  if constexpr (!FS && GQ == G && (G == 16 || G == 32)) {
    if (w == 2 && N / 16 <= 256) {
      launch_decode_w<FS, G, GQ, 1, 1>(1, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out);
      return;
    }
  }
  if (w == 2) {
    launch_decode_w<FS, G, GQ, 2, 1>(1, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out);
  } else if constexpr (G > 32) {
    // 96 or 112 groups: one row block on 4-wave workgroups (decode_padded)
    launch_decode_w<FS, G, GQ, 4, 1>(1, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out);
  } else {
    switch (w) {
      case 4: launch_decode_w<FS, G, GQ, 4, 4>(mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
      case 6: launch_decode_w<FS, G, GQ, 6, 4>(mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
      default: launch_decode_w<FS, G, GQ, 8, 4>(mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
    }
  }
}

// Split K of the 256 x 128 tile kernel (integer scale): when its tiles fill
// at most half of the CUs, the groups are split in 2, 4, ... (at least 4
// groups per split) while the workgroups still fit the CUs once; the splits'
// int32 sums meet in k_split_reduce. The float-scale control keeps one
// ascending fma chain per output (its rounding depends on the order).
static int split_count(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 127) / 128), cus = device_cus();
  const int G = K / kGroup;
  int s = 1;
  while (tiles * s * 2 <= cus && s * 2 * 4 <= G) s *= 2;
  return s;
}

size_t w4a8_split_bytes(int64_t M, int64_t N, int64_t K, bool float_scale) {
  if (float_scale) return 0;
  const W4Plan p = plan_w4a8((int)M, (int)N, (int)K, false);
  int64_t n = N;                                    // columns of the 256 x 128 launch
  if (p.path == W4Path::Wide) n = p.wide_cols > 0 ? N - p.wide_cols : 0;
  else if (p.path != W4Path::Tiled) n = 0;
  if (n == 0) return 0;
  const int s = split_count((int)M, (int)n, (int)K);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)n * sizeof(int32_t) : 0;
}

// The library's split-K workspace: one buffer per device, grown on demand
// (never while the stream is being captured into a graph: such a launch runs
// unsplit unless the buffer is already large enough). nullptr if unavailable.
int32_t* split_workspace(size_t bytes, hipStream_t stream) {
  struct Buf { int dev; void* p; size_t n; };
  static std::mutex mu;
  static std::vector<Buf> bufs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  Buf* b = nullptr;
  for (Buf& x : bufs)
    if (x.dev == dev) b = &x;
  if (b != nullptr && b->n >= bytes) return static_cast<int32_t*>(b->p);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  const size_t n = (bytes + (16u << 20) - 1) & ~((size_t)(16u << 20) - 1);
  void* p = nullptr;
  if (hipMalloc(&p, n) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (b != nullptr) {
    (void)hipFree(b->p);                           // waits for the device; earlier users are done
    b->p = p;
    b->n = n;
  } else {
    bufs.push_back({dev, p, n});
  }
  return static_cast<int32_t*>(p);
}

void launch_split_reduce(const int32_t* part, int splits, int M, int N, int ldn, const float* sx,
                         float inv_alpha, OutY y, int32_t* acc_out, hipStream_t stream) {
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream,
                     part, splits, MN, N, ldn, sx, inv_alpha, y, acc_out);
}

// Scratch of the no-allocation entry point (bgt_w4a8_gemm_is_noalloc): the
// split-K sums in a static device array. Each GPU the library runs on holds
// its own copy, at its own address, until the process ends; host code uses
// only the address hipGetSymbolAddress returns for the current device, looked
// up once per device. 32 MiB = 256 CUs x one 256 x 128 int32 tile each, the
// most a split launch writes on a 256-CU device (tiles x splits <= CUs).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

int32_t* noalloc_scratch(size_t* capacity) {
  constexpr int kMaxDev = 64;
  static std::atomic<int32_t*> ptrs[kMaxDev];
  *capacity = kNoAllocScratchBytes;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  int32_t* p = ptrs[dev].load();
  if (p != nullptr) return p;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  ptrs[dev].store(static_cast<int32_t*>(a));
  return static_cast<int32_t*>(a);
}

// 256 x 128 tiles, 8 waves of 64 x 64, over N columns whose scales, y and
// acc_out rows are ldn elements apart; split K when the tiles are few
template <bool FS, typename ST>
static void launch_tiled(const int8_t* qx, const float* sx, const uint8_t* packed,
                         const ST* iscale, const float* fscale, float inv_alpha, int M, int N,
                         int K, int ldn, OutY y, int32_t* acc_out, hipStream_t stream,
                         int32_t* ws) {
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const int tiles = ((M + 255) / 256) * ((N + 127) / 128);
  int splits = FS ? 1 : split_count(M, N, K);
  int32_t* part = nullptr;
  if (splits > 1) {
    part = ws != nullptr ? ws : split_workspace((size_t)splits * M * N * sizeof(int32_t), stream);
    if (part == nullptr) splits = 1;
  }
  hipLaunchKernelGGL((k_w4a8_prefill<4, 2, 2, 2, FS, ST>), dim3(tiles * splits), dim3(512), 0,
                     stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, K, ldn, y, acc_out,
                     Route{}, splits, part);
  if (splits > 1) launch_split_reduce(part, splits, M, N, ldn, sx, inv_alpha, y, acc_out, stream);
}

template <bool FS, typename ST>
static void launch_w4a8_t(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const ST* iscale, const float* fscale, float inv_alpha, int M, int N,
                          int K, OutY y, int32_t* acc_out, hipStream_t stream, int32_t* ws) {
  const W4Plan plan = plan_w4a8(M, N, K, FS);
  if (FS) acc_out = nullptr;
  if (plan.path == W4Path::Decode) {
    // one 16-column tile per wave, all rows per workgroup
    const uint4* pk = reinterpret_cast<const uint4*>(packed);
    switch (K / kGroup) {
      case 32: launch_decode<FS, 32, 32>(plan.mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
      case 16: launch_decode<FS, 16, 16>(plan.mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
      case 86: launch_decode<FS, 96, 86>(plan.mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
      default: launch_decode<FS, 112, 112>(plan.mr, stream, qx, sx, pk, iscale, fscale, inv_alpha, M, N, y, acc_out); break;
    }
  } else if (plan.path == W4Path::Wide) {
    const int nw = plan.wide_cols > 0 ? plan.wide_cols : N;
    launch_w4a8_wide(FS, qx, sx, packed, iscale, sizeof(ST), fscale, inv_alpha, M, nw, K, N, y,
                     acc_out, stream);
    if (nw < N) {                                   // the last round's columns
      const int G = K / kGroup;
      launch_tiled<FS, ST>(qx, sx, packed + (int64_t)(nw / 16) * G * 1024,
                           FS ? iscale : iscale + nw, FS ? fscale + nw : fscale, inv_alpha, M,
                           N - nw, K, N, y.cols(nw), acc_out ? acc_out + nw : nullptr, stream, ws);
    }
  } else if (plan.path != W4Path::Tiled) {
    launch_small_m<FS>(plan, qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out, stream);
  } else {
    launch_tiled<FS, ST>(qx, sx, packed, iscale, fscale, inv_alpha, M, N, K, N, y, acc_out, stream,
                         ws);
  }
}

hipError_t launch_w4a8(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                       const void* iscale, int iscale_bytes, const float* fscale, int alpha,
                       int64_t M64, int64_t N64, int64_t K64, OutY y, int32_t* acc_out,
                       hipStream_t stream, int32_t* ws) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  const float inv_alpha = 1.0f / (float)alpha;   // exact: alpha = 2^n
  if (float_scale)
    launch_w4a8_t<true>(qx, sx, packed, static_cast<const int32_t*>(nullptr), fscale, inv_alpha,
                        M, N, K, y, nullptr, stream, nullptr);
  else if (iscale_bytes == 4)
    launch_w4a8_t<false>(qx, sx, packed, static_cast<const int32_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream, ws);
  else if (iscale_bytes == 2)
    launch_w4a8_t<false>(qx, sx, packed, static_cast<const uint16_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream, ws);
  else
    launch_w4a8_t<false>(qx, sx, packed, static_cast<const uint8_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream, ws);
  return hipGetLastError();
}

// Quantize + GEMM in one launch for M <= 4 on the decode path (the decode
// kernel quantizes the fp32 rows itself); otherwise the quantizer and the GEMM.
// 16 or 32 groups: X staged in fragment order; waves per workgroup as for the
// unfused decode launch (workgroups of one or two tiles split K over four
// waves per tile; one tile where the 4 waves' share of the rows stays within
// 8 groups of 4 elements per thread), raised until a thread's share of the
// rows (held until they are quantized) is at most 8 groups of 4 elements,
// M*K/4 <= 8*64*waves: the quantizing prologue's critical path grows with
// that share. 86 groups (run as 96) and
// 112: the rows staged compactly, so any K fits LDS, on 2-wave workgroups
// splitting K in four (N/16 <= 512 tiles) or on 8-wave ones.
template <int IT, typename ST, int W, int GG, int GQQ>
static void launch_linear_fused_g(const void* x, int ldx, const uint4* pk, const ST* iscale,
                                  float inv_alpha, int M, int N, int8_t* q_out, float* s_out,
                                  OutY y, hipStream_t stream) {
  constexpr int KS = W <= 2 ? 4 : 1;
  constexpr bool CX = !(GG == 16 || GG == 32);
  const dim3 grid((N / 16 + W - 1) / W), block(W * KS * kWave);
  hipLaunchKernelGGL((k_w4a8_decode<false, W, decode_depth(1), GG, 1, ST, true, IT, false, GQQ, 1,
                                    KS, CX>),
                     grid, block, 0, stream, nullptr, nullptr, pk, iscale, nullptr, inv_alpha, M, N,
                     y, nullptr, x, ldx, q_out, s_out, Route{});
}

template <int IT, typename ST, int W>
static void launch_linear_fused_w(const void* x, int ldx, const uint4* pk, const ST* iscale,
                                  float inv_alpha, int M, int N, int K, int8_t* q_out,
                                  float* s_out, OutY y, hipStream_t stream) {
  if (K / kGroup == 32) {
    launch_linear_fused_g<IT, ST, W, 32, 32>(x, ldx, pk, iscale, inv_alpha, M, N, q_out, s_out, y, stream);
  } else if (K / kGroup == 16) {
    launch_linear_fused_g<IT, ST, W, 16, 16>(x, ldx, pk, iscale, inv_alpha, M, N, q_out, s_out, y, stream);
  } else if constexpr (W == 2 || W == 8) {           // compact rows (see launch_linear_fused)
    if (K / kGroup == 86)
      launch_linear_fused_g<IT, ST, W, 96, 86>(x, ldx, pk, iscale, inv_alpha, M, N, q_out, s_out, y, stream);
    else
      launch_linear_fused_g<IT, ST, W, 112, 112>(x, ldx, pk, iscale, inv_alpha, M, N, q_out, s_out, y, stream);
  }
}

template <int IT, typename ST>
static void launch_linear_fused(const void* x, int ldx, const uint8_t* packed, const ST* iscale,
                                float inv_alpha, int M, int N, int K, int8_t* q_out,
                                float* s_out, OutY y, hipStream_t stream) {
  int w = decode_waves(N / 16, 1);
  if (K / kGroup == 86 || K / kGroup == 112) w = w == 2 ? 2 : 8;   // 2 waves split K in 4, else 8
  else
    while (w < 8 && M * K > 2048 * w * decode_k_split(1, w, false, 32, 32)) w += 2;
  if (w == 2 && N / 16 <= 256 && (K / kGroup == 16 || K / kGroup == 32) && M * K <= 2048 * 4) w = 1;
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  if (w == 1)
    launch_linear_fused_w<IT, ST, 1>(x, ldx, pk, iscale, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else if (w == 2)
    launch_linear_fused_w<IT, ST, 2>(x, ldx, pk, iscale, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else if (w == 4)
    launch_linear_fused_w<IT, ST, 4>(x, ldx, pk, iscale, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else if (w == 6)
    launch_linear_fused_w<IT, ST, 6>(x, ldx, pk, iscale, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else
    launch_linear_fused_w<IT, ST, 8>(x, ldx, pk, iscale, inv_alpha, M, N, K, q_out, s_out, y, stream);
}

bool w4a8_linear_fused(int64_t M, int64_t K, const void* x, int64_t ldx) {
  const int64_t G = K / kGroup;
  return M <= 4 && (G == 16 || G == 32 || G == 86 || G == 112) && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 &&
         ldx % 4 == 0 && ldx <= (1ll << 28);
}

template <int IT>
static void launch_linear_fused_st(const void* x, int ld, const uint8_t* packed, const void* iscale,
                                   int iscale_bytes, float inv_alpha, int M, int N, int K,
                                   int8_t* q_out, float* s_out, OutY y, hipStream_t stream) {
  if (iscale_bytes == 4)
    launch_linear_fused<IT>(x, ld, packed, static_cast<const int32_t*>(iscale), inv_alpha, M, N, K,
                            q_out, s_out, y, stream);
  else if (iscale_bytes == 2)
    launch_linear_fused<IT>(x, ld, packed, static_cast<const uint16_t*>(iscale), inv_alpha, M, N, K,
                            q_out, s_out, y, stream);
  else
    launch_linear_fused<IT>(x, ld, packed, static_cast<const uint8_t*>(iscale), inv_alpha, M, N, K,
                            q_out, s_out, y, stream);
}

hipError_t launch_w4a8_linear(const void* x, int x_type, int64_t ldx, const uint8_t* packed,
                              const void* iscale, int iscale_bytes, int alpha, int64_t M64,
                              int64_t N64, int64_t K64, int8_t* q_out, float* s_out, OutY y,
                              hipStream_t stream) {
  if (!w4a8_linear_fused(M64, K64, x, ldx)) {
    hipError_t e = launch_quant_rows(x, x_type, M64, K64, ldx, false, q_out, s_out, nullptr,
                                     nullptr, stream);
    if (e != hipSuccess) return e;
    return launch_w4a8(false, q_out, s_out, packed, iscale, iscale_bytes, nullptr, alpha, M64, N64,
                       K64, y, nullptr, stream);
  }
  const int M = (int)M64, N = (int)N64, K = (int)K64, ld = (int)ldx;
  const float inv_alpha = 1.0f / (float)alpha;   // exact: alpha = 2^n
  if (x_type == kF16)
    launch_linear_fused_st<kF16>(x, ld, packed, iscale, iscale_bytes, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else if (x_type == kBF16)
    launch_linear_fused_st<kBF16>(x, ld, packed, iscale, iscale_bytes, inv_alpha, M, N, K, q_out, s_out, y, stream);
  else
    launch_linear_fused_st<kF32>(x, ld, packed, iscale, iscale_bytes, inv_alpha, M, N, K, q_out, s_out, y, stream);
  return hipGetLastError();
}

// Grouped (mixture-of-experts) integer-scale GEMM: with K/128 in {16, 32}
// (the expert w1/w3 shapes) or 112 (Mixtral's w2), routings within the rule
// of moe_decode_path take the decode kernel with one workgroup row per expert
// and row pass; otherwise the tiled kernel over the experts' row tiles.
// Row blocks per workgroup of the grouped decode kernel: enough for 1.5x the
// mean slots per expert (at most 4; at most 2 for 112 groups, whose scales
// leave LDS room for two); experts with more slots take further row passes
// (grid z), each streaming the expert's weights again.
static int moe_row_blocks(int64_t R, int64_t E, int64_t K) {
  const int64_t mean = (R + E - 1) / E;
  int mr = (int)((3 * mean / 2 + 15) / 16);
  mr = mr < 1 ? 1 : (mr == 3 ? 4 : (mr > 4 ? 4 : mr));
  return K / kGroup == 112 && mr > 2 ? 2 : mr;
}

// The grouped decode kernel streams each busy expert's weights once per row
// pass, the tiled kernel once per 256-row tile but with its MFMA tiles mostly
// empty at a few hundred slots per expert: the decode kernel serves every
// T <= 64 and, up to T = 1024, routings whose mean expert needs at most two
// row passes of 64 slots (16, 32 groups) or three of 32 slots (112 groups),
// while its worst-case grid (every expert with T slots; passes without slots
// exit at once) stays small. Crossovers measured at the Mixtral shapes (same
// call, decode / tiled us): w1 (32 groups) 196 / 204 at a mean of 128 slots
// (T = 512), 256 / 233 at 160 (T = 640); w2 (112 groups) 171 / 268 at 96
// (T = 384), 178 / 152 at 112 (T = 448).
static bool moe_decode_path(int64_t T, int64_t R, int64_t E, int64_t K) {
  const int64_t G = K / kGroup;
  if (!(G == 16 || G == 32 || G == 112)) return false;
  if (T <= 64) return true;
  const int64_t rows = 16 * moe_row_blocks(R, E, K);
  const int64_t mean = (R + E - 1) / E;
  return T <= 1024 && (mean + rows - 1) / rows <= (G == 112 ? 3 : 2) &&
         E * ((T + rows - 1) / rows) <= 2048;
}

// Past the decode range the experts' row tiles take the 256 x 256 tile kernel
// when K/128 <= 32 (and the gathered row offsets fit 32 bits), else the
// 256 x 128 one; set_prefill_kernel() forces either. With the row tiles dealt
// evenly over the XCDs, same call (us, 256 x 128 / 256 x 256): Mixtral w1
// (32 groups) T = 1024 343 / 311, T = 2048 546 / 531, T = 4096 888 / 823;
// w2 (112 groups) T = 1024 285 / 249, T = 2048 432 / 465, T = 4096 725 / 724.
static bool moe_wide_path(int64_t T, int64_t K) {
  const int f = g_prefill_kernel.load();
  if (f == kPrefillTiled || T * K >= ((int64_t)1 << 31)) return false;
  return f == kPrefillWide || K / kGroup <= 32;
}

template <typename ST>
static void launch_moe_t(const int8_t* qx, const float* sx, const uint8_t* packed,
                         const ST* iscale, float inv_alpha, int N, int K, const Route& rt,
                         OutY y, int32_t* acc_out, hipStream_t stream) {
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const int G = K / kGroup;
  if (moe_decode_path(rt.T, rt.R, rt.E, K)) {
    // every expert has at most T slots (a token reaches an expert once)
    const int mr = moe_row_blocks(rt.R, rt.E, K);
    const int passes = (rt.T + 16 * mr - 1) / (16 * mr);
    const dim3 grid((N / 16 + kDecodeW - 1) / kDecodeW, rt.E, passes), block(kDecodeW * kWave);
    const void* nx = nullptr;
    int8_t* nq = nullptr;
    float* ns = nullptr;
    const float* nf = nullptr;
#define BGT_MOE_DECODE(GG, MRR)                                                                  \
  hipLaunchKernelGGL((k_w4a8_decode<false, kDecodeW, decode_depth(MRR), GG, MRR, ST, false, kF32, \
                                    true>),                                                      \
                     grid, block, 0, stream, qx, sx, pk, iscale, nf, inv_alpha, 0, N, y, acc_out, \
                     nx, 0, nq, ns, rt)
    if (G == 112 && rt.R <= 4) {
      // at most four experts busy with narrow (N = 4096) layers: 4-wave
      // workgroups put each expert's tiles on twice as many CUs
      const dim3 g4((N / 16 + 3) / 4, rt.E, passes), b4(4 * kWave);
      hipLaunchKernelGGL((k_w4a8_decode<false, 4, decode_depth(1), 112, 1, ST, false, kF32, true>),
                         g4, b4, 0, stream, qx, sx, pk, iscale, nf, inv_alpha, 0, N, y, acc_out,
                         nx, 0, nq, ns, rt);
      return;
    }
    if (G == 32) {
      if (mr == 1) BGT_MOE_DECODE(32, 1);
      else if (mr == 2) BGT_MOE_DECODE(32, 2);
      else BGT_MOE_DECODE(32, 4);
    } else if (G == 112) {
      if (mr == 1) BGT_MOE_DECODE(112, 1);
      else BGT_MOE_DECODE(112, 2);
    } else {
      if (mr == 1) BGT_MOE_DECODE(16, 1);
      else if (mr == 2) BGT_MOE_DECODE(16, 2);
      else BGT_MOE_DECODE(16, 4);
    }
#undef BGT_MOE_DECODE
    return;
  }
  if (moe_wide_path(rt.T, K)) {
    launch_w4a8_wide_grouped(qx, sx, packed, iscale, sizeof(ST), inv_alpha, N, K, rt, y, acc_out,
                             stream);
    return;
  }
  const int tiles = ((rt.R + 255) / 256 + rt.E) * ((N + 127) / 128);
  hipLaunchKernelGGL((k_w4a8_prefill<4, 2, 2, 2, false, ST, true>), dim3(tiles), dim3(512), 0,
                     stream, qx, sx, pk, iscale, nullptr, inv_alpha, 0, N, K, N, y, acc_out, rt, 1,
                     nullptr);
}

hipError_t launch_w4a8_moe(const int8_t* qx, const float* sx, int64_t T, const int32_t* offs,
                           const int32_t* tok, int64_t E, int64_t R, const uint8_t* packed,
                           const void* iscale, int iscale_bytes, int alpha, int64_t N, int64_t K,
                           OutY y, int32_t* acc_out, hipStream_t stream) {
  const float inv_alpha = 1.0f / (float)alpha;   // exact: alpha = 2^n
  Route rt{offs, tok, (int)E, (int)T, (int)R, N * K / 2, (K / kGroup) * N};
  if (iscale_bytes == 4)
    launch_moe_t(qx, sx, packed, static_cast<const int32_t*>(iscale), inv_alpha, (int)N, (int)K,
                 rt, y, acc_out, stream);
  else if (iscale_bytes == 2)
    launch_moe_t(qx, sx, packed, static_cast<const uint16_t*>(iscale), inv_alpha, (int)N, (int)K,
                 rt, y, acc_out, stream);
  else
    launch_moe_t(qx, sx, packed, static_cast<const uint8_t*>(iscale), inv_alpha, (int)N, (int)K,
                 rt, y, acc_out, stream);
  return hipGetLastError();
}

const char* w4a8_moe_kernel_name(int64_t T, int64_t E, int64_t R, int64_t K) {
  if (moe_decode_path(T, R, E, K)) return "k_w4a8_decode<IS,grouped>";
  return moe_wide_path(T, K) ? "k_w4a8_wide<IS,grouped>" : "k_w4a8_prefill<4,2,2,2,IS,grouped>";
}

hipError_t launch_w8a8_zp(const uint8_t* qx, const float* sx, const int32_t* zx,
                          const int32_t* rowsum_x, const uint8_t* qw, const float* sw,
                          const int32_t* zw, const int32_t* colsum_w, int64_t M64, int64_t N64,
                          int64_t K64, float* y, int32_t* acc_out, hipStream_t stream) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int G = K / kGroup;
  constexpr int NW = kW8Waves;
  if (G == 32)
    hipLaunchKernelGGL((k_w8a8_zp<9, 32, NW>), dim3(tiles), dim3(NW * 64), 0, stream, qx, sx, zx,
                       rowsum_x, qw, sw, zw, colsum_w, M, N, K, OutY{y, kF32}, acc_out);
  else if (G == 16)
    hipLaunchKernelGGL((k_w8a8_zp<9, 16, NW>), dim3(tiles), dim3(NW * 64), 0, stream, qx, sx, zx,
                       rowsum_x, qw, sw, zw, colsum_w, M, N, K, OutY{y, kF32}, acc_out);
  else
    hipLaunchKernelGGL((k_w8a8_zp<9, 0, NW>), dim3(tiles), dim3(NW * 64), 0, stream, qx, sx, zx,
                       rowsum_x, qw, sw, zw, colsum_w, M, N, K, OutY{y, kF32}, acc_out);
  return hipGetLastError();
}

}  // namespace bgt
