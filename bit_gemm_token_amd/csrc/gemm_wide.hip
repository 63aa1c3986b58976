// gemm_wide.hip -- the W4A8 GEMM for large M (the compute-bound regime of the
// Integer Scale page, 5.2, Fig. 5(a)), integer-scale epilogue (方法, Fig. 3(c))
// and the float-scale control (Fig. 3(b)), for gfx950.
//
// One workgroup computes a 256 x 256 output tile with 8 waves (two per SIMD);
// wave w owns all 256 rows of the 32 columns 32w .. 32w+31, as 8 row blocks of
// v_mfma_i32_32x32x32_i8. One K step is one group of 128.
//
// Per group the workgroup copies into LDS (global_load_lds, no registers):
//   A: the 256 x 128 int8 activation tile, rows 144 bytes apart (128 + 16 of
//      padding), so the 16 rows an operand read touches at one 16-byte chunk
//      fall on distinct banks and every fragment address is one base register
//      plus an immediate;
//   B: the packed int4 group blocks of the 16 column tiles as stored (16 KiB,
//      half the bytes of int8 weights); wave w copies its own two tiles;
//   the group's 256 scales, wave w its own 32.
// Each wave reads its packed B fragments and its scales from LDS and unpacks
// the weights in registers to true int8: every packed byte is unpacked once.
// Per group and wave the VALU does 128 integer-scale multiply-adds and 56
// unpack operations for 32 MFMAs.
//
// Pipeline: three stages. In step s the waves run the MFMAs of group s; after
// the second row block they wait for their own copies of group s+1, meet at
// one barrier and request group s+2 into the stage group s-1 left. Each block
// runs one MFMA chain (one 32 x 32 block over the group's 128 k) with the
// epilogue of the previous block interleaved (one MFMA : four VALU) and reads
// the next block's activation fragments; the next group's packed weights and
// scales are read in the last blocks.
//
// MFMA operands (v_mfma_i32_32x32x32_i8): lane L = 32*hf + c supplies row
// (A) or column (B) c and 16 bytes of one of the two 16-k halves of the
// 32-wide K slice. The four K slices of a group are numbered q = 2h + j
// (h, j in {0, 1}); slice q takes k = 64h + 32j + 16hf + e, e = 0..15. In the
// packed layout lane 16s + c of a tile block holds column c, k = 16s + e
// (bytes 0..7) and 64 + 16s + e (bytes 8..15), so one 16-byte packed read at
// s = 2j + hf supplies slices (j, h = 0) and (j, h = 1) of a column.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bgt {

namespace {

constexpr int kWBM = 256, kWBN = 256, kWNW = 8;   // tile rows, columns; waves (each 256 x 32)
constexpr int kWPitch = 144;                      // LDS bytes per activation row: 128 + 16 pad
constexpr int kWA = kWBM * kWPitch;               // A stage: 256 padded rows (36 KiB)
constexpr int kWACopies = kWA / 1024;             // 1 KiB copies per A stage (36)
constexpr int kWB = (kWBN / 16) * 1024;           // B stage: 16 packed tile blocks (16 KiB)
constexpr int kWS = kWNW * 128;                   // scale stage: one 128-byte slot per wave
constexpr int kWW = kWB + kWS;                    // B + scale stage (17 KiB); three stages of
                                                  // A + B + scales: 159 KiB

}  // namespace

template <bool FS, typename ST, bool GR = false>
__global__ __launch_bounds__(kWNW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_w4a8_wide(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K, int ldn, OutY y,
    int32_t* __restrict__ acc_out, Route rt) {
  constexpr int NW = kWNW;
  constexpr int A_MAX = (kWACopies + NW - 1) / NW;   // 5 activation copies for waves 0..3,
  constexpr int A_FULL = kWACopies - NW * (A_MAX - 1);   // 4 for the others
  static_assert(A_MAX == 5 && A_FULL == 4, "activation copies per wave");
  __shared__ __align__(16) int8_t A0[kWA];
  __shared__ __align__(16) int8_t A1[kWA];
  __shared__ __align__(16) int8_t A2[kWA];
  __shared__ __align__(16) int8_t W0[kWW];
  __shared__ __align__(16) int8_t W1[kWW];
  __shared__ __align__(16) int8_t W2[kWW];

  const int G = K / kGroup, T = N / 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lr = lane % 32, hf = lane / 32;
  int tm, tn;
  // grouped GEMM: the grid covers ceil(R/256) + E row tiles, an upper bound on
  // the sum over experts of ceil(rows/256); the experts' row tiles (experts in
  // order) are dealt evenly over the XCDs and the spare workgroups exit.
  // The expert's slots r0 .. r0+M-1 are its rows; slot r reads activation row
  // tok[r] (row offsets fit 32 bits: T*K < 2^31, checked by the launcher)
  int r0 = 0;
  if constexpr (GR) {
    int e, a, rows;
    if (!grouped_tile(blockIdx.x, kWBM, (N + kWBN - 1) / kWBN, rt, e, a, rows, tm, tn)) return;
    M = rows;
    r0 = a;
    packed += e * rt.wstride;
    if (FS) fscale += e * rt.sstride;
    else iscale += e * rt.sstride;
  } else {
    tile_of(blockIdx.x, (M + kWBM - 1) / kWBM, (N + kWBN - 1) / kWBN, tm, tn);
  }
  const int m0 = tm * kWBM, n0 = tn * kWBN;

  // ---- copy sources. A: copy i = wave + NW*t fills the 64 16-byte units
  // 64i .. 64i+63 of the stage; unit u holds row u/9, chunk u%9 of the group
  // (chunk 8 is the row's padding: it gets chunk 0, never read). Rows past M
  // read row M-1 (their outputs are never stored).
  const int8_t* abase = GR ? qx : qx + (int64_t)m0 * K;
  uint32_t aoff[A_MAX];                            // unsigned: base + zero-extended offset
#pragma unroll
  for (int t = 0; t < A_MAX; ++t) {
    const int u = 64 * (wave + NW * t) + lane;
    const int r = u / 9, c = u % 9;
    const int rr = m0 + r < M ? r : M - 1 - m0;
    const int ro = GR ? clamp_route(rt.tok[r0 + m0 + rr], 0, rt.T - 1) : rr;
    aoff[t] = (uint32_t)ro * (uint32_t)K + (uint32_t)(16 * (c < 8 ? c : 0));
  }
  // B: wave w copies the packed group blocks of tiles 2w and 2w+1 (tiles past
  // N/16 read the last tile; their outputs are never stored)
  const uint8_t* bbase[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tg = n0 / 16 + 2 * wave + u;
    bbase[u] = packed + (int64_t)(tg < T ? tg : T - 1) * G * 1024;
  }
  const uint32_t lane16 = (uint32_t)lane * 16;
  // scales: wave w copies its 32 columns into its 128-byte slot with its first
  // 32 lanes, 4 bytes = CPL elements each (narrow elements leave the slot's
  // tail to clamped columns)
  using SL = typename std::conditional<FS, int32_t, ST>::type;   // scale element as stored
  constexpr int SB = sizeof(SL), CPL = 4 / SB;
  static_assert(SB == 1 || SB == 2 || SB == 4, "scale element of 1, 2 or 4 bytes");
  const char* ssrc = FS ? reinterpret_cast<const char*>(fscale) : reinterpret_cast<const char*>(iscale);
  const int scol = n0 + wave * 32 + lr * CPL;
  const uint32_t soff = (uint32_t)(scol <= N - CPL ? scol : N - CPL) * SB;

  auto issue = [&](int g, int8_t* as, int8_t* ws) {
    const int8_t* ab = abase + (int64_t)g * kGroup;
#pragma unroll
    for (int t = 0; t < A_MAX; ++t)
      if (t < A_MAX - 1 || wave < A_FULL)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(ab + aoff[t]),
            (__attribute__((address_space(3))) void*)(as + (wave + NW * t) * 1024), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bbase[u] + ((uint32_t)g * 1024u + lane16)),
          (__attribute__((address_space(3))) void*)(ws + (2 * wave + u) * 1024), 16, 0, 0);
    if (lane < 32)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)((ssrc + (int64_t)g * ldn * SB) + soff),
          (__attribute__((address_space(3))) void*)(ws + kWB + wave * 128), 4, 0, 0);
  };

  // ---- fragments. A slice q = 2h + j of row block rb: chunk 2q + hf of
  // tile row rb*32 + c.
  auto read_a = [&](const int8_t* as, int rb, v4i (&a)[4]) {
    const int8_t* p = as + (rb * 32 + lr) * kWPitch + hf * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = *reinterpret_cast<const v4i*>(p + 32 * q);
  };
  // The next group's packed B and scale are read by an asm block that waits
  // for its own reads: with compiler-visible reads of these stage regions the
  // wait-count pass cannot separate them from the copies in flight and waits
  // for all of them. Outputs are early-clobber: the later reads of the block
  // still need their address registers after the first result may have
  // landed. Packed read j: packed lane 16*(2j + hf) + c%16 of tile 2w + c/16
  // (this wave's own copies); scale: this lane's column, one aligned dword
  // (narrow elements are shifted out of it).
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const uint32_t boff = (uint32_t)((2 * wave + lr / 16) * 1024 + (16 * hf + lr % 16) * 16);
  const uint32_t sbyte = (uint32_t)(kWB + wave * 128 + lr * SB);
  auto read_bs = [&](const int8_t* ws, uint4& w0, uint4& w1, int32_t& sc) {
    u4v p0, p1;
    uint32_t wsc;
    uint32_t bo = boff, so = sbyte & ~3u;   // opaque copies: addresses formed here, not kept
    opaque_reg(bo);
    opaque_reg(so);
    const uint32_t ba = lds_addr(ws) + bo, sa = lds_addr(ws) + so;
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %3 offset:512\n\t"
        "ds_read_b32 %2, %4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p0), "=&v"(p1), "=&v"(wsc)
        : "v"(ba), "v"(sa)
        : "memory");
    w0 = make_uint4(p0.x, p0.y, p0.z, p0.w);
    w1 = make_uint4(p1.x, p1.y, p1.z, p1.w);
    const uint32_t mask = SB == 4 ? ~0u : (1u << (8 * SB)) - 1u;
    sc = (int32_t)((wsc >> (8 * (sbyte % 4))) & mask);
    // hide the narrow value range: with it the compiler rewrites the 24-bit
    // multiply-adds and re-associates them across groups (register blow-up)
    if (SB != 4) opaque_reg(sc);
  };
  // true int8 operands: slice (j, h = 0) from bytes 0..7 of read j, slice
  // (j, h = 1) from bytes 8..15
  auto unpack_b = [&](const uint4& w0, const uint4& w1, v4i (&b)[4]) {
    uint32_t l0, h0, l1, h1, l2, h2, l3, h3;
    unpack_i8(w0.x, l0, h0);
    unpack_i8(w0.y, l1, h1);
    unpack_i8(w0.z, l2, h2);
    unpack_i8(w0.w, l3, h3);
    b[0] = v4i{(int)l0, (int)h0, (int)l1, (int)h1};
    b[2] = v4i{(int)l2, (int)h2, (int)l3, (int)h3};
    unpack_i8(w1.x, l0, h0);
    unpack_i8(w1.y, l1, h1);
    unpack_i8(w1.z, l2, h2);
    unpack_i8(w1.w, l3, h3);
    b[1] = v4i{(int)l0, (int)h0, (int)l1, (int)h1};
    b[3] = v4i{(int)l2, (int)h2, (int)l3, (int)h3};
  };

  int acc[8][16];
  float facc[8][16];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[rb][r] = 0;
      facc[rb][r] = 0.0f;
    }

  auto chain = [&](const v4i (&a)[4], const v4i (&b)[4]) {
    v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], v16i{0}, 0, 0, 0);
#pragma unroll
    for (int q = 1; q < 4; ++q) p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[q], b[q], p, 0, 0, 0);
    return p;
  };
  // integer-scale epilogue of one group: acc += p * iscale (24-bit
  // multiply-add, exact mod 2^32); float-scale control: fma((float)p, s, acc)
  auto scale = [&](int rb, const v16i& p, int32_t sc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (FS) {
        facc[rb][r] = __builtin_fmaf((float)p[r], __int_as_float(sc), facc[rb][r]);
        opaque_reg(facc[rb][r]);
      } else {
        acc[rb][r] = mad24(p[r], sc, acc[rb][r]);
        opaque_reg(acc[rb][r]);
      }
    }
  };

  v4i a[4], an[4], b[4];
  int32_t sc = 0, scn = 0;
  // the partial of the previous block, scaled under the next block's MFMAs;
  // at a step's start it is block 7 of the previous step, with that group's
  // scale (zero before the first step: it adds nothing)
  v16i pend = v16i{0};
  int32_t pend_sc = 0;

  // block rb: the MFMA chain over the group's 128 k, the epilogue of the
  // previous block interleaved (one MFMA : four VALU), then `more` (LDS reads,
  // unpacking) placed after the chain's MFMAs are issued
  auto block = [&](auto rbk, auto more) {
    constexpr int RB = decltype(rbk)::value, PRB = (RB + 7) % 8;
    const v16i p = chain(a, b);
    scale(PRB, pend, pend_sc);
    more();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    pend = p;
    pend_sc = sc;
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = an[q];
  };

  // ---- step s on stage P = s % 3. Every step reads the next group's
  // fragments and requests the one after (clamped to the last group: the last
  // steps read a stage again and copy into one nobody reads), so every step is
  // the same straight-line code and the compiler can tell the stage arrays
  // apart (it adds no waits for copies in flight).
  auto step = [&](int s, auto pp) {
    constexpr int P = decltype(pp)::value;
    int8_t* cur = P == 0 ? A0 : (P == 1 ? A1 : A2);
    int8_t* nxt = P == 0 ? A1 : (P == 1 ? A2 : A0);
    int8_t* iss = P == 0 ? A2 : (P == 1 ? A0 : A1);
    int8_t* wnx = P == 0 ? W1 : (P == 1 ? W2 : W0);
    int8_t* wis = P == 0 ? W2 : (P == 1 ? W0 : W1);
    uint4 w0, w1;
    block(IC<0>{}, [&] { read_a(cur, 1, an); });
    block(IC<1>{}, [&] { read_a(cur, 2, an); });
    // own copies of group s+1 landed; after the barrier every wave's have, and
    // every wave is done with the stage of group s-1
    wait_vm<0>();
    lds_barrier();
    issue(s + 2 < G ? s + 2 : G - 1, iss, wis);
    block(IC<2>{}, [&] { read_a(cur, 3, an); });
    block(IC<3>{}, [&] { read_a(cur, 4, an); });
    block(IC<4>{}, [&] { read_a(cur, 5, an); });
    block(IC<5>{}, [&] { read_a(cur, 6, an); });
    block(IC<6>{}, [&] {
      read_a(cur, 7, an);
      read_bs(wnx, w0, w1, scn);
    });
    block(IC<7>{}, [&] {
      read_a(nxt, 0, an);
      unpack_b(w0, w1, b);
    });
    sc = scn;
  };

  // ---- prologue: groups 0 and 1 requested; group 0's fragments read
  issue(0, A0, W0);
  issue(G > 1 ? 1 : 0, A1, W1);
  if (wave < A_FULL) wait_vm<A_MAX + 3>();
  else wait_vm<A_MAX + 2>();
  lds_barrier();
  {
    uint4 w0, w1;
    read_bs(W0, w0, w1, sc);
    unpack_b(w0, w1, b);
    read_a(A0, 0, a);
  }

  for (int s = 0; s < G; s += 3) {
    step(s, IC<0>{});
    if (s + 1 >= G) break;
    step(s + 1, IC<1>{});
    if (s + 2 >= G) break;
    step(s + 2, IC<2>{});
  }
  scale(7, pend, pend_sc);                          // the last block's partial
  wait_vm<0>();                                     // clamped copies of the last steps

  // ---- one conversion per output; token scales loaded per row block before
  // its stores; full tiles store without per-element predicates. Outputs are
  // written non-temporally (each is written once; the 256 tiles of a round
  // finish together, and cached writes slowed the burst)
  const bool full = m0 + kWBM <= M && n0 + kWBN <= N;
  const int j = n0 + wave * 32 + lr;
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    float srow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + rb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
      const int ic = i < M ? i : M - 1;
      srow[r] = sx[GR ? clamp_route(rt.tok[r0 + ic], 0, rt.T - 1) : ic];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + rb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
      if (!full && (i >= M || j >= N)) continue;
      const int64_t o = (int64_t)(r0 + i) * ldn + j;
      if (FS) {
        y.put_nt(o, facc[rb][r] * srow[r]);
      } else {
        const float t0 = (float)acc[rb][r] * srow[r];
        y.put_nt(o, t0 * inv_alpha);
        if (acc_out) __builtin_nontemporal_store(acc[rb][r], acc_out + o);
      }
    }
  }
}

template <bool FS, typename ST>
static void launch_wide_t(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const ST* iscale, const float* fscale, float inv_alpha, int M, int N,
                          int K, int ldn, OutY y, int32_t* acc_out, hipStream_t stream) {
  const int tiles = ((M + kWBM - 1) / kWBM) * ((N + kWBN - 1) / kWBN);
  hipLaunchKernelGGL((k_w4a8_wide<FS, ST>), dim3(tiles), dim3(kWNW * 64), 0, stream, qx, sx,
                     packed, iscale, fscale, inv_alpha, M, N, K, ldn, y, acc_out, Route{});
}

template <typename ST>
static void launch_wide_grouped_t(const int8_t* qx, const float* sx, const uint8_t* packed,
                                  const ST* iscale, float inv_alpha, int N, int K, const Route& rt,
                                  OutY y, int32_t* acc_out, hipStream_t stream) {
  const int tiles = ((rt.R + kWBM - 1) / kWBM + rt.E) * ((N + kWBN - 1) / kWBN);
  hipLaunchKernelGGL((k_w4a8_wide<false, ST, true>), dim3(tiles), dim3(kWNW * 64), 0, stream, qx,
                     sx, packed, iscale, nullptr, inv_alpha, 0, N, K, N, y, acc_out, rt);
}

void launch_w4a8_wide(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                      const void* iscale, int iscale_bytes, const float* fscale, float inv_alpha,
                      int M, int N, int K, int ldn, OutY y, int32_t* acc_out, hipStream_t stream) {
  if (float_scale)
    launch_wide_t<true>(qx, sx, packed, static_cast<const int32_t*>(nullptr), fscale, inv_alpha,
                        M, N, K, ldn, y, nullptr, stream);
  else if (iscale_bytes == 4)
    launch_wide_t<false>(qx, sx, packed, static_cast<const int32_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, ldn, y, acc_out, stream);
  else if (iscale_bytes == 2)
    launch_wide_t<false>(qx, sx, packed, static_cast<const uint16_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, ldn, y, acc_out, stream);
  else
    launch_wide_t<false>(qx, sx, packed, static_cast<const uint8_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, ldn, y, acc_out, stream);
}

void launch_w4a8_wide_grouped(const int8_t* qx, const float* sx, const uint8_t* packed,
                              const void* iscale, int iscale_bytes, float inv_alpha, int N, int K,
                              const Route& rt, OutY y, int32_t* acc_out, hipStream_t stream) {
  if (iscale_bytes == 4)
    launch_wide_grouped_t(qx, sx, packed, static_cast<const int32_t*>(iscale), inv_alpha, N, K, rt,
                          y, acc_out, stream);
  else if (iscale_bytes == 2)
    launch_wide_grouped_t(qx, sx, packed, static_cast<const uint16_t*>(iscale), inv_alpha, N, K,
                          rt, y, acc_out, stream);
  else
    launch_wide_grouped_t(qx, sx, packed, static_cast<const uint8_t*>(iscale), inv_alpha, N, K, rt,
                          y, acc_out, stream);
}

}  // namespace bgt
