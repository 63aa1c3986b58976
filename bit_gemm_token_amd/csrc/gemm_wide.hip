// gemm_wide.hip -- the W4A8 GEMM for large M (the compute-bound regime of the
// Integer Scale page, 5.2, Fig. 5(a)), integer-scale epilogue (方法, Fig. 3(c))
// and the float-scale control (Fig. 3(b)), for gfx950.
//
// One workgroup computes a 256 x 256 output tile with 8 waves (two per SIMD)
// arranged 2 x 4; each wave owns 128 rows x 64 columns as 4 x 2 blocks of
// v_mfma_i32_32x32x32_i8. One K step is one group of 128.
//
// Per group the workgroup copies into LDS (global_load_lds, no registers):
//   A: the 256 x 128 int8 activation tile (32 KiB); each row's eight 16-byte
//      chunks are XOR-swizzled by (row / 2) % 8, so the 16 lanes of an operand
//      read phase hit distinct banks;
//   B: the packed int4 group blocks of its 16 column tiles as stored
//      (16 KiB: half the bytes of int8 weights);
//   the group's 256 scales.
// Each wave reads its packed B fragments from LDS and unpacks them in
// registers to true int8 (no unpacked LDS stage); every packed byte is read
// by the two waves that share its columns. Per group and wave the LDS is read
// for 16 KiB of activation fragments and 4 KiB of packed weights, half the
// bytes per multiply of a 256 x 128 tile with 64 x 64 waves.
//
// Pipeline: three stages. In step s the waves run the MFMAs of group s; after
// the first row block they wait for their own copies of group s+1, meet at one
// barrier and request group s+2 into the stage group s-1 left; the fragments
// of group s+1 (packed B, scales, the first A row block) are read at the end
// of step s. A wave runs one MFMA chain (one 32 x 32 block over the group's
// 128 k) and its epilogue at a time and rewrites operand registers only when
// none of its MFMAs is in flight; the other wave of the SIMD keeps the matrix
// core busy meanwhile.
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

constexpr int kWBM = 256, kWBN = 256, kWNW = 8;   // tile rows, columns; waves (2 x 4)
constexpr int kWA = kWBM * 128;                   // A stage bytes: 256 rows x 128 k
constexpr int kWB = (kWBN / 16) * 1024;           // B stage bytes: 16 packed tile blocks
constexpr int kWS = 8 * 128;                      // scale stage: 8 slots of 32 columns
constexpr int kWStage = kWA + kWB + kWS;          // 50176 bytes; three stages: 147 KiB

}  // namespace

template <bool FS, typename ST>
__global__ __launch_bounds__(kWNW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_w4a8_wide(
    const int8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ packed, const ST* __restrict__ iscale,
    const float* __restrict__ fscale, float inv_alpha, int M, int N, int K, OutY y,
    int32_t* __restrict__ acc_out) {
  constexpr int NW = kWNW;
  constexpr int A_INSTR = kWA / 1024 / NW;        // 1 KiB activation copies per wave per group
  constexpr int B_INSTR = kWB / 1024 / NW;        // 1 KiB weight copies per wave per group
  static_assert(A_INSTR == 4 && B_INSTR == 2, "tile and wave count");
  __shared__ __align__(16) int8_t L0[kWStage];
  __shared__ __align__(16) int8_t L1[kWStage];
  __shared__ __align__(16) int8_t L2[kWStage];

  const int G = K / kGroup, T = N / 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane % 32, hf = lane / 32;
  int tm, tn;
  tile_of(blockIdx.x, (M + kWBM - 1) / kWBM, (N + kWBN - 1) / kWBN, tm, tn);
  const int m0 = tm * kWBM, n0 = tn * kWBN;

  // ---- copy sources. A: copy i of wave w fills the 1 KiB block b = 4w... of
  // rows 8b .. 8b+7 (b = i*NW + w); lane L fills row 8b + L/8, chunk slot
  // L%8, with the row's global chunk (L%8) ^ ((row / 2) % 8). Rows past M
  // read row M-1 (their outputs are never stored).
  const int8_t* abase = qx + (int64_t)m0 * K;
  // (recomputed at each request from an opaque copy of the lane index, so the
  // four offsets do not occupy registers across the main loop)
  auto a_off = [&](int i, int ln) -> uint32_t {
    const int r = 8 * (i * NW + wave) + ln / 8;
    const int rr = m0 + r < M ? r : M - 1 - m0;
    return (uint32_t)(rr * K + 16 * ((ln % 8) ^ ((r >> 1) & 7)));
  };
  // B: copy u of wave w brings the packed group block of tile u*NW + w (tiles
  // past N/16 read the last tile; their outputs are never stored). The tile
  // bases are wave-uniform; lanes add 16*L.
  const uint8_t* bbase[B_INSTR];
#pragma unroll
  for (int u = 0; u < B_INSTR; ++u) {
    const int tg = n0 / 16 + u * NW + wave;
    bbase[u] = packed + (int64_t)(tg < T ? tg : T - 1) * G * 1024;
  }
  // scales: wave w copies the 32-column slice w into a 128-byte slot with its
  // first 32 lanes, 4 bytes = CPL elements each (narrow elements leave the
  // slot's tail to clamped columns), so every scale is copied once.
  using SL = typename std::conditional<FS, int32_t, ST>::type;   // scale element as stored
  constexpr int SB = sizeof(SL), CPL = 4 / SB;
  static_assert(SB == 1 || SB == 2 || SB == 4, "scale element of 1, 2 or 4 bytes");
  const char* ssrc = FS ? reinterpret_cast<const char*>(fscale) : reinterpret_cast<const char*>(iscale);
  const int scol = n0 + wave * 32 + (lane % 32) * CPL;
  const uint32_t soff = (uint32_t)(scol <= N - CPL ? scol : N - CPL) * SB;
  const uint32_t lane16 = (uint32_t)lane * 16;

  auto issue = [&](int g, int8_t* st) {
    const int8_t* ab = abase + (int64_t)g * kGroup;
    int ln = lane;
    opaque_reg(ln);
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(ab + a_off(i, ln)),
          (__attribute__((address_space(3))) void*)(st + (i * NW + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < B_INSTR; ++u)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bbase[u] + ((uint32_t)g * 1024u + lane16)),
          (__attribute__((address_space(3))) void*)(st + kWA + (u * NW + wave) * 1024), 16, 0, 0);
    if (lane < 32)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)((ssrc + (int64_t)g * N * SB) + soff),
          (__attribute__((address_space(3))) void*)(st + kWA + kWB + wave * 128), 4, 0, 0);
  };

  // ---- fragments. A slice q = 2h + j of row block rb: chunk 4h + 2j + hf of
  // tile row wm*128 + rb*32 + c.
  auto read_a = [&](const int8_t* st, int rb, v4i (&a)[4]) {
    const int row = wm * 128 + rb * 32 + lr;
    const int sw = (row >> 1) & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      a[q] = *reinterpret_cast<const v4i*>(st + row * 128 + 16 * ((2 * q + hf) ^ sw));
  };
  // true int8 operands of column block cb: slice (j, h = 0) from bytes 0..7 of
  // read j, slice (j, h = 1) from bytes 8..15
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
  // The next group's packed B and scales are read by asm blocks that wait for
  // their own reads (outputs early-clobber: the second read of a block still
  // needs the address register after the first one's result may have landed): with compiler-visible reads of these stage regions the
  // wait-count pass cannot separate them from the copies in flight and waits
  // for all of them. The compiler does not check an asm block's register
  // writes against MFMAs in flight, so they are issued only where this
  // wave has no MFMA in flight (after a chain's partials were consumed). Packed B of column block cb (columns wn*64 +
  // cb*32 + c), read j: packed lane 16*(2j + hf) + c%16 of tile 4wn + 2cb +
  // c/16. Scales: this lane's column in each column block, one aligned dword
  // each (narrow elements are shifted out of it).
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const uint32_t boff = (uint32_t)((4 * wn + lr / 16) * 1024 + (16 * hf + lr % 16) * 16);
  const uint32_t sbyte = (uint32_t)(wn * 256 + lr * SB);   // slot 2wn + cb, 128 bytes each
  auto read_b = [&](const int8_t* st, int cb, uint4& w0, uint4& w1) {
    u4v p0, p1;
    uint32_t bo = boff;   // opaque copy: the per-stage address is formed here, not kept
    opaque_reg(bo);
    const uint32_t ba = lds_addr(st + kWA + cb * 2048) + bo;
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:512\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p0), "=&v"(p1)
        : "v"(ba)
        : "memory");
    w0 = make_uint4(p0.x, p0.y, p0.z, p0.w);
    w1 = make_uint4(p1.x, p1.y, p1.z, p1.w);
  };
  auto read_s = [&](const int8_t* st, int32_t (&sc)[2]) {
    uint32_t w0, w1;
    uint32_t so = sbyte & ~3u;
    opaque_reg(so);
    const uint32_t sa = lds_addr(st + kWA + kWB) + so;
    asm volatile(
        "ds_read_b32 %0, %2\n\t"
        "ds_read_b32 %1, %2 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w0), "=&v"(w1)
        : "v"(sa)
        : "memory");
    const uint32_t sh = 8 * (sbyte % 4), mask = SB == 4 ? ~0u : (1u << (8 * SB)) - 1u;
    sc[0] = (int32_t)((w0 >> sh) & mask);
    sc[1] = (int32_t)((w1 >> sh) & mask);
    // hide the narrow value range: with it the compiler rewrites the 24-bit
    // multiply-adds and re-associates them across groups (register blow-up)
    if (SB != 4) {
      opaque_reg(sc[0]);
      opaque_reg(sc[1]);
    }
  };

  int acc[4][2][16];
  float facc[4][2][16];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[rb][cb][r] = 0;
        facc[rb][cb][r] = 0.0f;
      }

  auto chain = [&](const v4i (&a)[4], const v4i (&b)[4]) {
    v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], v16i{0}, 0, 0, 0);
#pragma unroll
    for (int q = 1; q < 4; ++q) p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[q], b[q], p, 0, 0, 0);
    return p;
  };
  // integer-scale epilogue of one group: acc += p * iscale (24-bit
  // multiply-add, exact mod 2^32); float-scale control: fma((float)p, s, acc)
  auto scale = [&](int rb, int cb, const v16i& p, int32_t sc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (FS) {
        facc[rb][cb][r] = __builtin_fmaf((float)p[r], __int_as_float(sc), facc[rb][cb][r]);
        opaque_reg(facc[rb][cb][r]);
      } else {
        acc[rb][cb][r] = mad24(p[r], sc, acc[rb][cb][r]);
        opaque_reg(acc[rb][cb][r]);
      }
    }
  };

  v4i a[4], b0[4], b1[4];
  int32_t sc[2], scn[2] = {0, 0};
  // The partial of the previous chain, scaled under the next chain's MFMAs;
  // at a step's start it is the last block (3, 1) of the previous step, with
  // that group's scale (zero before the first step: it adds nothing).
  v16i pend = v16i{0};
  int32_t pend_sc = 0;

  // block (rb, cb): the MFMA chain over the group's 128 k, with the epilogue
  // of the previous block's partial interleaved (one MFMA : four VALU), then
  // `more` (LDS reads, unpacking) placed after the chain's MFMAs are issued
  auto block = [&](auto rbk, auto cbk, auto more) {
    constexpr int RB = decltype(rbk)::value, CB = decltype(cbk)::value;
    constexpr int PRB = CB == 0 ? (RB + 3) % 4 : RB, PCB = 1 - CB;   // previous block
    const v16i p = chain(a, CB == 0 ? b0 : b1);
    scale(PRB, PCB, pend, pend_sc);
    more();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    pend = p;
    pend_sc = sc[CB];
  };

  // ---- step s on stage P = s % 3: blocks (rb, cb) of group s in order.
  // NEXT: every step reads the next group's fragments and requests the one
  // after (clamped to the last group: a clamped copy lands in a stage nobody
  // reads again). Steps are straight-line code so the compiler can tell the
  // stage arrays apart and adds no waits for copies in flight.
  auto step = [&](int s, auto pp) {
    constexpr int P = decltype(pp)::value;
    int8_t* cur = P == 0 ? L0 : (P == 1 ? L1 : L2);
    int8_t* nxt = P == 0 ? L1 : (P == 1 ? L2 : L0);
    int8_t* iss = P == 0 ? L2 : (P == 1 ? L0 : L1);
    auto none = [] {};
    block(IC<0>{}, IC<0>{}, none);
    block(IC<0>{}, IC<1>{}, [&] { read_a(cur, 1, a); });
    // own copies of group s+1 landed; after the barrier every wave's have, and
    // every wave is done with stage (s+2)%3 (it held group s-1)
    wait_vm<0>();
    lds_barrier();
    issue(s + 2 < G ? s + 2 : G - 1, iss);
    block(IC<1>{}, IC<0>{}, none);
    block(IC<1>{}, IC<1>{}, [&] { read_a(cur, 2, a); });
    block(IC<2>{}, IC<0>{}, none);
    block(IC<2>{}, IC<1>{}, [&] { read_a(cur, 3, a); });
    block(IC<3>{}, IC<0>{}, [&] {
      uint4 w0, w1;
      read_b(nxt, 0, w0, w1);
      unpack_b(w0, w1, b0);
    });
    block(IC<3>{}, IC<1>{}, [&] {
      uint4 w0, w1;
      read_b(nxt, 1, w0, w1);
      read_s(nxt, scn);
      unpack_b(w0, w1, b1);
      read_a(nxt, 0, a);
    });
    sc[0] = scn[0];
    sc[1] = scn[1];
  };

  // ---- prologue: groups 0 and 1 requested; group 0's fragments read
  issue(0, L0);
  issue(G > 1 ? 1 : 0, L1);
  wait_vm<A_INSTR + B_INSTR + 1>();
  lds_barrier();
  {
    uint4 w0, w1;
    read_b(L0, 0, w0, w1);
    unpack_b(w0, w1, b0);
    read_b(L0, 1, w0, w1);
    unpack_b(w0, w1, b1);
    read_s(L0, sc);
    read_a(L0, 0, a);
  }

  // every step reads the next group's fragments and requests the one after
  // (clamped to the last group): the last steps read a stage again and copy
  // into one nobody reads, so every step is the same straight-line code
  for (int s = 0; s < G; s += 3) {
    step(s, IC<0>{});
    if (s + 1 >= G) break;
    step(s + 1, IC<1>{});
    if (s + 2 >= G) break;
    step(s + 2, IC<2>{});
  }
  scale(3, 1, pend, pend_sc);                       // the last block's partial
  wait_vm<0>();                                     // clamped copies of the last steps

  // ---- one conversion per output; token scales loaded per row block before
  // its stores; full tiles store without per-element predicates
  const bool full = m0 + kWBM <= M && n0 + kWBN <= N;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    float srow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * 128 + rb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
      srow[r] = sx[i < M ? i : M - 1];
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int j = n0 + wn * 64 + cb * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 128 + rb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (!full && (i >= M || j >= N)) continue;
        const int64_t o = (int64_t)i * N + j;
        if (FS) {
          y.put(o, facc[rb][cb][r] * srow[r]);
        } else {
          const float t0 = (float)acc[rb][cb][r] * srow[r];
          y.put(o, t0 * inv_alpha);
          if (acc_out) acc_out[o] = acc[rb][cb][r];
        }
      }
    }
  }
}

template <bool FS, typename ST>
static void launch_wide_t(const int8_t* qx, const float* sx, const uint8_t* packed,
                          const ST* iscale, const float* fscale, float inv_alpha, int M, int N,
                          int K, OutY y, int32_t* acc_out, hipStream_t stream) {
  const int tiles = ((M + kWBM - 1) / kWBM) * ((N + kWBN - 1) / kWBN);
  hipLaunchKernelGGL((k_w4a8_wide<FS, ST>), dim3(tiles), dim3(kWNW * 64), 0, stream, qx, sx,
                     packed, iscale, fscale, inv_alpha, M, N, K, y, acc_out);
}

void launch_w4a8_wide(bool float_scale, const int8_t* qx, const float* sx, const uint8_t* packed,
                      const void* iscale, int iscale_bytes, const float* fscale, float inv_alpha,
                      int M, int N, int K, OutY y, int32_t* acc_out, hipStream_t stream) {
  if (float_scale)
    launch_wide_t<true>(qx, sx, packed, static_cast<const int32_t*>(nullptr), fscale, inv_alpha,
                        M, N, K, y, nullptr, stream);
  else if (iscale_bytes == 4)
    launch_wide_t<false>(qx, sx, packed, static_cast<const int32_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream);
  else if (iscale_bytes == 2)
    launch_wide_t<false>(qx, sx, packed, static_cast<const uint16_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream);
  else
    launch_wide_t<false>(qx, sx, packed, static_cast<const uint8_t*>(iscale), nullptr, inv_alpha,
                         M, N, K, y, acc_out, stream);
}

}  // namespace bgt
