// Prefill-shaped ternary product on int8 MFMA.
//
// The contraction acc[m, o] = sum_k q[m, k] * w[o, k] is the same integer
// product as the decode path (Hetman-2b s.7; BitRASP
// additive_ternary_linear_int8; Foundry "Native Matmul Kernel"), but with
// many tokens it is a dense matrix product, so it runs on the matrix cores.
// The qste project description ("Speed") records the two ways an
// unpack-in-the-K-loop GEMM loses: the dot product running off the matrix
// units and every packed byte being re-read for each of its values.  Here
// each packed word is read from global memory once per workgroup tile,
// decoded once into signed int8 in LDS, and fed to v_mfma_i32_32x32x32_i8.
//
// gfx950 mapping.  A workgroup computes a BM x BN tile with WM x WN waves.
// Each wave owns TM = BM/WM rows of the token matrix: its int8 activation
// fragments go straight from global memory into MFMA registers (16 bytes
// per lane per fragment), prefetched two K-stages ahead, with no LDS round
// trip.  The packed weight tile (BN rows x 16 bytes per 64-wide stage) is
// loaded once per workgroup, decoded to signed int8 and written to a
// double-buffered LDS tile (rows padded to 80 bytes so that 128-bit reads of
// eight consecutive rows touch disjoint banks); every wave reads its weight
// fragments from there.  Launch bounds allow two workgroups per CU, so one
// can compute while the other waits on memory.  Workgroup ids are mapped so
// that the workgroups resident on one XCD (ids congruent mod 8) share weight
// columns in that XCD's L2.  The epilogue applies y = acc * gamma * sx in
// fp32 and writes fp32, bf16 (round to nearest even) or the raw int32
// accumulator.

#include <type_traits>

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kBK = 64;
constexpr int kLD = kBK + 16;  // LDS row stride in bytes
constexpr int kXcds = 8;

template <bool ALIGNED>
__device__ inline v4i load_a_frag(const uint8_t* row, int64_t k, int64_t K, bool ok) {
  if (ALIGNED) {
    if (ok && k < K) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + k);
      v4i a;
      a.x = static_cast<int>(u.x);
      a.y = static_cast<int>(u.y);
      a.z = static_cast<int>(u.z);
      a.w = static_cast<int>(u.w);
      return a;
    }
    return v4i{0, 0, 0, 0};
  }
  int w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t kk = k + 4 * i + b;
      v |= static_cast<uint32_t>((ok && kk < K) ? row[kk] : 0u) << (8 * b);
    }
    w[i] = static_cast<int>(v);
  }
  return v4i{w[0], w[1], w[2], w[3]};
}

// one packed word (16 codes) at byte offset `kb` of a row with `rowbytes`
// bytes; bytes past the row read as zero codes (0x55)
template <bool ALIGNED>
__device__ inline uint32_t load_b_word(const uint8_t* row, int64_t kb, int64_t rowbytes,
                                       bool ok) {
  if (ALIGNED) {
    if (ok && kb < rowbytes) return *reinterpret_cast<const uint32_t*>(row + kb);
    return 0x55555555u;
  }
  uint32_t v = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t o = kb + b;
    v |= static_cast<uint32_t>((ok && o < rowbytes) ? row[o] : 0x55u) << (8 * b);
  }
  return v;
}

template <int BM, int BN, int WM, int WN, bool ALIGNED, int YT>
__global__ __launch_bounds__(WM* WN* kWave, 2) void k_gemm(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y) {
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CB = BN * 4 / NT;  // packed words per thread per stage
  static_assert(CB >= 1 && FM >= 1 && FN >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kLD];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  // ids congruent mod 8 run on one XCD: give them neighbouring weight columns
  const int64_t bid = blockIdx.x;
  const int64_t local = bid / kXcds;
  const int64_t tm = local % tiles_m;
  const int64_t tn = (local / tiles_m) * kXcds + bid % kXcds;
  if (tn >= tiles_n) return;  // padding ids (whole workgroup)
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K >> 2;
  const int fr = lane & 31, kg = lane >> 5;

  // activation rows of this lane's fragments
  const uint8_t* arow[FM];
  bool aok[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * TM + 32 * i + fr;
    aok[i] = m < M;
    arow[i] = reinterpret_cast<const uint8_t*>(q) + (aok[i] ? m : 0) * K;
  }
  // A fragments of a stage: [i][ks] for the two 32-wide K steps.  Three
  // register sets rotate (current stage, and two stages in flight); the loop
  // is unrolled by three so that every set is addressed statically.
  typedef v4i AFrags[FM][2];
  AFrags ra0, ra1, ra2;
  auto load_a = [&](int64_t kt, AFrags& dst) {
    const int64_t k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        dst[i][ks] = load_a_frag<ALIGNED>(arow[i], k0 + 32 * ks + 16 * kg, K, aok[i]);
  };
  uint32_t rb[CB];
  auto load_b = [&](int64_t kt) {
    const int64_t kb0 = kt * (kBK / 4);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, wi = c & 3;
      const int64_t n = n0 + r;
      const bool ok = n < N;
      rb[i] = load_b_word<ALIGNED>(packed + (ok ? n : 0) * rowbytes, kb0 + 4 * wi, rowbytes,
                                   ok);
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, wi = c & 3;
      *reinterpret_cast<v4i*>(&Bs[buf][r * kLD + 16 * wi]) = decode_signed_natural(rb[i]);
    }
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int64_t nk = (K + kBK - 1) / kBK;
  // one K stage: prefetch A two stages ahead and B one stage ahead, contract
  // the current stage, then publish the next B tile
  auto stage = [&](int64_t kt, AFrags& cur, AFrags& ahead) {
    const int buf = static_cast<int>(kt & 1);
    if (kt + 2 < nk) load_a(kt + 2, ahead);
    if (kt + 1 < nk) load_b(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i b[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const v4i*>(
            &Bs[buf][(wn * TN + 32 * j + fr) * kLD + 32 * ks + 16 * kg]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur[i][ks], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_b(buf ^ 1);
    __syncthreads();
  };

  load_a(0, ra0);
  if (nk > 1) load_a(1, ra1);
  load_b(0);
  store_b(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; kt += 3) {
    stage(kt, ra0, ra2);
    if (kt + 1 < nk) stage(kt + 1, ra1, ra0);
    if (kt + 2 < nk) stage(kt + 2, ra2, ra1);
  }

  // D layout of the 32x32 MFMA: lane l holds column l%32 and rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + 32 * j + fr;
    if (n >= N) continue;
    const float gam = YT == TQ_I32 ? 0.f : scale[per_row ? n : 0];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * TM + 32 * i + 8 * (v / 4) + 4 * kg + (v % 4);
        if (m >= M) continue;
        const int64_t o = m * N + n;
        const int accv = acc[i][j][v];
        if (YT == TQ_I32) {
          static_cast<int*>(Y)[o] = accv;
        } else {
          const float y = static_cast<float>(accv) * (gam * sx[m]);
          if (YT == TQ_F32)
            static_cast<float*>(Y)[o] = y;
          else
            static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// Fast path (K % 64 == 0, 16-byte aligned operands, both operands below
// 2 GiB).  Both operand tiles pass through LDS:
//   - activations: every 16-byte load of a stage covers 16 rows x 64
//     contiguous bytes (four lanes per row), the widest pattern a 64-wide
//     stage allows; an MFMA fragment loaded straight from global memory
//     would touch 32 rows (32 cache lines) per instruction, and on gfx950
//     the address path is limited by lines per instruction, not bytes;
//   - packed weights: one 32-bit word (16 codes) per lane, decoded to signed
//     int8 once per workgroup.
// Small grids (fewer than 384 tiles of 128 x 128) use 128 x 64 tiles with
// two groups of four waves: a stage holds 128 of K, each group contracts one
// 64-deep half, and the two int32 sums meet in LDS at the end, so a tile gets
// eight waves instead of four.
// Global loads are raw buffer loads whose per-lane offset is fixed for the
// K loop and whose K position rides in the scalar offset (no address
// arithmetic in the loop; reads past the end return zero).  Loads run two
// stages ahead in registers; each stage stores the next stage's tiles into
// the other half of a double-buffered LDS tile.  LDS rows are 64 bytes with
// the four 16-byte chunks XOR-swizzled by ((row >> 1) ^ (row >> 4)) & 3:
// measured on gfx950 with the LDS bank-conflict counter, this is free of
// conflicts for the tile stores (four lanes per row) and for the MFMA
// fragment reads of both 32-wide K steps (32 rows, two chunks).  Fragment reads for the next 32-wide K step are issued
// before the MFMAs of the current one.

constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kKS = kBK / 32;          // MFMA K steps per stage

__device__ inline int swz(int row, int chunk) {
  return row * kBK + 16 * (chunk ^ (((row >> 1) ^ (row >> 4)) & 3));
}

// LDS bytes of one BM x BN tile: double-buffered activation and weight tiles
// of KG 64-deep sub-tiles each.
template <int BM, int BN, int KG = 1>
constexpr int fast_lds_bytes() { return 2 * KG * (BM + BN) * kBK; }

// One BM x BN output tile (tile coordinates tm, tn in units of BM, BN) by a
// workgroup of KG groups of WM x WN waves, staging through `lds`.  A stage
// covers KG x 64 of K; group g contracts the stage's 64-deep sub-tile g into
// its own accumulators, and the groups' sums meet in LDS at the end (exact
// int32 additions).  KG = 2 gives small grids twice the waves per tile.
template <int BM, int BN, int WM, int WN, int YT, int KG = 1>
__device__ __forceinline__ void gemm_fast_tile(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y, int64_t tm, int64_t tn, uint8_t* lds) {
  constexpr int NW = WM * WN;                 // waves per group
  constexpr int NT = NW * KG * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CPR = KG * (kBK / 16);       // 16-byte chunks per row and stage
  constexpr int CA = BM * CPR / NT;          // 16-byte activation chunks per thread
  constexpr int CB = BN * CPR / NT;          // packed words per thread
  constexpr int ASZ = BM * kBK, BSZ = BN * kBK;  // bytes of one 64-deep sub-tile
  static_assert(CA >= 1 && CB >= 1 && FM >= 1 && FN >= 1, "tile shape");
  static_assert(KG == 1 || NW * FM * FN * 16 * kWave * 4 <= 2 * KG * (ASZ + BSZ),
                "group sums must fit in the staging LDS");
  constexpr int SA = KG * ASZ, SB = KG * BSZ;  // bytes of one stage
  uint8_t* const As = lds;                     // [2][KG][BM * kBK]
  uint8_t* const Bs = lds + 2 * SA;            // [2][KG][BN * kBK]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform in the wave
  const int grp = wave / NW, wl = wave % NW;
  const int wm = wl / WN, wn = wl % WN;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K >> 2;
  const int fr = lane & 31, kg = lane >> 5;

  const __amdgpu_buffer_rsrc_t ra_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q), static_cast<short>(0), static_cast<int>(M * K), kBufFlags);
  const __amdgpu_buffer_rsrc_t rb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed), static_cast<short>(0), static_cast<int>(N * rowbytes),
      kBufFlags);
  // per-thread global offsets and LDS slots, fixed for the K loop
  uint32_t aoff[CA];
  int ast[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + NT * i;
    const int r = c / CPR, ch = c % CPR;
    aoff[i] = static_cast<uint32_t>((m0 + r) * K + 16 * ch);
    ast[i] = (ch / 4) * ASZ + swz(r, ch % 4);
  }
  uint32_t boff[CB];
  int bst[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + NT * i;
    const int r = c / CPR, wi = c % CPR;
    boff[i] = static_cast<uint32_t>((n0 + r) * rowbytes + 4 * wi);
    bst[i] = (wi / 4) * BSZ + swz(r, wi % 4);
  }
  // this group's fragments: sub-tile grp of each stage
  int ard[FM][kKS], brd[FN][kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i) ard[i][ks] = grp * ASZ + swz(wm * TM + 32 * i + fr, 2 * ks + kg);
#pragma unroll
    for (int j = 0; j < FN; ++j) brd[j][ks] = grp * BSZ + swz(wn * TN + 32 * j + fr, 2 * ks + kg);
  }

  typedef v4i ARegs[CA];
  typedef uint32_t BRegs[CB];
  ARegs ra0, ra1, ra2;
  BRegs rb0, rb1, rb2;
  auto load_stage = [&](int64_t kt, ARegs& a, BRegs& b) {
    const int soa = static_cast<int>(kt * kBK * KG), sob = static_cast<int>(kt * (kBK / 4) * KG);
#pragma unroll
    for (int i = 0; i < CA; ++i)
      a[i] = __builtin_bit_cast(v4i,
                                __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff[i], soa, 0));
#pragma unroll
    for (int i = 0; i < CB; ++i) b[i] = __builtin_amdgcn_raw_buffer_load_b32(rb_rsrc, boff[i], sob, 0);
  };
  auto store_stage = [&](int buf, ARegs& a, BRegs& b) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<v4i*>(&As[(buf) * SA + ast[i]]) = a[i];
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *reinterpret_cast<v4i*>(&Bs[(buf) * SB + bst[i]]) = decode_signed_natural(b[i]);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int64_t nk = K / (kBK * KG);
  // one stage: start the loads of stage kt+2, contract stage kt from LDS,
  // publish stage kt+1 (loaded during the previous stage).  In the main loop
  // (GUARD false) every stage issues its loads and stores unconditionally:
  // a branch around the loads would leave the compiler unable to count the
  // loads in flight, and it would then wait for all of them, the ones just
  // issued included.  Loads past stage nk-1 read zeros or data that is never
  // stored; a store of stage nk goes to the LDS half no later stage reads.
  auto stage = [&](int64_t kt, ARegs& a_next, BRegs& b_next, ARegs& a_far, BRegs& b_far,
                   auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    const int buf = static_cast<int>(kt & 1);
    if (!GUARD || kt + 2 < nk) load_stage(kt + 2, a_far, b_far);
    v4i ac[FM], an[FM], bc[FN], bn[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ac[i] = *reinterpret_cast<const v4i*>(&As[(buf) * SA + ard[i][0]]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bc[j] = *reinterpret_cast<const v4i*>(&Bs[(buf) * SB + brd[j][0]]);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks + 1 < kKS) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          an[i] = *reinterpret_cast<const v4i*>(&As[(buf) * SA + ard[i][ks + 1]]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bn[j] = *reinterpret_cast<const v4i*>(&Bs[(buf) * SB + brd[j][ks + 1]]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ac[i], bc[j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < FM; ++i) ac[i] = an[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) bc[j] = bn[j];
    }
    // keep the decode of stage kt+1 here: hoisted above the MFMAs it would
    // wait for that stage's loads one stage early
    __builtin_amdgcn_sched_barrier(0);
    if (!GUARD || kt + 1 < nk) store_stage(buf ^ 1, a_next, b_next);
    __syncthreads();
  };
  using Free = std::false_type;
  using Guarded = std::true_type;

  load_stage(0, ra0, rb0);
  load_stage(1, ra1, rb1);
  store_stage(0, ra0, rb0);
  __syncthreads();
  // register sets rotate with period three: stage kt reads set (kt+1)%3 and
  // fills set (kt+2)%3
  int64_t kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    stage(kt, ra1, rb1, ra2, rb2, Free{});
    stage(kt + 1, ra2, rb2, ra0, rb0, Free{});
    stage(kt + 2, ra0, rb0, ra1, rb1, Free{});
  }
  if (kt < nk) stage(kt, ra1, rb1, ra2, rb2, Guarded{});
  if (kt + 1 < nk) stage(kt + 1, ra2, rb2, ra0, rb0, Guarded{});

  if constexpr (KG > 1) {
    // groups 1.. leave their sums in LDS (the staging tiles are free after
    // the last stage's barrier); group 0 adds them in group order
    int* const red = reinterpret_cast<int*>(lds);
    const int slot = (wl * FM * FN) * 16 * kWave + lane;
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            red[(grp - 1) * NW * FM * FN * 16 * kWave + slot + ((i * FN + j) * 16 + v) * kWave] =
                acc[i][j][v];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[i][j][v] +=
                red[(g - 1) * NW * FM * FN * 16 * kWave + slot + ((i * FN + j) * 16 + v) * kWave];
  }

  // D layout of the 32x32 MFMA: lane l holds column l%32 and rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + 32 * j + fr;
    if (n >= N) continue;
    const float gam = YT == TQ_I32 ? 0.f : scale[per_row ? n : 0];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * TM + 32 * i + 8 * (v / 4) + 4 * kg + (v % 4);
        if (m >= M) continue;
        const int64_t o = m * N + n;
        const int accv = acc[i][j][v];
        if (YT == TQ_I32) {
          static_cast<int*>(Y)[o] = accv;
        } else {
          const float y = static_cast<float>(accv) * (gam * sx[m]);
          if (YT == TQ_F32)
            static_cast<float*>(Y)[o] = y;
          else
            static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int YT, int KG>
__global__ __launch_bounds__(WM* WN* KG* kWave, 2) void k_gemm_fast(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[fast_lds_bytes<BM, BN, KG>()];
  const int64_t tiles_m = (M + BM - 1) / BM;
  gemm_fast_tile<BM, BN, WM, WN, YT, KG>(q, sx, M, packed, scale, per_row, N, K, Y,
                                         blockIdx.x % tiles_m, blockIdx.x / tiles_m, lds);
}

template <int BM, int BN, int WM, int WN, int KG = 1>
hipError_t gemm_fast_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int NT = WM * WN * KG * kWave;
#define TQ_GEMM_FAST(YTV)                                                                      \
  hipLaunchKernelGGL((k_gemm_fast<BM, BN, WM, WN, YTV, KG>), dim3(grid), dim3(NT), 0, s, a.q, \
                     a.sx, a.M, a.packed, a.scale, a.per_row, a.N, a.K, a.Y)
  if (a.ydt == TQ_F32) TQ_GEMM_FAST(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMM_FAST(TQ_BF16);
  else TQ_GEMM_FAST(TQ_I32);
#undef TQ_GEMM_FAST
  return hipGetLastError();
}

hipError_t gemm_fast_dispatch(const GemmArgs& a, hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  constexpr int64_t kEnough = 384;
  if (tiles(256, 128) >= kEnough) return gemm_fast_launch<256, 128, 4, 2>(a, s);
  if (tiles(128, 128) >= kEnough) return gemm_fast_launch<128, 128, 2, 2>(a, s);
  // small grids: two wave groups split each 128-deep stage (needs K % 128)
  if (a.K % 128 == 0) return gemm_fast_launch<128, 64, 4, 1, 2>(a, s);
  return gemm_fast_launch<128, 64, 4, 1>(a, s);
}

template <int BM, int BN, int WM, int WN, bool ALIGNED>
hipError_t gemm_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t tiles_n = (a.N + BN - 1) / BN;
  const int64_t grid = tiles_m * ((tiles_n + kXcds - 1) / kXcds) * kXcds;
  constexpr int NT = WM * WN * kWave;
#define TQ_GEMM(YTV)                                                                    \
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, ALIGNED, YTV>), dim3(grid), dim3(NT), 0, s, \
                     a.q, a.sx, a.M, a.packed, a.scale, a.per_row, a.N, a.K, a.Y)
  if (a.ydt == TQ_F32) TQ_GEMM(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMM(TQ_BF16);
  else TQ_GEMM(TQ_I32);
#undef TQ_GEMM
  return hipGetLastError();
}

template <bool ALIGNED>
hipError_t gemm_dispatch(const GemmArgs& a, hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  constexpr int64_t kEnough = 384;  // 1.5 workgroups per CU on 256 CUs
  if (tiles(256, 128) >= kEnough) return gemm_launch<256, 128, 4, 1, ALIGNED>(a, s);
  if (tiles(128, 128) >= kEnough) return gemm_launch<128, 128, 4, 1, ALIGNED>(a, s);
  return gemm_launch<128, 64, 4, 1, ALIGNED>(a, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  const bool aligned = (a.K % 64) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.packed) & 15u) == 0u &&
                       (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0u;
  // buffer offsets are 32-bit: rows up to one tile past the end must stay
  // below 2^31 bytes
  constexpr int64_t kLim = int64_t{1} << 31;
  const bool small = (a.M + 256) * a.K < kLim && (a.N + 256) * (a.K / 4) < kLim;
  if (aligned && small) return gemm_fast_dispatch(a, s);
  return aligned ? gemm_dispatch<true>(a, s) : gemm_dispatch<false>(a, s);
}

}  // namespace tq
