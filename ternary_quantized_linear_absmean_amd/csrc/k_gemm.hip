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
// Four kernels, picked by shape:
//   - k_gemm_reg (K % 128 == 0, aligned, at most one 32 x 64 tile per CU):
//     four waves split K over one tile, operands in registers several
//     blocks ahead, tokens re-laid through a private LDS slot per wave and
//     codes decoded per product (to 0..2, with the token sums subtracted);
//   - k_gemm_fast (K % 64 == 0, aligned): both operand tiles staged through a
//     double-buffered, swizzled LDS tile, eight- or four-wave workgroups,
//     two workgroups per CU (see the fast-path notes below);
//   - k_gemm_wide (K % 256 == 0, aligned, every round of 256 x 256 tiles at
//     least half full): 256 x 256 per workgroup of four 128 x 128 waves, one
//     workgroup per CU, half the LDS reads per MFMA of the fast tiles;
//   - k_gemm (any shape): each wave owns TM = BM/WM token rows whose int8
//     fragments go straight from global memory into MFMA registers (byte
//     loads where K or the pointers are unaligned); the packed weight tile is
//     decoded to signed int8 into a double-buffered LDS tile with 80-byte rows.
// In k_gemm, workgroup ids are mapped so that the workgroups resident on one
// XCD (ids congruent mod 8) share weight columns in that XCD's L2; the fast
// and wide kernels take tiles with the token-row index fastest.  The epilogue
// applies y = acc * gamma * sx in fp32 and writes fp32, bf16 (round to
// nearest even) or the raw int32 accumulator.  The fast and wide kernels
// pass each wave's tile through LDS so that every lane stores 16 contiguous
// bytes (8 for bf16): element-wise stores straight from the MFMA layout cost
// more than the main loop's last third.

#include <type_traits>
#include <utility>

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kBK = 64;
constexpr int kLD = kBK + 16;  // LDS row stride in bytes
constexpr int kXcds = 8;

// Tile of workgroup `bid` for the fast and wide kernels.  Workgroup ids are
// handed to the eight XCDs round-robin (ids congruent mod 8 share an XCD and
// its L2), so XCD x takes a contiguous share of the tiles in an order that
// walks gm token-row tiles fastest inside each column: its share is a patch
// of about gm token-row slabs by T/(8 gm) weight-column slabs, and each L2
// streams only that patch's operands instead of every weight column.  The
// map is a bijection of [0, T) onto the tiles.
__device__ inline void xcd_tile(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t gm,
                                int64_t& tm, int64_t& tn) {
  const int64_t T = tiles_m * tiles_n;
  const int64_t x = bid % kXcds, li = bid / kXcds;
  const int64_t per = T / kXcds, extra = T % kXcds;
  const int64_t t = x * per + (x < extra ? x : extra) + li;
  const int64_t g = t / (gm * tiles_n);            // group of gm token-row tiles
  const int64_t m_first = g * gm;
  const int64_t rows = tiles_m - m_first < gm ? tiles_m - m_first : gm;
  const int64_t r = t - g * gm * tiles_n;
  tm = m_first + r % rows;
  tn = r / rows;
}

// Group size for xcd_tile: the gm in 1..min(tiles_m, 16) whose map gives the
// eight XCDs the fewest operand bytes per K step in all (an XCD's share
// counts gm-row token slabs at BM bytes and weight-column slabs at BN / 4
// bytes; a share that spans two groups counts the slabs of each piece).
inline int64_t xcd_group_m(int64_t tiles_m, int64_t tiles_n, int BM, int BN) {
  const int64_t T = tiles_m * tiles_n, per = T / kXcds, extra = T % kXcds;
  int64_t best = 1, best_cost = INT64_MAX;
  for (int64_t g = 1; g <= tiles_m && g <= 16; ++g) {
    int64_t cost = 0;
    for (int64_t x = 0; x < kXcds; ++x) {
      int64_t t = x * per + (x < extra ? x : extra);
      const int64_t end = t + per + (x < extra ? 1 : 0);
      while (t < end) {  // one piece per group the share touches
        const int64_t grp = t / (g * tiles_n), first = grp * g * tiles_n;
        const int64_t rows = tiles_m - grp * g < g ? tiles_m - grp * g : g;
        const int64_t stop = first + rows * tiles_n < end ? first + rows * tiles_n : end;
        const int64_t r0 = t - first, r1 = stop - first;
        const int64_t nm = r1 - r0 >= rows ? rows : r1 - r0;
        const int64_t nn = (r1 - 1) / rows - r0 / rows + 1;
        cost += nm * BM + nn * (BN / 4);
        t = stop;
      }
    }
    if (cost < best_cost) { best_cost = cost; best = g; }
  }
  return best;
}

// Epilogue of a wave holding FM x FN accumulators of the 32x32 MFMA, whose
// top-left output is (mb, nb).  D layout: lane l holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.  y = acc * (gamma * sx) in fp32,
// stored as fp32, bf16 (round to nearest even) or the raw int32.  Stores and
// loads share one memory counter on this chip, so a load issued between two
// stores would wait for every store before it: all scale factors are loaded
// first (rows and columns past the end read the last valid one and are not
// stored).
template <int YT, int FM, int FN>
__device__ inline void store_acc32(const v16i (&acc)[FM][FN], int64_t mb, int64_t nb, int lane,
                                   const float* __restrict__ sx,
                                   const float* __restrict__ scale, int per_row, int64_t M,
                                   int64_t N, void* __restrict__ Y) {
  const int fr = lane & 31, kg = lane >> 5;
  float sv[FM][16], gv[FN];
  if (YT != TQ_I32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mb + 32 * i + 8 * (v / 4) + 4 * kg + (v % 4);
        sv[i][v] = sx[m < M ? m : M - 1];
      }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = nb + 32 * j + fr;
      gv[j] = scale[per_row ? (n < N ? n : N - 1) : 0];
    }
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = nb + 32 * j + fr;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mb + 32 * i + 8 * (v / 4) + 4 * kg + (v % 4);
        if (m >= M) continue;
        const int64_t o = m * N + n;
        const int accv = acc[i][j][v];
        if (YT == TQ_I32) {
          static_cast<int*>(Y)[o] = accv;
        } else {
          const float y = static_cast<float>(accv) * (gv[j] * sv[i][v]);
          if (YT == TQ_F32)
            static_cast<float*>(Y)[o] = y;
          else
            static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
        }
      }
    }
  }
}

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

  store_acc32<YT>(acc, m0 + wm * TM, n0 + wn * TN, lane, sx, scale, per_row, M, N, Y);
}

// The same epilogue staged through LDS, for a wave with FM x FN fragments
// and a private LDS area of 32 x (32 FN + 8) words.  Each 32-row block of the
// wave tile goes into LDS as raw int32 (lanes 0..31 and 32..63 land on
// disjoint banks), then is read back four columns per lane, so that every
// lane stores 16 contiguous bytes (8 for bf16) instead of single elements.
// The row factors sx and column factors gamma of the wave tile are read from
// LDS copies (sxl[r], gml[c] for tile row r and column c), so that no global
// load sits between the stores.
template <int FN>
constexpr int staged_lds_words() { return 32 * (32 * FN + 8); }

// The output is written once and not read again by the kernel: its 16-byte
// stores are non-temporal (measured 3% faster at 4096^3, 7% at 512 x 4096 x
// 4096, where every tile's epilogue falls in the same few microseconds).
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

template <int YT, int FM, int FN>
__device__ inline void store_acc32_staged(const v16i (&acc)[FM][FN], int64_t mb, int64_t nb,
                                          int lane, const float* sxl, const float* gml,
                                          int64_t M, int64_t N, void* __restrict__ Y,
                                          int* buf) {
  constexpr int W = 32 * FN;    // columns of the wave tile
  constexpr int LDW = W + 8;    // LDS row stride in words
  constexpr int CPR = W / 4;    // four-column chunks per row
  constexpr int RPI = 64 / CPR; // rows one wave-wide pass covers
  constexpr int T = 32 / RPI;   // passes per 32-row block
  const int fr = lane & 31, kg = lane >> 5;
  const int c4 = lane % CPR, rr = lane / CPR;
  const int64_t n = nb + 4 * c4;
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15u) == 0;
  float gv[4] = {0.f, 0.f, 0.f, 0.f};
  if (YT != TQ_I32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[e] = gml[4 * c4 + e];
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        buf[(8 * (v / 4) + 4 * kg + (v % 4)) * LDW + 32 * j + fr] = acc[i][j][v];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    v4i av[T];
    float sv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      av[t] = *reinterpret_cast<const v4i*>(buf + (RPI * t + rr) * LDW + 4 * c4);
      sv[t] = YT == TQ_I32 ? 0.f : sxl[32 * i + RPI * t + rr];
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t m = mb + 32 * i + RPI * t + rr;
      const v4i a = av[t];
      if (m >= M || n >= N) continue;
      const int64_t o = m * N + n;
      if (YT == TQ_I32) {
        if (vec && n + 3 < N) {
          __builtin_nontemporal_store(a, reinterpret_cast<v4i*>(static_cast<int*>(Y) + o));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) static_cast<int*>(Y)[o + e] = a[e];
        }
      } else {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = static_cast<float>(a[e]) * (gv[e] * sv[t]);
        if (YT == TQ_F32) {
          if (vec && n + 3 < N) {
            const v4f t = {y[0], y[1], y[2], y[3]};
            __builtin_nontemporal_store(t, reinterpret_cast<v4f*>(static_cast<float*>(Y) + o));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) static_cast<float*>(Y)[o + e] = y[e];
          }
        } else {
          if (vec && n + 3 < N) {
            const v2u t = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            __builtin_nontemporal_store(t, reinterpret_cast<v2u*>(static_cast<uint16_t*>(Y) + o));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) static_cast<uint16_t*>(Y)[o + e] = f32_to_bf16(y[e]);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
// the other half of a double-buffered LDS tile, both spread over the
// stage's MFMAs.  LDS rows are 64 bytes with the four 16-byte chunks
// XOR-swizzled by ((row >> 1) ^ (row >> 4)) & 3: measured on gfx950 with the
// LDS bank-conflict counter, this is free of conflicts for the tile stores
// (four lanes per row) and for the MFMA fragment reads of both 32-wide K
// steps (32 rows, two chunks).  Fragment reads for the next 32-wide K step
// are issued before the MFMAs of the current one.

constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kKS = kBK / 32;          // MFMA K steps per stage

template <int I>
using ic = std::integral_constant<int, I>;
// f(ic<0>{}), ..., f(ic<N-1>{}) in order
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(ic<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ inline int swz(int row, int chunk) {
  return row * kBK + 16 * (chunk ^ (((row >> 1) ^ (row >> 4)) & 3));
}

// LDS bytes of one BM x BN tile: double-buffered activation and weight tiles
// of KG 64-deep sub-tiles each.
template <int BM, int BN, int KG = 1>
constexpr int fast_lds_bytes() { return 2 * KG * (BM + BN) * kBK; }
template <int BM, int BN, int WM, int WN>
constexpr int fast_epi_bytes() {
  return (WM * WN * staged_lds_words<BN / WN / 32>() + BM + BN) * 4;
}
template <int BM, int BN, int WM, int WN, int KG>
constexpr int fast_lds_size() {
  return fast_lds_bytes<BM, BN, KG>() > fast_epi_bytes<BM, BN, WM, WN>()
             ? fast_lds_bytes<BM, BN, KG>()
             : fast_epi_bytes<BM, BN, WM, WN>();
}

// One BM x BN output tile (tile coordinates tm, tn in units of BM, BN) by a
// workgroup of KG groups of WM x WN waves, staging through `lds`.  A stage
// covers KG x 64 of K; group g contracts the stage's 64-deep sub-tile g into
// its own accumulators, and the groups' sums meet in LDS at the end (exact
// int32 additions).  KG = 2 gives small grids twice the waves per tile.
// The loads of stage kt+D go out while stage kt is contracted, so D-1 stages
// of compute cover a load's latency; D+1 register sets hold the stages in
// flight.
template <int BM, int BN, int WM, int WN, int YT, int KG = 1, int D = 2>
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
  // per-thread global offsets and LDS slots, fixed for the K loop.  Chunks
  // are numbered sub-tile by sub-tile, four to a row: the 16 lanes of a
  // quarter-wave store four consecutive rows of one sub-tile, a pattern free
  // of bank conflicts under the swizzle.  (Rows of two sub-tiles lie a
  // multiple of 256 bytes apart, on the same banks.)
  uint32_t aoff[CA];
  int ast[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + NT * i;
    const int sub = c / (4 * BM), r = (c / 4) % BM, cc = c % 4;
    aoff[i] = static_cast<uint32_t>((m0 + r) * K + 64 * sub + 16 * cc);
    ast[i] = sub * ASZ + swz(r, cc);
  }
  uint32_t boff[CB];
  int bst[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + NT * i;
    const int sub = c / (4 * BN), r = (c / 4) % BN, cc = c % 4;
    boff[i] = static_cast<uint32_t>((n0 + r) * rowbytes + 16 * sub + 4 * cc);
    bst[i] = sub * BSZ + swz(r, cc);
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
  constexpr int P = D + 1;
  static_assert(D >= 2 && D <= 5, "load distance");
  // named sets, picked by compile-time index (an array of sets allocates
  // worse once the loop is unrolled)
  ARegs ra0, ra1, ra2, ra3, ra4, ra5;
  BRegs rb0, rb1, rb2, rb3, rb4, rb5;
  auto aset = [&](auto I) -> ARegs& {
    constexpr int i = decltype(I)::value % P;
    if constexpr (i == 0) return ra0;
    else if constexpr (i == 1) return ra1;
    else if constexpr (i == 2) return ra2;
    else if constexpr (i == 3) return ra3;
    else if constexpr (i == 4) return ra4;
    else return ra5;
  };
  auto bset = [&](auto I) -> BRegs& {
    constexpr int i = decltype(I)::value % P;
    if constexpr (i == 0) return rb0;
    else if constexpr (i == 1) return rb1;
    else if constexpr (i == 2) return rb2;
    else if constexpr (i == 3) return rb3;
    else if constexpr (i == 4) return rb4;
    else return rb5;
  };
  // piece p of a stage: p < CA an activation chunk, else a packed word
  auto load_piece = [&](int64_t kt, ARegs& a, BRegs& b, int p) {
    const int soa = static_cast<int>(kt * kBK * KG), sob = static_cast<int>(kt * (kBK / 4) * KG);
    if (p < CA)
      a[p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff[p], soa, 0));
    else
      b[p - CA] = __builtin_amdgcn_raw_buffer_load_b32(rb_rsrc, boff[p - CA], sob, 0);
  };
  auto store_piece = [&](int buf, ARegs& a, BRegs& b, int p) {
    if (p < CA)
      *reinterpret_cast<v4i*>(&As[(buf) * SA + ast[p]]) = a[p];
    else
      *reinterpret_cast<v4i*>(&Bs[(buf) * SB + bst[p - CA]]) = decode_signed_natural(b[p - CA]);
  };
  auto load_stage = [&](int64_t kt, ARegs& a, BRegs& b) {
#pragma unroll
    for (int p = 0; p < CA + CB; ++p) load_piece(kt, a, b, p);
  };
  auto store_stage = [&](int buf, ARegs& a, BRegs& b) {
#pragma unroll
    for (int p = 0; p < CA + CB; ++p) store_piece(buf, a, b, p);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int64_t nk = K / (kBK * KG);
  // one stage: contract stage kt from LDS, move stage kt+1 (loaded D-1
  // stages earlier) from registers into the other LDS half, load stage
  // kt+D.  The pieces of the move and the loads go out after each group of
  // FN products, so that neither arrives in one burst from every wave.  In
  // the main loop (GUARD false) every stage issues its
  // loads and stores unconditionally: a branch around the loads would leave
  // the compiler unable to count the loads in flight, and it would then wait
  // for all of them, the ones just issued included.  Loads past stage nk-1
  // read zeros or data that is never stored; a store of stage nk goes to the
  // LDS half no later stage reads.
  constexpr int kGroups = kKS * FM, kPieces = CA + CB;
  auto stage = [&](int64_t kt, ARegs& a_next, BRegs& b_next, ARegs& a_far, BRegs& b_far,
                   auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    const int buf = static_cast<int>(kt & 1);
    const bool do_load = !GUARD || kt + D < nk, do_store = !GUARD || kt + 1 < nk;
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
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ac[i], bc[j], acc[i][j], 0, 0, 0);
        const int g = ks * FM + i;
#pragma unroll
        for (int p = g; p < kPieces; p += kGroups) {
          if (do_store) store_piece(buf ^ 1, a_next, b_next, p);
          if (do_load) load_piece(kt + D, a_far, b_far, p);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) ac[i] = an[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) bc[j] = bn[j];
    }
    __syncthreads();
  };
  using Free = std::false_type;
  using Guarded = std::true_type;

  static_for<D>([&](auto J) { load_stage(J.value, aset(J), bset(J)); });
  store_stage(0, ra0, rb0);
  __syncthreads();
  // register sets rotate with period P: stage kt reads set (kt+1)%P and
  // fills set (kt+D)%P
  int64_t kt = 0;
  for (; kt + P <= nk; kt += P) {
    static_for<P>([&](auto J) {
      stage(kt + J.value, aset(ic<J.value + 1>{}), bset(ic<J.value + 1>{}), aset(ic<J.value + D>{}),
            bset(ic<J.value + D>{}), Free{});
    });
  }
  static_for<P - 1>([&](auto J) {
    if (kt + J.value < nk)
      stage(kt + J.value, aset(ic<J.value + 1>{}), bset(ic<J.value + 1>{}), aset(ic<J.value + D>{}),
            bset(ic<J.value + D>{}), Guarded{});
  });

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
    if (grp == 0) {
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
  }

  // staged epilogue: the wave areas, then the tile's row and column factors
  // (every wave is past its last LDS read once the barrier below is passed)
  static_assert(fast_epi_bytes<BM, BN, WM, WN>() <= fast_lds_size<BM, BN, WM, WN, KG>(),
                "epilogue LDS");
  int* const ep = reinterpret_cast<int*>(lds);
  float* const sxs = reinterpret_cast<float*>(ep + NW * staged_lds_words<FN>());
  float* const gms = sxs + BM;
  __syncthreads();
  if (YT != TQ_I32) {
    for (int r = tid; r < BM; r += NT) {
      const int64_t m = m0 + r;
      sxs[r] = sx[m < M ? m : M - 1];
    }
    for (int c = tid; c < BN; c += NT) {
      const int64_t n = n0 + c;
      gms[c] = scale[per_row ? (n < N ? n : N - 1) : 0];
    }
  }
  __syncthreads();
  if (grp == 0)
    store_acc32_staged<YT>(acc, m0 + wm * TM, n0 + wn * TN, lane, sxs + wm * TM, gms + wn * TN,
                           M, N, Y, ep + wl * staged_lds_words<FN>());
}

template <int BM, int BN, int WM, int WN, int YT, int KG, int D>
__global__ __launch_bounds__(WM* WN* KG* kWave, WM* WN* KG >= 16 ? 1 : 2) void k_gemm_fast(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y, int64_t gm) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[fast_lds_size<BM, BN, WM, WN, KG>()];
  int64_t tm, tn;
  xcd_tile(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, gm, tm, tn);
  gemm_fast_tile<BM, BN, WM, WN, YT, KG, D>(q, sx, M, packed, scale, per_row, N, K, Y, tm, tn,
                                            lds);
}

template <int BM, int BN, int WM, int WN, int KG = 1, int D = 2>
hipError_t gemm_fast_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t grid = tiles_m * tiles_n;
  const int64_t gm = xcd_group_m(tiles_m, tiles_n, BM, BN);
  constexpr int NT = WM * WN * KG * kWave;
#define TQ_GEMM_FAST(YTV)                                                                      \
  hipLaunchKernelGGL((k_gemm_fast<BM, BN, WM, WN, YTV, KG, D>), dim3(grid), dim3(NT), 0, s, a.q, \
                     a.sx, a.M, a.packed, a.scale, a.per_row, a.N, a.K, a.Y, gm)
  if (a.ydt == TQ_F32) TQ_GEMM_FAST(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMM_FAST(TQ_BF16);
  else TQ_GEMM_FAST(TQ_I32);
#undef TQ_GEMM_FAST
  return hipGetLastError();
}

// Small grids with few token rows (at most one 32 x 64 tile per CU, e.g. 128
// x 4096): the tiles are too few to hide a load's latency behind other
// workgroups, and each tile walks a long K.  Four waves hold the same
// 32 FM x 32 FN tile and split K between them: wave w takes the 128-deep
// blocks w, w + KG, w + 2 KG, ..., keeps D of them in flight in registers,
// and meets the other waves only once, at the end.
//   - tokens: loaded eight lanes to a 128-byte row (16 bytes each, whole
//     cache lines), written into one of the wave's two private LDS slots and
//     read back as MFMA fragments.  A fragment read straight from global
//     memory would touch 32 rows per load, four times the cache-line lookups
//     of the row-wise load; the slot is the wave's own, so no barrier is
//     needed.  Rows are 128 bytes apart and chunk c of row w sits at
//     position c ^ sw(w): both the row writes and the fragment reads (16
//     consecutive rows, one chunk) fall on distinct banks;
//   - codes: lane (r, h) = (l % 32, l / 32) loads the 16 packed bytes of
//     column 32 j + r that cover K offsets 64 h .. 64 h + 63 of the block,
//     and MFMA step s decodes word s of them: the 16 codes of K offsets
//     64 h + 16 s .., the same 16 K values as the token chunk 4 h + s that
//     the lane's fragment holds.  The codes stay 0..2 in the strided order
//     (seven operations per word); each token chunk is byte-transposed to
//     match on its way into the slot, and one more product per step, of the
//     token fragment and an all-ones operand, accumulates the tokens' sums,
//     subtracted at the end: sum q (c - 1).  (Decoding every word to signed
//     values in natural order cost about 23 operations; same-box A/B
//     128 x 4096 x 4096 10.2 -> 9.1 us, 64 x 2560 x 6912 12.8 -> 11.0 us.)
// The products pair equal K values, so the sums are exact whatever order the
// matrix unit takes inside a step.  Loads past a wave's last block go
// through a buffer descriptor of zero size: they return zeros and touch no
// memory, and stay unconditional so that the compiler can count the loads
// in flight.  At the end wave w owns the column fragments [w FN / KG,
// (w + 1) FN / KG) (fragment w when FN < KG), adds the other waves' partial
// sums of them from LDS (exact int32 additions) and stores them with the
// staged epilogue.
constexpr int kRBK = 128;  // K per block

template <int FM, int FN, int KG>
constexpr int reg_own() { return FN >= KG ? FN / KG : 1; }
template <int FM, int FN, int KG>
constexpr int reg_lds_bytes() {
  constexpr int slots = KG * 2 * FM * 32 * kRBK;
  constexpr int red = FN * (KG - 1) * FM * 16 * kWave * 4;
  constexpr int epi = (KG * staged_lds_words<reg_own<FM, FN, KG>()>() + 32 * FM + 32 * FN) * 4;
  return slots > red ? (slots > epi ? slots : epi) : (red > epi ? red : epi);
}

template <int FM, int FN, int KG, int D, int YT>
__global__ __launch_bounds__(KG* kWave) void k_gemm_reg(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y, int64_t gm) {
  constexpr int BM = 32 * FM, BN = 32 * FN;
  constexpr int OWN = reg_own<FM, FN, KG>();
  constexpr int SLOT = FM * 32 * kRBK;  // bytes of one token slot
  static_assert(FN % KG == 0 || KG % FN == 0, "column ownership");
  static_assert(D >= 2 && D <= 5, "blocks in flight");
  __shared__ __attribute__((aligned(16))) uint8_t lds[reg_lds_bytes<FM, FN, KG>()];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int64_t tm, tn;
  xcd_tile(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, gm, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K >> 2;
  const int r = lane & 31, h = lane >> 5;

  const __amdgpu_buffer_rsrc_t ra_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q), static_cast<short>(0), static_cast<int>(M * K), kBufFlags);
  const __amdgpu_buffer_rsrc_t rb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed), static_cast<short>(0), static_cast<int>(N * rowbytes),
      kBufFlags);
  const __amdgpu_buffer_rsrc_t ra_none = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q), static_cast<short>(0), 0, kBufFlags);
  const __amdgpu_buffer_rsrc_t rb_none = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed), static_cast<short>(0), 0, kBufFlags);
  // token chunk t of a block: rows 8t .. 8t+7 of the tile, chunk lane % 8
  auto sw = [](int w) { return (w ^ (w >> 3)) & 7; };
  uint32_t aoff[4 * FM], boff[FN];
  int wst[4 * FM], frd[FM][4];
#pragma unroll
  for (int t = 0; t < 4 * FM; ++t) {
    const int w = 8 * t + lane / 8;
    aoff[t] = static_cast<uint32_t>((m0 + w) * K + 16 * (lane % 8));
    wst[t] = w * kRBK + 16 * ((lane % 8) ^ sw(w));
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int w = 32 * i + r;
      frd[i][s] = w * kRBK + 16 * ((4 * h + s) ^ sw(w));
    }
#pragma unroll
  for (int j = 0; j < FN; ++j)
    boff[j] = static_cast<uint32_t>((n0 + 32 * j + r) * rowbytes + 16 * h);
  const int nb = static_cast<int>(K / kRBK);
  const int nbw = wave < nb ? (nb - wave + KG - 1) / KG : 0;  // this wave's blocks

  v16i acc[FM][FN], acc1[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc1[i][v] = 0;
  }
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  struct Blk {
    v4i a[4 * FM];
    v4i b[FN];
  };
  Blk s0, s1, s2, s3, s4;
  auto set = [&](auto I) -> Blk& {
    constexpr int i = decltype(I)::value % D;
    if constexpr (i == 0) return s0;
    else if constexpr (i == 1) return s1;
    else if constexpr (i == 2) return s2;
    else if constexpr (i == 3) return s3;
    else return s4;
  };
  // block jw of this wave (K offset (wave + KG jw) * 128)
  auto load_blk = [&](int jw, Blk& x) {
    const bool live = jw < nbw;
    const int blk = wave + KG * jw;
    const __amdgpu_buffer_rsrc_t ra = live ? ra_rsrc : ra_none;
    const __amdgpu_buffer_rsrc_t rb = live ? rb_rsrc : rb_none;
    const int sa = live ? blk * kRBK : 0, sb = live ? blk * (kRBK / 4) : 0;
#pragma unroll
    for (int t = 0; t < 4 * FM; ++t)
      x.a[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[t], sa, 0));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      x.b[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, boff[j], sb, 0));
  };
  auto compute_blk = [&](const Blk& x, int jw) {
    uint8_t* const slot = lds + (wave * 2 + (jw & 1)) * SLOT;
#pragma unroll
    for (int t = 0; t < 4 * FM; ++t)
      *reinterpret_cast<v4i*>(slot + wst[t]) = transpose_bytes4x4(
          static_cast<uint32_t>(x.a[t].x), static_cast<uint32_t>(x.a[t].y),
          static_cast<uint32_t>(x.a[t].z), static_cast<uint32_t>(x.a[t].w));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i af[FM], bd[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const v4i*>(slot + frd[i][s]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bd[j] = decode_codes_strided(static_cast<uint32_t>(x.b[j][s]));
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bd[j], acc[i][j], 0, 0, 0);
        acc1[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], ones, acc1[i], 0, 0, 0);
      }
    }
  };

  static_for<D>([&](auto J) { load_blk(J.value, set(J)); });
  int jw = 0;
  // the scheduling barriers keep each block's refill right after its
  // products (left free, the scheduler sinks every load below the last
  // block's products, and each pass then waits for all of them)
  for (; jw + D <= nbw; jw += D) {
    static_for<D>([&](auto J) {
      compute_blk(set(J), jw + J.value);
      __builtin_amdgcn_sched_barrier(0);
      load_blk(jw + J.value + D, set(J));
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  static_for<D - 1>([&](auto J) {
    if (jw + J.value < nbw) compute_blk(set(J), jw + J.value);
  });
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] -= acc1[i];
  __syncthreads();  // the slots overlap the exchange area

  // exchange: every fragment goes to its owner; the others leave it in LDS
  auto owner = [](int j) { return FN >= KG ? j / OWN : j; };
  int* const red = reinterpret_cast<int*>(lds);
  auto slot_of = [&](int j, int w) {  // partial sums of fragment j from wave w
    const int o = owner(j);
    return ((j * (KG - 1) + (w < o ? w : w - 1)) * FM) * 16 * kWave;
  };
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (owner(j) == wave) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[slot_of(j, wave) + (i * 16 + v) * kWave + lane] = acc[i][j][v];
  }
  __syncthreads();
  v16i own[FM][OWN];
  const int j0 = FN >= KG ? wave * OWN : wave;
  const bool owns = j0 < FN;
#pragma unroll
  for (int t = 0; t < OWN; ++t)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      v16i x = acc[i][0];
#pragma unroll
      for (int j = 1; j < FN; ++j)
        if (j == j0 + t) x = acc[i][j];
      if (owns) {
#pragma unroll
        for (int w = 0; w < KG; ++w) {
          if (w == wave) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            x[v] += red[slot_of(j0 + t, w) + (i * 16 + v) * kWave + lane];
        }
      }
      own[i][t] = x;
    }

  // staged epilogue (the exchange area is free once every wave is past it)
  int* const ep = reinterpret_cast<int*>(lds);
  float* const sxs = reinterpret_cast<float*>(ep + KG * staged_lds_words<OWN>());
  float* const gms = sxs + BM;
  __syncthreads();
  if (YT != TQ_I32) {
    for (int x = tid; x < BM; x += KG * kWave) {
      const int64_t m = m0 + x;
      sxs[x] = sx[m < M ? m : M - 1];
    }
    for (int x = tid; x < BN; x += KG * kWave) {
      const int64_t n = n0 + x;
      gms[x] = scale[per_row ? (n < N ? n : N - 1) : 0];
    }
  }
  __syncthreads();
  if (owns)
    store_acc32_staged<YT>(own, m0, n0 + 32 * j0, lane, sxs, gms + 32 * j0, M, N, Y,
                           ep + wave * staged_lds_words<OWN>());
}

template <int FM, int FN, int KG, int D>
hipError_t gemm_reg_launch(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 32 * FM, BN = 32 * FN;
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t gm = xcd_group_m(tiles_m, tiles_n, BM, BN);
#define TQ_GEMM_REG(YTV)                                                                    \
  hipLaunchKernelGGL((k_gemm_reg<FM, FN, KG, D, YTV>), dim3(tiles_m * tiles_n),              \
                     dim3(KG * kWave), 0, s, a.q, a.sx, a.M, a.packed, a.scale, a.per_row, a.N, \
                     a.K, a.Y, gm)
  if (a.ydt == TQ_F32) TQ_GEMM_REG(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMM_REG(TQ_BF16);
  else TQ_GEMM_REG(TQ_I32);
#undef TQ_GEMM_REG
  return hipGetLastError();
}

// Wide tiles for large grids: 256 x 256 outputs per workgroup of four waves,
// each wave 128 x 128 (4 x 4 accumulators of 32 x 32, held in the
// accumulation registers), 128 of K per stage, one workgroup per CU.  A wave
// issues 64 MFMAs per stage against 32 fragment reads: half the LDS feed per
// MFMA of a 64 x 64 wave tile, and one barrier per 64 MFMAs.  LDS rows are
// 144 bytes (128 + 16 of padding): the 16 rows a fragment read touches per
// quarter-wave fall on distinct banks, and every LDS offset is a base plus a
// constant, which keeps the architectural registers free for the loads in
// flight and the fragments read ahead.
constexpr int kWBM = 256, kWBN = 256, kWBK = 128;
constexpr int kWNT = 4 * kWave;
constexpr int kWLD = kWBK + 16;                      // LDS row stride
constexpr int kWTile = kWBM * kWLD;                  // one operand tile (A or B)
constexpr int kWStage = 2 * kWTile;

template <int YT>
__global__ __launch_bounds__(kWNT, 1) void k_gemm_wide(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y, int64_t gm) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kWStage];
  constexpr int FM = 4, FN = 4;
  constexpr int CA = kWBM * (kWBK / 16) / kWNT;  // 8 activation chunks per thread
  constexpr int CB = kWBN * (kWBK / 16) / kWNT;  // 8 packed words per thread
  constexpr int LB = CB / 4;                      // in 2 loads of 16 bytes
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  int64_t tm, tn;
  xcd_tile(blockIdx.x, (M + kWBM - 1) / kWBM, (N + kWBN - 1) / kWBN, gm, tm, tn);
  const int64_t m0 = tm * kWBM, n0 = tn * kWBN;
  const int64_t rowbytes = K >> 2;
  const int fr = lane & 31, kg = lane >> 5;

  const __amdgpu_buffer_rsrc_t ra_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q), static_cast<short>(0), static_cast<int>(M * K), kBufFlags);
  const __amdgpu_buffer_rsrc_t rb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed), static_cast<short>(0), static_cast<int>(N * rowbytes),
      kBufFlags);
  // staging: eight consecutive threads cover a row's 128 bytes of tokens,
  // chunk i of a thread 32 rows further; two threads cover a row's 32 bytes
  // of packed codes, 16 bytes (four words) each, load i 128 rows further
  const int sr = tid / 8, sc = tid % 8;
  const int br = tid / 2, bh = tid % 2;
  const uint32_t aoff = static_cast<uint32_t>((m0 + sr) * K + 16 * sc);
  const uint32_t boff = static_cast<uint32_t>((n0 + br) * rowbytes + 16 * bh);
  const uint32_t astep = static_cast<uint32_t>(32 * K), bstep = static_cast<uint32_t>(128 * rowbytes);
  const int st_off = sr * kWLD + 16 * sc;
  const int bst_off = kWTile + br * kWLD + 64 * bh;
  // fragment reads: row l%32 of each 32-row fragment, bytes 16*(l/32) of a
  // 32-wide K step
  const int ard = (wm * 128 + fr) * kWLD + 16 * kg;
  const int brd = kWTile + (wn * 128 + fr) * kWLD + 16 * kg;

  // two register sets: the loads run two stages ahead of the products
  struct Regs {
    v4i a[CA];
    v4i b[LB];
  };
  Regs r0, r1;
  const int64_t nk = K / kWBK;
  // load slot p of a stage: even p an activation chunk; odd p = 2q + 1 the
  // packed load q / 4 when q % 4 == 0 (ten loads per stage)
  auto load_piece = [&](Regs& r, int64_t kt, int p) {
    kt = kt < nk ? kt : nk - 1;  // past the end: reload the last stage (unused)
    const int soa = static_cast<int>(kt * kWBK), sob = static_cast<int>(kt * (kWBK / 4));
    const int q = p >> 1;
    if (!(p & 1))
      r.a[q] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff + q * astep, soa, 0));
    else if (q % 4 == 0)
      r.b[q / 4] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rb_rsrc, boff + (q / 4) * bstep, sob, 0));
  };
  auto load_stage = [&](Regs& r, int64_t kt) {
#pragma unroll
    for (int p = 0; p < CA + CB; ++p) load_piece(r, kt, p);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  // one of the sixteen pieces of moving a stage from registers into LDS:
  // even pieces store an activation chunk, odd ones decode and store a
  // packed word
  auto put_piece = [&](Regs& r, int buf, int p) {
    const int q = p >> 1;
    if (p & 1) {
      uint32_t w = static_cast<uint32_t>(r.b[q / 4][q % 4]);
      asm volatile("" : "+v"(w));
      *reinterpret_cast<v4i*>(lds + buf * kWStage + bst_off + (q / 4) * 128 * kWLD +
                              16 * (q % 4)) = decode_signed_natural(w);
    } else {
      *reinterpret_cast<v4i*>(lds + buf * kWStage + st_off + q * 32 * kWLD) = r.a[q];
    }
  };
  auto store_stage = [&](Regs& r, int buf) {
#pragma unroll
    for (int p = 0; p < CA + CB; ++p) put_piece(r, buf, p);
  };
  // multiply stage kt out of LDS half buf; between groups of four products
  // the next stage moves from registers st into the other half and one load
  // of stage kld goes out into registers ld (sixteen of each per stage:
  // spread over the stage, the loads do not reach the memory system in one
  // burst from every wave at once)
  static_assert(CA + CB == 4 * FM && CA == CB, "one load and one store piece per group");
  static_assert(FM == FN, "one A and one B fragment read per group");
  auto compute = [&](int buf, Regs& st, Regs& ld, int64_t kld) {
    const uint8_t* sa = lds + buf * kWStage + ard;
    const uint8_t* sb = lds + buf * kWStage + brd;
    v4i ac[FM], an[FM], bc[FN], bn[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ac[i] = *reinterpret_cast<const v4i*>(sa + i * 32 * kWLD);
#pragma unroll
    for (int j = 0; j < FN; ++j) bc[j] = *reinterpret_cast<const v4i*>(sb + j * 32 * kWLD);
#pragma unroll
    for (int kk = 0; kk < kWBK / 32; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ac[i], bc[j], acc[i][j], 0, 0, 0);
        // the next K step's fragments, two reads per group of products: a
        // burst of eight per wave fills the LDS command queue and stalls
        // the products behind it
        if (kk + 1 < kWBK / 32) {
          an[i] = *reinterpret_cast<const v4i*>(sa + i * 32 * kWLD + 32 * (kk + 1));
          bn[i] = *reinterpret_cast<const v4i*>(sb + i * 32 * kWLD + 32 * (kk + 1));
        }
        put_piece(st, buf ^ 1, kk * FM + i);
        load_piece(ld, kld, kk * FM + i);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) ac[i] = an[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) bc[j] = bn[j];
    }
  };
  // one stage: multiply stage kt while stage kt + 1 moves into the other LDS
  // half and stage kt + 2 is loaded into the set stage kt came from
  auto stage = [&](Regs& ld, Regs& st, int64_t kt) {
    compute(static_cast<int>(kt & 1), st, ld, kt + 2);
    __syncthreads();
  };

  load_stage(r0, 0);
  load_stage(r1, 1);
  store_stage(r0, 0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; kt += 2) {  // nk is even
    stage(r0, r1, kt);
    stage(r1, r0, kt + 1);
  }

  // the last stage ended on a barrier: LDS is free for the staged epilogue,
  // four wave areas followed by the tile's row and column factors
  constexpr int kEpi = 4 * staged_lds_words<FN>();
  static_assert((kEpi + kWBM + kWBN) * 4 <= 2 * kWStage, "epilogue LDS");
  static_assert(kWNT == kWBM && kWNT == kWBN, "one row and one column factor per thread");
  int* ep = reinterpret_cast<int*>(lds);
  float* sxs = reinterpret_cast<float*>(ep + kEpi);
  float* gms = sxs + kWBM;
  if (YT != TQ_I32) {
    const int64_t m = m0 + tid, n = n0 + tid;
    sxs[tid] = sx[m < M ? m : M - 1];
    gms[tid] = scale[per_row ? (n < N ? n : N - 1) : 0];
  }
  __syncthreads();
  store_acc32_staged<YT>(acc, m0 + wm * 128, n0 + wn * 128, lane, sxs + wm * 128,
                         gms + wn * 128, M, N, Y, ep + wave * staged_lds_words<FN>());
}

hipError_t gemm_wide_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + kWBM - 1) / kWBM, tiles_n = (a.N + kWBN - 1) / kWBN;
  const int64_t grid = tiles_m * tiles_n;
  const int64_t gm = xcd_group_m(tiles_m, tiles_n, kWBM, kWBN);
#define TQ_GEMM_WIDE(YTV)                                                                   \
  hipLaunchKernelGGL((k_gemm_wide<YTV>), dim3(grid), dim3(kWNT), 0, s, a.q, a.sx, a.M,      \
                     a.packed, a.scale, a.per_row, a.N, a.K, a.Y, gm)
  if (a.ydt == TQ_F32) TQ_GEMM_WIDE(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMM_WIDE(TQ_BF16);
  else TQ_GEMM_WIDE(TQ_I32);
#undef TQ_GEMM_WIDE
  return hipGetLastError();
}

hipError_t gemm_fast_dispatch(const GemmArgs& a, hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  constexpr int64_t kEnough = 384;
  // wide tiles run one workgroup per CU: they pay off when every round of
  // tiles, the last one included, fills at least half of the chip
  const int64_t cus = device_cus() > 0 ? device_cus() : 256;
  // at most one 32 x 64 tile per CU: K split over four waves (measured
  // 9.1 against 12.0 us at 128 x 4096 x 4096 and 11.0 against 16.3 us at
  // 64 x 2560 x 6912; with up to two tiles per CU the staged tiles below
  // stay 2-7% faster, e.g. 11.9 against 12.2-12.3 us at 160-256 x 4096 x 4096)
  if (a.K % kRBK == 0 && tiles(32, 64) <= cus) return gemm_reg_launch<1, 2, 4, 4>(a, s);
  const int64_t tw = tiles(kWBM, kWBN), last = tw % cus;
  if (tw >= cus && (last == 0 || 2 * last >= cus) && a.K % (2 * kWBK) == 0)
    return gemm_wide_launch(a, s);
  // 256 x 128 tiles (four waves of 128 x 64) from one per CU on (measured:
  // 2048 x 4096 runs 7% faster on 256 of them than on 512 tiles of
  // 128 x 128; eight waves of 64 x 64 per tile measured 3% slower)
  if (tiles(256, 128) >= cus) return gemm_fast_launch<256, 128, 2, 2>(a, s);
  if (tiles(128, 128) >= kEnough) return gemm_fast_launch<128, 128, 2, 2>(a, s);
  // small grids: two wave groups split each 128-deep stage (needs K % 128)
  // at most one 64 x 64 tile per CU (e.g. 256 x 4096): four K groups of two
  // waves per tile (measured 11.8 against 15.1 us at 256 x 4096 x 4096; with
  // more tiles, e.g. 512 x 2560 x 6912, the 128 x 64 tile below is faster)
  if (tiles(64, 64) <= cus && a.K % 256 == 0) return gemm_fast_launch<64, 64, 2, 1, 4>(a, s);
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
