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
// decoded once into signed int8 in LDS, and every wave then feeds LDS
// fragments to v_mfma_i32_32x32x32_i8.
//
// Tile: BM x BN outputs per workgroup, BK = 64 per stage, double-buffered
// LDS (rows padded to 80 bytes so that 128-bit fragment reads from 8
// consecutive rows touch disjoint banks).  Global loads of stage k+1 are in
// flight while stage k is contracted.  The epilogue applies
// y = acc * gamma * sx in fp32 and writes fp32, bf16 (round to nearest even)
// or the raw int32 accumulator.

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kBK = 64;
constexpr int kLD = kBK + 16;  // LDS row stride in bytes

template <bool ALIGNED>
__device__ inline uint4 load_a_chunk(const uint8_t* row, int64_t k, int64_t K, bool ok) {
  if (ALIGNED) {
    if (ok && k < K) return *reinterpret_cast<const uint4*>(row + k);
    return make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t kk = k + 4 * i + b;
      v |= static_cast<uint32_t>((ok && kk < K) ? row[kk] : 0u) << (8 * b);
    }
    w[i] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
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
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int64_t M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y) {
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CA = BM * 4 / NT;   // 16-byte A chunks per thread per stage
  constexpr int CB = BN * 4 / NT;   // packed B words per thread per stage
  static_assert(CA >= 1 && CB >= 1, "tile too small for the thread count");
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * kLD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kLD];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tm = blockIdx.x % tiles_m;
  const int64_t tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K >> 2;
  const uint8_t* qb = reinterpret_cast<const uint8_t*>(q);

  uint4 ra[CA];
  uint32_t rb[CB];

  auto load_stage = [&](int64_t kt) {
    const int64_t k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, cc = c & 3;
      const int64_t m = m0 + r;
      const bool ok = m < M;
      ra[i] = load_a_chunk<ALIGNED>(qb + (ok ? m : 0) * K, k0 + 16 * cc, K, ok);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, wi = c & 3;
      const int64_t n = n0 + r;
      const bool ok = n < N;
      rb[i] = load_b_word<ALIGNED>(packed + (ok ? n : 0) * rowbytes, k0 / 4 + 4 * wi,
                                   rowbytes, ok);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, cc = c & 3;
      *reinterpret_cast<uint4*>(&As[buf][r * kLD + 16 * cc]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 2, wi = c & 3;
      const v4i d = decode_signed_natural(rb[i]);
      *reinterpret_cast<v4i*>(&Bs[buf][r * kLD + 16 * wi]) = d;
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
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int fr = lane & 31, kg = lane >> 5;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    if (kt + 1 < nk) load_stage(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      v4i a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const v4i*>(
            &As[buf][(wm * TM + 32 * i + fr) * kLD + kk + 16 * kg]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const v4i*>(
            &Bs[buf][(wn * TN + 32 * j + fr) * kLD + kk + 16 * kg]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
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

template <int BM, int BN, int WM, int WN, bool ALIGNED>
hipError_t gemm_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int NT = WM * WN * kWave;
#define TQ_GEMM(YTV)                                                                     \
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, ALIGNED, YTV>), dim3(tiles), dim3(NT), 0, s, \
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
  if (tiles(256, 128) >= kEnough) return gemm_launch<256, 128, 2, 2, ALIGNED>(a, s);
  if (tiles(128, 128) >= kEnough) return gemm_launch<128, 128, 2, 2, ALIGNED>(a, s);
  return gemm_launch<128, 64, 2, 2, ALIGNED>(a, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  const bool aligned = (a.K % 64) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.packed) & 15u) == 0u &&
                       (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0u;
  return aligned ? gemm_dispatch<true>(a, s) : gemm_dispatch<false>(a, s);
}

}  // namespace tq
