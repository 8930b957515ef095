// Backward through the ternary layer (Foundry, docs/quantization.md,
// "Ternary Training (Backward Pass + Stochastic Flip) / Backward Pass").
//
// The forward is y[m, o] = gamma_o * sum_k x[m, k] w[o, k] with w in
// {-1, 0, +1} held as 2-bit codes, W = [N, K] rows of K/4 bytes.  The input
// gradient contracts the output gradient with the same codes over the output
// index:
//     dX[m, k] = sum_n dY[m, n] * gamma_n * w[n, k]
// which reads the packed rows transposed (the contraction runs down the
// columns of W).
//
// Matrix-core mapping (gfx950).  The products dY * w are exact in any float
// format that holds dY exactly, because w is -1, 0 or +1.  An fp32 value
// splits exactly into three bf16 terms, h = bf16(v), m = bf16(v - h),
// l = bf16(v - h - m) (each residual is exact in fp32 and has at most 16,
// then 8 significant bits), so sum_n v_n w_n is three bf16 MFMA contractions
// into one fp32 accumulator: the products stay exact and only the fp32
// accumulation rounds, the same arithmetic as an fp32 dot product, at three
// bf16 matrix-core passes instead of the 8x slower fp32 matrix path.  A bf16
// dY with one scale per tensor is exact in one term, and the scale is applied
// to the finished sum; a per-row scale multiplies dY in fp32 first and takes
// the three-term split.
//
// A workgroup (8 waves, 2 x 4) owns a 128-token x 256-column dX tile and
// walks the contraction in steps of 32 rows of W.  Each step it stages
//   - the dY tile (128 x 32), split into its bf16 planes once per workgroup,
//     in 64-byte LDS rows whose 16-byte chunks are XOR-swizzled by row so that
//     the 16 rows of an MFMA operand read hit disjoint banks;
//   - the code tile (32 rows x 64 bytes, loaded a byte per lane and row)
//     transposed to [column byte][row], 40-byte rows, so that one 8-byte read gives a lane the codes of eight
//     consecutive W rows for four adjacent dX columns (a byte holds four
//     columns).  Each lane decodes them to four bf16 B operands with byte
//     permutes; B fragment f covers columns 4j + f (j = lane % 16), so a lane
//     ends with four adjacent columns of each output row, stored as one
//     16-byte write.
// Global loads are raw buffer loads issued two steps ahead into rotating
// register sets (bytes past a buffer read as zero); the dY columns past N are
// zeroed on staging.

#include <type_traits>

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kXcds = 8;

constexpr int kBM = 128;                  // dX rows (tokens) per workgroup
constexpr int kBK = 256;                  // dX columns per workgroup
constexpr int kBN = 32;                   // W rows per contraction step
constexpr int kWM = 2, kWK = 4;           // waves
constexpr int kNT = kWM * kWK * kWave;    // 512 threads
constexpr int kArow = kBN * 2;            // bytes of one bf16 plane row
constexpr int kPlane = kBM * kArow;       // bytes of one bf16 plane
constexpr int kWrow = 40;                 // bytes of one transposed code row
constexpr int kWbytes = (kBK / 4) * kWrow;

#ifndef TQ_BWD_SPREAD
#define TQ_BWD_SPREAD 1
#endif
#ifndef TQ_BWD_KS3
#define TQ_BWD_KS3 2
#endif
#ifndef TQ_BWD_KS1
#define TQ_BWD_KS1 4
#endif
// MFMA steps (of kBN rows) per LDS stage, with three bf16 planes or one
constexpr int kBwdKS3 = TQ_BWD_KS3, kBwdKS1 = TQ_BWD_KS1;

template <int P>
constexpr int bwd_stage_bytes() { return P * kPlane + kWbytes; }

// two fp32 -> two bf16 (round to nearest even), and back
__device__ inline uint32_t pk_bf16(float a, float b) {
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// x = h + m + l exactly, each as packed bf16 pairs (element 2i in the low half)
__device__ inline void split3(const float (&x)[8], v4i& h, v4i& m, v4i& l) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[2 * i], b = x[2 * i + 1];
    const uint32_t hu = pk_bf16(a, b);
    const float ra = a - bf_lo(hu), rb = b - bf_hi(hu);
    const uint32_t mu = pk_bf16(ra, rb);
    const uint32_t lu = pk_bf16(ra - bf_lo(mu), rb - bf_hi(mu));
    h[i] = static_cast<int>(hu);
    m[i] = static_cast<int>(mu);
    l[i] = static_cast<int>(lu);
  }
}

// Offset of 16-byte chunk `chunk` of row `row` in a tile of 64-byte rows.
// The XOR swizzle keeps both the 16x16x32 operand reads (16 consecutive rows
// at one chunk per lane group) and the staging writes (whole rows) free of
// LDS bank conflicts (measured with the LDS bank-conflict counter and by
// timing; the plain (row >> 2) swizzle costs the reads 40%).
__device__ inline int swz64(int row, int chunk) {
  return row * 64 + 16 * (chunk ^ (((row >> 1) ^ (row >> 4)) & 3));
}

// bf16 bit patterns of the codes 0, 1, 2 (-1, 0, +1): low bytes in LUT_LO
// bytes 0..2, high bytes in LUT_HI bytes 0..2 (byte-permute indices 4..6)
constexpr uint32_t kLutLo = 0x00800080u;
constexpr uint32_t kLutHi = 0x003F00BFu;

// Codes of eight consecutive W rows for one column (u0: rows 0..3, u1: rows
// 4..7, one byte per row, the column's code at bits 2F..2F+1) as eight bf16.
template <int F>
__device__ inline bf16x8 decode_column(uint32_t u0, uint32_t u1) {
  const uint32_t t0 = (u0 >> (2 * F)) & 0x03030303u;
  const uint32_t t1 = (u1 >> (2 * F)) & 0x03030303u;
  const uint32_t s0 = t0 + 0x04040404u, s1 = t1 + 0x04040404u;
  v4i o;
  o.x = static_cast<int>(__builtin_amdgcn_perm(kLutHi, kLutLo, __builtin_amdgcn_perm(s0, t0, 0x05010400u)));
  o.y = static_cast<int>(__builtin_amdgcn_perm(kLutHi, kLutLo, __builtin_amdgcn_perm(s0, t0, 0x07030602u)));
  o.z = static_cast<int>(__builtin_amdgcn_perm(kLutHi, kLutLo, __builtin_amdgcn_perm(s1, t1, 0x05010400u)));
  o.w = static_cast<int>(__builtin_amdgcn_perm(kLutHi, kLutLo, __builtin_amdgcn_perm(s1, t1, 0x07030602u)));
  return __builtin_bit_cast(bf16x8, o);
}

// DT: 0 = fp32 dY, 1 = bf16 dY.  ROWG: one scale per W row.  ACC: add into dX.
// W4: stage the codes by words (needs K % 16 == 0, so that rows start on
// 4-byte boundaries and no word straddles the end of the codes).
template <int DT, bool ROWG, bool ACC, bool W4>
__global__ __launch_bounds__(kNT, 1) void k_bwd_input(
    const void* __restrict__ dY, int64_t M, const uint8_t* __restrict__ packed,
    const float* __restrict__ scale, int64_t N, int64_t K, float* __restrict__ dX) {
  constexpr int P = (DT == 0 || ROWG) ? 3 : 1;  // bf16 planes
  constexpr int ES = DT == 0 ? 4 : 2;           // bytes per dY element
  constexpr int KS = P == 3 ? kBwdKS3 : kBwdKS1;  // MFMA steps per stage
  constexpr int kStep = bwd_stage_bytes<P>();   // LDS bytes of one MFMA step
  constexpr int kStage = KS * kStep;
  constexpr int YL = ES == 4 ? 2 : 1;           // 16-byte dY loads per step
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform in the wave
  const int wm = wave / kWK, wk = wave % kWK;
  const int64_t tiles_m = (M + kBM - 1) / kBM;
  const int64_t tiles_k = (K + kBK - 1) / kBK;
  // ids congruent mod 8 run on one XCD: give them the same dY rows
  const int64_t bid = blockIdx.x;
  const int64_t local = bid / kXcds;
  const int64_t tk = local % tiles_k;
  const int64_t tm = (local / tiles_k) * kXcds + bid % kXcds;
  if (tm >= tiles_m) return;  // padding ids (whole workgroup)
  const int64_t m0 = tm * kBM, k0 = tk * kBK;
  const int64_t rows = M - m0 < kBM ? M - m0 : kBM;
  const int64_t rowbytes = K / 4;

  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(dY) + m0 * N * ES), static_cast<short>(0),
      static_cast<int>(rows * N * ES), kBufFlags);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed + k0 / 4), static_cast<short>(0),
      static_cast<int>(N * rowbytes - k0 / 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scale), static_cast<short>(0), static_cast<int>(ROWG ? N * 4 : 4),
      kBufFlags);

  // staging roles, per MFMA step: every thread one row x 8 columns of dY,
  // and one code byte (column byte `lane`) of four consecutive W rows.  With
  // 128 W rows per stage (four steps) a thread instead loads one word (four
  // column bytes 4d..4d+3) of four rows 4g..4g+3 and transposes the 4 x 4
  // bytes in registers: four loads per stage instead of sixteen.
  constexpr bool kW4 = W4 && KS * kBN == 128;
  const int sr = tid >> 2, sc = tid & 3;
  const uint32_t yoff = static_cast<uint32_t>((sr * N + 8 * sc) * ES);
  const int yst = swz64(sr, sc);
  const int wg4 = tid >> 4, wd4 = tid & 15;
  const uint32_t woff = kW4 ? static_cast<uint32_t>(4 * wg4 * rowbytes + 4 * wd4)
                            : static_cast<uint32_t>(4 * wave * rowbytes + lane);
  const int wst = kW4 ? (wg4 / 8) * kStep + P * kPlane + 4 * wd4 * kWrow + 4 * (wg4 % 8)
                      : P * kPlane + lane * kWrow + 4 * wave;

  // fragment reads
  const int fr = lane & 15, fg = lane >> 4;
  int ard[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = wm * 64 + 16 * a + fr;
    ard[a] = swz64(r, fg);
  }
  const int brd = P * kPlane + (wk * 16 + fr) * kWrow + 8 * fg;

  struct Regs {
    v4i y[KS][YL];
    uint32_t w[KS][4];  // one code byte each
  };
  typedef v4i Gam[ROWG ? KS : 1][2];
  auto load_stage = [&](int64_t kt, Regs& r) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int64_t j = kt * KS + ks;
      const int so = static_cast<int>(j * kBN * ES);
#pragma unroll
      for (int i = 0; i < YL; ++i)
        r.y[ks][i] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(ry, yoff + 16 * i, so, 0));
      if constexpr (!kW4) {
        const int sw = static_cast<int>(j * kBN * rowbytes);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r.w[ks][i] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(
              rw, woff + static_cast<uint32_t>(i * rowbytes), sw, 0));
      }
    }
    if constexpr (kW4) {
      const int sw = static_cast<int>(kt * KS * kBN * rowbytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.w[0][i] = __builtin_amdgcn_raw_buffer_load_b32(
            rw, woff + static_cast<uint32_t>(i * rowbytes), sw, 0);
    }
  };
  // per-row scales of a stage's columns (issued before the far loads of the
  // same step, so that waiting for them leaves those in flight)
  auto load_gamma = [&](int64_t kt, Gam& g) {
    if constexpr (ROWG) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t go = static_cast<uint32_t>(((kt * KS + ks) * kBN + 8 * sc) * 4);
        g[ks][0] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rg, go, 0, 0));
        g[ks][1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rg, go + 16, 0, 0));
      }
    }
  };
  // staging of step ks of a stage (and, with word-loaded codes, ks == KS:
  // the transposed codes of the whole stage)
  auto put_step = [&](int buf, int64_t kt, Regs& r, Gam& g, int ks) {
    if (ks < KS) {
      uint8_t* st = lds + buf * kStage + ks * kStep;
      // the loaded values enter here: without this the compiler combines the
      // code bytes right after their loads and waits for them a step early
      if constexpr (!kW4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(r.w[ks][i]));
      }
      const bool ok = (kt * KS + ks) * kBN + 8 * sc < N;
      if constexpr (P == 1) {
        const v4i z = {0, 0, 0, 0};
        *reinterpret_cast<v4i*>(st + yst) = ok ? r.y[ks][0] : z;
      } else {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (ES == 4) {
            x[e] = __int_as_float(r.y[ks][e / 4][e % 4]);
          } else {
            const uint32_t u = static_cast<uint32_t>(r.y[ks][0][e / 2]);
            x[e] = (e & 1) ? bf_hi(u) : bf_lo(u);
          }
          x[e] = ok ? x[e] : 0.f;
          if constexpr (ROWG) x[e] *= __int_as_float(g[ks][e / 4][e % 4]);
        }
        v4i h, m, l;
        split3(x, h, m, l);
        *reinterpret_cast<v4i*>(st + yst) = h;
        *reinterpret_cast<v4i*>(st + kPlane + yst) = m;
        *reinterpret_cast<v4i*>(st + 2 * kPlane + yst) = l;
      }
      if constexpr (!kW4)
        *reinterpret_cast<uint32_t*>(st + wst) =
            r.w[ks][0] | (r.w[ks][1] << 8) | (r.w[ks][2] << 16) | (r.w[ks][3] << 24);
    } else if constexpr (kW4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(r.w[0][i]));
      // out[s] holds column byte 4d+s of rows 4g..4g+3
      const v4i t = transpose_bytes4x4(r.w[0][0], r.w[0][1], r.w[0][2], r.w[0][3]);
      uint8_t* st = lds + buf * kStage;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) *reinterpret_cast<int*>(st + wst + s4 * kWrow) = t[s4];
    }
  };
  constexpr int NPUT = KS + (kW4 ? 1 : 0);  // staging pieces per stage
  auto store_stage = [&](int buf, int64_t kt, Regs& r, Gam& g) {
#pragma unroll
    for (int q = 0; q < NPUT; ++q) put_step(buf, kt, r, g, q);
  };
  // load q of a stage: the dY loads first (KS x YL), then the code loads
  // (four words, or KS x 4 bytes)
  constexpr int NLD = KS * YL + (kW4 ? 4 : KS * 4);
  auto load_one = [&](int64_t kt, Regs& r, int q) {
    if (q < KS * YL) {
      const int ks = q / YL, i = q % YL;
      const int so = static_cast<int>((kt * KS + ks) * kBN * ES);
      r.y[ks][i] =
          __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ry, yoff + 16 * i, so, 0));
    } else if constexpr (kW4) {
      const int i = q - KS * YL;
      const int sw = static_cast<int>(kt * KS * kBN * rowbytes);
      r.w[0][i] = __builtin_amdgcn_raw_buffer_load_b32(
          rw, woff + static_cast<uint32_t>(i * rowbytes), sw, 0);
    } else {
      const int ks = (q - KS * YL) / 4, i = (q - KS * YL) % 4;
      const int sw = static_cast<int>((kt * KS + ks) * kBN * rowbytes);
      r.w[ks][i] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(
          rw, woff + static_cast<uint32_t>(i * rowbytes), sw, 0));
    }
  };

  f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[a][f] = f4{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = (N + KS * kBN - 1) / (KS * kBN);  // stages
  // one stage: start the loads of stage kt+2, contract stage kt from LDS,
  // publish stage kt+1.  In the main loop every stage loads and stores
  // unconditionally (a branch around the loads would make the compiler wait
  // for all loads in flight); loads past the last stage read zeros or data
  // that is never used (columns past N are zeroed on staging), and a store of
  // stage nk goes to the LDS half that no later stage reads.
  // With TQ_BWD_SPREAD the far loads and the staging are issued in pieces
  // after each group of four MFMAs instead of in one block each.
  constexpr bool kSpread = TQ_BWD_SPREAD;
  constexpr int NG = KS * P * 4;  // MFMA groups per stage
  auto step = [&](int64_t kt, Regs& r_next, Regs& r_far, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    const int buf = static_cast<int>(kt & 1);
    const bool do_load = !GUARD || kt + 2 < nk, do_store = !GUARD || kt + 1 < nk;
    Gam g;
    if (!GUARD || kt + 1 < nk) load_gamma(kt + 1, g);
    if (!kSpread && do_load) load_stage(kt + 2, r_far);
    __builtin_amdgcn_sched_barrier(0);
    int grp = 0;
    auto pieces = [&]() {
      if constexpr (kSpread) {
#pragma unroll
        for (int q = grp * NLD / NG; q < (grp + 1) * NLD / NG; ++q)
          if (do_load) load_one(kt + 2, r_far, q);
#pragma unroll
        for (int q = grp * NPUT / NG; q < (grp + 1) * NPUT / NG; ++q)
          if (do_store) put_step(buf ^ 1, kt + 1, r_next, g, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++grp;
    };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* st = lds + buf * kStage + ks * kStep;
      const uint2 wb = *reinterpret_cast<const uint2*>(st + brd);
      bf16x8 av[P][4];
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          av[p][a] = *reinterpret_cast<const bf16x8*>(st + p * kPlane + ard[a]);
      bf16x8 b[4];
      b[0] = decode_column<0>(wb.x, wb.y);
      b[1] = decode_column<1>(wb.x, wb.y);
      b[2] = decode_column<2>(wb.x, wb.y);
      b[3] = decode_column<3>(wb.x, wb.y);
#pragma unroll
      for (int p = P - 1; p >= 0; --p)  // smallest terms first
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
          for (int f = 0; f < 4; ++f)
            acc[a][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[p][a], b[f], acc[a][f], 0, 0, 0);
          pieces();
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!kSpread && do_store) store_stage(buf ^ 1, kt + 1, r_next, g);
    __syncthreads();
  };
  using Free = std::false_type;
  using Guarded = std::true_type;

  Regs r0, r1, r2;
  Gam g0;
  load_gamma(0, g0);
  load_stage(0, r0);
  load_stage(1, r1);
  store_stage(0, 0, r0, g0);
  __syncthreads();
  int64_t kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, r1, r2, Free{});
    step(kt + 1, r2, r0, Free{});
    step(kt + 2, r0, r1, Free{});
  }
  if (kt < nk) step(kt, r1, r2, Guarded{});
  if (kt + 1 < nk) step(kt + 1, r2, r0, Guarded{});

  // D of the 16x16 MFMA: lane l holds rows 4(l/16)+i of column l%16, and
  // fragment f is column 4(l%16)+f of the wave's 64
  // (when accumulating, every old value is loaded before the first store:
  // loads and stores share one memory counter, so a load issued after a
  // store would wait for it)
  const float gt = ROWG ? 1.f : scale[0];
  const int64_t col = k0 + wk * 64 + 4 * fr;
  if (col >= K) return;
  f4 old[4][4];
  if (ACC) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 64 + 16 * a + 4 * fg + i;
        if (row < M) old[a][i] = *reinterpret_cast<const f4*>(dX + row * K + col);
      }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + wm * 64 + 16 * a + 4 * fg + i;
      if (row >= M) continue;
      f4 v = {acc[a][0][i], acc[a][1][i], acc[a][2][i], acc[a][3][i]};
      if (!ROWG) v = v * gt;
      if (ACC) v = v + old[a][i];
      *reinterpret_cast<f4*>(dX + row * K + col) = v;
    }
  }
}

// Any shape: one thread per dX element, the contraction in fp32 in row order.
template <int DT, bool ACC>
__global__ __launch_bounds__(256) void k_bwd_input_generic(
    const void* __restrict__ dY, int64_t M, const uint8_t* __restrict__ packed,
    const float* __restrict__ scale, int per_row, int64_t N, int64_t K, float* __restrict__ dX) {
  const int64_t total = M * K;
  const int64_t rowbytes = K / 4;
  for (int64_t idx = blockIdx.x * int64_t{256} + threadIdx.x; idx < total;
       idx += int64_t{gridDim.x} * 256) {
    const int64_t m = idx / K, k = idx % K;
    float acc = 0.f;
    for (int64_t n = 0; n < N; ++n) {
      const uint32_t c = (packed[n * rowbytes + k / 4] >> (2 * (k % 4))) & 3u;
      if (c != 0u && c != 2u) continue;
      float v = DT == 0 ? static_cast<const float*>(dY)[m * N + n]
                        : bf16_to_f32(static_cast<const uint16_t*>(dY)[m * N + n]);
      if (per_row) v *= scale[n];
      acc += c == 2u ? v : -v;
    }
    if (!per_row) acc *= scale[0];
    dX[idx] = ACC ? dX[idx] + acc : acc;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t{256} + threadIdx.x; i < n;
       i += int64_t{gridDim.x} * 256)
    p[i] = 0.f;
}

template <int DT, bool ROWG, bool ACC, bool W4>
hipError_t bwd_input_fast(const BwdInputArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + kBM - 1) / kBM;
  const int64_t tiles_k = (a.K + kBK - 1) / kBK;
  const int64_t grid = tiles_k * ((tiles_m + kXcds - 1) / kXcds) * kXcds;
  hipLaunchKernelGGL((k_bwd_input<DT, ROWG, ACC, W4>), dim3(grid), dim3(kNT), 0, s, a.dY, a.M,
                     a.packed, a.scale, a.N, a.K, a.dX);
  return hipGetLastError();
}

template <int DT>
hipError_t bwd_input_fast_dt(const BwdInputArgs& a, hipStream_t s) {
  if (a.per_row) return a.accumulate ? bwd_input_fast<DT, true, true, false>(a, s)
                                     : bwd_input_fast<DT, true, false, false>(a, s);
  // word staging of the codes only where it applies (one bf16 plane)
  if (DT == 1 && a.K % 16 == 0)
    return a.accumulate ? bwd_input_fast<DT, false, true, true>(a, s)
                        : bwd_input_fast<DT, false, false, true>(a, s);
  return a.accumulate ? bwd_input_fast<DT, false, true, false>(a, s)
                      : bwd_input_fast<DT, false, false, false>(a, s);
}

int64_t grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return g < 65536 ? g : 65536;
}

// ------------------------------------------------------------ weight gradient
//
// dW[n, k] = sum_m dY[m, n] * X[m, k]: the float product X^T dY of the page,
// with no codes and no scale.  Both operands run down their rows (the
// contraction is over tokens), so each workgroup transposes its tiles while
// staging them: a thread loads 8 consecutive token rows of two adjacent
// columns (one 8- or 4-byte load per row; 64 lanes read 512 or 256
// contiguous bytes of a row) and writes, per column, the 8 values as one
// 16-byte chunk of that column's LDS row.  fp32 operands are split into
// three bf16 terms (a = a1 + a2 + a3 exactly); with both operands fp32 the
// products a_p * b_q with p + q <= 2 (six MFMA passes) are kept, the dropped
// terms adding at most about 2^-23 |a b| per product; with a bf16 operand
// the kept terms give every product exactly.  The terms are accumulated
// smallest first: with a bf16 operand the partial sums of one product's terms
// are then exact (a2 + a3 = a - a1 has at most 16 significant bits), so a
// single token's contribution is its product with a single rounding (the
// matrix cores' accumulation rounds faithfully, not always to nearest).
//
// A workgroup (8 waves, 4 x 2, 32 x 64 each) owns a 128 x 128 dW tile.  A
// stage holds KS MFMA steps of 32 tokens, as many as double-buffered LDS
// allows (4 with two bf16 operands, 2 with one fp32 operand, 1 with two);
// with KS >= 2 every thread stages KS/2 units (8 rows x 2 columns) of each
// operand, with one step threads 0..255 stage dY and 256..511 stage X.
// Either way all threads issue the same loads.

constexpr int kGK = 128;             // dW columns per tile
constexpr int kGPlane = 128 * 64;    // one plane: 128 rows of 32 bf16
constexpr int kPN = 4, kPK = 8;      // tiles of a patch (one per CU of an XCD)

__host__ __device__ constexpr int planes_of(int dt) { return dt == 0 ? 3 : 1; }
#ifndef TQ_WGT_WIDE
#define TQ_WGT_WIDE 1
#endif
#ifndef TQ_WGT_SPREAD
#define TQ_WGT_SPREAD 1
#endif
// dW rows per tile: 256 with two bf16 operands (64 x 64 per wave, half the
// LDS fragment reads per MFMA of a 32 x 64 wave tile), else 128
__host__ __device__ constexpr int wgt_gn(int da, int db) {
  return (TQ_WGT_WIDE && da == 1 && db == 1) ? 256 : 128;
}
// MFMA steps per LDS stage: as many as 160 KiB of double-buffered LDS allow
__host__ __device__ constexpr int wgt_ks(int da, int db) {
  return (da == 0 && db == 0) ? 1 : (da == 1 && db == 1) ? (wgt_gn(da, db) == 256 ? 2 : 4) : 2;
}
template <int DA, int DB>
constexpr int wgt_lds_bytes() {
  return 2 * wgt_ks(DA, DB) * (planes_of(DA) * wgt_gn(DA, DB) * 64 + planes_of(DB) * kGPlane);
}

// DA: dtype of dY, DB: dtype of X (0 = fp32, 1 = bf16).  ACC: add into dW.
template <int DA, int DB, bool ACC>
__global__ __launch_bounds__(kNT, 1) void k_bwd_weight(
    const void* __restrict__ dY, const void* __restrict__ X, int64_t M, int64_t N, int64_t K,
    float* __restrict__ dW) {
  constexpr int PA = planes_of(DA), PB = planes_of(DB);
  constexpr int KS = wgt_ks(DA, DB);
  constexpr int GN = wgt_gn(DA, DB);           // dW rows (dY columns) per tile
  constexpr int TW = GN / 4;                   // rows per wave
  constexpr int FA = TW / 16;                  // A fragments per wave
  constexpr int kAPlane = GN * 64;             // one A plane: GN rows of 32 bf16
  constexpr int kGM = 32 * KS;                 // tokens per stage
  constexpr int kStep = PA * kAPlane + PB * kGPlane;  // LDS bytes of one MFMA step
  constexpr int kStage = KS * kStep;
  constexpr bool kRoles = KS == 1;             // half the threads per operand
  constexpr int ESA = DA == 0 ? 4 : 2, ESB = DB == 0 ? 4 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform in the wave
  const int wn = wave / 2, wk = wave % 2;
  const int64_t tiles_n = (N + GN - 1) / GN;
  const int64_t tiles_k = (K + kGK - 1) / kGK;
  // ids congruent mod 8 run on one XCD: its 32 workgroups in flight take a
  // 4 x 8 patch of tiles, which share 4 dY and 8 X column blocks in its L2
  const int64_t pcols = (tiles_n + kPN - 1) / kPN;
  const int64_t bid = blockIdx.x;
  const int64_t local = bid / kXcds;
  const int64_t patch = (local / (kPN * kPK)) * kXcds + bid % kXcds;
  const int64_t q = local % (kPN * kPK);
  const int64_t tn = (patch % pcols) * kPN + q % kPN;
  const int64_t tk = (patch / pcols) * kPK + q / kPN;
  if (tn >= tiles_n || tk >= tiles_k) return;  // padding ids (whole workgroup)
  const int64_t n0 = tn * GN, k0 = tk * kGK;

  // staging units of this thread: columns 2cp, 2cp+1, token rows 8o..8o+7 of
  // the stage for o = uo + 8u (u < U); an A tile of 256 columns takes a
  // second unit for columns 128 + 2cp, 128 + 2cp + 1; with roles, waves
  // 0..3 stage dY and 4..7 stage X
  constexpr int U = kRoles ? 1 : KS / 2;
  constexpr int PRA = GN / 128;                // A column blocks of 128
  const bool role_a = !kRoles || wave < 4;
  const int ut = kRoles ? (tid & 255) : tid;
  const int cp = ut & 63, uo = ut >> 6;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(dY) + n0 * ESA), static_cast<short>(0),
      static_cast<int>(M * N * ESA - n0 * ESA), kBufFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(X) + k0 * ESB), static_cast<short>(0),
      static_cast<int>(M * K * ESB - k0 * ESB), kBufFlags);
  const uint32_t aoff = static_cast<uint32_t>((8 * uo * N + 2 * cp) * ESA);
  const uint32_t boff = static_cast<uint32_t>((8 * uo * K + 2 * cp) * ESB);
  // LDS offsets of unit 0's two column rows within its operand's plane 0;
  // unit u sits 2u MFMA steps further
  const int ubase = (uo >> 2) * kStep;
  const int wo0 = ubase + swz64(2 * cp, uo & 3), wo1 = ubase + swz64(2 * cp + 1, uo & 3);

  // a unit: 8 rows of two fp32 (two words) or two bf16 (one word) columns
  struct Regs {
    uint32_t a[U * PRA][8][ESA / 2];
    uint32_t b[kRoles ? 1 : U][8][ESB / 2];
  };
  auto load_unit = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t str, int so, auto es,
                       auto& v) {
    constexpr int E = decltype(es)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (E == 4) {
        const uint2 t = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off + i * str, so, 0));
        v[i][0] = t.x;
        v[i][E / 2 - 1] = t.y;
      } else {
        v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(r, off + i * str, so, 0);
      }
    }
  };
  using EA = std::integral_constant<int, ESA>;
  using EB = std::integral_constant<int, ESB>;
  auto load_stage = [&](int64_t st, Regs& r) {
    if constexpr (kRoles) {
      // both operands fp32: the same loads, buffer and offsets by role
      const int64_t rl = role_a ? N : K;
      load_unit(role_a ? ra : rb, role_a ? aoff : boff, static_cast<uint32_t>(rl * 4),
                static_cast<int>(st * kGM * rl * 4), EA{}, r.a[0]);
    } else {
      const uint32_t sa = static_cast<uint32_t>(N * ESA), sb = static_cast<uint32_t>(K * ESB);
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int pb = 0; pb < PRA; ++pb)
          load_unit(ra, aoff + 64 * u * sa + 128 * pb * ESA, sa,
                    static_cast<int>(st * kGM * N * ESA), EA{}, r.a[u * PRA + pb]);
        load_unit(rb, boff + 64 * u * sb, sb, static_cast<int>(st * kGM * K * ESB), EB{},
                  r.b[u]);
      }
    }
  };
  // one unit -> its operand's planes (plane 0 at `base`)
  auto put_unit = [&](uint8_t* base, int plane, auto es, auto& v) {
    constexpr int E = decltype(es)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < E / 2; ++j) asm volatile("" : "+v"(v[i][j]));
    if constexpr (E == 4) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(v[i][c * (E / 2 - 1)]);
        v4i h, m, l;
        split3(x, h, m, l);
        const int o = c ? wo1 : wo0;
        *reinterpret_cast<v4i*>(base + o) = h;
        *reinterpret_cast<v4i*>(base + plane + o) = m;
        *reinterpret_cast<v4i*>(base + 2 * plane + o) = l;
      }
    } else {
      // bf16 pairs (column 2cp in the low half): each column's 8 halves
      v4i c0, c1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        c0[t] = static_cast<int>(__builtin_amdgcn_perm(v[2 * t + 1][0], v[2 * t][0], 0x05040100u));
        c1[t] = static_cast<int>(__builtin_amdgcn_perm(v[2 * t + 1][0], v[2 * t][0], 0x07060302u));
      }
      *reinterpret_cast<v4i*>(base + wo0) = c0;
      *reinterpret_cast<v4i*>(base + wo1) = c1;
    }
  };
  auto store_stage = [&](int buf, Regs& r) {
    uint8_t* st = lds + buf * kStage;
    if constexpr (kRoles) {
      put_unit(st + (role_a ? 0 : PA * kAPlane), role_a ? kAPlane : kGPlane, EA{}, r.a[0]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int pb = 0; pb < PRA; ++pb)
          put_unit(st + 2 * u * kStep + pb * 128 * 64, kAPlane, EA{}, r.a[u * PRA + pb]);
        put_unit(st + 2 * u * kStep + PA * kAPlane, kGPlane, EB{}, r.b[u]);
      }
    }
  };
  // the same work in pieces: with roles, one unit per thread; without,
  // unit `uid` < U*PRA is A unit (uid / PRA, uid % PRA), the rest B units.
  // Row i of a unit is one load.
  constexpr int NU = kRoles ? 1 : U * PRA + U;
  auto load_row = [&](int64_t st, Regs& r, int uid, int i) {
    if constexpr (kRoles) {
      const int64_t rl = role_a ? N : K;
      const uint32_t off = (role_a ? aoff : boff) + i * static_cast<uint32_t>(rl * 4);
      const uint2 t = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(role_a ? ra : rb, off,
                                                      static_cast<int>(st * kGM * rl * 4), 0));
      r.a[0][i][0] = t.x;
      r.a[0][i][1] = t.y;
    } else {
      const uint32_t sa = static_cast<uint32_t>(N * ESA), sb = static_cast<uint32_t>(K * ESB);
      if (uid < U * PRA) {
        const int u = uid / PRA, pb = uid % PRA;
        auto& v = r.a[uid];
        const uint32_t off = aoff + 64 * u * sa + 128 * pb * ESA + i * sa;
        const int so = static_cast<int>(st * kGM * N * ESA);
        if constexpr (ESA == 4) {
          const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ra, off, so, 0));
          v[i][0] = t.x;
          v[i][ESA / 2 - 1] = t.y;
        } else {
          v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(ra, off, so, 0);
        }
      } else {
        const int u = uid - U * PRA;
        auto& v = r.b[u];
        const uint32_t off = boff + 64 * u * sb + i * sb;
        const int so = static_cast<int>(st * kGM * K * ESB);
        if constexpr (ESB == 4) {
          const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rb, off, so, 0));
          v[i][0] = t.x;
          v[i][ESB / 2 - 1] = t.y;
        } else {
          v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rb, off, so, 0);
        }
      }
    }
  };
  auto put_one = [&](int buf, Regs& r, int uid) {
    if constexpr (kRoles) {
      uint8_t* st = lds + buf * kStage;
      put_unit(st + (role_a ? 0 : PA * kAPlane), role_a ? kAPlane : kGPlane, EA{}, r.a[0]);
    } else {
      uint8_t* st = lds + buf * kStage;
      if (uid < U * PRA) {
        const int u = uid / PRA, pb = uid % PRA;
        put_unit(st + 2 * u * kStep + pb * 128 * 64, kAPlane, EA{}, r.a[uid]);
      } else {
        const int u = uid - U * PRA;
        put_unit(st + 2 * u * kStep + PA * kAPlane, kGPlane, EB{}, r.b[u]);
      }
    }
  };

  const int fr = lane & 15, fg = lane >> 4;
  int ard[FA], brd[4];
#pragma unroll
  for (int a = 0; a < FA; ++a) ard[a] = swz64(wn * TW + 16 * a + fr, fg);
#pragma unroll
  for (int b = 0; b < 4; ++b) brd[b] = PA * kAPlane + swz64(wk * 64 + 16 * b + fr, fg);

  f4 acc[FA][4];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  const int64_t ns = (M + kGM - 1) / kGM;
  // the loads of stage s+2 and the LDS moves of stage s+1 are spread over
  // the MFMA groups of stage s (one group = 4 MFMAs)
  constexpr bool kSpread = TQ_WGT_SPREAD;
  constexpr int NC = [] {  // (pa, pb) terms per k step
    int n = 0;
    for (int pa = 0; pa < PA; ++pa)
      for (int pb = 0; pb < PB; ++pb) n += pa + pb <= 2;
    return n;
  }();
  constexpr int NG = KS * NC * FA;                   // MFMA groups per stage
  constexpr int NL = NU * 8;                         // loads per stage
  auto step = [&](int64_t s, Regs& r_next, Regs& r_far, auto guard) {
    constexpr bool GUARD = decltype(guard)::value;
    const int buf = static_cast<int>(s & 1);
    const bool do_load = !GUARD || s + 2 < ns, do_store = !GUARD || s + 1 < ns;
    if (!kSpread && do_load) load_stage(s + 2, r_far);
    __builtin_amdgcn_sched_barrier(0);
    int g = 0;
    auto pieces = [&]() {
      if constexpr (kSpread) {
#pragma unroll
        for (int q = g * NL / NG; q < (g + 1) * NL / NG; ++q)
          if (do_load) load_row(s + 2, r_far, q / 8, q % 8);
#pragma unroll
        for (int q = g * NU / NG; q < (g + 1) * NU / NG; ++q)
          if (do_store) put_one(buf ^ 1, r_next, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++g;
    };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* st = lds + buf * kStage + ks * kStep;
      bf16x8 av[PA][FA], bv[PB][4];
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int a = 0; a < FA; ++a)
          av[p][a] = *reinterpret_cast<const bf16x8*>(st + p * kAPlane + ard[a]);
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          bv[p][b] = *reinterpret_cast<const bf16x8*>(st + p * kGPlane + brd[b]);
      // smallest terms first (see above)
#pragma unroll
      for (int lvl = 2; lvl >= 0; --lvl)
#pragma unroll
        for (int pa = PA - 1; pa >= 0; --pa) {
          const int pb = lvl - pa;
          if (pb < 0 || pb >= PB) continue;
#pragma unroll
          for (int a = 0; a < FA; ++a) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[pa][a], bv[pb][b],
                                                                  acc[a][b], 0, 0, 0);
            pieces();
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!kSpread && do_store) store_stage(buf ^ 1, r_next);
    __syncthreads();
  };
  using Free = std::false_type;
  using Guarded = std::true_type;

  Regs r0, r1, r2;
  load_stage(0, r0);
  load_stage(1, r1);
  store_stage(0, r0);
  __syncthreads();
  int64_t s = 0;
  for (; s + 3 <= ns; s += 3) {
    step(s, r1, r2, Free{});
    step(s + 1, r2, r0, Free{});
    step(s + 2, r0, r1, Free{});
  }
  if (s < ns) step(s, r1, r2, Guarded{});
  if (s + 1 < ns) step(s + 1, r2, r0, Guarded{});

  // D of the 16x16 MFMA: lane l holds rows 4(l/16)+i of column l%16.  When
  // accumulating, all old values are loaded before the first store.
  float old[4][FA][4];
  if (ACC) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t k = k0 + wk * 64 + 16 * b + fr;
#pragma unroll
      for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t n = n0 + wn * TW + 16 * a + 4 * fg + i;
          if (k < K && n < N) old[b][a][i] = dW[n * K + k];
        }
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t k = k0 + wk * 64 + 16 * b + fr;
    if (k >= K) continue;
#pragma unroll
    for (int a = 0; a < FA; ++a) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + wn * TW + 16 * a + 4 * fg + i;
        if (n >= N) continue;
        dW[n * K + k] = ACC ? old[b][a][i] + acc[a][b][i] : acc[a][b][i];
      }
    }
  }
}

// Any shape: one thread per dW element, products and sum in fp32, token order.
template <int DA, int DB, bool ACC>
__global__ __launch_bounds__(256) void k_bwd_weight_generic(
    const void* __restrict__ dY, const void* __restrict__ X, int64_t M, int64_t N, int64_t K,
    float* __restrict__ dW) {
  const int64_t total = N * K;
  for (int64_t idx = blockIdx.x * int64_t{256} + threadIdx.x; idx < total;
       idx += int64_t{gridDim.x} * 256) {
    const int64_t n = idx / K, k = idx % K;
    float acc = 0.f;
    for (int64_t m = 0; m < M; ++m) {
      const float a = DA == 0 ? static_cast<const float*>(dY)[m * N + n]
                              : bf16_to_f32(static_cast<const uint16_t*>(dY)[m * N + n]);
      const float b = DB == 0 ? static_cast<const float*>(X)[m * K + k]
                              : bf16_to_f32(static_cast<const uint16_t*>(X)[m * K + k]);
      acc += a * b;
    }
    dW[idx] = ACC ? dW[idx] + acc : acc;
  }
}

template <int DA, int DB, bool ACC>
hipError_t bwd_weight_fast(const BwdWeightArgs& a, hipStream_t s) {
  constexpr int lds_bytes = wgt_lds_bytes<DA, DB>();
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bwd_weight<DA, DB, ACC>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  const int64_t tiles_n = (a.N + wgt_gn(DA, DB) - 1) / wgt_gn(DA, DB);
  const int64_t tiles_k = (a.K + kGK - 1) / kGK;
  const int64_t patches = ((tiles_n + kPN - 1) / kPN) * ((tiles_k + kPK - 1) / kPK);
  const int64_t grid = ((patches + kXcds - 1) / kXcds) * kXcds * kPN * kPK;
  hipLaunchKernelGGL((k_bwd_weight<DA, DB, ACC>), dim3(grid), dim3(kNT), lds_bytes, s, a.dY,
                     a.X, a.M, a.N, a.K, a.dW);
  return hipGetLastError();
}

template <int DA, int DB>
hipError_t bwd_weight_dispatch(const BwdWeightArgs& a, bool fast, hipStream_t s) {
  if (fast) return a.accumulate ? bwd_weight_fast<DA, DB, true>(a, s)
                                : bwd_weight_fast<DA, DB, false>(a, s);
  const int64_t g = grid_for(a.N * a.K);
  if (a.accumulate)
    hipLaunchKernelGGL((k_bwd_weight_generic<DA, DB, true>), dim3(g), dim3(256), 0, s, a.dY, a.X,
                       a.M, a.N, a.K, a.dW);
  else
    hipLaunchKernelGGL((k_bwd_weight_generic<DA, DB, false>), dim3(g), dim3(256), 0, s, a.dY,
                       a.X, a.M, a.N, a.K, a.dW);
  return hipGetLastError();
}

}  // namespace

bool bwd_weight_fast_ok(const BwdWeightArgs& a) {
  const int64_t ea = a.dy_bf16 ? 2 : 4, eb = a.x_bf16 ? 2 : 4;
  constexpr int64_t kLim = int64_t{1} << 31;
  return (a.N % 8) == 0 && (a.K % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(a.dY) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(a.X) & 15u) == 0u &&
         (a.M + 384) * a.N * ea < kLim && (a.M + 384) * a.K * eb < kLim;
}

hipError_t launch_backward_weight(const BwdWeightArgs& a, hipStream_t s) {
  if (a.N == 0 || a.K == 0) return hipSuccess;
  if (a.M == 0) {
    if (a.accumulate) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(a.N * a.K)), dim3(256), 0, s, a.dW,
                       a.N * a.K);
    return hipGetLastError();
  }
  const bool fast = bwd_weight_fast_ok(a);
  if (a.dy_bf16) return a.x_bf16 ? bwd_weight_dispatch<1, 1>(a, fast, s)
                                 : bwd_weight_dispatch<1, 0>(a, fast, s);
  return a.x_bf16 ? bwd_weight_dispatch<0, 1>(a, fast, s) : bwd_weight_dispatch<0, 0>(a, fast, s);
}

bool bwd_input_fast_ok(const BwdInputArgs& a) {
  const int64_t es = a.bf16 ? 2 : 4;
  constexpr int64_t kLim = int64_t{1} << 31;
  return (a.N % 8) == 0 && (reinterpret_cast<uintptr_t>(a.dY) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(a.dX) & 15u) == 0u &&
         (!a.per_row || (reinterpret_cast<uintptr_t>(a.scale) & 15u) == 0u) &&
         int64_t{kBM} * a.N * es < kLim && (a.N + 3 * 4 * kBN) * (a.K / 4) < kLim &&
         (a.N + 3 * 4 * kBN) * 4 < kLim;
}

hipError_t launch_backward_input(const BwdInputArgs& a, hipStream_t s) {
  if (a.M == 0 || a.K == 0) return hipSuccess;
  if (a.N == 0) {
    if (a.accumulate) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(a.M * a.K)), dim3(256), 0, s, a.dX,
                       a.M * a.K);
    return hipGetLastError();
  }
  if (bwd_input_fast_ok(a)) return a.bf16 ? bwd_input_fast_dt<1>(a, s) : bwd_input_fast_dt<0>(a, s);
#define TQ_BWD_GENERIC(DTV, ACCV)                                                          \
  hipLaunchKernelGGL((k_bwd_input_generic<DTV, ACCV>), dim3(grid_for(a.M * a.K)), dim3(256), \
                     0, s, a.dY, a.M, a.packed, a.scale, a.per_row, a.N, a.K, a.dX)
  if (a.bf16) {
    if (a.accumulate) TQ_BWD_GENERIC(1, true);
    else TQ_BWD_GENERIC(1, false);
  } else {
    if (a.accumulate) TQ_BWD_GENERIC(0, true);
    else TQ_BWD_GENERIC(0, false);
  }
#undef TQ_BWD_GENERIC
  return hipGetLastError();
}

}  // namespace tq
