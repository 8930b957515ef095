// Decode-shaped ternary product for 1 <= M <= 16 tokens.
//
// Hetman-2b, src/quantization.py, section 7 (the integer GEMV emulator): per
// output row, decode the packed bytes four weights at a time and accumulate
// int8 x ternary products in an int32 accumulator, then apply one fp32
// scale.  Foundry, docs/quantization.md, "Native Matmul Kernel": the weights
// are unpacked on the fly, never into a dequantised buffer, and the result
// is scaled by gamma afterwards.
//
// gfx950 mapping.  A workgroup (4 waves) owns 16 output rows; the waves
// split K in 256-wide sub-blocks.  Per sub-block a lane loads 16 packed bytes
// (64 codes) of one row with a single 128-bit load, so a wave load covers
// 16 rows x 64 contiguous bytes.  Each 32-bit word (16 codes) is decoded in
// registers with shifts, masks and byte permutes into 16 int8 values 0..2
// (code c = w + 1) and fed as the B operand of v_mfma_i32_16x16x64_i8; the
// A operand holds the int8 tokens (rows beyond M are zero).  Since
// sum_k q*(c-1) = sum_k q*c - sum_k q, the per-token sum of q (formed from
// the same A registers with v_dot4) is subtracted once at the end, which
// keeps the decode to 15 integer operations per word.  Waves combine their
// int32 partial tiles through LDS, and the epilogue applies
// y = acc * gamma * sx in fp32.

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kNT = 256;
constexpr int kWaves = kNT / kWave;
constexpr int kUnroll = 4;  // sub-blocks in flight per wave

template <bool ALIGNED>
__device__ inline uint4 load_chunk16(const uint8_t* base, int64_t off, int64_t limit,
                                     bool ok, uint32_t fill) {
  if (ALIGNED) {
    if (ok && off + 16 <= limit) return *reinterpret_cast<const uint4*>(base + off);
    return make_uint4(fill, fill, fill, fill);
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t o = off + 4 * i + b;
      const uint32_t byte = (ok && o < limit) ? base[o] : ((fill >> (8 * b)) & 0xFFu);
      v |= byte << (8 * b);
    }
    w[i] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool ALIGNED, int YT>
__global__ __launch_bounds__(kNT) void k_gemv(const int8_t* __restrict__ q,
                                              const float* __restrict__ sx, int M,
                                              const uint8_t* __restrict__ packed,
                                              const float* __restrict__ scale, int per_row,
                                              int64_t N, int64_t K, void* __restrict__ Y) {
  __shared__ v4i red_acc[kWaves][kWave];
  __shared__ int red_xs[kWaves][kWave];
  __shared__ int tok_sum[16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;  // output row in the tile (B column) / token (A row)
  const int g = lane >> 4;    // 64-wide K group inside a sub-block
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 16 + col;
  const bool n_ok = n < N;
  const int64_t rowbytes = K >> 2;
  const uint8_t* wrow = packed + (n_ok ? n : 0) * rowbytes;
  const bool m_ok = col < M;
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(q) + (m_ok ? col : 0) * K;
  const int64_t nsb = (K + 255) >> 8;

  v4i acc = {0, 0, 0, 0};
  int xs = 0;
  for (int64_t sb0 = wave; sb0 < nsb; sb0 += kWaves * kUnroll) {
    uint4 wv[kUnroll];
    uint4 xv[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t sb = sb0 + kWaves * u;
      const bool sb_ok = sb < nsb;
      // 0x55 bytes are zero codes; they meet zero activations past K anyway
      wv[u] = load_chunk16<ALIGNED>(wrow, sb * 64 + g * 16, rowbytes, n_ok && sb_ok,
                                    0x55555555u);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xv[u][j] = load_chunk16<ALIGNED>(xrow, sb * 256 + g * 64 + 16 * j, K,
                                         m_ok && sb_ok, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i b = decode_codes_natural(words[j]);
        v4i a;
        a.x = static_cast<int>(xv[u][j].x);
        a.y = static_cast<int>(xv[u][j].y);
        a.z = static_cast<int>(xv[u][j].z);
        a.w = static_cast<int>(xv[u][j].w);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        xs = byte_sum(xv[u][j].x, xs);
        xs = byte_sum(xv[u][j].y, xs);
        xs = byte_sum(xv[u][j].z, xs);
        xs = byte_sum(xv[u][j].w, xs);
      }
    }
  }
  red_acc[wave][lane] = acc;
  red_xs[wave][lane] = xs;
  __syncthreads();
  if (threadIdx.x < 16) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) t += red_xs[w][16 * gg + threadIdx.x];
    tok_sum[threadIdx.x] = t;
  }
  __syncthreads();
  // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16) + i (tokens) of
  // column l%16 (output row).  Wave w finishes element i = w.
  const int i = wave;
  const int m = 4 * g + i;
  if (m >= M || !n_ok) return;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += red_acc[w][lane][i];
  const int accv = total - tok_sum[m];
  const int64_t o = static_cast<int64_t>(m) * N + n;
  if (YT == TQ_I32) {
    static_cast<int*>(Y)[o] = accv;
  } else {
    const float gam = scale[per_row ? n : 0];
    const float y = static_cast<float>(accv) * (gam * sx[m]);
    if (YT == TQ_F32)
      static_cast<float*>(Y)[o] = y;
    else
      static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
  }
}

template <bool ALIGNED>
hipError_t gemv_dispatch(const GemmArgs& a, hipStream_t s) {
  const int64_t grid = (a.N + 15) / 16;
#define TQ_GEMV(YTV)                                                                  \
  hipLaunchKernelGGL((k_gemv<ALIGNED, YTV>), dim3(grid), dim3(kNT), 0, s, a.q, a.sx, \
                     static_cast<int>(a.M), a.packed, a.scale, a.per_row, a.N, a.K, a.Y)
  if (a.ydt == TQ_F32) TQ_GEMV(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMV(TQ_BF16);
  else TQ_GEMV(TQ_I32);
#undef TQ_GEMV
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const GemmArgs& a, hipStream_t s) {
  const bool aligned = (a.K % 64) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.packed) & 15u) == 0u &&
                       (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0u;
  return aligned ? gemv_dispatch<true>(a, s) : gemv_dispatch<false>(a, s);
}

}  // namespace tq
