// Decode-shaped ternary product for 1 <= M <= 16 tokens.
//
// Hetman-2b, src/quantization.py, section 7 (the integer GEMV emulator): per
// output row, decode the packed bytes four weights at a time and accumulate
// int8 x ternary products in an int32 accumulator, then apply one fp32
// scale.  Foundry, docs/quantization.md, "Native Matmul Kernel": the weights
// are unpacked on the fly, never into a dequantised buffer, and the result
// is scaled by gamma afterwards.
//
// gfx950 mapping (general path, M <= 16).  A workgroup (4 waves) owns 16
// output rows; the waves
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

#include <type_traits>

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

// ------------------------------------------------------------------------
// Small-M path (M <= 4): the activations of the workgroup's whole K range are
// staged once in LDS with each 16-byte chunk byte-transposed, which lets the
// packed words be decoded with seven operations (decode_codes_strided)
// instead of fifteen.  Eight waves split K; two accumulators alternate so
// that consecutive MFMAs do not wait on each other.  With SRC != 0 the
// kernel also performs the per-token int8 quantisation of X itself (the same
// operations as k_quant_plain: eta = max(max|x|, eps), optional clamp,
// s = 127/eta, q = clamp(rint(x*s)), sx = eta/127); every workgroup derives
// the same codes, and workgroup 0 writes q and sx out.
#ifndef TQ_GEMV_LDS_WAVES
#define TQ_GEMV_LDS_WAVES 8
#endif
constexpr int kWavesS = TQ_GEMV_LDS_WAVES;
constexpr int kNTs = kWavesS * kWave;
#ifndef TQ_GEMV_LDS_UNROLL
#define TQ_GEMV_LDS_UNROLL 4
#endif
constexpr int kUnrollS = TQ_GEMV_LDS_UNROLL;

template <int SRC>
__device__ inline void load16_act(const void* src, int64_t off, float (&v)[16]) {
  if constexpr (SRC == 1) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = p[i];
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 a = p[i];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  }
}

template <int SRC, int YT>
__global__ __launch_bounds__(kNTs) void k_gemv_lds(
    const void* __restrict__ src, int M, float eps, int clamp, float lo, float hi,
    int8_t* __restrict__ q_out, float* __restrict__ sx_io,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xt[];  // [M][K], chunks transposed
  __shared__ v4i red[kWavesS][kWave];
  __shared__ int tok_sum[4];
  __shared__ uint32_t tok_max[4];
  __shared__ float tok_eta[4];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 16 + col;
  const bool n_ok = n < N;
  const int64_t rowbytes = K >> 2;
  const uint8_t* wrow = packed + (n_ok ? n : 0) * rowbytes;
  const int64_t nsb = (K + 255) >> 8;

  auto load_w = [&](int64_t sb0, uint4 (&wv)[kUnrollS]) {
#pragma unroll
    for (int u = 0; u < kUnrollS; ++u) {
      const int64_t sb = sb0 + kWavesS * u;
      const int64_t off = sb * 64 + g * 16;
      typedef unsigned v4u __attribute__((ext_vector_type(4)));
      if (n_ok && sb < nsb && off + 16 <= rowbytes) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wrow + off));
        wv[u] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        wv[u] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
      }
    }
  };
  uint4 wv[kUnrollS];
  load_w(wave, wv);  // weight loads are in flight while the activations are staged

  if (tid < 4) {
    tok_sum[tid] = 0;
    tok_max[tid] = 0u;
  }
  const int64_t cpr = K / 16;  // 16-byte chunks per token
  const int64_t nchunk = static_cast<int64_t>(M) * cpr;
  __syncthreads();
  if (SRC != 0) {
    for (int64_t c = tid; c < nchunk; c += kNTs) {
      const int m = static_cast<int>(c / cpr);
      float v[16];
      load16_act<SRC>(src, m * K + (c - m * cpr) * 16, v);
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
      atomicMax(&tok_max[m], __float_as_uint(amax));  // non-negative: bit order = value order
    }
    __syncthreads();
    if (tid < M) {
      float eta = fmaxf(__uint_as_float(tok_max[tid]), eps);
      if (clamp) eta = fminf(fmaxf(eta, lo), hi);
      tok_eta[tid] = eta;
      if (blockIdx.x == 0) sx_io[tid] = eta / 127.f;
    }
    __syncthreads();
  }
  for (int64_t c = tid; c < nchunk; c += kNTs) {
    const int m = static_cast<int>(c / cpr);
    const int64_t off = m * K + (c - m * cpr) * 16;
    uint32_t d[4];
    if (SRC == 0) {
      const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(src) + off);
      d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    } else {
      const float s = 127.f / tok_eta[m];
      float v[16];
      load16_act<SRC>(src, off, v);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        d[b] = quant_word(v[4 * b], v[4 * b + 1], v[4 * b + 2], v[4 * b + 3], s);
      if (blockIdx.x == 0)
        *reinterpret_cast<uint4*>(q_out + off) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    *reinterpret_cast<v4i*>(xt + off) = transpose_bytes4x4(d[0], d[1], d[2], d[3]);
    atomicAdd(&tok_sum[m], byte_sum(d[3], byte_sum(d[2], byte_sum(d[1], byte_sum(d[0], 0)))));
  }
  __syncthreads();

  const bool m_ok = col < M;
  v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int64_t sb0 = wave; sb0 < nsb; sb0 += kWavesS * kUnrollS) {
    if (sb0 != wave) load_w(sb0, wv);
#pragma unroll
    for (int u = 0; u < kUnrollS; ++u) {
      const int64_t sb = sb0 + kWavesS * u;
      if (sb >= nsb) break;  // uniform across the wave
      const uint32_t words[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k0 = sb * 256 + 64 * g + 16 * j;
        v4i a = {0, 0, 0, 0};
        if (m_ok && k0 < K) a = *reinterpret_cast<const v4i*>(xt + col * K + k0);
        const v4i b = decode_codes_strided(words[j]);
        if (j & 1)
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc1, 0, 0, 0);
        else
          acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc0, 0, 0, 0);
      }
    }
  }
  red[wave][lane] = acc0 + acc1;
  __syncthreads();
  // D layout: lane l holds tokens 4*(l/16) + i of output column l%16; with
  // M <= 4 only g == 0 carries tokens.  Wave w < 4 finishes element i = w.
  if (wave >= 4 || g != 0) return;
  const int m = wave;
  if (m >= M || !n_ok) return;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWavesS; ++w) total += red[w][lane][m];
  const int accv = total - tok_sum[m];
  const int64_t o = static_cast<int64_t>(m) * N + n;
  if (YT == TQ_I32) {
    static_cast<int*>(Y)[o] = accv;
  } else {
    const float sxm = SRC == 0 ? sx_io[m] : tok_eta[m] / 127.f;
    const float gam = scale[per_row ? n : 0];
    const float y = static_cast<float>(accv) * (gam * sxm);
    if (YT == TQ_F32)
      static_cast<float*>(Y)[o] = y;
    else
      static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
  }
}

// ------------------------------------------------------------------------
// Row-per-wave path (M == 1, K <= 16384).  A single-token weight stream read
// once is latency-bound: its time falls with the number of waves that each
// hold one load in flight, not with the loads per wave, so every wave owns
// one output row and fetches it with one 16-byte buffer load per lane per
// 4096-wide K slice (64 codes a lane).  The loads are ordered so that no wave
// waits on its weights before it must: the thread's share of the token
// first, then the weights, then the epilogue operands.  The token work
// (quantising fp32 / bf16 input exactly as k_quant_plain does when SRC != 0)
// is done by four staging waves and leaves the int8 token in LDS,
// byte-transposed to the strided code order and swizzled so that the lanes'
// 16-byte reads fall in distinct banks.  The weights decode with
// decode_codes_scaled (five operations per 32-bit word): the products with
// codes 4b + 1 and 4b + 2 come out scaled by 4 and 16, go to accumulators of
// their own and are shifted back once per row (exact: int32 sums of
// multiples of 4 or 16; same-box A/B against the seven-operation decode,
// 4096 x 4096: int8 codes in 2.89 -> 2.82 us, fused 3.16-3.21 -> 3.14-3.15 us,
// 4096 x 16384 fused 6.61 -> 6.38 us, the SwiGLU pair 2-7% faster).  With
// ternary codes a staging lane takes whole 16-value units: 16-byte loads,
// the transposed unit built in registers and stored with one 16-byte LDS
// write.  Per-wave maxima and byte sums go through small LDS arrays, so the
// token costs two barriers.  Products use v_dot4 and
// sum_k q*(c-1) = sum_k q*c - sum_k q as in the tiled kernels; the wave sum
// is a DPP reduction.
#ifndef TQ_GEMV_DOT_WAVES
#define TQ_GEMV_DOT_WAVES 16
#endif
constexpr int kRowsD = TQ_GEMV_DOT_WAVES;
constexpr int kNTd = kRowsD * kWave;
// The token is quantised and staged by four waves, one per SIMD: its fixed
// per-wave cost (reductions, the exact divide) is then paid once per SIMD.
constexpr int kStageWaves = 4;
constexpr int kStageNT = kStageWaves * kWave;
static_assert(kRowsD >= kStageWaves, "row-per-wave kernel needs at least four waves");
constexpr int kMaxSlices = 4;        // K <= 16384
constexpr int kBufRaw = 0x00020000;  // raw buffer resource, 32-bit data format
// Cache policy of the packed-weight loads: non-temporal.  A launch reads each
// weight byte once; marked so, the 4 MiB decode stream arrived sooner (same-box
// A/B, 4096 x 4096: 3.34 -> 3.17 us fused, 3.00 -> 2.88 us from int8 codes).
constexpr int kStreamAux = 2;

// Four consecutive token values in their storage type.
template <int SRC>
struct RawQuad {
  uint32_t w[SRC == 1 ? 4 : SRC == 2 ? 2 : 1];
};

template <int SRC>
__device__ inline RawQuad<SRC> load_quad(__amdgpu_buffer_rsrc_t r, int q) {
  RawQuad<SRC> out;
  if constexpr (SRC == 1) {
    const v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * q, 0, 0));
    out.w[0] = v.x; out.w[1] = v.y; out.w[2] = v.z; out.w[3] = v.w;
  } else if constexpr (SRC == 2) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, 8 * q, 0, 0));
    out.w[0] = v.x; out.w[1] = v.y;
  } else {
    out.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, 4 * q, 0, 0);
  }
  return out;
}

template <int SRC>
__device__ inline void quad_to_f32(const RawQuad<SRC>& r, float (&v)[4]) {
  if constexpr (SRC == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v[2 * i] = __uint_as_float(r.w[i] << 16);
      v[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
    }
  }
}

// LDS slot of 16-byte unit u of the staged token.  Reads take units 4l + j
// (lane l, fixed j); XOR-ing the low two bits with bits 3 and 4 spreads any 8
// or 16 consecutive lanes over distinct bank groups.
__device__ inline int dot_slot(int u) { return (u ^ (((u >> 3) ^ (u >> 4)) & 3)) * 16; }

// BITS 2: ternary codes, 64 per 16-byte lane chunk.  BITS 1: the signs of
// binary weights, 64 per 8-byte lane chunk (one 64-bit load), so a slice is
// 4096 codes for both widths; each packed word decodes to eight words of 0/1
// bytes, (w >> s) & 0x01010101 holding the signs of codes 8b + s, the token
// is staged as the matching 8 x 4 byte transpose of each 32-value group, and
// sum_k q*(2b - 1) = 2 * sum_k q*b - sum_k q.
// DUAL (SwiGLU, BITS 2): every wave also contracts the row of a second
// matrix (packed2, scale2) against the same staged token, and the epilogue
// writes h = clamp(silu(g) * u, -clampv, clampv) from the two outputs g and u.
template <int SRC, int S, int BITS, bool DUAL, bool EARLY = true>
__global__ __launch_bounds__(kNTd) void k_gemv_dot(
    const void* __restrict__ src, float eps, int clamp, float lo, float hi,
    int8_t* __restrict__ q_out, float* __restrict__ sx_io,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int K, void* __restrict__ Y, int ydt,
    const uint8_t* __restrict__ packed2, const float* __restrict__ scale2, float clampv) {
  static_assert(!DUAL || BITS == 2, "the SwiGLU pair takes ternary codes");
  extern __shared__ __attribute__((aligned(16))) uint8_t xt[];  // K bytes
  __shared__ float wave_max_part[kStageWaves];
  __shared__ int wave_sum_part[kStageWaves];
  __shared__ float tok_sx;
  // S: K <= 4096 * S, one 4096-code slice of the 64 lanes' chunks each
  constexpr int kRounds = S * 4096 / 4 / kStageNT;    // quads per staging lane
  constexpr int kSl = S;                              // weight slices
  constexpr int kEl = SRC == 1 ? 4 : SRC == 2 ? 2 : 1;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool stager = wave < kStageWaves;
  const int rowbytes = BITS == 2 ? K >> 2 : K >> 3;
  const int64_t nrg = (N + kRowsD - 1) / kRowsD;  // row groups, one per workgroup pass
  const int nquad = K >> 2;

  // 1. the staging waves' quads of the token (reads past K return zero)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(src), static_cast<short>(0), K * kEl, kBufRaw);
  // BITS 2: a staging lane takes whole 16-value units (16 * kEl bytes in
  // kEl 16-byte loads); BITS 1: quads, as the 8 x 4 layout needs
  constexpr int kUnitsL = S * 4096 / 16 / kStageNT;
  constexpr int kLdU = kEl;
  RawQuad<SRC> rq[BITS == 2 ? 1 : kRounds];
  v4i ru[BITS == 2 ? kUnitsL * kLdU : 1];
  if (stager) {
    if constexpr (BITS == 2) {
#pragma unroll
      for (int i = 0; i < kUnitsL; ++i)
#pragma unroll
        for (int j = 0; j < kLdU; ++j)
          ru[i * kLdU + j] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(
                       xr, ((tid + kStageNT * i) * kLdU + j) * 16, 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < kRounds; ++i) rq[i] = load_quad<SRC>(xr, tid + kStageNT * i);
    }
  }
  // 2. the wave's row in row group rg: chunk lane + 64*sl of each slice,
  // and the row's scale.  Rows >= N (also whole groups past the end) read
  // zeros, so the loads are never conditional.
  struct Row {
    uint4 w[kSl];
    uint4 w2[DUAL ? kSl : 1];
    float g, g2;
  };
  auto load_one = [&](const uint8_t* base, const float* sc, int64_t rg,
                      uint4 (&w)[kSl]) -> float {
    const int64_t n = rg * kRowsD + wave;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base + (n < N ? n : 0) * rowbytes), static_cast<short>(0),
        n < N ? rowbytes : 0, kBufRaw);
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      if (BITS == 2) {
        w[sl] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, (lane + kWave * sl) * 16, 0, kStreamAux));
      } else {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_bit_cast(
            u2, __builtin_amdgcn_raw_buffer_load_b64(wr, (lane + kWave * sl) * 8, 0, kStreamAux));
        w[sl] = make_uint4(v.x, v.y, 0u, 0u);
      }
    }
    return ydt == TQ_I32 ? 0.f : sc[per_row ? (n < N ? n : N - 1) : 0];
  };
  auto load_row = [&](int64_t rg, Row& r) {
    r.g = load_one(packed, scale, rg, r.w);
    if constexpr (DUAL) r.g2 = load_one(packed2, scale2, rg, r.w2);
  };
  Row ra, rb;
  int64_t rg = blockIdx.x;
  load_row(rg, ra);
  // 3. epilogue operand of the token
  const float sx_in = SRC == 0 ? sx_io[0] : 0.f;

  // 4. token scale (SRC != 0): staging-wave maxima, folded by each stager
  float sc = 0.f;
  if (SRC != 0) {
    if (stager) {
      float mx = 0.f;
      if constexpr (BITS == 2 && SRC == 2) {
        // bf16: for finite values the order of |x| is that of the unsigned
        // integer of its 15 low bits, so two values at a time by a packed max
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = {0, 0};
#pragma unroll
        for (int i = 0; i < kUnitsL * kLdU; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m = __builtin_elementwise_max(
                m, __builtin_bit_cast(u16x2, static_cast<uint32_t>(ru[i][e]) & 0x7FFF7FFFu));
        mx = __uint_as_float(static_cast<uint32_t>(m.x > m.y ? m.x : m.y) << 16);
      } else if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < kUnitsL * kLdU; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mx = fmaxf(mx, fabsf(__uint_as_float(static_cast<uint32_t>(ru[i][e]))));
      } else {
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
          float v[4];
          quad_to_f32<SRC>(rq[i], v);  // zeros past K
          mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        }
      }
      mx = wave_max_last(mx);
      if (lane == kWave - 1) wave_max_part[wave] = mx;
    }
    __syncthreads();
    // the staging waves need 127 / eta; eta / 127 (for the epilogue) is
    // formed by the first wave that does not stage, off their path
    constexpr int kSxTid = (kRowsD > kStageWaves ? kStageWaves : 0) * kWave;
    if (stager || tid == kSxTid) {
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < kStageWaves; ++w) amax = fmaxf(amax, wave_max_part[w]);
      float eta = fmaxf(amax, eps);
      if (clamp) eta = fminf(fmaxf(eta, lo), hi);
      if (stager) sc = 127.f / eta;
      if (tid == kSxTid) {
        const float sxv = eta / 127.f;
        tok_sx = sxv;
        if (blockIdx.x == 0) sx_io[0] = sxv;
      }
    }
  }
  // The codes workgroup 0 writes back (SRC != 0) are stored once the whole
  // token is staged: stores and loads share one counter, so a store issued
  // between the staging steps would make the next wait for a token load
  // also wait for the weights (same-box A/B, 4096 x 4096 fused: 2.97 ->
  // 2.86 us; at the end of the kernel instead, 2.85 us, but the SwiGLU
  // decode FFN at one token 8.93 -> 9.17 us).
  uint32_t qk[BITS == 2 && SRC != 0 ? kUnitsL : 1][4];
  auto flush_q = [&]() {
    if constexpr (BITS == 2 && SRC != 0) {
      if (stager && blockIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kUnitsL; ++i) {
          const int u = tid + kStageNT * i;
          if (u < (K >> 4))
            *reinterpret_cast<uint4*>(q_out + 16 * static_cast<int64_t>(u)) =
                make_uint4(qk[i][0], qk[i][1], qk[i][2], qk[i][3]);
        }
      }
    }
  };
  // 5. int8 token -> transposed, swizzled LDS; byte sums.  Without an eta
  // clamp every |x| <= eta and the codes need no clamp (quant_word_unclamped).
  auto stage_units = [&](auto clamped) {
    constexpr bool CL = decltype(clamped)::value;
    int bsum = 0;
    const int nunit = K >> 4;
#pragma unroll
    for (int i = 0; i < kUnitsL; ++i) {
      const int u = tid + kStageNT * i;
      if (u < nunit) {
        uint32_t d[4];  // quad b: values 4b .. 4b+3 as int8 codes
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if constexpr (SRC == 0) {
            d[b] = static_cast<uint32_t>(ru[i][b]);
          } else {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int val = 4 * b + e;  // value of the unit
              if constexpr (SRC == 1) {
                v[e] = __uint_as_float(static_cast<uint32_t>(ru[i * kLdU + val / 4][val % 4]));
              } else {
                const uint32_t w = static_cast<uint32_t>(ru[i * kLdU + val / 8][(val % 8) / 2]);
                v[e] = __uint_as_float((val & 1) ? (w & 0xFFFF0000u) : (w << 16));
              }
            }
            d[b] = CL ? quant_word(v[0], v[1], v[2], v[3], sc)
                      : quant_word_unclamped(v[0], v[1], v[2], v[3], sc);
            qk[i][b] = d[b];
          }
          bsum = byte_sum(d[b], bsum);
        }
        *reinterpret_cast<v4i*>(xt + dot_slot(u)) = transpose_bytes4x4(d[0], d[1], d[2], d[3]);
      }
    }
    bsum = wave_isum_last(bsum);
    if (lane == kWave - 1) wave_sum_part[wave] = bsum;
  };
  if (stager && BITS == 2) {
    if (SRC == 0 || clamp)
      stage_units(std::true_type{});
    else
      stage_units(std::false_type{});
    flush_q();
  } else if (stager) {
    int bsum = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int qi = tid + kStageNT * i;
      if (qi < nquad) {
        uint32_t d;
        if (SRC == 0) {
          d = rq[i].w[0];
        } else {
          float v[4];
          quad_to_f32<SRC>(rq[i], v);
          d = quant_word(v[0], v[1], v[2], v[3], sc);
          if (blockIdx.x == 0) reinterpret_cast<uint32_t*>(q_out)[qi] = d;
        }
        // BITS 2: quad qi is word b = qi % 4 of unit qi / 4; its byte s goes
        // to byte b of word s of the transposed unit.  BITS 1: value
        // v = 4 qi + s of group v / 32 goes to byte (v % 32) / 8 of word v % 8
        // of the group's two units.
        uint8_t* dst = BITS == 2 ? xt + dot_slot(qi >> 2) + (qi & 3)
                                 : xt + dot_slot(2 * (qi >> 3) + (qi & 1)) + ((qi >> 1) & 3);
        dst[0] = static_cast<uint8_t>(d);
        dst[4] = static_cast<uint8_t>(d >> 8);
        dst[8] = static_cast<uint8_t>(d >> 16);
        dst[12] = static_cast<uint8_t>(d >> 24);
        bsum = byte_sum(d, bsum);
      }
    }
    bsum = wave_isum_last(bsum);
    if (lane == kWave - 1) wave_sum_part[wave] = bsum;
  }
  asm volatile("" ::"v"(ra.g));
  if constexpr (DUAL) asm volatile("" ::"v"(ra.g2));
  asm volatile("" ::"v"(sx_in));
  // With the token quantised here (SRC != 0), the first row's weights have
  // mostly landed by the time the staging waves finish, and every wave would
  // then decode at once.  The other waves, idle until the barrier, decode
  // their first row before it (EARLY).  The barrier then also waits for the
  // slowest of the workgroup's weights; where every lane's slices are full
  // (K = 4096 or 8192) the launcher measured the plain order faster.
  // (Not for the SwiGLU pair: there the split first row group measured
  // slower, with or without the early decode.)
  constexpr bool PRE = EARLY && SRC != 0 && BITS == 2 && !DUAL;
  v4i pre[PRE ? kSl : 1][4], pre2[PRE && DUAL ? kSl : 1][4];
  if constexpr (PRE) {
    if (!stager) {
#pragma unroll
      for (int sl = 0; sl < kSl; ++sl) {
        const uint32_t words[4] = {ra.w[sl].x, ra.w[sl].y, ra.w[sl].z, ra.w[sl].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[sl][j] = decode_codes_scaled(words[j]);
        if constexpr (DUAL) {
          const uint32_t words2[4] = {ra.w2[sl].x, ra.w2[sl].y, ra.w2[sl].z, ra.w2[sl].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) pre2[sl][j] = decode_codes_strided(words2[j]);
        }
      }
    }
  }
  __syncthreads();
  int tsum = 0;
#pragma unroll
  for (int w = 0; w < kStageWaves; ++w) tsum += wave_sum_part[w];
  const float sxv = SRC == 0 ? sx_in : tok_sx;

  // 6. contraction of the wave's row in group rg (P: its codes are in `pre`)
  auto finish_p = [&](int64_t rg, const Row& r, auto predecoded) {
    constexpr bool P = decltype(predecoded)::value;
    const int64_t n = rg * kRowsD + wave;
    int acc = 0, acc2 = 0, a4 = 0, a16 = 0, b4 = 0, b16 = 0;
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      const int chunk = lane + kWave * sl;
      const uint32_t words[4] = {r.w[sl].x, r.w[sl].y, r.w[sl].z, r.w[sl].w};
      if (BITS == 2) {
        const int unit = 4 * chunk;   // first 16-code unit of the chunk
        if (16 * unit >= K) break;    // this chunk, and every later one, is past K
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v4i cd;
          if constexpr (P && PRE)
            cd = pre[sl][j];
          else
            cd = decode_codes_scaled(words[j]);
          const v4i x = *reinterpret_cast<const v4i*>(xt + dot_slot(unit + j));
          acc = __builtin_amdgcn_sdot4(x.x, cd.x, acc, false);
          a4 = __builtin_amdgcn_sdot4(x.y, cd.y, a4, false);
          a16 = __builtin_amdgcn_sdot4(x.z, cd.z, a16, false);
          acc = __builtin_amdgcn_sdot4(x.w, cd.w, acc, false);
          if constexpr (DUAL) {
            const uint32_t words2[4] = {r.w2[sl].x, r.w2[sl].y, r.w2[sl].z, r.w2[sl].w};
            v4i cu;
            if constexpr (P && PRE)
              cu = pre2[sl][j];
            else
              cu = decode_codes_scaled(words2[j]);
            acc2 = __builtin_amdgcn_sdot4(x.x, cu.x, acc2, false);
            b4 = __builtin_amdgcn_sdot4(x.y, cu.y, b4, false);
            b16 = __builtin_amdgcn_sdot4(x.z, cu.z, b16, false);
            acc2 = __builtin_amdgcn_sdot4(x.w, cu.w, acc2, false);
          }
        }
      } else {
        const int group = 2 * chunk;  // first 32-code group of the chunk
        if (32 * group >= K) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v4i x0 = *reinterpret_cast<const v4i*>(xt + dot_slot(2 * (group + j)));
          const v4i x1 = *reinterpret_cast<const v4i*>(xt + dot_slot(2 * (group + j) + 1));
          const uint32_t wj = words[j];
          acc = __builtin_amdgcn_sdot4(x0.x, static_cast<int>(wj & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x0.y, static_cast<int>((wj >> 1) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x0.z, static_cast<int>((wj >> 2) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x0.w, static_cast<int>((wj >> 3) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x1.x, static_cast<int>((wj >> 4) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x1.y, static_cast<int>((wj >> 5) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x1.z, static_cast<int>((wj >> 6) & 0x01010101u), acc, false);
          acc = __builtin_amdgcn_sdot4(x1.w, static_cast<int>((wj >> 7) & 0x01010101u), acc, false);
        }
      }
    }
    if (BITS == 2) {
      acc += (a4 >> 2) + (a16 >> 4);
      if constexpr (DUAL) acc2 += (b4 >> 2) + (b16 >> 4);
    }
    acc = wave_isum_last(acc);
    if constexpr (DUAL) acc2 = wave_isum_last(acc2);
    if (lane != kWave - 1 || n >= N) return;
    const int accv = BITS == 2 ? acc - tsum : 2 * acc - tsum;
    if constexpr (DUAL) {
      const float gv = static_cast<float>(accv) * (r.g * sxv);
      const float uv = static_cast<float>(acc2 - tsum) * (r.g2 * sxv);
      const float h = fminf(fmaxf(gv / (1.f + expf(-gv)) * uv, -clampv), clampv);
      if (ydt == TQ_F32)
        static_cast<float*>(Y)[n] = h;
      else
        static_cast<uint16_t*>(Y)[n] = f32_to_bf16(h);
    } else if (ydt == TQ_I32) {
      static_cast<int*>(Y)[n] = accv;
    } else {
      const float y = static_cast<float>(accv) * (r.g * sxv);
      if (ydt == TQ_F32)
        static_cast<float*>(Y)[n] = y;
      else
        static_cast<uint16_t*>(Y)[n] = f32_to_bf16(y);
    }
  };
  auto finish = [&](int64_t rg, const Row& r) { finish_p(rg, r, std::false_type{}); };
  // the first row group: decoded before the barrier unless a staging wave
  auto finish_first = [&](int64_t rg, const Row& r) {
    if (PRE && !stager)
      finish_p(rg, r, std::true_type{});
    else
      finish_p(rg, r, std::false_type{});
  };
  // Row groups rg, rg + gridDim.x, ...: the next group's row is loaded
  // before the current one is contracted, alternating two named register
  // sets so that no copy of a load in flight is needed.  The last group
  // issues no load: a load past the end would still have to return before
  // the wave may end.
  const int64_t step = gridDim.x;
  if constexpr (PRE) {
    if (rg + step >= nrg) {
      finish_first(rg, ra);
      return;
    }
    load_row(rg + step, rb);
    finish_first(rg, ra);
    rg += step;
    for (;;) {
      if (rg + step >= nrg) {
        finish(rg, rb);
        break;
      }
      load_row(rg + step, ra);
      finish(rg, rb);
      rg += step;
      if (rg + step >= nrg) {
        finish(rg, ra);
        break;
      }
      load_row(rg + step, rb);
      finish(rg, ra);
      rg += step;
    }
  } else {
    for (;;) {
      if (rg + step >= nrg) {
        finish(rg, ra);
        break;
      }
      load_row(rg + step, rb);
      finish(rg, ra);
      rg += step;
      if (rg + step >= nrg) {
        finish(rg, rb);
        break;
      }
      load_row(rg + step, ra);
      finish(rg, rb);
      rg += step;
    }
  }
}

// Second matrix of the SwiGLU pair (DUAL launches only).
struct DualArgs {
  const uint8_t* packed2 = nullptr;
  const float* scale2 = nullptr;
  float clampv = 0.f;
};

template <int SRC, int S, int BITS, bool DUAL, bool EARLY = true>
hipError_t gemv_dot_launch_s(const void* src, const ActParams* p, int8_t* q_out, float* sx,
                             const GemmArgs& a, const DualArgs& d, hipStream_t s) {
  // one workgroup per row group up to two per compute unit (the resident
  // limit of 1024-thread workgroups); past that, workgroups loop over groups
  const int64_t groups = (a.N + kRowsD - 1) / kRowsD;
  const int64_t cap = 2 * static_cast<int64_t>(device_cus() > 0 ? device_cus() : 256);
  const int64_t grid = groups < cap ? groups : cap;
  const float eps = p ? p->eps : 0.f, lo = p ? p->eta_min : 0.f, hi = p ? p->eta_max : 0.f;
  const int clamp = p ? p->clamp : 0;
  hipLaunchKernelGGL((k_gemv_dot<SRC, S, BITS, DUAL, EARLY>), dim3(grid), dim3(kNTd),
                     static_cast<size_t>(a.K), s, src, eps, clamp, lo, hi, q_out, sx, a.packed,
                     a.scale, a.per_row, a.N, static_cast<int>(a.K), a.Y, a.ydt, d.packed2,
                     d.scale2, d.clampv);
  return hipGetLastError();
}

template <int SRC, int BITS = 2, bool DUAL = false>
hipError_t gemv_dot_launch(const void* src, const ActParams* p, int8_t* q_out, float* sx,
                           const GemmArgs& a, hipStream_t s, const DualArgs& d = DualArgs()) {
  // The early decode of the first row (quantising kernels only) measured
  // slower where the slices are exactly full at one or two slices (same-box
  // A/B: 4096 x 4096 3.16 -> 3.05 us, 11008 x 4096 5.11 -> 4.71, 4096 x 8192
  // 4.17 -> 4.11) and faster elsewhere (K = 1024, 2560, 3072, 6912, 16384:
  // 1-4%).
  constexpr bool kEarlyMatters = SRC != 0 && BITS == 2 && !DUAL;
  if (a.K <= 4096) {
    if constexpr (kEarlyMatters)
      if (a.K == 4096) return gemv_dot_launch_s<SRC, 1, BITS, DUAL, false>(src, p, q_out, sx, a, d, s);
    return gemv_dot_launch_s<SRC, 1, BITS, DUAL>(src, p, q_out, sx, a, d, s);
  }
  if (a.K <= 8192) {
    if constexpr (kEarlyMatters)
      if (a.K == 8192) return gemv_dot_launch_s<SRC, 2, BITS, DUAL, false>(src, p, q_out, sx, a, d, s);
    return gemv_dot_launch_s<SRC, 2, BITS, DUAL>(src, p, q_out, sx, a, d, s);
  }
  return gemv_dot_launch_s<SRC, kMaxSlices, BITS, DUAL>(src, p, q_out, sx, a, d, s);
}

// One token, K a multiple of 64 up to 16384 (the token and its LDS copy are
// then at most 64 KiB, offsets 32-bit; the row offset n*K/4 is 64-bit).
bool dot_path_ok(int64_t M, int64_t K, const void* packed, const void* act) {
  return M == 1 && (K % 64) == 0 && K <= 4096 * kMaxSlices &&
         (reinterpret_cast<uintptr_t>(packed) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(act) & 15u) == 0u;
}

template <int SRC>
hipError_t gemv_lds_launch(const void* src, int M, const ActParams* p, int8_t* q_out,
                           float* sx, const GemmArgs& a, hipStream_t s) {
  const int64_t grid = (a.N + 15) / 16;
  const size_t lds = static_cast<size_t>(M) * static_cast<size_t>(a.K);
  const float eps = p ? p->eps : 0.f, lo = p ? p->eta_min : 0.f, hi = p ? p->eta_max : 0.f;
  const int clamp = p ? p->clamp : 0;
#define TQ_GEMV_LDS(YTV)                                                                 \
  hipLaunchKernelGGL((k_gemv_lds<SRC, YTV>), dim3(grid), dim3(kNTs), lds, s, src, M, eps, \
                     clamp, lo, hi, q_out, sx, a.packed, a.scale, a.per_row, a.N, a.K, a.Y)
  if (a.ydt == TQ_F32) TQ_GEMV_LDS(TQ_F32);
  else if (a.ydt == TQ_BF16) TQ_GEMV_LDS(TQ_BF16);
  else TQ_GEMV_LDS(TQ_I32);
#undef TQ_GEMV_LDS
  return hipGetLastError();
}

bool lds_path_ok(int64_t M, int64_t K, const void* packed, const void* act) {
  return M >= 1 && M <= 4 && (K % 64) == 0 && M * K <= kGemvLdsBytes &&
         (reinterpret_cast<uintptr_t>(packed) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(act) & 15u) == 0u;
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

// ------------------------------------------------------------------------
// 2..16 tokens on matrix cores (K % 256 == 0).  A workgroup owns 16 output
// rows and W = min(16, K/256) waves; wave w takes the 256-code K blocks
// w, w + W, ...  Per block a lane holds 16 packed bytes, 64 codes, of row
// l % 16 at byte offset 16 * (l / 16) of the block (one 128-bit buffer load
// per lane, rows past N read zeros).  Its four words feed four
// v_mfma_i32_16x16x64_i8: in MFMA j, lane l's 16-slot group stands for the
// codes 64 * (l / 16) + 16 * j + 0..15 of the block.  Because the dot product
// is unchanged by any permutation of K applied to both operands, the token
// fragment for that MFMA is the matching 16 token bytes, a contiguous
// 16-byte read.  Weight words decode in 7 operations to codes 0..2 (the
// strided order, matched by staging the tokens byte-transposed); the same
// token fragments times an all-ones operand accumulate each token's sum over
// the wave's blocks, subtracted at the end, so the tiles are the exact int32
// sums of q (c - 1) (the extra product replaced 8 operations per word that
// mapped the codes to c - 1: same-box A/B 1-3% faster, the SwiGLU pair 3-4%).
// The workgroup stages the M int8 tokens once in LDS with a row pitch of
// K + 16 bytes (lanes of a fragment read then fall in distinct banks); rows
// M..15 of the MFMA read zeros.  With int8 tokens each thread's S units
// (S = 1, 2, 4 or 8 by the launcher: the fewest that cover the tokens) are
// loaded ahead of the weights and staged as each lands, so that the tokens
// are in LDS when the weights arrive (same-box A/B against a loop that
// loaded one unit at a time once the weights had landed: 16 tokens on the
// FFN shapes 5.3 -> 4.8 us and 5.8 -> 5.6 us, on 4096 x 4096 4.7 -> 4.4 us;
// 4 tokens 1.5-3% faster).  The waves' 16 x 16 partial tiles are summed
// through LDS and the threads apply the epilogue, 256 outputs a tile.
constexpr int kMfmaRows = 16;
constexpr int kMfmaMaxWaves = 16;

// 16 consecutive token values in their storage type: int8 (one 16-byte
// word), fp32 (four) or bf16 (two).
template <int SRC>
struct RawUnit {
  static constexpr int kWords = SRC == 1 ? 4 : SRC == 2 ? 2 : 1;
  v4i w[kWords];
};

template <int SRC>
__device__ inline RawUnit<SRC> load_unit(__amdgpu_buffer_rsrc_t r, int c) {
  RawUnit<SRC> u;
#pragma unroll
  for (int i = 0; i < RawUnit<SRC>::kWords; ++i)
    u.w[i] = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (RawUnit<SRC>::kWords * c + i), 0, 0));
  return u;
}

template <int SRC>
__device__ inline void unit_to_f32(const RawUnit<SRC>& u, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < RawUnit<SRC>::kWords; ++i) {
    const uint32_t w[4] = {static_cast<uint32_t>(u.w[i].x), static_cast<uint32_t>(u.w[i].y),
                           static_cast<uint32_t>(u.w[i].z), static_cast<uint32_t>(u.w[i].w)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (SRC == 1) {
        v[4 * i + k] = __uint_as_float(w[k]);
      } else {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  }
}

// BITS 1 (signs of binary weights): a lane holds 8 packed bytes, 64 signs,
// of its row per block (one 64-bit load).  MFMA j takes 32-bit word j / 2 and
// its operand word t is (w >> (4 (j % 2) + t)) & 0x01010101, byte b holding
// the sign of code 8 b + 4 (j % 2) + t of the word, mapped to -1 / +1 by one
// byte permute.  The matching token operand is the 4 x 4 byte transpose of
// the quads 4 (j % 2) / 4 + {0, 2, 4, 6} of the 32 values, so each 32-value
// group is staged as two transposes, in place.
// DUAL (SwiGLU, BITS 2): the row block of a second matrix (packed2, scale2)
// is contracted against the same token fragments into a second tile, and the
// epilogue writes h = clamp(silu(g) * u, -clampv, clampv).
template <int SRC, int KBW, int BITS, bool DUAL, int S>
__global__ __launch_bounds__(kMfmaMaxWaves* kWave) void k_gemv_mfma(
    const void* __restrict__ src, float eps, int clamp, float lo, float hi,
    int8_t* __restrict__ q_out, float* __restrict__ sx_io, int M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int K, void* __restrict__ Y, int ydt,
    const uint8_t* __restrict__ packed2, const float* __restrict__ scale2, float clampv) {
  static_assert(!DUAL || BITS == 2, "the SwiGLU pair takes ternary codes");
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // M x (K + 16) bytes
  __shared__ uint32_t tok_max[kMfmaRows];
  __shared__ float tok_sc[kMfmaRows];  // 127 / eta
  __shared__ float tok_sx[kMfmaRows];  // eta / 127
  constexpr int kEl = SRC == 1 ? 4 : SRC == 2 ? 2 : 1;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nw = blockDim.x / kWave;
  const int nt = blockDim.x;
  const int pitch = K + 16;
  const int upr = K >> 4;          // 16-value units per token
  const int nkb = K >> 8;          // 256-code blocks
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kMfmaRows;
  const int rowbytes = BITS == 2 ? K >> 2 : K >> 3;

  // 1. the thread's first token unit (a read past the end returns zero),
  // then its weight blocks and the epilogue operands of its output (token
  // m, row n0 + n).  With int8 tokens and ternary codes the epilogue
  // operands go first, and for S > 1 the thread's other S - 1 units go out
  // with the first,
  // unconditionally, so that each is staged as soon as it lands, while the
  // weights are in flight (a branch around them would leave the compiler
  // unable to count the loads ahead of each one).
  const int em = tid >> 4, en = tid & 15;
  const bool eout = tid < kMfmaRows * kMfmaRows && em < M && n0 + en < N;
  float egam = 0.f, egam2 = 0.f, esx = 0.f;
  auto load_epi = [&]() {
    if (eout && ydt != TQ_I32) {
      egam = scale[per_row ? n0 + en : 0];
      if (DUAL) egam2 = scale2[per_row ? n0 + en : 0];
      if (SRC == 0) esx = sx_io[em];
    }
  };
  if constexpr (SRC == 0 && BITS == 2) load_epi();
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(src), static_cast<short>(0), M * K * kEl, kBufRaw);
  const int nunits = M * upr;
  static_assert(BITS == 2 || SRC == 0, "1-bit weights take int8 tokens");
  // BITS 2: one 16-value unit per thread per round; BITS 1: a 32-value
  // group (two units) per thread per round
  const RawUnit<SRC> u0 = load_unit<SRC>(qr, BITS == 2 ? tid : 2 * tid);
  const RawUnit<SRC> u1 = BITS == 2 ? u0 : load_unit<SRC>(qr, 2 * tid + 1);
  static_assert(S == 1 || (SRC == 0 && BITS == 2), "unit slots: int8 tokens, ternary codes");
  RawUnit<SRC> ux[S > 1 ? S - 1 : 1];
  if constexpr (S > 1) {
#pragma unroll
    for (int j = 1; j < S; ++j) ux[j - 1] = load_unit<SRC>(qr, tid + j * nt);
  }
  const int64_t rows_here = N - n0 < kMfmaRows ? N - n0 : kMfmaRows;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed + n0 * rowbytes), static_cast<short>(0),
      static_cast<int>(rows_here * rowbytes), kBufRaw);
  const int fr = lane & 15, fg = lane >> 4;
  const __amdgpu_buffer_rsrc_t wr2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(DUAL ? packed2 + n0 * rowbytes : packed), static_cast<short>(0),
      DUAL ? static_cast<int>(rows_here * rowbytes) : 0, kBufRaw);
  uint4 wv[KBW];
  uint4 wv2[DUAL ? KBW : 1];
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int kb = wave + nw * i;  // blocks past the end read zeros and are skipped
    const int kbl = kb < nkb ? kb : 0;
    if (BITS == 2) {
      wv[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, fr * rowbytes + 64 * kbl + 16 * fg, 0,
                                                       kStreamAux));
      if constexpr (DUAL)
        wv2[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               wr2, fr * rowbytes + 64 * kbl + 16 * fg, 0,
                                               kStreamAux));
    } else {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      const u2 v = __builtin_bit_cast(
          u2, __builtin_amdgcn_raw_buffer_load_b64(wr, fr * rowbytes + 32 * kbl + 8 * fg, 0,
                                                   kStreamAux));
      wv[i] = make_uint4(v.x, v.y, 0u, 0u);
    }
  }
  if constexpr (SRC != 0 || BITS != 2) load_epi();

  // 2. (fp32 / bf16 tokens) per-token absmax and scale, as k_quant_plain
  if (SRC != 0) {
    if (tid < kMfmaRows) tok_max[tid] = 0u;
    __syncthreads();
    auto unit_max = [&](const RawUnit<SRC>& u, int c) {
      float v[16];
      unit_to_f32<SRC>(u, v);
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
      atomicMax(&tok_max[c / upr], __float_as_uint(mx));
    };
    // The first unit of every thread: the 64 units of a wave are
    // consecutive, so with at least 63 units a token they span two tokens
    // at most, m0 and m0 + 1; the wave reduces both maxima and one lane
    // writes them (an atomic from every lane on one LDS word serialises:
    // same-box A/B, 4 x 4096 fused 5.70 -> 5.01 us, 4 x 2560 6.05 -> 5.77).
    // Later units (none where the launcher fuses: M K <= 16384 with M <= 4
    // gives each thread one unit) take one atomic each.
    if (upr >= kWave - 1) {
      float v[16];
      unit_to_f32<SRC>(u0, v);
      float mx = 0.f;  // zero past the end (the load read zeros)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
      const int cw = wave * kWave;  // the wave's first unit
      if (cw < nunits) {
        const int m0 = cw / upr;
        const bool lo = tid / upr == m0;
        const float a0 = wave_max_last(lo ? mx : 0.f);
        const float a1 = wave_max_last(lo ? 0.f : mx);
        if (lane == kWave - 1) {
          atomicMax(&tok_max[m0], __float_as_uint(a0));
          if (m0 + 1 < M) atomicMax(&tok_max[m0 + 1], __float_as_uint(a1));
        }
      }
    } else if (tid < nunits) {
      unit_max(u0, tid);
    }
    for (int c = tid + nt; c < nunits; c += nt) unit_max(load_unit<SRC>(qr, c), c);
    __syncthreads();
    if (tid < M) {
      float eta = fmaxf(__uint_as_float(tok_max[tid]), eps);
      if (clamp) eta = fminf(fmaxf(eta, lo), hi);
      tok_sc[tid] = 127.f / eta;
      const float sxv = eta / 127.f;
      tok_sx[tid] = sxv;
      if (blockIdx.x == 0) sx_io[tid] = sxv;
    }
    __syncthreads();
  }
  // 3. int8 tokens -> LDS, each 16-byte unit byte-transposed
  auto stage = [&](const RawUnit<SRC>& u, int c) {
    const int m = c / upr, uu = c - m * upr;
    uint32_t d[4];
    if (SRC == 0) {
      d[0] = u.w[0].x; d[1] = u.w[0].y; d[2] = u.w[0].z; d[3] = u.w[0].w;
    } else {
      float v[16];
      unit_to_f32<SRC>(u, v);
      const float sc = tok_sc[m];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        d[b] = quant_word(v[4 * b], v[4 * b + 1], v[4 * b + 2], v[4 * b + 3], sc);
      if (blockIdx.x == 0)
        *reinterpret_cast<uint4*>(q_out + 16 * static_cast<int64_t>(c)) =
            make_uint4(d[0], d[1], d[2], d[3]);
    }
    *reinterpret_cast<v4i*>(xs + m * pitch + 16 * uu) = transpose_bytes4x4(d[0], d[1], d[2], d[3]);
  };
  if (BITS == 2) {
    if constexpr (SRC == 0) {
      // int8 units staged unconditionally (a branch would let the compiler
      // move a load into it, behind the weights): a unit past the end, read
      // as zeros, goes to the 16 padding bytes of row 0, which no product
      // reads
      // unit c = tid + j nt is unit r of token m (m >= M past the end); one
      // more j adds nt, so (m, r) advances without another division
      int m = tid / upr, r = tid - m * upr;
      auto stage_int8 = [&](const RawUnit<SRC>& uv) {
        const int off = m < M ? m * pitch + 16 * r : K;
        *reinterpret_cast<v4i*>(xs + off) =
            transpose_bytes4x4(uv.w[0].x, uv.w[0].y, uv.w[0].z, uv.w[0].w);
      };
      stage_int8(u0);
      if constexpr (S > 1) {
        const int adv_m = nt / upr, adv_r = nt - adv_m * upr;
#pragma unroll
        for (int j = 1; j < S; ++j) {
          r += adv_r;
          m += adv_m;
          if (r >= upr) {
            r -= upr;
            ++m;
          }
          stage_int8(ux[j - 1]);
        }
      } else {
        for (int c = tid + nt; c < nunits; c += nt) {
          m = c / upr;
          r = c - m * upr;
          stage_int8(load_unit<SRC>(qr, c));
        }
      }
    } else {
      if (tid < nunits) stage(u0, tid);
      for (int c = tid + nt; c < nunits; c += nt) stage(load_unit<SRC>(qr, c), c);
    }
  } else {
    // group g: quads Q0..Q7 = a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w
    auto stage1 = [&](const RawUnit<SRC>& a, const RawUnit<SRC>& b, int g) {
      const int gpr = upr >> 1;
      const int m = g / gpr, gg = g - m * gpr;
      uint8_t* dst = xs + m * pitch + 32 * gg;
      *reinterpret_cast<v4i*>(dst) =
          transpose_bytes4x4(a.w[0].x, a.w[0].z, b.w[0].x, b.w[0].z);
      *reinterpret_cast<v4i*>(dst + 16) =
          transpose_bytes4x4(a.w[0].y, a.w[0].w, b.w[0].y, b.w[0].w);
    };
    const int ngroups = nunits >> 1;
    if (tid < ngroups) stage1(u0, u1, tid);
    for (int g = tid + nt; g < ngroups; g += nt)
      stage1(load_unit<SRC>(qr, 2 * g), load_unit<SRC>(qr, 2 * g + 1), g);
  }
  __syncthreads();
  if (SRC != 0 && eout) esx = tok_sx[em];

  // 4. contraction of the wave's blocks.  Ternary codes enter the products
  // as 0..2; a product with an all-ones operand gives the wave's share of
  // each token's sum, subtracted once at the end (sum q (c - 1)).
  v4i acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const bool arow = fr < M;
  const uint8_t* abase = xs + (arow ? fr : 0) * pitch + 64 * fg;
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int kb = wave + nw * i;
    if (kb >= nkb) break;
    const uint32_t words[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4i b;
      if (BITS == 2) {
        b = decode_codes_strided(words[j]);
      } else {
        // bytes 0 / 1 select 0xFF (-1) / 0x01 (+1) from the permute pool
        auto pm = [](uint32_t x) {
          return static_cast<int>(__builtin_amdgcn_perm(0u, 0x000001FFu, x & 0x01010101u));
        };
        const uint32_t wj = words[j >> 1] >> (4 * (j & 1));
        b.x = pm(wj);
        b.y = pm(wj >> 1);
        b.z = pm(wj >> 2);
        b.w = pm(wj >> 3);
      }
      v4i a = *reinterpret_cast<const v4i*>(abase + 256 * kb + 16 * j);
      if (!arow) a = v4i{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
      if constexpr (BITS == 2) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, ones, acc1, 0, 0, 0);
      if constexpr (DUAL) {
        const uint32_t words2[4] = {wv2[i].x, wv2[i].y, wv2[i].z, wv2[i].w};
        const v4i b2 = decode_codes_strided(words2[j]);
        acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b2, acc2, 0, 0, 0);
      }
    }
  }
  if constexpr (BITS == 2) {
    acc -= acc1;
    if constexpr (DUAL) acc2 -= acc1;
  }
  __syncthreads();  // every wave is done with the tokens: reuse LDS

  // 5. sum the waves' tiles; D layout: lane l holds rows 4 * (l / 16) + i,
  // column l % 16
  int* red = reinterpret_cast<int*>(xs);  // [nw][16 x 16], then the second tile
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave * 256 + (4 * fg + i) * 16 + fr] = acc[i];
  if constexpr (DUAL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(nw + wave) * 256 + (4 * fg + i) * 16 + fr] = acc2[i];
  }
  __syncthreads();
  // output t = 16 m + n of the tile: token m, row n0 + n
  auto emit = [&](int t, float gam, float gam2, float sxe) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += red[w * 256 + t];
    const int64_t o = static_cast<int64_t>(t >> 4) * N + n0 + (t & 15);
    if constexpr (DUAL) {
      int tot2 = 0;
      for (int w = 0; w < nw; ++w) tot2 += red[(nw + w) * 256 + t];
      const float gv = static_cast<float>(tot) * (gam * sxe);
      const float uv = static_cast<float>(tot2) * (gam2 * sxe);
      const float h = fminf(fmaxf(gv / (1.f + expf(-gv)) * uv, -clampv), clampv);
      if (ydt == TQ_F32)
        static_cast<float*>(Y)[o] = h;
      else
        static_cast<uint16_t*>(Y)[o] = f32_to_bf16(h);
      return;
    }
    if (ydt == TQ_I32) {
      static_cast<int*>(Y)[o] = tot;
    } else {
      const float y = static_cast<float>(tot) * (gam * sxe);
      if (ydt == TQ_F32)
        static_cast<float*>(Y)[o] = y;
      else
        static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
    }
  };
  if (eout) emit(tid, egam, egam2, esx);
  // fewer than 256 threads (one to three waves, K < 1024): the rest of the
  // tile, its operands loaded here
  for (int t = tid + nt; t < kMfmaRows * kMfmaRows; t += nt) {
    const int m = t >> 4, n = t & 15;
    if (m >= M || n0 + n >= N) continue;
    float gam = 0.f, gam2 = 0.f, sxe = 0.f;
    if (ydt != TQ_I32) {
      gam = scale[per_row ? n0 + n : 0];
      if (DUAL) gam2 = scale2[per_row ? n0 + n : 0];
      sxe = SRC == 0 ? sx_io[m] : tok_sx[m];
    }
    emit(t, gam, gam2, sxe);
  }
}

constexpr int64_t kMfmaLdsMax = 120 * 1024;

int64_t mfma_lds_bytes(int64_t M, int64_t K, bool dual = false) {
  const int64_t stage = M * (K + 16);
  const int64_t red = static_cast<int64_t>(kMfmaMaxWaves) * 256 * 4 * (dual ? 2 : 1);
  return stage > red ? stage : red;
}

bool mfma_path_ok(int64_t M, int64_t K, const void* packed, const void* act) {
  return M >= 2 && M <= 16 && (K % 256) == 0 && K <= 16384 &&
         mfma_lds_bytes(M, K) <= kMfmaLdsMax &&
         (reinterpret_cast<uintptr_t>(packed) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(act) & 15u) == 0u;
}

template <int SRC, int KBW, int BITS, bool DUAL, int S>
hipError_t gemv_mfma_launch_k(const void* src, const ActParams* p, int8_t* q_out, float* sx,
                              const GemmArgs& a, const DualArgs& d, int waves, hipStream_t s) {
  const size_t lds = static_cast<size_t>(mfma_lds_bytes(a.M, a.K, DUAL));
  // allow the kernel more than 64 KiB of dynamic LDS, once per device
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_mfma<SRC, KBW, BITS, DUAL, S>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kMfmaLdsMax));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  const int64_t grid = (a.N + kMfmaRows - 1) / kMfmaRows;
  const float eps = p ? p->eps : 0.f, lo = p ? p->eta_min : 0.f, hi = p ? p->eta_max : 0.f;
  const int clamp = p ? p->clamp : 0;
  hipLaunchKernelGGL((k_gemv_mfma<SRC, KBW, BITS, DUAL, S>), dim3(grid), dim3(waves * kWave), lds, s,
                     src, eps, clamp, lo, hi, q_out, sx, static_cast<int>(a.M), a.packed,
                     a.scale, a.per_row, a.N, static_cast<int>(a.K), a.Y, a.ydt, d.packed2,
                     d.scale2, d.clampv);
  return hipGetLastError();
}

template <int SRC, int BITS = 2, bool DUAL = false>
hipError_t gemv_mfma_launch(const void* src, const ActParams* p, int8_t* q_out, float* sx,
                            const GemmArgs& a, hipStream_t s, const DualArgs& d = DualArgs()) {
  const int64_t nkb = a.K / 256;
  const int waves = static_cast<int>(nkb < kMfmaMaxWaves ? nkb : kMfmaMaxWaves);
  const int64_t per = (nkb + waves - 1) / waves;  // blocks per wave
  auto by_kbw = [&](auto slots) {
    constexpr int S = decltype(slots)::value;
    if (per <= 1) return gemv_mfma_launch_k<SRC, 1, BITS, DUAL, S>(src, p, q_out, sx, a, d, waves, s);
    if (per <= 2) return gemv_mfma_launch_k<SRC, 2, BITS, DUAL, S>(src, p, q_out, sx, a, d, waves, s);
    return gemv_mfma_launch_k<SRC, 4, BITS, DUAL, S>(src, p, q_out, sx, a, d, waves, s);
  };
  if constexpr (SRC == 0 && BITS == 2) {
    // token units per thread, loaded together
    const int64_t nsl = (a.M * (a.K / 16) + waves * kWave - 1) / (waves * kWave);
    if (nsl > 8) return hipErrorInvalidValue;  // kMfmaLdsMax keeps M K / 16 <= 7680
    if (nsl <= 1) return by_kbw(std::integral_constant<int, 1>{});
    if (nsl <= 2) return by_kbw(std::integral_constant<int, 2>{});
    if (nsl <= 4) return by_kbw(std::integral_constant<int, 4>{});
    return by_kbw(std::integral_constant<int, 8>{});
  } else {
    return by_kbw(std::integral_constant<int, 1>{});
  }
}

// ------------------------------------------------------------------------
// 1-bit sign-packed binary weights, any K % 8 == 0, 1 <= M <= 16, any
// alignment: one wave per output row, lanes stride over the row's packed
// bytes and read the tokens from global memory.  The shapes the two fast
// kernels do not take.
__global__ __launch_bounds__(256) void k_gemv1_generic(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int M,
    const uint8_t* __restrict__ packed, const float* __restrict__ scale, int per_row,
    int64_t N, int64_t K, void* __restrict__ Y, int ydt) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (n >= N) return;  // no barriers in this kernel
  const int64_t nb = K / 8;
  const uint8_t* row = packed + n * nb;
  int acc[kGemvMaxM];
#pragma unroll
  for (int m = 0; m < kGemvMaxM; ++m) acc[m] = 0;
  for (int64_t j = lane; j < nb; j += kWave) {
    const uint32_t byte = row[j];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bool plus = (byte >> t) & 1u;
#pragma unroll
      for (int m = 0; m < kGemvMaxM; ++m) {
        if (m < M) {
          const int x = q[m * K + 8 * j + t];
          acc[m] += plus ? x : -x;
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kGemvMaxM; ++m)
    if (m < M) acc[m] = wave_isum_last(acc[m]);
  if (lane != kWave - 1) return;
  const float gam = ydt == TQ_I32 ? 0.f : scale[per_row ? n : 0];
  for (int m = 0; m < M; ++m) {
    const int64_t o = static_cast<int64_t>(m) * N + n;
    if (ydt == TQ_I32) {
      static_cast<int*>(Y)[o] = acc[m];
    } else {
      const float y = static_cast<float>(acc[m]) * (gam * sx[m]);
      if (ydt == TQ_F32)
        static_cast<float*>(Y)[o] = y;
      else
        static_cast<uint16_t*>(Y)[o] = f32_to_bf16(y);
    }
  }
}

// ------------------------------------------------------------------------
// SwiGLU pair, any K % 4 == 0, 1 <= M <= 16, any alignment: one wave per
// output row contracts the gate and up rows (natural decode, tokens from
// global memory) and writes h = clamp(silu(g) * u, -clampv, clampv).  The
// shapes the two fast kernels do not take.
__global__ __launch_bounds__(256) void k_gemv_swiglu_generic(
    const int8_t* __restrict__ q, const float* __restrict__ sx, int M,
    const uint8_t* __restrict__ pg, const float* __restrict__ sg,
    const uint8_t* __restrict__ pu, const float* __restrict__ su, int per_row, int64_t N,
    int64_t K, void* __restrict__ H, int hdt, float clampv) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (n >= N) return;  // no barriers in this kernel
  const int64_t nb = K / 4;
  const uint8_t* rg = pg + n * nb;
  const uint8_t* ru = pu + n * nb;
  int ag[kGemvMaxM], au[kGemvMaxM];
#pragma unroll
  for (int m = 0; m < kGemvMaxM; ++m) ag[m] = au[m] = 0;
  for (int64_t j = lane; j < nb; j += kWave) {
    const uint32_t bg = rg[j], bu = ru[j];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int cg = static_cast<int>((bg >> (2 * t)) & 3u) - 1;
      const int cu = static_cast<int>((bu >> (2 * t)) & 3u) - 1;
#pragma unroll
      for (int m = 0; m < kGemvMaxM; ++m) {
        if (m < M) {
          const int x = q[m * K + 4 * j + t];
          ag[m] += cg * x;
          au[m] += cu * x;
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kGemvMaxM; ++m) {
    if (m < M) {
      ag[m] = wave_isum_last(ag[m]);
      au[m] = wave_isum_last(au[m]);
    }
  }
  if (lane != kWave - 1) return;
  const float gg = sg[per_row ? n : 0], gu = su[per_row ? n : 0];
  for (int m = 0; m < M; ++m) {
    const float gv = static_cast<float>(ag[m]) * (gg * sx[m]);
    const float uv = static_cast<float>(au[m]) * (gu * sx[m]);
    const float h = fminf(fmaxf(gv / (1.f + expf(-gv)) * uv, -clampv), clampv);
    const int64_t o = static_cast<int64_t>(m) * N + n;
    if (hdt == TQ_F32)
      static_cast<float*>(H)[o] = h;
    else
      static_cast<uint16_t*>(H)[o] = f32_to_bf16(h);
  }
}

// One token, 1-bit weights: 64-code lane chunks, K <= 16384.
bool dot1_path_ok(int64_t M, int64_t K, const void* packed, const void* act) {
  return M == 1 && (K % 64) == 0 && K <= 16384 &&
         (reinterpret_cast<uintptr_t>(packed) & 15u) == 0u &&
         (reinterpret_cast<uintptr_t>(act) & 15u) == 0u;
}

}  // namespace

// Compute units of the current device (0 if the query fails), cached per
// device.
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0 &&
      hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t s) {
  if (dot_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_dot_launch<0>(a.q, nullptr, nullptr, const_cast<float*>(a.sx), a, s);
  if (mfma_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_mfma_launch<0>(a.q, nullptr, nullptr, const_cast<float*>(a.sx), a, s);
  if (lds_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_lds_launch<0>(a.q, static_cast<int>(a.M), nullptr, nullptr,
                              const_cast<float*>(a.sx), a, s);
  const bool aligned = (a.K % 64) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.packed) & 15u) == 0u &&
                       (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0u;
  return aligned ? gemv_dispatch<true>(a, s) : gemv_dispatch<false>(a, s);
}

// Fusing the quantiser costs every workgroup the whole token work (M*K
// values); past four tokens or 16384 values that is more than a separate
// quantiser launch (measured at the FFN and 4096 x 4096 shapes).
constexpr int64_t kFusedMfmaMaxM = 4;
constexpr int64_t kFusedMfmaMaxMK = 16384;

bool fused_mfma_ok(int64_t M, int64_t K, const void* packed, const void* X) {
  return M <= kFusedMfmaMaxM && M * K <= kFusedMfmaMaxMK && mfma_path_ok(M, K, packed, X);
}

bool fused_quant_gemv_ok(int64_t M, int64_t K, const void* packed, const void* X) {
  // the LDS-tiled fused kernel only where no matrix-core GEMV takes the shape
  return dot_path_ok(M, K, packed, X) || fused_mfma_ok(M, K, packed, X) ||
         (!mfma_path_ok(M, K, packed, X) && lds_path_ok(M, K, packed, X));
}

hipError_t launch_quant_gemv(const void* X, int bf16, const ActParams& p, int8_t* q,
                             float* sx, const GemmArgs& a, hipStream_t s) {
  const int M = static_cast<int>(a.M);
  if (dot_path_ok(a.M, a.K, a.packed, X))
    return bf16 ? gemv_dot_launch<2>(X, &p, q, sx, a, s) : gemv_dot_launch<1>(X, &p, q, sx, a, s);
  if (fused_mfma_ok(a.M, a.K, a.packed, X))
    return bf16 ? gemv_mfma_launch<2>(X, &p, q, sx, a, s) : gemv_mfma_launch<1>(X, &p, q, sx, a, s);
  return bf16 ? gemv_lds_launch<2>(X, M, &p, q, sx, a, s)
              : gemv_lds_launch<1>(X, M, &p, q, sx, a, s);
}

hipError_t launch_gemv1(const GemmArgs& a, hipStream_t s) {
  if (dot1_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_dot_launch<0, 1>(a.q, nullptr, nullptr, const_cast<float*>(a.sx), a, s);
  if (mfma_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_mfma_launch<0, 1>(a.q, nullptr, nullptr, const_cast<float*>(a.sx), a, s);
  const int64_t grid = (a.N + 3) / 4;
  hipLaunchKernelGGL(k_gemv1_generic, dim3(grid), dim3(256), 0, s, a.q, a.sx,
                     static_cast<int>(a.M), a.packed, a.scale, a.per_row, a.N, a.K, a.Y, a.ydt);
  return hipGetLastError();
}

bool fused_quant_swiglu_ok(int64_t M, int64_t K, const void* pg, const void* pu, const void* X) {
  const bool up_ok = (reinterpret_cast<uintptr_t>(pu) & 15u) == 0u;
  return up_ok && (dot_path_ok(M, K, pg, X) || fused_mfma_ok(M, K, pg, X));
}

hipError_t launch_quant_swiglu_gemv(const void* X, int bf16, const ActParams& p, int8_t* q,
                                    float* sx, const GemmArgs& a, const uint8_t* packed_up,
                                    const float* scale_up, float clampv, hipStream_t s) {
  DualArgs d;
  d.packed2 = packed_up;
  d.scale2 = scale_up;
  d.clampv = clampv;
  if (dot_path_ok(a.M, a.K, a.packed, X))
    return bf16 ? gemv_dot_launch<2, 2, true>(X, &p, q, sx, a, s, d)
                : gemv_dot_launch<1, 2, true>(X, &p, q, sx, a, s, d);
  return bf16 ? gemv_mfma_launch<2, 2, true>(X, &p, q, sx, a, s, d)
              : gemv_mfma_launch<1, 2, true>(X, &p, q, sx, a, s, d);
}

hipError_t launch_swiglu_gemv(const GemmArgs& a, const uint8_t* packed_up, const float* scale_up,
                              float clampv, hipStream_t s) {
  DualArgs d;
  d.packed2 = packed_up;
  d.scale2 = scale_up;
  d.clampv = clampv;
  const bool up_ok = (reinterpret_cast<uintptr_t>(packed_up) & 15u) == 0u;
  float* sxm = const_cast<float*>(a.sx);
  if (up_ok && dot_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_dot_launch<0, 2, true>(a.q, nullptr, nullptr, sxm, a, s, d);
  if (up_ok && mfma_path_ok(a.M, a.K, a.packed, a.q))
    return gemv_mfma_launch<0, 2, true>(a.q, nullptr, nullptr, sxm, a, s, d);
  const int64_t grid = (a.N + 3) / 4;
  hipLaunchKernelGGL(k_gemv_swiglu_generic, dim3(grid), dim3(256), 0, s, a.q, a.sx,
                     static_cast<int>(a.M), a.packed, a.scale, packed_up, scale_up, a.per_row,
                     a.N, a.K, a.Y, a.ydt, clampv);
  return hipGetLastError();
}

}  // namespace tq
