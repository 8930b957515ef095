// Per-token int8 activation quantisation, the fused BitLinear prologue
// (RMSNorm -> blockwise FWHT-512 -> int8) and the standalone FWHT-512.
//
// Hetman-2b, src/quantization.py:
//   section 2, SymmetricActivationQuantizer: eta = max|x| per token (floored
//     at eps, optionally clamped to [eta_min, eta_max]), scale = 127/eta,
//     q = clamp(round(x*scale), -127, 127), all in fp32, round half to even;
//   section 1, fast_walsh_hadamard_transform_512: nine butterfly stages with
//     half-widths 1, 2, ..., 256, (a, b) -> (a + b, a - b) in fp32, then the
//     factor 1/sqrt(512); blockwise over consecutive 512-wide blocks;
//   section 4, SubLayerRMSNorm: x * rsqrt(mean(x^2) + eps) * weight;
//   section 5, BitLinear.forward: RMSNorm, then FWHT, then the quantiser
//     with (1e-6, 0.05, 40).
// BitRASP core_math.py, fake_quant_int, is the same per-token absmax scheme.
//
// The fused prologue uses the cancellation of positive per-token factors in
// absmax quantisation: the normalised, rotated token is r*c*z with
// z = FWHT_unnormalised(g*x), so while neither the eps floor nor the gain
// clamp moves eta_true = r*c*max|z| the codes are those of z itself and only
// the dequantisation scale carries r*c.  Codes then depend on no
// order-sensitive reduction.

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kNT = 256;
constexpr int kWavesPerBlock = kNT / kWave;
constexpr float kFwhtNorm = 0x1.6a09e6p-5f;  // fp32 nearest 1/sqrt(512) = 0x3D3504F3

// ------------------------------------------------------------- element I/O

template <typename T>
__device__ inline float to_f32(T v);
template <>
__device__ inline float to_f32<float>(float v) { return v; }
template <>
__device__ inline float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

// eight consecutive elements starting at p (16-byte aligned when VEC)
template <typename T, bool VEC>
__device__ inline void load8(const T* p, int64_t valid, float (&v)[8]) {
  if (VEC && valid >= 8) {
    if constexpr (sizeof(T) == 4) {
      const float4 a = reinterpret_cast<const float4*>(p)[0];
      const float4 b = reinterpret_cast<const float4*>(p)[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 a = reinterpret_cast<const uint4*>(p)[0];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < valid ? to_f32<T>(p[i]) : 0.f;
  }
}

template <bool VEC>
__device__ inline void store8_q(int8_t* p, int64_t valid, const uint32_t (&b)[8]) {
  if (VEC && valid >= 8) {
    uint2 o;
    o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    *reinterpret_cast<uint2*>(p) = o;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < valid) p[i] = static_cast<int8_t>(static_cast<uint8_t>(b[i]));
  }
}

// ------------------------------------------------------------- plain path

template <typename T, bool VEC>
__global__ __launch_bounds__(kNT) void k_quant_plain(const T* __restrict__ X, int64_t K,
                                                     float eps, int clamp, float lo,
                                                     float hi, int8_t* __restrict__ q,
                                                     float* __restrict__ sx) {
  __shared__ float sh[kWavesPerBlock];
  const int64_t row = blockIdx.x;
  const T* x = X + row * K;
  int8_t* qo = q + row * K;
  const int64_t nchunk = (K + 7) / 8;
  float amax = 0.f;
  for (int64_t c = threadIdx.x; c < nchunk; c += kNT) {
    float v[8];
    load8<T, VEC>(x + 8 * c, K - 8 * c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max<kNT>(amax, sh);
  float eta = fmaxf(amax, eps);
  if (clamp) eta = fminf(fmaxf(eta, lo), hi);
  const float s = 127.f / eta;
  for (int64_t c = threadIdx.x; c < nchunk; c += kNT) {
    float v[8];
    load8<T, VEC>(x + 8 * c, K - 8 * c, v);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = quant_byte(v[i], s);
    store8_q<VEC>(qo + 8 * c, K - 8 * c, b);
  }
  if (threadIdx.x == 0) sx[row] = eta / 127.f;
}

// A token's values read once: NT threads per token, each holding CH chunks
// of 8 values in registers; wave maxima (DPP) meet in LDS.  Same eta, scale
// and codes as k_quant_plain (the max is exact).  Few tokens take 1024
// threads per token (more waves in flight per token), many tokens 256.
constexpr int kNTs = 1024;

template <typename T, bool VEC, int CH, int NT = kNTs>
__global__ __launch_bounds__(NT) void k_quant_small(const T* __restrict__ X, int64_t K,
                                                    float eps, int clamp, float lo, float hi,
                                                    int8_t* __restrict__ q,
                                                    float* __restrict__ sx) {
  constexpr int kNTs = NT;
  __shared__ float part[kNTs / kWave];
  const int64_t row = blockIdx.x;
  const T* x = X + row * K;
  int8_t* qo = q + row * K;
  const int64_t nchunk = (K + 7) / 8;
  const int tid = threadIdx.x;
  float v[CH][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = tid + static_cast<int64_t>(kNTs) * i;
    if (c < nchunk) {
      load8<T, VEC>(x + 8 * c, K - 8 * c, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    }
  }
  amax = wave_max_last(amax);
  if ((tid & (kWave - 1)) == kWave - 1) part[tid / kWave] = amax;
  __syncthreads();
  amax = 0.f;
#pragma unroll
  for (int w = 0; w < kNTs / kWave; ++w) amax = fmaxf(amax, part[w]);
  float eta = fmaxf(amax, eps);
  if (clamp) eta = fminf(fmaxf(eta, lo), hi);
  const float s = 127.f / eta;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = tid + static_cast<int64_t>(kNTs) * i;
    if (c < nchunk) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = quant_byte(v[i][e], s);
      store8_q<VEC>(qo + 8 * c, K - 8 * c, b);
    }
  }
  if (tid == 0) sx[row] = eta / 127.f;
}

// ---------------------------------------------------------------- FWHT-512

// v from lane l ^ LM: DPP row operations for LM = 1, 2 (quad swaps), 4 (half
// mirror, then quad reversal) and 8 (row mirror, then half mirror);
// v_permlane16_swap / v_permlane32_swap of v with itself for 16 / 32 (the
// first result holds, in the upper lane of each pair, the lower one's value,
// the second result the reverse).  The moves leave the values untouched.
template <int LM>
__device__ inline float lane_xor(float v) {
  const int i = __float_as_int(v);
  if constexpr (LM == 1) {
    return __int_as_float(dpp_get<0xB1>(i));
  } else if constexpr (LM == 2) {
    return __int_as_float(dpp_get<0x4E>(i));
  } else if constexpr (LM == 4) {
    return __int_as_float(dpp_get<0x1B>(dpp_get<0x141>(i)));
  } else if constexpr (LM == 8) {
    return __int_as_float(dpp_get<0x141>(dpp_get<0x140>(i)));
  } else {
    static_assert(LM == 16 || LM == 32, "lane distance");
    const unsigned u = static_cast<unsigned>(i);
    unsigned r0, r1;
    if constexpr (LM == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      r0 = r[0];
      r1 = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      r0 = r[0];
      r1 = r[1];
    }
    const bool upper = (threadIdx.x & LM) != 0;
    return __uint_as_float(upper ? r0 : r1);
  }
}

template <int LM>
__device__ inline void fwht_lane_stage(float (&v)[8], int lane) {
  const bool upper = (lane & LM) != 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float other = lane_xor<LM>(v[e]);
    v[e] = upper ? (other - v[e]) : (v[e] + other);
  }
}

// In-place FWHT of one 512-block held by a wave: lane l holds elements
// 8l .. 8l+7.  Stages h = 1, 2, 4 pair elements inside a lane; stages
// h = 8 .. 256 pair lane l with lane l ^ (h/8).  The lower index of a pair
// takes a + b and the upper a - b, a being the lower element.
__device__ inline void fwht512_wave(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  fwht_lane_stage<1>(v, lane);
  fwht_lane_stage<2>(v, lane);
  fwht_lane_stage<4>(v, lane);
  fwht_lane_stage<8>(v, lane);
  fwht_lane_stage<16>(v, lane);
  fwht_lane_stage<32>(v, lane);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kNT) void k_fwht512(const T* __restrict__ X, int64_t nseg,
                                                 int normalize, float* __restrict__ Y) {
  const int64_t seg = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                      threadIdx.x / kWave;
  if (seg >= nseg) return;  // whole wave leaves together
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t off = seg * 512 + 8 * lane;
  float v[8];
  load8<T, VEC>(X + off, 8, v);
  fwht512_wave(v);
  if (normalize) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * kFwhtNorm;
  }
  float* y = Y + off;
  if (VEC) {
    reinterpret_cast<float4*>(y)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(y)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = v[e];
  }
}

// ------------------------------------------------------------ prologue path

// One block per token.  Each wave holds NB 512-element segments in
// registers (segment wave + 4*j), lane l holding elements 8l .. 8l+7 of each.
template <typename T, int NB, bool VEC>
__global__ __launch_bounds__(kNT) void k_quant_prologue(
    const T* __restrict__ X, int64_t K, float eps, int clamp, float lo, float hi,
    int rmsnorm, float rms_eps, const float* __restrict__ gweight, int fwht,
    int8_t* __restrict__ q, float* __restrict__ sx) {
  __shared__ float sh[kWavesPerBlock];
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const T* x = X + row * K;
  const int64_t nseg = (K + 511) / 512;
  float v[NB][8];
  float ss = 0.f;
  // every segment's load goes out before the first one is used
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t seg = wave + kWavesPerBlock * j;
    const int64_t base = seg * 512 + 8 * lane;
    if (seg < nseg) {
      load8<T, VEC>(x + base, K - base, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t seg = wave + kWavesPerBlock * j;
    const int64_t base = seg * 512 + 8 * lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    if (gweight != nullptr && seg < nseg) {
      float g[8];
      load8<float, false>(gweight + base, K - base, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * g[e];
    }
    if (fwht) fwht512_wave(v[j]);
  }
  float r = 1.f;
  if (rmsnorm) {
    const float sum_sq = block_sum<kNT>(ss, sh);
    const float ms = sum_sq / static_cast<float>(K);
    const float t = ms + rms_eps;
    r = 1.f / sqrtf(t);
  }
  float zmax = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) zmax = fmaxf(zmax, fabsf(v[j][e]));
  // block max of |z| (non-negative: DPP wave maxima, lane 63 holds them)
  zmax = wave_max_last(zmax);
  if (lane == kWave - 1) sh[wave] = zmax;
  __syncthreads();
  zmax = sh[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) zmax = fmaxf(zmax, sh[w]);
  const float rc = r * (fwht ? kFwhtNorm : 1.f);
  const float eta_true = rc * zmax;
  float eta = fmaxf(eta_true, eps);
  if (clamp) eta = fminf(fmaxf(eta, lo), hi);
  float mult, sxv;
  if (eta == eta_true) {
    mult = zmax > 0.f ? 127.f / zmax : 0.f;
    sxv = eta_true / 127.f;
  } else {
    mult = rc * (127.f / eta);
    sxv = eta / 127.f;
  }
  int8_t* qo = q + row * K;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t seg = wave + kWavesPerBlock * j;
    if (seg >= nseg) continue;
    const int64_t base = seg * 512 + 8 * lane;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = quant_byte(v[j][e], mult);
    store8_q<VEC>(qo + base, K - base, b);
  }
  if (threadIdx.x == 0) sx[row] = sxv;
}

template <typename T, bool VEC>
hipError_t prologue_dispatch(const T* X, int64_t M, int64_t K, const ActParams& p,
                             int8_t* q, float* sx, hipStream_t s) {
  const int64_t per_wave = (K + 2047) / 2048;  // segments per wave
#define TQ_PROLOGUE(NBV)                                                            \
  hipLaunchKernelGGL((k_quant_prologue<T, NBV, VEC>), dim3(M), dim3(kNT), 0, s, X, K, \
                     p.eps, p.clamp, p.eta_min, p.eta_max, p.rmsnorm, p.rms_eps,    \
                     p.rms_weight, p.fwht, q, sx)
  if (per_wave <= 1) TQ_PROLOGUE(1);
  else if (per_wave <= 2) TQ_PROLOGUE(2);
  else if (per_wave <= 4) TQ_PROLOGUE(4);
  else if (per_wave <= 8) TQ_PROLOGUE(8);
  else TQ_PROLOGUE(16);
#undef TQ_PROLOGUE
  return hipGetLastError();
}

}  // namespace

template <typename T, bool VEC, int NT = kNTs>
hipError_t quant_small_launch(const T* x, int64_t M, int64_t K, const ActParams& p, int8_t* q,
                              float* sx, hipStream_t s) {
  const int64_t ch = ((K + 7) / 8 + NT - 1) / NT;  // chunks per thread
#define TQ_QSMALL(C)                                                                        \
  hipLaunchKernelGGL((k_quant_small<T, VEC, C, NT>), dim3(M), dim3(NT), 0, s, x, K, p.eps, \
                     p.clamp, p.eta_min, p.eta_max, q, sx)
  if (ch <= 1) TQ_QSMALL(1);
  else if (ch <= 2) TQ_QSMALL(2);
  else if (ch <= 4) TQ_QSMALL(4);
  else TQ_QSMALL(8);
#undef TQ_QSMALL
  return hipGetLastError();
}

// Tokens below which one workgroup per token leaves the GPU latency-bound:
// there, each token's values are read once (k_quant_small, K <= 32768).
constexpr int64_t kQuantSmallM = 64;
constexpr int64_t kQuantSmallMaxK = 4 * 8 * kNTs;

hipError_t launch_quant_plain(const void* X, int bf16, int64_t M, int64_t K,
                              const ActParams& p, int8_t* q, float* sx, hipStream_t s) {
  const bool vec = (K % 8) == 0 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0u &&
                   (reinterpret_cast<uintptr_t>(q) & 7u) == 0u;
  if (M < kQuantSmallM && K <= kQuantSmallMaxK) {
    if (bf16) {
      const uint16_t* x = static_cast<const uint16_t*>(X);
      return vec ? quant_small_launch<uint16_t, true>(x, M, K, p, q, sx, s)
                 : quant_small_launch<uint16_t, false>(x, M, K, p, q, sx, s);
    }
    const float* x = static_cast<const float*>(X);
    return vec ? quant_small_launch<float, true>(x, M, K, p, q, sx, s)
               : quant_small_launch<float, false>(x, M, K, p, q, sx, s);
  }
  // many tokens, K up to 8 chunks of 8 per thread of 256: the values stay in
  // registers between the max and the codes (k_quant_plain reads them twice)
  if (K <= 8 * 8 * kNT) {
    if (bf16) {
      const uint16_t* x = static_cast<const uint16_t*>(X);
      return vec ? quant_small_launch<uint16_t, true, kNT>(x, M, K, p, q, sx, s)
                 : quant_small_launch<uint16_t, false, kNT>(x, M, K, p, q, sx, s);
    }
    const float* x = static_cast<const float*>(X);
    return vec ? quant_small_launch<float, true, kNT>(x, M, K, p, q, sx, s)
               : quant_small_launch<float, false, kNT>(x, M, K, p, q, sx, s);
  }
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    if (vec)
      hipLaunchKernelGGL((k_quant_plain<uint16_t, true>), dim3(M), dim3(kNT), 0, s, x, K,
                         p.eps, p.clamp, p.eta_min, p.eta_max, q, sx);
    else
      hipLaunchKernelGGL((k_quant_plain<uint16_t, false>), dim3(M), dim3(kNT), 0, s, x, K,
                         p.eps, p.clamp, p.eta_min, p.eta_max, q, sx);
  } else {
    const float* x = static_cast<const float*>(X);
    if (vec)
      hipLaunchKernelGGL((k_quant_plain<float, true>), dim3(M), dim3(kNT), 0, s, x, K,
                         p.eps, p.clamp, p.eta_min, p.eta_max, q, sx);
    else
      hipLaunchKernelGGL((k_quant_plain<float, false>), dim3(M), dim3(kNT), 0, s, x, K,
                         p.eps, p.clamp, p.eta_min, p.eta_max, q, sx);
  }
  return hipGetLastError();
}

hipError_t launch_quant_prologue(const void* X, int bf16, int64_t M, int64_t K,
                                 const ActParams& p, int8_t* q, float* sx,
                                 hipStream_t s) {
  const bool vec = (K % 8) == 0 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0u &&
                   (reinterpret_cast<uintptr_t>(q) & 7u) == 0u;
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    return vec ? prologue_dispatch<uint16_t, true>(x, M, K, p, q, sx, s)
               : prologue_dispatch<uint16_t, false>(x, M, K, p, q, sx, s);
  }
  const float* x = static_cast<const float*>(X);
  return vec ? prologue_dispatch<float, true>(x, M, K, p, q, sx, s)
             : prologue_dispatch<float, false>(x, M, K, p, q, sx, s);
}

hipError_t launch_fwht512(const void* X, int bf16, int64_t M, int64_t K, int normalize,
                          float* Y, hipStream_t s) {
  const int64_t nseg = M * (K / 512);
  const int64_t grid = (nseg + kWavesPerBlock - 1) / kWavesPerBlock;
  const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0u &&
                   (reinterpret_cast<uintptr_t>(Y) & 15u) == 0u;
  if (bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    if (vec)
      hipLaunchKernelGGL((k_fwht512<uint16_t, true>), dim3(grid), dim3(kNT), 0, s, x, nseg,
                         normalize, Y);
    else
      hipLaunchKernelGGL((k_fwht512<uint16_t, false>), dim3(grid), dim3(kNT), 0, s, x,
                         nseg, normalize, Y);
  } else {
    const float* x = static_cast<const float*>(X);
    if (vec)
      hipLaunchKernelGGL((k_fwht512<float, true>), dim3(grid), dim3(kNT), 0, s, x, nseg,
                         normalize, Y);
    else
      hipLaunchKernelGGL((k_fwht512<float, false>), dim3(grid), dim3(kNT), 0, s, x, nseg,
                         normalize, Y);
  }
  return hipGetLastError();
}

}  // namespace tq
