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
// The fused prologue runs the three steps in that order on fp32 values held
// in registers: RMSNorm (var = mean of the fp32 squares, r = 1/sqrt(var +
// eps) as a correctly rounded square root and division, x * r * g), the
// FWHT and its factor, then the quantiser.  var is the fp32 nearest to the
// exact mean of the squares: an fp64 sum decides it unless it lies within
// its error bound of an fp32 rounding midpoint, and then the squares are
// summed exactly in integer exponent bins.  Every later step is a fixed
// sequence of correctly rounded fp32 operations, so codes and scales do not
// depend on the reduction order.

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

// b[i]: code i in the low byte (quant_bits)
template <bool VEC>
__device__ inline void store8_q(int8_t* p, int64_t valid, const uint32_t (&b)[8]) {
  if (VEC && valid >= 8) {
    uint2 o;
    o.x = pack_low_bytes(b[0], b[1], b[2], b[3]);
    o.y = pack_low_bytes(b[4], b[5], b[6], b[7]);
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
    for (int i = 0; i < 8; ++i) b[i] = quant_bits(v[i], s);
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
      for (int e = 0; e < 8; ++e) b[e] = quant_bits(v[i][e], s);
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
// a row permutation that has a source lane for every lane (the mirrors):
// no old value to keep, so no move to initialise one
template <int CTRL>
__device__ inline int dpp_all(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

template <int LM>
__device__ inline float lane_xor(float v) {
  const int i = __float_as_int(v);
  if constexpr (LM == 1) {
    return __int_as_float(dpp_get<0xB1>(i));
  } else if constexpr (LM == 2) {
    return __int_as_float(dpp_get<0x4E>(i));
  } else if constexpr (LM == 4) {
    return __int_as_float(dpp_get<0x1B>(dpp_all<0x141>(i)));
  } else if constexpr (LM == 8) {
    return __int_as_float(dpp_get<0x141>(dpp_all<0x140>(i)));
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

// Cross-lane butterflies with the sign carried: a lane takes own + k * other
// with k = +1 in the lower lane of a pair and -1 in the upper one, one fused
// multiply-add of an exact product, so one rounding, that of the sum or
// difference.  The upper lane's result is the negated butterfly difference
// (round to nearest even is symmetric); partners of a stage differ only in
// that stage's lane bit, so they always carry the same sign, and after the
// six stages lane l holds its values times (-1)^popcount(l).  For lane
// distances 1 and 2 the lane move is the fma's own DPP source operand
// (v_fmac_f32 with DPP, written out: the compiler does not fold a move into
// it), for 4 and 8 a DPP move and then the fma with the second DPP step;
// each block starts with the two wait states a DPP read of a VGPR written by
// the instruction before it needs.  16 and 32 move through permlane swaps.
#define TQ_FMAC_DPP8(CTRL)                                                              \
  asm volatile("s_nop 1\n\t"                                                            \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"      \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),     \
                 "+v"(v[6]), "+v"(v[7])                                                   \
               : "v"(k))
#define TQ_MOV_FMAC_DPP8(CTRL1, CTRL2)                                                   \
  do {                                                                                  \
    float t0, t1, t2, t3, t4, t5, t6, t7;                                               \
    asm volatile("s_nop 1\n\t"                                                          \
                 "v_mov_b32_dpp %0, %8 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %1, %9 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %2, %10 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %3, %11 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %4, %12 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %5, %13 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %6, %14 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_mov_b32_dpp %7, %15 " CTRL1 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "s_nop 1\n\t"                                                          \
                 "v_fmac_f32_dpp %8, %0, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %9, %1, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %10, %2, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %11, %3, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %12, %4, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %13, %5, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %14, %6, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                 "v_fmac_f32_dpp %15, %7, %16 " CTRL2 " row_mask:0xf bank_mask:0xf bound_ctrl:1" \
                 : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5),        \
                   "=&v"(t6), "=&v"(t7), "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]),    \
                   "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])                           \
                 : "v"(k));                                                             \
  } while (0)

// The plain form for the standalone transform, whose fp32 output keeps the
// butterflies' signed zeros: the lower lane of a pair takes other + v, the
// upper other - v (other + (+-1 * v): the product is exact, so the one
// rounding is that of the sum; the lane move folds into the add).  The
// carried-sign form below can turn a zero difference into -0.0, which only
// the prologue, whose codes and maximum do not see the sign of zero, takes.
template <int LM>
__device__ inline void fwht_lane_stage_plain(float (&v)[8], int lane) {
  const float sgn = (lane & LM) != 0 ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = lane_xor<LM>(v[e]) + sgn * v[e];
}

template <int LM>
__device__ inline void fwht_lane_stage(float (&v)[8], int lane) {
  const float k = (lane & LM) != 0 ? -1.f : 1.f;
  if constexpr (LM == 1) {
    TQ_FMAC_DPP8("quad_perm:[1,0,3,2]");
  } else if constexpr (LM == 2) {
    TQ_FMAC_DPP8("quad_perm:[2,3,0,1]");
  } else if constexpr (LM == 4) {  // half-row mirror, then quad reversal: lane ^ 4
    TQ_MOV_FMAC_DPP8("row_half_mirror", "quad_perm:[3,2,1,0]");
  } else if constexpr (LM == 8) {  // row mirror, then half-row mirror: lane ^ 8
    TQ_MOV_FMAC_DPP8("row_mirror", "row_half_mirror");
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(lane_xor<LM>(v[e]), k, v[e]);
  }
}
#undef TQ_FMAC_DPP8
#undef TQ_MOV_FMAC_DPP8

// In-place FWHT of one 512-block held by a wave: lane l holds elements
// 8l .. 8l+7.  Stages h = 1, 2, 4 pair elements inside a lane; stages
// h = 8 .. 256 pair lane l with lane l ^ (h/8).  The lower index of a pair
// takes a + b and the upper a - b, a being the lower element.  Returns the
// lane's sign s (+-1): v then holds s times the transform.
__device__ inline void fwht8_in_lane(float (&v)[8]) {
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
}

__device__ inline float fwht512_wave(float (&v)[8]) {
  fwht8_in_lane(v);
  const int lane = threadIdx.x & (kWave - 1);
  fwht_lane_stage<1>(v, lane);
  fwht_lane_stage<2>(v, lane);
  fwht_lane_stage<4>(v, lane);
  fwht_lane_stage<8>(v, lane);
  fwht_lane_stage<16>(v, lane);
  fwht_lane_stage<32>(v, lane);
  return (__builtin_popcount(lane) & 1) ? -1.f : 1.f;
}

// the same transform in the plain form, signed zeros as the butterflies give
__device__ inline void fwht512_wave_plain(float (&v)[8]) {
  fwht8_in_lane(v);
  const int lane = threadIdx.x & (kWave - 1);
  fwht_lane_stage_plain<1>(v, lane);
  fwht_lane_stage_plain<2>(v, lane);
  fwht_lane_stage_plain<4>(v, lane);
  fwht_lane_stage_plain<8>(v, lane);
  fwht_lane_stage_plain<16>(v, lane);
  fwht_lane_stage_plain<32>(v, lane);
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
  fwht512_wave_plain(v);
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

// Relative error bound of the fp64 mean of squares: each fp32 square is exact
// in fp64 and passes through at most NB * 8 sequential additions in a
// thread, six in the wave tree and sixteen across waves, then one division
// by K: under 160 roundings of 2^-53 each, far below 2^-40.
constexpr double kVarThr = 0x1p-40;

// fp32 nearest (ties to even) to (sum_b bins[b] * 2^(b-1)) / n quanta of
// 2^-149, over the whole fp32 range (subnormals included).  One thread, on
// LDS words `T` (kVarLimbs of scratch).  bins[b] < 2^40 (a token of at most
// 2^16 squares of 24-bit significands) shifted by at most 253 bits fit 11
// limbs of 32 bits.
constexpr int kVarLimbs = 11;
__device__ float exact_mean_squares(const unsigned long long* bins, uint32_t n, uint32_t* T) {
  for (int i = 0; i < kVarLimbs; ++i) T[i] = 0u;
  for (int b = 1; b < 255; ++b) {
    const unsigned long long v = bins[b];
    if (v == 0ull) continue;
    const int sh = b - 1, li = sh >> 5, bo = sh & 31;
    const unsigned long long lo = v << bo;
    const unsigned long long hi = bo ? (v >> (64 - bo)) : 0ull;
    const uint32_t add[3] = {static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                             static_cast<uint32_t>(hi)};
    unsigned long long carry = 0ull;
    for (int j = 0; li + j < kVarLimbs; ++j) {
      if (j >= 3 && carry == 0ull) break;
      const unsigned long long t =
          static_cast<unsigned long long>(T[li + j]) + (j < 3 ? add[j] : 0u) + carry;
      T[li + j] = static_cast<uint32_t>(t);
      carry = t >> 32;
    }
  }
  // long division by n, limb by limb from the top: T becomes the quotient
  unsigned long long rem = 0ull;
  for (int i = kVarLimbs - 1; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | T[i];
    T[i] = static_cast<uint32_t>(cur / n);
    rem = cur % n;
  }
  int lead = -1;
  for (int i = kVarLimbs - 1; i >= 0 && lead < 0; --i)
    if (T[i]) lead = i * 32 + 31 - __clz(static_cast<int>(T[i]));
  const bool half = 2ull * rem == n, above = 2ull * rem > n;
  if (lead < 24) {
    // below 2^-125 the fp32 spacing is one quantum: round the quotient
    uint32_t u = T[0];
    if (above || (half && (u & 1u))) ++u;
    return __uint_as_float(u);  // u <= 2^24 is that value's bit pattern
  }
  const int shift = lead - 23;
  auto bit = [&](int p) { return (T[p >> 5] >> (p & 31)) & 1u; };
  uint32_t mant = 0u;
  for (int p = lead; p >= shift; --p) mant = (mant << 1) | bit(p);
  const uint32_t guard = bit(shift - 1);
  bool sticky = rem != 0ull;
  for (int p = shift - 2; p >= 0 && !sticky; --p) sticky = bit(p) != 0u;
  int e = shift;
  if (guard && (sticky || (mant & 1u))) ++mant;
  if (mant == (1u << 24)) {
    mant >>= 1;
    ++e;
  }
  // mant * 2^(e - 149) with mant in [2^23, 2^24): biased exponent e + 1
  return __uint_as_float((static_cast<uint32_t>(e + 1) << 23) | (mant & 0x7FFFFFu));
}

// fp32 rounding of an fp64 mean of squares whose relative error is at most
// kVarThr; true when it lies too close to an fp32 rounding midpoint to
// decide (then *v is not final).
__device__ inline bool var_from_fp64(double mean, float* v) {
  const float f = __double2float_rn(mean);
  *v = f;
  if (mean == 0.0) return false;  // every square is zero
  const uint32_t fb = __float_as_uint(f);
  const double fd = static_cast<double>(f);
  const double up = static_cast<double>(__uint_as_float(fb + 1u));
  double dist = fabs(0.5 * (fd + up) - mean);
  if (fb != 0u) dist = fmin(dist, fabs(mean - 0.5 * (fd + static_cast<double>(__uint_as_float(fb - 1u)))));
  return dist <= kVarThr * mean;
}

__device__ inline void square_bin_add(unsigned long long* bins, float sq) {
  const uint32_t u = __float_as_uint(sq);
  const uint32_t e = u >> 23;
  const uint32_t m = (u & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  atomicAdd(&bins[e ? e : 1u], static_cast<unsigned long long>(m));
}

// fp64 wave sum in the six DPP levels of wave_isum_last, each double moved
// as its two words; lane 63 holds the sum.
template <int CTRL, int ROWS = 0xF>
__device__ inline double dpp_get_f64(double v) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(dpp_get<CTRL, ROWS>(static_cast<int>(u)));
  const uint32_t hi = static_cast<uint32_t>(dpp_get<CTRL, ROWS>(static_cast<int>(u >> 32)));
  return __longlong_as_double(
      static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ inline double wave_sum_last(double v) {
  v += dpp_get_f64<0xB1>(v);
  v += dpp_get_f64<0x4E>(v);
  v += dpp_get_f64<0x141>(v);
  v += dpp_get_f64<0x140>(v);
  v += dpp_get_f64<0x142, 0xA>(v);
  v += dpp_get_f64<0x143, 0xC>(v);
  return v;
}

// One block of NW waves per token.  Each wave holds NB 512-element segments
// in registers (segment wave + NW * j), lane l holding elements 8l .. 8l+7
// of each; the token is read once.
template <typename T, int NW, int NB, bool VEC>
__global__ __launch_bounds__(NW * kWave) void k_quant_prologue(
    const T* __restrict__ X, int64_t K, float eps, int clamp, float lo, float hi,
    int rmsnorm, float rms_eps, const float* __restrict__ gweight, int fwht,
    int8_t* __restrict__ q, float* __restrict__ sx) {
  __shared__ double part[NW];
  __shared__ float pmax[NW];
  __shared__ unsigned long long bins[256];
  __shared__ uint32_t limbs[kVarLimbs];
  __shared__ float var_sh;
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const T* x = X + row * K;
  const int64_t nseg = (K + 511) / 512;
  float v[NB][8], g[NB][8];
  // every segment's load goes out before the first one is used, the RMSNorm
  // weight's too (it does not depend on the token)
  const bool gw = rmsnorm && gweight != nullptr;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t seg = wave + NW * j;
    const int64_t base = seg * 512 + 8 * lane;
    if (seg < nseg) {
      load8<T, VEC>(x + base, K - base, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    }
  }
  if (gw) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t seg = wave + NW * j;
      const int64_t base = seg * 512 + 8 * lane;
      if (seg < nseg) load8<float, false>(gweight + base, K - base, g[j]);
    }
  }
  if (rmsnorm) {
    // var: the fp32 nearest to the exact mean of the fp32 squares
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += static_cast<double>(v[j][e] * v[j][e]);
    acc = wave_sum_last(acc);
    if (lane == kWave - 1) part[wave] = acc;
    __syncthreads();
    double S = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) S += part[w];
    // S / K; for K a power of two S scaled by 2^-log2(K), the same
    // correctly rounded value without the division's instruction sequence
    const double mean = (K & (K - 1)) == 0 ? ldexp(S, -__builtin_ctzll(static_cast<unsigned long long>(K)))
                                           : S / static_cast<double>(K);
    float var;
    if (var_from_fp64(mean, &var)) {  // uniform over the block
      for (int b = threadIdx.x; b < 256; b += NW * kWave) bins[b] = 0ull;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) square_bin_add(bins, v[j][e] * v[j][e]);
      __syncthreads();
      if (threadIdx.x == 0) var_sh = exact_mean_squares(bins, static_cast<uint32_t>(K), limbs);
      __syncthreads();
      var = var_sh;
    }
    // sqrtf and / are the correctly rounded operations under the build's
    // -fhip-fp32-correctly-rounded-divide-sqrt (__fsqrt_rn is the hardware
    // approximation on this toolchain unless rounded OCML operations are on)
    const float r = 1.f / sqrtf(var + rms_eps);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * r;
      if (gw && wave + NW * j < nseg) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * g[j][e];
      }
    }
  }
  if (fwht) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float f = fwht512_wave(v[j]) * kFwhtNorm;  // +-kFwhtNorm, exact
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * f;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
  // block max of |x| (non-negative: DPP wave maxima, lane 63 holds them)
  amax = wave_max_last(amax);
  if (lane == kWave - 1) pmax[wave] = amax;
  __syncthreads();
  amax = pmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) amax = fmaxf(amax, pmax[w]);
  float eta = fmaxf(amax, eps);
  if (clamp) eta = fminf(fmaxf(eta, lo), hi);
  const float s = 127.f / eta;
  int8_t* qo = q + row * K;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t seg = wave + NW * j;
    if (seg >= nseg) continue;
    const int64_t base = seg * 512 + 8 * lane;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = quant_bits(v[j][e], s);
    store8_q<VEC>(qo + base, K - base, b);
  }
  if (threadIdx.x == 0) sx[row] = eta / 127.f;
}

template <typename T, bool VEC>
hipError_t prologue_dispatch(const T* X, int64_t M, int64_t K, const ActParams& p,
                             int8_t* q, float* sx, hipStream_t s) {
  const int64_t nseg = (K + 511) / 512;
#define TQ_PROLOGUE(NWV, NBV)                                                             \
  hipLaunchKernelGGL((k_quant_prologue<T, NWV, NBV, VEC>), dim3(M), dim3(NWV * kWave), 0, \
                     s, X, K, p.eps, p.clamp, p.eta_min, p.eta_max, p.rmsnorm, p.rms_eps, \
                     p.rms_weight, p.fwht, q, sx)
  if (nseg <= 4) TQ_PROLOGUE(4, 1);
  else if (nseg <= 8) TQ_PROLOGUE(8, 1);
  else if (nseg <= 16) TQ_PROLOGUE(16, 1);
  else if (nseg <= 32) TQ_PROLOGUE(16, 2);
  else TQ_PROLOGUE(16, 4);
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
