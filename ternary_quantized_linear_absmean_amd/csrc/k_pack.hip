// Absmean scale, ternarization and 2-bit packing of a weight matrix.
//
// Foundry, docs/quantization.md, "Ternary Quantization (BitNet b1.58) / How
// It Works": gamma = mean|w|, q = round(w/gamma) clamped to {-1, 0, +1},
// four codes per byte; "Ternary Format / Encoding": -1 = 0b00, 0 = 0b01,
// +1 = 0b10, LSB-first.  Hetman-2b, src/quantization.py, section 2: the mean
// is floored at 1e-6 and the rounding is round-half-to-even.
//
// gamma is the fp32 value nearest to the exact mean of |w| (ties to even),
// then floored.  The sum is carried in fp64; when the fp64 mean lies within
// its error bound of an fp32 rounding boundary the group is summed again
// exactly: each |w| is M * 2^(b-150) with b = max(biased exponent, 1) and M
// the 24-bit significand, the M are added per b in 64-bit integers, and the
// total is divided by the element count in multi-word integer arithmetic.
//
// Ternarization uses a comparison instead of the quotient: for normal fp32
// w and gamma, rint(fp32(w/gamma)) is +1 exactly when w > gamma/2 (the next
// fp32 above gamma/2 exceeds it by more than gamma * 2^-25, half the fp32
// spacing just above 0.5), and -1 exactly when w < -gamma/2.  The same
// kernels take other thresholds h = fp32(f * gamma) (Foundry "Absmean
// Thresholding": f = 1; BitRASP ternarize_weight: f = 0.55) or a manual h
// (Foundry fq_quantize_ternary_threshold, whose scale is h itself).
//
// The end of the file converts packed codes between this library's format
// and Hetman-2b's Formats 0 and 1 (src/quantization.py, section 3).

#include "tq_device.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kNT = 256;
constexpr int kMaxPartials = 1024;
constexpr size_t kWsPartials = 0;                                  // double[1024]
constexpr size_t kWsFlag = kMaxPartials * sizeof(double);          // uint32
constexpr size_t kWsBins = kWsFlag + 256;                          // uint64[256]
constexpr size_t kWsTotal = kWsBins + 256 * sizeof(unsigned long long);

constexpr float kGammaEps = 1e-6f;

// --------------------------------------------------------------- exact mean

// value of the fp32 nearest (ties to even) to (sum_b bins[b] * 2^(b-150)) / n,
// or 0 when that value is below 2^-20 (callers floor at 1e-6 anyway).
__device__ float exact_mean_from_bins(const unsigned long long* bins,
                                      unsigned long long n) {
  constexpr int kLimbs = 11;  // 352 bits: bins < 2^64 shifted by at most 253
  uint32_t T[kLimbs];
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) T[i] = 0u;
  for (int b = 1; b < 255; ++b) {
    const unsigned long long v = bins[b];
    if (v == 0ull) continue;
    const int s = b - 1;
    const int li = s >> 5, bo = s & 31;
    const unsigned long long lo = v << bo;
    const unsigned long long hi = bo ? (v >> (64 - bo)) : 0ull;
    const uint32_t add[3] = {static_cast<uint32_t>(lo),
                             static_cast<uint32_t>(lo >> 32),
                             static_cast<uint32_t>(hi)};
    unsigned long long carry = 0ull;
    for (int j = 0; li + j < kLimbs; ++j) {
      if (j >= 3 && carry == 0ull) break;
      const unsigned long long t = static_cast<unsigned long long>(T[li + j]) +
                                   (j < 3 ? add[j] : 0u) + carry;
      T[li + j] = static_cast<uint32_t>(t);
      carry = t >> 32;
    }
  }
  int top = -1;
  for (int i = kLimbs - 1; i >= 0; --i) {
    if (T[i]) {
      top = i * 32 + 31 - __clz(static_cast<int>(T[i]));
      break;
    }
  }
  if (top < 0) return 0.f;
  // restoring division, one quotient bit per step, from T's top bit down and
  // on into fraction bits; stop after the leading bit + 23 + a guard bit
  unsigned long long rem = 0ull, mant = 0ull;
  int count = 0, lead = 0, pos = top;
  bool started = false;
  for (;; --pos) {
    const unsigned bit = pos >= 0 ? (T[pos >> 5] >> (pos & 31)) & 1u : 0u;
    rem = (rem << 1) | bit;
    const unsigned qb = rem >= n ? 1u : 0u;
    if (qb) rem -= n;
    if (!started && qb) {
      started = true;
      lead = pos;
    }
    if (started) {
      mant = (mant << 1) | qb;
      if (++count == 25) break;
    }
  }
  bool sticky = rem != 0ull;
  for (int p = pos - 1; p >= 0 && !sticky; --p)
    if ((T[p >> 5] >> (p & 31)) & 1u) sticky = true;
  uint32_t m24 = static_cast<uint32_t>(mant >> 1);
  const uint32_t guard = static_cast<uint32_t>(mant & 1ull);
  if (guard && (sticky || (m24 & 1u))) ++m24;
  if (m24 == (1u << 24)) {
    m24 >>= 1;
    ++lead;
  }
  // the quotient's leading bit is 2^lead quanta of 2^-149
  const int biased = lead - 149 + 127;
  if (biased < 107) return 0.f;  // below 2^-20
  return __uint_as_float((static_cast<uint32_t>(biased) << 23) | (m24 & 0x7FFFFFu));
}

// gamma from an fp64 sum S of |w| over n elements whose relative error is at
// most thr.  Returns true when S/n is too close to an fp32 rounding boundary
// to decide, in which case *g is not final.
__device__ inline bool gamma_from_fp64(double S, double n, double thr, float* g) {
  const double mean = S / n;
  if (mean < 0.5 * static_cast<double>(kGammaEps)) {
    *g = kGammaEps;
    return false;
  }
  const float f = __double2float_rn(mean);
  const uint32_t fb = __float_as_uint(f);
  const double fd = static_cast<double>(f);
  const double up = static_cast<double>(__uint_as_float(fb + 1u)) - fd;
  const double dn = fd - static_cast<double>(__uint_as_float(fb - 1u));
  const double dist = fmin((fd + 0.5 * up) - mean, mean - (fd - 0.5 * dn));
  *g = fmaxf(f, kGammaEps);
  return dist <= thr * mean;
}

__device__ inline void bin_add(unsigned long long* lb, float w) {
  const uint32_t u = __float_as_uint(w) & 0x7FFFFFFFu;
  const uint32_t e = u >> 23;
  const uint32_t m = (u & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  const uint32_t b = e ? e : 1u;
  atomicAdd(&lb[b], static_cast<unsigned long long>(m));
}

__device__ inline uint32_t code_of(float w, float h, int binary) {
  if (binary) return w >= 0.f ? 2u : 0u;
  return w > h ? 2u : (w < -h ? 0u : 1u);
}

__device__ inline uint32_t byte_of(float4 v, float h, int binary) {
  return code_of(v.x, h, binary) | (code_of(v.y, h, binary) << 2) |
         (code_of(v.z, h, binary) << 4) | (code_of(v.w, h, binary) << 6);
}

template <bool VEC>
__device__ inline float4 load4(const float* p, int64_t i4) {
  if (VEC) return reinterpret_cast<const float4*>(p)[i4];
  return make_float4(p[4 * i4], p[4 * i4 + 1], p[4 * i4 + 2], p[4 * i4 + 3]);
}

// ------------------------------------------------------------ per tensor

template <bool VEC>
__global__ __launch_bounds__(kNT) void k_abssum_partial(const float* __restrict__ W,
                                                        int64_t n4,
                                                        double* __restrict__ partials) {
  __shared__ double sh[kNT / kWave];
  double acc = 0.0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x; i < n4;
       i += stride) {
    const float4 v = load4<VEC>(W, i);
    acc += fabs(static_cast<double>(v.x));
    acc += fabs(static_cast<double>(v.y));
    acc += fabs(static_cast<double>(v.z));
    acc += fabs(static_cast<double>(v.w));
  }
  const double s = block_sum<kNT>(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kNT) void k_gamma_finalize(
    const double* __restrict__ partials, int P, int64_t n, double thr,
    uint32_t* __restrict__ flag, unsigned long long* __restrict__ bins,
    float* __restrict__ scale) {
  __shared__ double sh[kNT / kWave];
  __shared__ int near_sh;
  double v = 0.0;
  for (int i = threadIdx.x; i < P; i += kNT) v += partials[i];
  const double S = block_sum<kNT>(v, sh);
  if (threadIdx.x == 0) {
    float g;
    const bool near = gamma_from_fp64(S, static_cast<double>(n), thr, &g);
    near_sh = near ? 1 : 0;
    *flag = near ? 1u : 0u;
    if (!near) scale[0] = g;
  }
  __syncthreads();
  if (near_sh) bins[threadIdx.x] = 0ull;
}

template <bool VEC>
__global__ __launch_bounds__(kNT) void k_gamma_bins(const float* __restrict__ W,
                                                    int64_t n4,
                                                    const uint32_t* __restrict__ flag,
                                                    unsigned long long* __restrict__ bins) {
  if (*flag == 0u) return;
  __shared__ unsigned long long lb[256];
  lb[threadIdx.x] = 0ull;
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x; i < n4;
       i += stride) {
    const float4 v = load4<VEC>(W, i);
    bin_add(lb, v.x);
    bin_add(lb, v.y);
    bin_add(lb, v.z);
    bin_add(lb, v.w);
  }
  __syncthreads();
  if (lb[threadIdx.x]) atomicAdd(&bins[threadIdx.x], lb[threadIdx.x]);
}

__global__ void k_gamma_exact_final(const uint32_t* __restrict__ flag,
                                    const unsigned long long* __restrict__ bins,
                                    int64_t n, float* __restrict__ scale) {
  if (*flag == 0u || threadIdx.x != 0) return;
  scale[0] = fmaxf(exact_mean_from_bins(bins, static_cast<unsigned long long>(n)),
                   kGammaEps);
}

// One packed byte (four weights) per lane and step; VEC: W 16-byte aligned.
template <bool VEC>
__global__ __launch_bounds__(kNT) void k_ternarize_pack(const float* __restrict__ W,
                                                        int64_t nbytes, int binary, float hf,
                                                        const float* __restrict__ scale,
                                                        uint8_t* __restrict__ packed) {
  const float h = scale[0] * hf;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x;
  int64_t j = tid;
  if (VEC) {
    // one byte (four weights, one 16-byte load) per lane and step: a wave's
    // load reads 1 KiB of consecutive weights; four loads in flight.  The
    // bytes are taken from the end of W backwards: the sum pass just read W
    // from the front, so its last lines are the likeliest still in the
    // memory-side cache (measured 2-3% faster than front to back)
    for (; j + 3 * stride < nbytes; j += 4 * stride) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = load4<true>(W, nbytes - 1 - (j + u * stride));
#pragma unroll
      for (int u = 0; u < 4; ++u)
        packed[nbytes - 1 - (j + u * stride)] = static_cast<uint8_t>(byte_of(v[u], h, binary));
    }
  }
  for (; j < nbytes; j += stride)
    packed[nbytes - 1 - j] = static_cast<uint8_t>(byte_of(load4<VEC>(W, nbytes - 1 - j), h, binary));
}

// 1-bit sign packing of binary weights: bit t of byte j is 1 when weight
// 8j + t is >= 0 (+1), LSB-first; 32 weights -> one 32-bit word per step.
__device__ inline uint32_t sign_bits4(float4 v) {
  return (v.x >= 0.f ? 1u : 0u) | (v.y >= 0.f ? 2u : 0u) | (v.z >= 0.f ? 4u : 0u) |
         (v.w >= 0.f ? 8u : 0u);
}

template <bool VEC>
__global__ __launch_bounds__(kNT) void k_sign_pack(const float* __restrict__ W, int64_t nbytes,
                                                   uint8_t* __restrict__ packed) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x;
  int64_t done = 0;
  if (VEC) {
    const int64_t nwords = nbytes / 4;
    for (int64_t i = tid; i < nwords; i += stride) {
      uint32_t word = 0u;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= sign_bits4(load4<true>(W, 8 * i + n)) << (4 * n);
      reinterpret_cast<uint32_t*>(packed)[i] = word;
    }
    done = nwords * 4;
  }
  for (int64_t j = done + tid; j < nbytes; j += stride)
    packed[j] = static_cast<uint8_t>(sign_bits4(load4<false>(W, 2 * j)) |
                                     (sign_bits4(load4<false>(W, 2 * j + 1)) << 4));
}

// --------------------------------------------------------------- per row

// BITS 2: ternary or binary codes, four per byte; BITS 1: signs, eight per
// byte (binary weights only).  R > 0 (BITS 2, K <= 4 R kNT): each thread keeps
// its R four-weight groups of the row in registers, so the row is read from
// memory once for the sum, the exact mean and the codes.
template <bool VEC, int BITS, int R = 0>
__global__ __launch_bounds__(kNT) void k_pack_rows(const float* __restrict__ W,
                                                   int64_t K, int binary, float hf, double thr,
                                                   uint8_t* __restrict__ packed,
                                                   float* __restrict__ scale) {
  __shared__ double sh[kNT / kWave];
  __shared__ float g_sh;
  __shared__ int near_sh;
  __shared__ unsigned long long lb[256];
  const int64_t row = blockIdx.x;
  const float* w = W + row * K;
  uint8_t* out = packed + row * (K * BITS / 8);
  const int64_t nb = K / 4;
  double acc = 0.0;
  float4 rv[R > 0 ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t j = threadIdx.x + int64_t{kNT} * r;
      rv[r] = j < nb ? load4<VEC>(w, j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {  // the same order as the loop below
      if (threadIdx.x + int64_t{kNT} * r >= nb) break;
      acc += fabs(static_cast<double>(rv[r].x));
      acc += fabs(static_cast<double>(rv[r].y));
      acc += fabs(static_cast<double>(rv[r].z));
      acc += fabs(static_cast<double>(rv[r].w));
    }
  } else {
    for (int64_t j = threadIdx.x; j < nb; j += kNT) {
      const float4 v = load4<VEC>(w, j);
      acc += fabs(static_cast<double>(v.x));
      acc += fabs(static_cast<double>(v.y));
      acc += fabs(static_cast<double>(v.z));
      acc += fabs(static_cast<double>(v.w));
    }
  }
  const double S = block_sum<kNT>(acc, sh);
  if (threadIdx.x == 0) {
    float g;
    near_sh = gamma_from_fp64(S, static_cast<double>(K), thr, &g) ? 1 : 0;
    g_sh = g;
  }
  __syncthreads();
  if (near_sh) {  // block-uniform
    lb[threadIdx.x] = 0ull;
    __syncthreads();
    if constexpr (R > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (threadIdx.x + int64_t{kNT} * r >= nb) break;
        bin_add(lb, rv[r].x);
        bin_add(lb, rv[r].y);
        bin_add(lb, rv[r].z);
        bin_add(lb, rv[r].w);
      }
    } else {
      for (int64_t j = threadIdx.x; j < nb; j += kNT) {
        const float4 v = load4<VEC>(w, j);
        bin_add(lb, v.x);
        bin_add(lb, v.y);
        bin_add(lb, v.z);
        bin_add(lb, v.w);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0)
      g_sh = fmaxf(exact_mean_from_bins(lb, static_cast<unsigned long long>(K)),
                   kGammaEps);
    __syncthreads();
  }
  const float g = g_sh;
  if (threadIdx.x == 0) scale[row] = g;
  const float h = g * hf;
  if constexpr (BITS == 2 && R > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t j = threadIdx.x + int64_t{kNT} * r;
      if (j < nb) out[j] = static_cast<uint8_t>(byte_of(rv[r], h, binary));
    }
  } else if constexpr (BITS == 2) {
    for (int64_t j = threadIdx.x; j < nb; j += kNT)
      out[j] = static_cast<uint8_t>(byte_of(load4<VEC>(w, j), h, binary));
  } else {
    for (int64_t j = threadIdx.x; j < K / 8; j += kNT)
      out[j] = static_cast<uint8_t>(sign_bits4(load4<VEC>(w, 2 * j)) |
                                    (sign_bits4(load4<VEC>(w, 2 * j + 1)) << 4));
  }
}

__global__ void k_set_scale(float* __restrict__ scale, float v) {
  if (threadIdx.x == 0) scale[0] = v;
}

// ------------------------------------------------------------ code formats

// Per 2-bit field of a word (bits at even positions): +1 and -1 masks of
// this library's codes (fmt 0: -1 = 00, 0 = 01, +1 = 10), Format 0 (fmt 1:
// +1 = 01, -1 = 11) and Format 1 (fmt 2: +1 = 01, -1 = 10); the reserved
// code of each format is a zero.
__device__ inline void code_masks(uint32_t w, int fmt, uint32_t& plus, uint32_t& minus) {
  const uint32_t lo = w & 0x55555555u, hi = (w >> 1) & 0x55555555u;
  if (fmt == 0) {
    plus = hi & ~lo;
    minus = ~hi & ~lo & 0x55555555u;
  } else if (fmt == 1) {
    plus = lo & ~hi;
    minus = lo & hi;
  } else {
    plus = lo & ~hi;
    minus = hi & ~lo;
  }
}

__device__ inline uint32_t encode_masks(uint32_t plus, uint32_t minus, int fmt) {
  if (fmt == 0) return (plus << 1) | (~plus & ~minus & 0x55555555u);
  if (fmt == 1) return plus | minus | (minus << 1);
  return plus | (minus << 1);
}

__device__ inline uint32_t convert_word(uint32_t w, int sf, int df) {
  uint32_t p, m;
  code_masks(w, sf, p, m);
  return encode_masks(p, m, df);
}

// VEC: 16 bytes per step (both pointers 16-byte aligned), then single bytes.
template <bool VEC>
__global__ __launch_bounds__(kNT) void k_convert_codes(const uint8_t* src, int sf, uint8_t* dst,
                                                       int df, int64_t nbytes) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x;
  int64_t done = 0;
  if (VEC) {
    const int64_t n16 = nbytes / 16;
    for (int64_t i = tid; i < n16; i += stride) {
      uint4 v = reinterpret_cast<const uint4*>(src)[i];
      v.x = convert_word(v.x, sf, df);
      v.y = convert_word(v.y, sf, df);
      v.z = convert_word(v.z, sf, df);
      v.w = convert_word(v.w, sf, df);
      reinterpret_cast<uint4*>(dst)[i] = v;
    }
    done = n16 * 16;
  }
  for (int64_t j = done + tid; j < nbytes; j += stride)
    dst[j] = static_cast<uint8_t>(convert_word(src[j], sf, df));
}

// one packed byte (its masks in the low 8 bits) -> four int8 values
__device__ inline uint32_t values_of_byte(uint32_t p, uint32_t m) {
  const uint32_t ps = (p & 1u) | ((p & 4u) << 6) | ((p & 16u) << 12) | ((p & 64u) << 18);
  const uint32_t ms = (m & 1u) | ((m & 4u) << 6) | ((m & 16u) << 12) | ((m & 64u) << 18);
  return ps | (ms * 0xFFu);  // bytes 0, 1 or 0xFF (-1)
}

// VEC: a 32-bit word (16 values) per step, 16-byte stores (packed 4-byte and
// out 16-byte aligned); then single bytes, the last one partial.
template <bool VEC>
__global__ __launch_bounds__(kNT) void k_unpack_codes(const uint8_t* __restrict__ packed, int fmt,
                                                      int64_t numel, int8_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNT;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kNT + threadIdx.x;
  int64_t done = 0;
  if (VEC) {
    const int64_t nw = numel / 16;
    for (int64_t i = tid; i < nw; i += stride) {
      uint32_t p, m;
      code_masks(reinterpret_cast<const uint32_t*>(packed)[i], fmt, p, m);
      uint4 o;
      o.x = values_of_byte(p, m);
      o.y = values_of_byte(p >> 8, m >> 8);
      o.z = values_of_byte(p >> 16, m >> 16);
      o.w = values_of_byte(p >> 24, m >> 24);
      reinterpret_cast<uint4*>(out)[i] = o;
    }
    done = nw * 4;  // bytes
  }
  const int64_t nb = (numel + 3) / 4;
  for (int64_t j = done + tid; j < nb; j += stride) {
    uint32_t p, m;
    code_masks(packed[j], fmt, p, m);
    const uint32_t v = values_of_byte(p, m);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (4 * j + t < numel) out[4 * j + t] = static_cast<int8_t>((v >> (8 * t)) & 0xFFu);
  }
}

int64_t elementwise_grid(int64_t work) {
  int64_t g = (work + kNT - 1) / kNT;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  return g;
}

// Relative error bound of an fp64 sum of non-negative terms whose longest
// chain of additions has `depth` steps, including the final division,
// doubled for margin.
double sum_error_bound(int64_t depth) {
  return 2.0 * static_cast<double>(depth + 2) * 0x1p-53;
}

}  // namespace

size_t pack_tensor_ws_bytes() { return kWsTotal; }

hipError_t launch_pack_tensor(const float* W, int64_t numel, tq_wmode mode,
                              uint8_t* packed, float* scale, void* ws,
                              hipStream_t s, int bits, float hf) {
  const int binary = mode == TQ_BINARY_SIGN ? 1 : 0;
  char* base = static_cast<char*>(ws);
  double* partials = reinterpret_cast<double*>(base + kWsPartials);
  uint32_t* flag = reinterpret_cast<uint32_t*>(base + kWsFlag);
  unsigned long long* bins = reinterpret_cast<unsigned long long*>(base + kWsBins);
  const int64_t n4 = numel / 4;
  int64_t P = (n4 + kNT * 4 - 1) / (kNT * 4);
  if (P < 1) P = 1;
  if (P > kMaxPartials) P = kMaxPartials;
  const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0u;
  // longest addition chain: per-thread loop (4 adds per float4), wave (6) and
  // block (4) reductions, then the same in the finalising block
  const int64_t per_thread = (n4 + P * kNT - 1) / (P * kNT);
  const int64_t depth = 4 * per_thread + 10 + (P + kNT - 1) / kNT + 10;
  const double thr = sum_error_bound(depth);
  if (vec)
    hipLaunchKernelGGL(k_abssum_partial<true>, dim3(P), dim3(kNT), 0, s, W, n4, partials);
  else
    hipLaunchKernelGGL(k_abssum_partial<false>, dim3(P), dim3(kNT), 0, s, W, n4, partials);
  hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(kNT), 0, s, partials,
                     static_cast<int>(P), numel, thr, flag, bins, scale);
  if (vec)
    hipLaunchKernelGGL(k_gamma_bins<true>, dim3(P), dim3(kNT), 0, s, W, n4, flag, bins);
  else
    hipLaunchKernelGGL(k_gamma_bins<false>, dim3(P), dim3(kNT), 0, s, W, n4, flag, bins);
  hipLaunchKernelGGL(k_gamma_exact_final, dim3(1), dim3(kWave), 0, s, flag, bins,
                     numel, scale);
  if (bits == 1) {
    const int64_t nb1 = numel / 8;
    const bool vec1 = vec && (reinterpret_cast<uintptr_t>(packed) & 3u) == 0u;
    int64_t grid1 = ((vec1 ? nb1 / 4 : nb1) + kNT - 1) / kNT;
    if (grid1 < 1) grid1 = 1;
    if (grid1 > 8192) grid1 = 8192;
    if (vec1)
      hipLaunchKernelGGL(k_sign_pack<true>, dim3(grid1), dim3(kNT), 0, s, W, nb1, packed);
    else
      hipLaunchKernelGGL(k_sign_pack<false>, dim3(grid1), dim3(kNT), 0, s, W, nb1, packed);
    return hipGetLastError();
  }
  const int64_t nbytes = numel / 4;
  const bool vec_pack = vec && (reinterpret_cast<uintptr_t>(packed) & 3u) == 0u;
  int64_t work = vec_pack ? nbytes / 4 : nbytes;
  int64_t grid = (work + kNT - 1) / kNT;
  if (grid < 1) grid = 1;
  if (grid > 8192) grid = 8192;
  if (vec_pack)
    hipLaunchKernelGGL(k_ternarize_pack<true>, dim3(grid), dim3(kNT), 0, s, W, nbytes,
                       binary, hf, scale, packed);
  else
    hipLaunchKernelGGL(k_ternarize_pack<false>, dim3(grid), dim3(kNT), 0, s, W, nbytes,
                       binary, hf, scale, packed);
  return hipGetLastError();
}

hipError_t launch_pack_manual(const float* W, int64_t numel, float t, uint8_t* packed,
                              float* scale, hipStream_t s) {
  hipLaunchKernelGGL(k_set_scale, dim3(1), dim3(kWave), 0, s, scale, t);
  const int64_t nbytes = numel / 4;
  const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0u &&
                   (reinterpret_cast<uintptr_t>(packed) & 3u) == 0u;
  const int64_t grid = elementwise_grid(vec ? nbytes / 4 : nbytes);
  if (vec)
    hipLaunchKernelGGL(k_ternarize_pack<true>, dim3(grid), dim3(kNT), 0, s, W, nbytes, 0, 1.0f,
                       scale, packed);
  else
    hipLaunchKernelGGL(k_ternarize_pack<false>, dim3(grid), dim3(kNT), 0, s, W, nbytes, 0, 1.0f,
                       scale, packed);
  return hipGetLastError();
}

hipError_t launch_convert_codes(const uint8_t* src, int sf, uint8_t* dst, int df, int64_t nbytes,
                                hipStream_t s) {
  const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) == 0u;
  const int64_t grid = elementwise_grid(vec ? nbytes / 16 : nbytes);
  if (vec)
    hipLaunchKernelGGL(k_convert_codes<true>, dim3(grid), dim3(kNT), 0, s, src, sf, dst, df, nbytes);
  else
    hipLaunchKernelGGL(k_convert_codes<false>, dim3(grid), dim3(kNT), 0, s, src, sf, dst, df, nbytes);
  return hipGetLastError();
}

hipError_t launch_unpack_codes(const uint8_t* packed, int fmt, int64_t numel, int8_t* out,
                               hipStream_t s) {
  const bool vec = (reinterpret_cast<uintptr_t>(packed) & 3u) == 0u &&
                   (reinterpret_cast<uintptr_t>(out) & 15u) == 0u;
  const int64_t grid = elementwise_grid(vec ? numel / 16 : (numel + 3) / 4);
  if (vec)
    hipLaunchKernelGGL(k_unpack_codes<true>, dim3(grid), dim3(kNT), 0, s, packed, fmt, numel, out);
  else
    hipLaunchKernelGGL(k_unpack_codes<false>, dim3(grid), dim3(kNT), 0, s, packed, fmt, numel, out);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const float* W, int64_t N, int64_t K, tq_wmode mode,
                            uint8_t* packed, float* scale, hipStream_t s, int bits, float hf) {
  const int binary = mode == TQ_BINARY_SIGN ? 1 : 0;
  const bool vec = (reinterpret_cast<uintptr_t>(W) & 15u) == 0u;
  const int64_t per_thread = (K / 4 + kNT - 1) / kNT;
  const double thr = sum_error_bound(4 * per_thread + 10);
#define TQ_PACK_ROWS(V, B)                                                                  \
  hipLaunchKernelGGL((k_pack_rows<V, B>), dim3(N), dim3(kNT), 0, s, W, K, binary, hf, thr, \
                     packed, scale)
  if (bits == 1) {
    if (vec) TQ_PACK_ROWS(true, 1);
    else TQ_PACK_ROWS(false, 1);
  } else if (per_thread <= 8) {  // the row fits in registers
#define TQ_PACK_ROWS_R(V, RV)                                                                   \
  hipLaunchKernelGGL((k_pack_rows<V, 2, RV>), dim3(N), dim3(kNT), 0, s, W, K, binary, hf, thr, \
                     packed, scale)
    if (per_thread <= 1) { if (vec) TQ_PACK_ROWS_R(true, 1); else TQ_PACK_ROWS_R(false, 1); }
    else if (per_thread <= 2) { if (vec) TQ_PACK_ROWS_R(true, 2); else TQ_PACK_ROWS_R(false, 2); }
    else if (per_thread <= 4) { if (vec) TQ_PACK_ROWS_R(true, 4); else TQ_PACK_ROWS_R(false, 4); }
    else { if (vec) TQ_PACK_ROWS_R(true, 8); else TQ_PACK_ROWS_R(false, 8); }
#undef TQ_PACK_ROWS_R
  } else {
    if (vec) TQ_PACK_ROWS(true, 2);
    else TQ_PACK_ROWS(false, 2);
  }
#undef TQ_PACK_ROWS
  return hipGetLastError();
}

}  // namespace tq
