// Device-side helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- reductions

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ inline int wave_isum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Wave reductions through DPP row operations (no LDS round trips): pair and
// quad swaps, half-row and row mirrors give every lane its 16-lane row's
// value; row_bcast:15 and row_bcast:31 then fold rows 0..2 into row 3.  Only
// lane 63 holds the wave's result.  Lanes a row_mask leaves out read the
// identity 0, so the max form is for non-negative, non-NaN floats.
template <int CTRL, int ROWS = 0xF>
__device__ inline int dpp_get(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}

__device__ inline int wave_isum_last(int v) {
  v += dpp_get<0xB1>(v);        // quad_perm 1,0,3,2
  v += dpp_get<0x4E>(v);        // quad_perm 2,3,0,1
  v += dpp_get<0x141>(v);       // row_half_mirror
  v += dpp_get<0x140>(v);       // row_mirror
  v += dpp_get<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_get<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Non-negative, non-NaN floats order as their bit patterns, so their wave
// max is an unsigned integer max.
__device__ inline float wave_max_last(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, static_cast<uint32_t>(dpp_get<0xB1>(static_cast<int>(u))));
  u = max(u, static_cast<uint32_t>(dpp_get<0x4E>(static_cast<int>(u))));
  u = max(u, static_cast<uint32_t>(dpp_get<0x141>(static_cast<int>(u))));
  u = max(u, static_cast<uint32_t>(dpp_get<0x140>(static_cast<int>(u))));
  u = max(u, static_cast<uint32_t>(dpp_get<0x142, 0xA>(static_cast<int>(u))));
  u = max(u, static_cast<uint32_t>(dpp_get<0x143, 0xC>(static_cast<int>(u))));
  return __uint_as_float(u);
}

// Block-wide sum / max for blockDim.x == NT (multiple of 64).  `scratch`
// holds NT/64 entries.  Every thread gets the result.  The partials of the
// waves are combined in wave order, so the result does not depend on timing.
template <int NT>
__device__ inline double block_sum(double v, double* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

template <int NT>
__device__ inline float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

template <int NT>
__device__ inline float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float t = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) t = fmaxf(t, scratch[i]);
  __syncthreads();
  return t;
}

// ------------------------------------------------------------------ numbers

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even: the chip's own conversion
// (v_cvt_pk_bf16_f32; NaN stays NaN, subnormals are rounded, not flushed).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two values in one conversion: lo in bits 0..15, hi in bits 16..31
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// round half to even, clamp to [-127, 127], as a byte
// The code rint(x * s) clamped to [-127, 127], as int8 in the low byte of
// the result (the upper bytes are not zero).  Clamping first and adding
// 1.5 * 2^23 gives that code: for |t| < 2^22 the fp32 sum rounds to the
// nearest integer, ties to even, as rint does, and holds it in two's
// complement in its low bits (the clamp also sends NaN to -127 either way).
__device__ inline uint32_t quant_bits(float x, float s) {
  const float t = fminf(fmaxf(x * s, -127.f), 127.f);
  return __float_as_uint(t + 12582912.f);
}

// the low bytes of b0..b3 as one word, b0 in byte 0
__device__ inline uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// four codes, the first in byte 0
__device__ inline uint32_t quant_word(float a, float b, float c, float d, float s) {
  return pack_low_bytes(quant_bits(a, s), quant_bits(b, s), quant_bits(c, s), quant_bits(d, s));
}

// quant_bits without the clamp, for s = 127 / eta with eta >= |x|: then
// |x * s| <= 127 * (1 + 2^-24) before its rounding, so the product rounds to
// at most 127 + 2^-17 and the code to at most 127 in magnitude.
__device__ inline uint32_t quant_bits_unclamped(float x, float s) {
  const float t = x * s;
  return __float_as_uint(t + 12582912.f);
}

__device__ inline uint32_t quant_word_unclamped(float a, float b, float c, float d, float s) {
  return pack_low_bytes(quant_bits_unclamped(a, s), quant_bits_unclamped(b, s),
                        quant_bits_unclamped(c, s), quant_bits_unclamped(d, s));
}

// --------------------------------------------------------- 2-bit decoding

// 4x4 byte transpose: out[s] holds byte s of d0, d1, d2, d3 (in that order).
// Applied to 16 consecutive int8 values (d_b = values 4b..4b+3) it gives
// out[s] byte b = value 4b + s, the order decode_codes_strided produces.
__device__ inline v4i transpose_bytes4x4(uint32_t d0, uint32_t d1, uint32_t d2,
                                         uint32_t d3) {
  const uint32_t a_lo = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
  const uint32_t a_hi = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
  const uint32_t b_lo = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
  v4i out;
  out.x = static_cast<int>(__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u));
  out.y = static_cast<int>(__builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u));
  out.z = static_cast<int>(__builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u));
  out.w = static_cast<int>(__builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u));
  return out;
}

// One packed 32-bit word holds 16 codes, code i in bits 2i..2i+1 (-1 = 0,
// 0 = 1, +1 = 2).  Returns the 16 codes (values 0..2) as bytes in natural
// order: byte j of out[t] is code 4t + j.  (w >> 2s) & 0x03030303 holds codes
// s, 4+s, 8+s, 12+s; a 4x4 byte transpose puts them in order.
__device__ inline v4i decode_codes_natural(uint32_t w) {
  return transpose_bytes4x4(w & 0x03030303u, (w >> 2) & 0x03030303u,
                            (w >> 4) & 0x03030303u, (w >> 6) & 0x03030303u);
}

// The 16 codes of a packed word, values 0..2, in strided order: byte b of
// out[s] is code 4b + s.  Seven integer operations; the matching activation
// operand is the byte transpose above.
__device__ inline v4i decode_codes_strided(uint32_t w) {
  v4i out;
  out.x = static_cast<int>(w & 0x03030303u);
  out.y = static_cast<int>((w >> 2) & 0x03030303u);
  out.z = static_cast<int>((w >> 4) & 0x03030303u);
  out.w = static_cast<int>((w >> 6) & 0x03030303u);
  return out;
}

// The 16 codes of a packed word in strided order as above, but without
// shifting codes 4b + 1 and 4b + 2 down: out.y holds 4 * code, out.z
// 16 * code (both still positive bytes), so a product with them is scaled by
// 4 or 16 and is accumulated apart.  Five integer operations.
__device__ inline v4i decode_codes_scaled(uint32_t w) {
  v4i out;
  out.x = static_cast<int>(w & 0x03030303u);
  out.y = static_cast<int>(w & 0x0C0C0C0Cu);
  out.z = static_cast<int>(w & 0x30303030u);
  out.w = static_cast<int>((w >> 6) & 0x03030303u);
  return out;
}

// Codes 0..2 in each byte -> signed values -1..+1 (0x7F + c never carries
// out of its byte; flipping the top bit then gives c - 1 in two's complement).
__device__ inline uint32_t codes_to_signed(uint32_t c) {
  return (c + 0x7F7F7F7Fu) ^ 0x80808080u;
}

__device__ inline v4i decode_signed_natural(uint32_t w) {
  v4i c = decode_codes_natural(w);
  v4i s;
  s.x = static_cast<int>(codes_to_signed(static_cast<uint32_t>(c.x)));
  s.y = static_cast<int>(codes_to_signed(static_cast<uint32_t>(c.y)));
  s.z = static_cast<int>(codes_to_signed(static_cast<uint32_t>(c.z)));
  s.w = static_cast<int>(codes_to_signed(static_cast<uint32_t>(c.w)));
  return s;
}

// sum of the four signed bytes of v, added to acc
__device__ inline int byte_sum(uint32_t v, int acc) {
  return __builtin_amdgcn_sdot4(static_cast<int>(v), 0x01010101, acc, false);
}

}  // namespace tq
