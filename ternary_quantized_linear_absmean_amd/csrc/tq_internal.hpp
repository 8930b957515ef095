// Internal launch interface between the C ABI (tq_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

// ---- absmean + ternarize + pack (k_pack.hip)
size_t pack_tensor_ws_bytes();
// bits: 2 (codes, four per byte) or 1 (signs of binary weights, eight per
// byte); hf: the ternarization threshold as a factor of gamma (0.5 is the
// rounding rule)
hipError_t launch_pack_tensor(const float* W, int64_t numel, tq_wmode mode,
                              uint8_t* packed, float* scale, void* ws,
                              hipStream_t s, int bits = 2, float hf = 0.5f);
hipError_t launch_pack_rows(const float* W, int64_t N, int64_t K, tq_wmode mode,
                            uint8_t* packed, float* scale, hipStream_t s, int bits = 2,
                            float hf = 0.5f);
// manual threshold t: codes by |w| > t, scale[0] = t
hipError_t launch_pack_manual(const float* W, int64_t numel, float t, uint8_t* packed,
                              float* scale, hipStream_t s);
// code formats: 0 this library's, 1 Format 0, 2 Format 1
hipError_t launch_convert_codes(const uint8_t* src, int sf, uint8_t* dst, int df, int64_t nbytes,
                                hipStream_t s);
hipError_t launch_unpack_codes(const uint8_t* packed, int fmt, int64_t numel, int8_t* out,
                               hipStream_t s);

// ---- activations (k_quant.hip)
struct ActParams {
  float eps;
  int clamp;
  float eta_min, eta_max;
  int rmsnorm;
  float rms_eps;
  const float* rms_weight;
  int fwht;
};
hipError_t launch_quant_plain(const void* X, int bf16, int64_t M, int64_t K,
                              const ActParams& p, int8_t* q, float* sx,
                              hipStream_t s);
hipError_t launch_quant_prologue(const void* X, int bf16, int64_t M, int64_t K,
                                 const ActParams& p, int8_t* q, float* sx,
                                 hipStream_t s);
hipError_t launch_fwht512(const void* X, int bf16, int64_t M, int64_t K,
                          int normalize, float* Y, hipStream_t s);
constexpr int64_t kPrologueMaxK = 32768;

// ---- contraction (k_gemv.hip, k_gemm.hip)
struct GemmArgs {
  const int8_t* q;
  const float* sx;
  const uint8_t* packed;
  const float* scale;
  int per_row;
  int64_t M, N, K;
  void* Y;
  int ydt;  // tq_dtype
};
constexpr int kGemvMaxM = 16;
constexpr int64_t kGemvLdsBytes = 65536;  // activation staging of the small-M GEMV
hipError_t launch_gemv(const GemmArgs& a, hipStream_t s);
// the same product with 1-bit sign-packed binary weights ([N][K/8] bytes)
hipError_t launch_gemv1(const GemmArgs& a, hipStream_t s);
// SwiGLU pair (a.packed / a.scale = gate, the second matrix = up):
// h = clamp(silu(g) * u, -clampv, clampv) into a.Y (fp32 or bf16), from int8
// tokens, or (fused, when fused_quant_swiglu_ok holds) from fp32/bf16 tokens
// quantised in the same launch
hipError_t launch_swiglu_gemv(const GemmArgs& a, const uint8_t* packed_up, const float* scale_up,
                              float clampv, hipStream_t s);
bool fused_quant_swiglu_ok(int64_t M, int64_t K, const void* pg, const void* pu, const void* X);
hipError_t launch_quant_swiglu_gemv(const void* X, int bf16, const ActParams& p, int8_t* q,
                                    float* sx, const GemmArgs& a, const uint8_t* packed_up,
                                    const float* scale_up, float clampv, hipStream_t s);
// quantise X (plain path) and apply the GEMV in one launch; only when
// fused_quant_gemv_ok() holds
bool fused_quant_gemv_ok(int64_t M, int64_t K, const void* packed, const void* X);
hipError_t launch_quant_gemv(const void* X, int bf16, const ActParams& p, int8_t* q,
                             float* sx, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// compute units of the current device (0 if the query fails), cached per device
int device_cus();

// ---- backward through the packed weights (k_bwd.hip)
struct BwdInputArgs {
  const void* dY;  // [M, N] fp32 or bf16
  int bf16;
  const uint8_t* packed;
  const float* scale;
  int per_row;
  int64_t M, N, K;
  float* dX;       // [M, K]
  int accumulate;
};
bool bwd_input_fast_ok(const BwdInputArgs& a);
hipError_t launch_backward_input(const BwdInputArgs& a, hipStream_t s);
struct BwdWeightArgs {
  const void* X;   // [M, K] fp32 or bf16
  int x_bf16;
  const void* dY;  // [M, N] fp32 or bf16
  int dy_bf16;
  int64_t M, N, K;
  float* dW;       // [N, K]
  int accumulate;
};
bool bwd_weight_fast_ok(const BwdWeightArgs& a);
hipError_t launch_backward_weight(const BwdWeightArgs& a, hipStream_t s);

}  // namespace tq
