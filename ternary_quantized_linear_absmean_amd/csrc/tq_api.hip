// C ABI of libtq: argument checks, then launches on the caller's stream.
// Every check runs before any HIP call, so an error status means nothing was
// enqueued.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "tq.h"
#include "tq_internal.hpp"

// Scratch of tq_pack_ternary_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  In host code `scratch` names only a
// host-side stand-in; the device address comes from hipGetSymbolAddress
// (scratch_ptr below), resolved once per device with that device current.
constexpr size_t kNoallocScratchBytes = 16384;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local const char* g_last_hip_error = "hipSuccess";

constexpr int64_t kMaxNumelPack = int64_t{1} << 40;  // exact-bin headroom
constexpr int64_t kMaxKContract = (int64_t{1} << 24) / 127;  // |acc| < 2^24

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

tq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  g_last_hip_error = hipGetErrorName(e);
  return TQ_ERR_HIP;
}

tq_status check_contract(const int8_t* q, const float* sx, int64_t M,
                         const uint8_t* packed, const float* scale, tq_gran g,
                         int64_t N, int64_t K, void* Y, tq_dtype ydt) {
  if (M < 0 || N < 0 || K <= 0 || (K % 4) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (ydt != TQ_F32 && ydt != TQ_BF16 && ydt != TQ_I32) return TQ_ERR_DTYPE;
  if (K > kMaxKContract) return TQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return TQ_OK;
  if (!q || !sx || !packed || !scale || !Y) return TQ_ERR_NULL;
  if (!aligned(sx, 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  if (!aligned(Y, ydt == TQ_BF16 ? 2 : 4)) return TQ_ERR_ALIGN;
  return TQ_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of `scratch`, its address looked up on the
// device's first call.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

tq::GemmArgs make_args(const int8_t* q, const float* sx, int64_t M, const uint8_t* packed,
                       const float* scale, tq_gran g, int64_t N, int64_t K, void* Y,
                       tq_dtype ydt) {
  tq::GemmArgs a;
  a.q = q;
  a.sx = sx;
  a.packed = packed;
  a.scale = scale;
  a.per_row = g == TQ_PER_ROW ? 1 : 0;
  a.M = M;
  a.N = N;
  a.K = K;
  a.Y = Y;
  a.ydt = static_cast<int>(ydt);
  return a;
}

}  // namespace

extern "C" {

size_t tq_packed_bytes(int64_t numel) {
  if (numel <= 0) return 0;
  return static_cast<size_t>((numel + 3) / 4);
}

size_t tq_pack_workspace_bytes(int64_t N, int64_t K, tq_gran g) {
  if (N < 0 || K <= 0 || (K % 4) != 0) return 0;
  if (g == TQ_PER_TENSOR) return tq::pack_tensor_ws_bytes();
  return 0;
}

tq_status tq_pack_ternary(const float* W, int64_t N, int64_t K, tq_gran g, tq_wmode mode,
                          uint8_t* packed, float* scale, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (N < 0 || K <= 0 || (K % 4) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (mode != TQ_TERNARY_ABSMEAN && mode != TQ_BINARY_SIGN) return TQ_ERR_UNSUPPORTED;
  if (K >= kMaxNumelPack || N >= kMaxNumelPack / K) return TQ_ERR_UNSUPPORTED;
  if (N == 0) return TQ_OK;
  if (!W || !packed || !scale) return TQ_ERR_NULL;
  if (!aligned(W, 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  if (g == TQ_PER_TENSOR) {
    const size_t need = tq::pack_tensor_ws_bytes();
    if (!ws || ws_bytes < need) return TQ_ERR_WORKSPACE;
    if (!aligned(ws, 8)) return TQ_ERR_ALIGN;
    return hip_status(tq::launch_pack_tensor(W, N * K, mode, packed, scale, ws, stream));
  }
  return hip_status(tq::launch_pack_rows(W, N, K, mode, packed, scale, stream));
}

tq_status tq_pack_ternary_noalloc(const float* W, int64_t N, int64_t K, tq_gran g,
                                  tq_wmode mode, uint8_t* packed, float* scale,
                                  hipStream_t stream) {
  if (N < 0 || K <= 0 || (K % 4) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (mode != TQ_TERNARY_ABSMEAN && mode != TQ_BINARY_SIGN) return TQ_ERR_UNSUPPORTED;
  if (K >= kMaxNumelPack || N >= kMaxNumelPack / K) return TQ_ERR_UNSUPPORTED;
  if (N == 0) return TQ_OK;
  if (!W || !packed || !scale) return TQ_ERR_NULL;
  if (!aligned(W, 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  if (g == TQ_PER_ROW) return hip_status(tq::launch_pack_rows(W, N, K, mode, packed, scale, stream));
  if (tq::pack_tensor_ws_bytes() > kNoallocScratchBytes) return TQ_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(tq::launch_pack_tensor(W, N * K, mode, packed, scale, ws, stream));
}

// Checks of tq_quant_act_int8; fills p and tells whether a prologue is on.
static tq_status check_quant(const void* X, tq_dtype xdt, int64_t M, int64_t K,
                             const tq_act_opts* opts, int8_t* q, float* sx,
                             tq::ActParams* p, bool* prologue) {
  if (M < 0 || K <= 0) return TQ_ERR_SHAPE;
  if (xdt != TQ_F32 && xdt != TQ_BF16) return TQ_ERR_DTYPE;
  p->eps = 1e-6f;
  p->clamp = 0;
  p->eta_min = 0.f;
  p->eta_max = 0.f;
  p->rmsnorm = 0;
  p->rms_eps = 1e-6f;
  p->rms_weight = nullptr;
  p->fwht = 0;
  if (opts) {
    p->eps = opts->eps;
    p->clamp = opts->clamp ? 1 : 0;
    p->eta_min = opts->eta_min;
    p->eta_max = opts->eta_max;
    p->rmsnorm = opts->rmsnorm ? 1 : 0;
    p->rms_eps = opts->rms_eps;
    p->rms_weight = opts->rms_weight;
    if (opts->fwht_block != 0 && opts->fwht_block != 512) return TQ_ERR_UNSUPPORTED;
    p->fwht = opts->fwht_block == 512 ? 1 : 0;
  }
  if (!(p->eps > 0.f) || !isfinite(p->eps)) return TQ_ERR_UNSUPPORTED;
  if (p->clamp && !(p->eta_min > 0.f && p->eta_min <= p->eta_max && isfinite(p->eta_max)))
    return TQ_ERR_UNSUPPORTED;
  if (p->rmsnorm && (!(p->rms_eps >= 0.f) || !isfinite(p->rms_eps))) return TQ_ERR_UNSUPPORTED;
  if (p->fwht && (K % 512) != 0) return TQ_ERR_SHAPE;
  *prologue = p->rmsnorm || p->fwht;
  if (*prologue && K > tq::kPrologueMaxK) return TQ_ERR_UNSUPPORTED;
  if (M == 0) return TQ_OK;
  if (!X || !q || !sx) return TQ_ERR_NULL;
  if (!aligned(X, xdt == TQ_F32 ? 4 : 2) || !aligned(sx, 4)) return TQ_ERR_ALIGN;
  if (p->rms_weight && !aligned(p->rms_weight, 4)) return TQ_ERR_ALIGN;
  return TQ_OK;
}

static hipError_t launch_quant(const void* X, tq_dtype xdt, int64_t M, int64_t K,
                               const tq::ActParams& p, bool prologue, int8_t* q, float* sx,
                               hipStream_t stream) {
  const int bf16 = xdt == TQ_BF16 ? 1 : 0;
  return prologue ? tq::launch_quant_prologue(X, bf16, M, K, p, q, sx, stream)
                  : tq::launch_quant_plain(X, bf16, M, K, p, q, sx, stream);
}

size_t tq_packed1_bytes(int64_t numel) {
  if (numel <= 0) return 0;
  return static_cast<size_t>((numel + 7) / 8);
}

tq_status tq_pack_binary1(const float* W, int64_t N, int64_t K, tq_gran g, uint8_t* packed,
                          float* scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (N < 0 || K <= 0 || (K % 8) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (K >= kMaxNumelPack || N >= kMaxNumelPack / K) return TQ_ERR_UNSUPPORTED;
  if (N == 0) return TQ_OK;
  if (!W || !packed || !scale) return TQ_ERR_NULL;
  if (!aligned(W, 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  if (g == TQ_PER_TENSOR) {
    const size_t need = tq::pack_tensor_ws_bytes();
    if (!ws || ws_bytes < need) return TQ_ERR_WORKSPACE;
    if (!aligned(ws, 8)) return TQ_ERR_ALIGN;
    return hip_status(
        tq::launch_pack_tensor(W, N * K, TQ_BINARY_SIGN, packed, scale, ws, stream, 1));
  }
  return hip_status(tq::launch_pack_rows(W, N, K, TQ_BINARY_SIGN, packed, scale, stream, 1));
}

tq_status tq_binary1_gemv(const int8_t* q, const float* sx, int64_t M, const uint8_t* packed,
                          const float* scale, tq_gran g, int64_t N, int64_t K, void* Y,
                          tq_dtype ydt, hipStream_t stream) {
  if (M > tq::kGemvMaxM) return TQ_ERR_SHAPE;
  if (K > 0 && (K % 8) != 0) return TQ_ERR_SHAPE;
  const tq_status st = check_contract(q, sx, M, packed, scale, g, N, K, Y, ydt);
  if (st != TQ_OK || M == 0 || N == 0) return st;
  return hip_status(tq::launch_gemv1(make_args(q, sx, M, packed, scale, g, N, K, Y, ydt),
                                     stream));
}

tq_status tq_quant_act_int8(const void* X, tq_dtype xdt, int64_t M, int64_t K,
                            const tq_act_opts* opts, int8_t* q, float* sx,
                            hipStream_t stream) {
  tq::ActParams p;
  bool prologue = false;
  const tq_status st = check_quant(X, xdt, M, K, opts, q, sx, &p, &prologue);
  if (st != TQ_OK || M == 0) return st;
  return hip_status(launch_quant(X, xdt, M, K, p, prologue, q, sx, stream));
}

tq_status tq_quant_ternary_gemv(const void* X, tq_dtype xdt, int64_t M,
                                const tq_act_opts* opts, const uint8_t* packed,
                                const float* scale, tq_gran g, int64_t N, int64_t K,
                                int8_t* q, float* sx, void* Y, tq_dtype ydt,
                                hipStream_t stream) {
  if (M > tq::kGemvMaxM) return TQ_ERR_SHAPE;
  tq::ActParams p;
  bool prologue = false;
  tq_status st = check_quant(X, xdt, M, K, opts, q, sx, &p, &prologue);
  if (st != TQ_OK) return st;
  st = check_contract(q, sx, M, packed, scale, g, N, K, Y, ydt);
  if (st != TQ_OK || M == 0) return st;
  if (N == 0) return hip_status(launch_quant(X, xdt, M, K, p, prologue, q, sx, stream));
  const tq::GemmArgs a = make_args(q, sx, M, packed, scale, g, N, K, Y, ydt);
  if (!prologue && tq::fused_quant_gemv_ok(M, K, packed, X))
    return hip_status(
        tq::launch_quant_gemv(X, xdt == TQ_BF16 ? 1 : 0, p, q, sx, a, stream));
  const hipError_t e = launch_quant(X, xdt, M, K, p, prologue, q, sx, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(tq::launch_gemv(a, stream));
}

// Checks of tq_swiglu_gemv; fills p and tells whether a prologue is on.
static tq_status check_swiglu(const void* X, tq_dtype xdt, int64_t M, const tq_act_opts* opts,
                              const uint8_t* pg, const float* sg, const uint8_t* pu,
                              const float* su, tq_gran g, int64_t N, int64_t K, float clampv,
                              int8_t* q, float* sx, void* H, tq_dtype hdt, tq::ActParams* p,
                              bool* prologue) {
  if (M > tq::kGemvMaxM) return TQ_ERR_SHAPE;
  if (hdt != TQ_F32 && hdt != TQ_BF16) return TQ_ERR_DTYPE;
  if (!(clampv > 0.f) || !isfinite(clampv)) return TQ_ERR_UNSUPPORTED;
  tq_status st = check_quant(X, xdt, M, K, opts, q, sx, p, prologue);
  if (st != TQ_OK) return st;
  st = check_contract(q, sx, M, pg, sg, g, N, K, H, hdt);
  if (st != TQ_OK) return st;
  return check_contract(q, sx, M, pu, su, g, N, K, H, hdt);
}

static hipError_t launch_swiglu(const void* X, tq_dtype xdt, int64_t M, const tq::ActParams& p,
                                bool prologue, const uint8_t* pg, const float* sg,
                                const uint8_t* pu, const float* su, tq_gran g, int64_t N,
                                int64_t K, float clampv, int8_t* q, float* sx, void* H,
                                tq_dtype hdt, hipStream_t stream) {
  if (N == 0) return launch_quant(X, xdt, M, K, p, prologue, q, sx, stream);
  const tq::GemmArgs a = make_args(q, sx, M, pg, sg, g, N, K, H, hdt);
  if (!prologue && tq::fused_quant_swiglu_ok(M, K, pg, pu, X))
    return tq::launch_quant_swiglu_gemv(X, xdt == TQ_BF16 ? 1 : 0, p, q, sx, a, pu, su, clampv,
                                        stream);
  const hipError_t e = launch_quant(X, xdt, M, K, p, prologue, q, sx, stream);
  if (e != hipSuccess) return e;
  return tq::launch_swiglu_gemv(a, pu, su, clampv, stream);
}

tq_status tq_swiglu_gemv(const void* X, tq_dtype xdt, int64_t M, const tq_act_opts* opts,
                         const uint8_t* packed_gate, const float* scale_gate,
                         const uint8_t* packed_up, const float* scale_up, tq_gran g, int64_t N,
                         int64_t K, float clamp_val, int8_t* q, float* sx, void* H, tq_dtype hdt,
                         hipStream_t stream) {
  tq::ActParams p;
  bool prologue = false;
  const tq_status st = check_swiglu(X, xdt, M, opts, packed_gate, scale_gate, packed_up,
                                    scale_up, g, N, K, clamp_val, q, sx, H, hdt, &p, &prologue);
  if (st != TQ_OK || M == 0) return st;
  return hip_status(launch_swiglu(X, xdt, M, p, prologue, packed_gate, scale_gate, packed_up,
                                  scale_up, g, N, K, clamp_val, q, sx, H, hdt, stream));
}

tq_status tq_ffn_swiglu_decode(const void* X, tq_dtype xdt, int64_t M, const tq_act_opts* opts,
                               const uint8_t* packed_gate, const float* scale_gate,
                               const uint8_t* packed_up, const float* scale_up,
                               const uint8_t* packed_down, const float* scale_down, tq_gran g,
                               int64_t d_model, int64_t d_ffn, float clamp_val, int8_t* q_x,
                               float* sx_x, float* H, int8_t* q_h, float* sx_h, void* Y,
                               tq_dtype ydt, hipStream_t stream) {
  // every check of both stages before anything is launched
  tq::ActParams p, ph;
  bool prologue = false, prologue_h = false;
  tq_status st = check_swiglu(X, xdt, M, opts, packed_gate, scale_gate, packed_up, scale_up, g,
                              d_ffn, d_model, clamp_val, q_x, sx_x, H, TQ_F32, &p, &prologue);
  if (st != TQ_OK) return st;
  st = check_quant(H, TQ_F32, M, d_ffn, nullptr, q_h, sx_h, &ph, &prologue_h);
  if (st != TQ_OK) return st;
  st = check_contract(q_h, sx_h, M, packed_down, scale_down, g, d_model, d_ffn, Y, ydt);
  if (st != TQ_OK || M == 0) return st;
  hipError_t e = launch_swiglu(X, xdt, M, p, prologue, packed_gate, scale_gate, packed_up,
                               scale_up, g, d_ffn, d_model, clamp_val, q_x, sx_x, H, TQ_F32,
                               stream);
  if (e != hipSuccess) return hip_status(e);
  if (d_model == 0) return hip_status(launch_quant(H, TQ_F32, M, d_ffn, ph, false, q_h, sx_h,
                                                   stream));
  const tq::GemmArgs a = make_args(q_h, sx_h, M, packed_down, scale_down, g, d_model, d_ffn, Y,
                                   ydt);
  if (tq::fused_quant_gemv_ok(M, d_ffn, packed_down, H))
    return hip_status(tq::launch_quant_gemv(H, 0, ph, q_h, sx_h, a, stream));
  e = launch_quant(H, TQ_F32, M, d_ffn, ph, false, q_h, sx_h, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(tq::launch_gemv(a, stream));
}

tq_status tq_fwht512(const void* X, tq_dtype xdt, int64_t M, int64_t K, int normalize,
                     float* Y, hipStream_t stream) {
  if (M < 0 || K <= 0 || (K % 512) != 0) return TQ_ERR_SHAPE;
  if (xdt != TQ_F32 && xdt != TQ_BF16) return TQ_ERR_DTYPE;
  if (M == 0) return TQ_OK;
  if (!X || !Y) return TQ_ERR_NULL;
  if (!aligned(X, xdt == TQ_F32 ? 4 : 2) || !aligned(Y, 4)) return TQ_ERR_ALIGN;
  return hip_status(tq::launch_fwht512(X, xdt == TQ_BF16 ? 1 : 0, M, K, normalize ? 1 : 0,
                                       Y, stream));
}

tq_status tq_ternary_gemv(const int8_t* q, const float* sx, int64_t M, const uint8_t* packed,
                          const float* scale, tq_gran g, int64_t N, int64_t K, void* Y,
                          tq_dtype ydt, hipStream_t stream) {
  if (M > tq::kGemvMaxM) return TQ_ERR_SHAPE;
  const tq_status st = check_contract(q, sx, M, packed, scale, g, N, K, Y, ydt);
  if (st != TQ_OK || M == 0 || N == 0) return st;
  return hip_status(tq::launch_gemv(make_args(q, sx, M, packed, scale, g, N, K, Y, ydt),
                                    stream));
}

tq_status tq_ternary_gemm(const int8_t* q, const float* sx, int64_t M, const uint8_t* packed,
                          const float* scale, tq_gran g, int64_t N, int64_t K, void* Y,
                          tq_dtype ydt, hipStream_t stream) {
  const tq_status st = check_contract(q, sx, M, packed, scale, g, N, K, Y, ydt);
  if (st != TQ_OK || M == 0 || N == 0) return st;
  return hip_status(tq::launch_gemm(make_args(q, sx, M, packed, scale, g, N, K, Y, ydt),
                                    stream));
}

tq_status tq_ternary_backward_input(const void* dY, tq_dtype dydt, int64_t M,
                                    const uint8_t* packed, const float* scale, tq_gran g,
                                    int64_t N, int64_t K, float* dX, int accumulate,
                                    hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || (K % 4) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (dydt != TQ_F32 && dydt != TQ_BF16) return TQ_ERR_DTYPE;
  if (M == 0) return TQ_OK;
  if (!dX) return TQ_ERR_NULL;
  if (!aligned(dX, 4)) return TQ_ERR_ALIGN;
  if (N > 0) {
    if (!dY || !packed || !scale) return TQ_ERR_NULL;
    if (!aligned(dY, dydt == TQ_BF16 ? 2 : 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  }
  tq::BwdInputArgs a;
  a.dY = dY;
  a.bf16 = dydt == TQ_BF16 ? 1 : 0;
  a.packed = packed;
  a.scale = scale;
  a.per_row = g == TQ_PER_ROW ? 1 : 0;
  a.M = M;
  a.N = N;
  a.K = K;
  a.dX = dX;
  a.accumulate = accumulate ? 1 : 0;
  return hip_status(tq::launch_backward_input(a, stream));
}

tq_status tq_ternary_backward_weight(const void* X, tq_dtype xdt, const void* dY, tq_dtype dydt,
                                     int64_t M, int64_t N, int64_t K, float* dW, int accumulate,
                                     hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return TQ_ERR_SHAPE;
  if ((xdt != TQ_F32 && xdt != TQ_BF16) || (dydt != TQ_F32 && dydt != TQ_BF16))
    return TQ_ERR_DTYPE;
  if (N == 0 || K == 0) return TQ_OK;
  if (!dW) return TQ_ERR_NULL;
  if (!aligned(dW, 4)) return TQ_ERR_ALIGN;
  if (M > 0) {
    if (!X || !dY) return TQ_ERR_NULL;
    if (!aligned(X, xdt == TQ_BF16 ? 2 : 4) || !aligned(dY, dydt == TQ_BF16 ? 2 : 4))
      return TQ_ERR_ALIGN;
  }
  tq::BwdWeightArgs a;
  a.X = X;
  a.x_bf16 = xdt == TQ_BF16 ? 1 : 0;
  a.dY = dY;
  a.dy_bf16 = dydt == TQ_BF16 ? 1 : 0;
  a.M = M;
  a.N = N;
  a.K = K;
  a.dW = dW;
  a.accumulate = accumulate ? 1 : 0;
  return hip_status(tq::launch_backward_weight(a, stream));
}

tq_status tq_pack_ternary_threshold(const float* W, int64_t N, int64_t K, tq_gran g,
                                    tq_thresh kind, float value, uint8_t* packed, float* scale,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (N < 0 || K <= 0 || (K % 4) != 0) return TQ_ERR_SHAPE;
  if (g != TQ_PER_TENSOR && g != TQ_PER_ROW) return TQ_ERR_UNSUPPORTED;
  if (kind != TQ_THRESH_RELATIVE && kind != TQ_THRESH_ABSOLUTE) return TQ_ERR_UNSUPPORTED;
  if (!isfinite(value) || value < 0.f) return TQ_ERR_UNSUPPORTED;
  if (kind == TQ_THRESH_ABSOLUTE && (g != TQ_PER_TENSOR || !(value > 0.f)))
    return TQ_ERR_UNSUPPORTED;
  if (K >= kMaxNumelPack || N >= kMaxNumelPack / K) return TQ_ERR_UNSUPPORTED;
  if (N == 0) return TQ_OK;
  if (!W || !packed || !scale) return TQ_ERR_NULL;
  if (!aligned(W, 4) || !aligned(scale, 4)) return TQ_ERR_ALIGN;
  if (kind == TQ_THRESH_ABSOLUTE)
    return hip_status(tq::launch_pack_manual(W, N * K, value, packed, scale, stream));
  if (g == TQ_PER_TENSOR) {
    const size_t need = tq::pack_tensor_ws_bytes();
    if (!ws || ws_bytes < need) return TQ_ERR_WORKSPACE;
    if (!aligned(ws, 8)) return TQ_ERR_ALIGN;
    return hip_status(tq::launch_pack_tensor(W, N * K, TQ_TERNARY_ABSMEAN, packed, scale, ws,
                                             stream, 2, value));
  }
  return hip_status(tq::launch_pack_rows(W, N, K, TQ_TERNARY_ABSMEAN, packed, scale, stream, 2,
                                         value));
}

static bool valid_codes(tq_codes f) {
  return f == TQ_CODES_NATIVE || f == TQ_CODES_F0 || f == TQ_CODES_F1;
}

tq_status tq_convert_codes(const uint8_t* src, tq_codes src_fmt, uint8_t* dst, tq_codes dst_fmt,
                           int64_t nbytes, hipStream_t stream) {
  if (nbytes < 0) return TQ_ERR_SHAPE;
  if (!valid_codes(src_fmt) || !valid_codes(dst_fmt)) return TQ_ERR_UNSUPPORTED;
  if (nbytes == 0) return TQ_OK;
  if (!src || !dst) return TQ_ERR_NULL;
  return hip_status(tq::launch_convert_codes(src, static_cast<int>(src_fmt), dst,
                                             static_cast<int>(dst_fmt), nbytes, stream));
}

tq_status tq_unpack_codes(const uint8_t* packed, tq_codes fmt, int64_t numel, int8_t* out,
                          hipStream_t stream) {
  if (numel < 0) return TQ_ERR_SHAPE;
  if (!valid_codes(fmt)) return TQ_ERR_UNSUPPORTED;
  if (numel == 0) return TQ_OK;
  if (!packed || !out) return TQ_ERR_NULL;
  return hip_status(tq::launch_unpack_codes(packed, static_cast<int>(fmt), numel, out, stream));
}

const char* tq_status_str(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "null pointer";
    case TQ_ERR_SHAPE: return "invalid shape";
    case TQ_ERR_DTYPE: return "unsupported dtype";
    case TQ_ERR_ALIGN: return "misaligned pointer";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_UNSUPPORTED: return "unsupported option or size";
    case TQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* tq_last_hip_error(void) { return g_last_hip_error; }

const char* tq_version(void) { return "0.1.0"; }

}  // extern "C"
