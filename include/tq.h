/*
 * tq.h -- C ABI of libtq, a ternary (absmean, 2-bit) linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer follows the BitNet-b1.58 recipe as the pages state it:
 *   - Foundry, docs/quantization.md, "Ternary Quantization (BitNet b1.58) /
 *     How It Works": gamma = mean|w|, q = round(w/gamma) clamped to
 *     {-1, 0, +1}, pack four per byte, integer add/sub contraction, scale by
 *     gamma afterwards; "Ternary Format / Encoding": -1 = 0b00, 0 = 0b01,
 *     +1 = 0b10, byte = v0 | v1<<2 | v2<<4 | v3<<6, (numel+3)/4 bytes.
 *   - Hetman-2b, src/quantization.py, sections 1, 2, 4, 5 and 7: FWHT-512,
 *     absmean weight quantizer, per-token symmetric int8 activations with
 *     scale 127/eta and codes in [-127, 127], RMSNorm, the BitLinear order
 *     RMSNorm -> FWHT -> int8 -> integer contraction -> y*(gamma/s_x), and
 *     the int32 GEMV emulator.
 *   - BitRASP, core_math.py, ``additive_ternary_linear_int8``: the integer
 *     identity y[o] = sum(x where W=+1) - sum(x where W=-1).
 *
 * Conventions shared by every call
 *   - W is [N, K] row-major (N output rows, K inputs), as a PyTorch Linear
 *     weight.  Packed weights are [N, K/4] bytes, row o holding the codes of
 *     W[o, 0..K-1] in order, so K must be a multiple of 4.  With K % 4 == 0
 *     this is byte-for-byte the flat LSB-first packing of the whole tensor.
 *   - Activations X are [M, K] row-major (M tokens); int8 codes q are [M, K];
 *     sx[m] is the dequantisation scale of token m (eta_m / 127).
 *   - Outputs Y are [M, N] row-major: y[m, o] = acc[m, o] * scale_o * sx[m],
 *     acc the exact int32 sum over k of q[m, k] * w[o, k].
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; libtq
 *     never allocates, frees or retains device memory.  Work is enqueued
 *     asynchronously on `stream` (0 = the null stream); results are ready
 *     once the caller synchronises that stream.
 *   - Arguments are checked before anything is enqueued; on an error status
 *     nothing is launched and no output is written.  TQ_ERR_HIP reports a
 *     failed launch (the HIP error is available from tq_last_hip_error()).
 *   - M == 0 or N == 0 is a valid empty call: TQ_OK, nothing launched.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified (but in-bounds)
 *     results.
 *   - No call keeps state between calls; calls on different streams may run
 *     concurrently as long as their output buffers do not overlap.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_NULL = 1,        /* a required pointer is NULL                      */
  TQ_ERR_SHAPE = 2,       /* negative size, K % 4 != 0, M out of range, ...  */
  TQ_ERR_DTYPE = 3,       /* dtype not accepted by this call                 */
  TQ_ERR_ALIGN = 4,       /* pointer misaligned for its element type         */
  TQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required      */
  TQ_ERR_UNSUPPORTED = 6, /* option combination or size beyond stated limits */
  TQ_ERR_HIP = 7          /* the HIP runtime refused a launch                */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1, TQ_I32 = 2 } tq_dtype;

/* Granularity of the absmean scale: one for the whole tensor, or one per
 * output row (Foundry "fq_quantize_ternary_per_channel"; BitRASP
 * ``ternarize_weight`` keeps one scale per output row). */
typedef enum tq_gran { TQ_PER_TENSOR = 0, TQ_PER_ROW = 1 } tq_gran;

/* TQ_TERNARY_ABSMEAN: q = clamp(round_half_even(fp32(w / gamma)), -1, 1).
 * TQ_BINARY_SIGN: q = +1 where w >= 0 else -1 (the +-1 weights with a
 * per-row scale of the qste project description, "What it costs and what it
 * buys"); stored in the same 2-bit codes (0b10 / 0b00). */
typedef enum tq_wmode { TQ_TERNARY_ABSMEAN = 0, TQ_BINARY_SIGN = 1 } tq_wmode;

/* Options of tq_quant_act_int8 (NULL = plain per-token absmax, eps 1e-6). */
typedef struct tq_act_opts {
  float eps;               /* floor on eta (Hetman-2b s.2 uses 1e-6)           */
  int clamp;               /* 1: clamp eta to [eta_min, eta_max] (gain clamp)  */
  float eta_min, eta_max;  /* BitLinear uses 0.05 and 40 (Hetman-2b s.0, s.5)  */
  int rmsnorm;             /* 1: RMSNorm prologue (Hetman-2b s.4)              */
  float rms_eps;           /* 1e-6 in Hetman-2b s.4                            */
  const float* rms_weight; /* [K] device pointer, or NULL for all ones         */
  int fwht_block;          /* 0 (off) or 512: blockwise FWHT-512 prologue      */
} tq_act_opts;

/* Bytes of a packed ternary tensor of `numel` values: (numel + 3) / 4
 * (Foundry "Ternary Format / Encoding").  Returns 0 for numel <= 0. */
size_t tq_packed_bytes(int64_t numel);

/* Device workspace that tq_pack_ternary needs for an [N, K] weight at
 * granularity g (0 for TQ_PER_ROW).  Returns 0 for invalid sizes. */
size_t tq_pack_workspace_bytes(int64_t N, int64_t K, tq_gran g);

/* Absmean scale + ternarize (or binarize) + 2-bit pack.
 * (Foundry "How It Works" steps 1-3 and "Ternary Format / Encoding";
 *  Hetman-2b s.2 AbsmeanWeightQuantizer forward and s.5 export_packed_weights.)
 *
 *   W       [N, K] fp32, 4-byte aligned.
 *   packed  [N, K/4] bytes (output).
 *   scale   fp32 output: [1] for TQ_PER_TENSOR, [N] for TQ_PER_ROW.
 *           gamma = max(fp32 nearest to the exact mean of |w| over the group
 *           (ties to even), fp32(1e-6)).  The mean is accumulated in fp64 and
 *           re-computed exactly (integer exponent bins) whenever the fp64
 *           value lies too close to an fp32 rounding boundary, so gamma does
 *           not depend on the launch shape.
 *   ws      device workspace of at least tq_pack_workspace_bytes(N, K, g)
 *           bytes (may be NULL when that is 0); contents are scratch.
 * Errors: NULL pointers, N < 0, K <= 0 or K % 4 != 0, N*K >= 2^40
 * (TQ_ERR_UNSUPPORTED), short workspace, misaligned W. */
tq_status tq_pack_ternary(const float* W, int64_t N, int64_t K, tq_gran g,
                          tq_wmode mode, uint8_t* packed, float* scale,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* tq_pack_ternary without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same inputs, outputs, results (bit for
 * bit) and errors as tq_pack_ternary.  The per-tensor path's partial sums,
 * flag and exponent bins live in a static device array of the library,
 * 16 KiB per GPU (the path needs 10.5 KiB, independent of N and K; a larger
 * need would be TQ_ERR_WORKSPACE), kept until the process ends; the per-row
 * path uses no scratch.  The array's device address is looked up on a
 * device's first call (hipGetSymbolAddress, a host query: make that first
 * call outside graph capture if the capture mode forbids it).  No call
 * allocates or frees memory.  All calls on one GPU share its array: calls
 * that overlap in time on that GPU (other streams, other host threads) race
 * and give undefined results; calls ordered on one stream are safe, each
 * writing every scratch word it reads first. */
tq_status tq_pack_ternary_noalloc(const float* W, int64_t N, int64_t K, tq_gran g,
                                  tq_wmode mode, uint8_t* packed, float* scale,
                                  hipStream_t stream);

/* Per-token symmetric int8 quantisation (Hetman-2b s.2
 * SymmetricActivationQuantizer, reduced per token as its code does; BitRASP
 * ``fake_quant_int``), with an optional BitLinear prologue (Hetman-2b s.5).
 *
 *   X     [M, K] fp32 or bf16 (xdt = TQ_F32 / TQ_BF16), element-aligned.
 *   q     [M, K] int8 output, codes in [-127, 127].
 *   sx    [M] fp32 output, the dequantisation scale eta_eff / 127.
 * Plain path (opts NULL, or rmsnorm == 0 and fwht_block == 0):
 *   eta = max(max_k |x|, eps), clamped to [eta_min, eta_max] when clamp;
 *   s = fp32(127/eta); q = clamp(rint(fp32(x*s)), -127, 127);
 *   sx = fp32(eta/127).  Bit-exact: q and sx.
 * Prologue path (rmsnorm and/or fwht_block = 512, K % 512 == 0 for FWHT):
 *   Hetman-2b s.5 BitLinear.forward's order, every step in fp32:
 *   1. RMSNorm (s.4): var = the fp32 nearest to the exact mean of the fp32
 *      squares fp32(x*x) (ties to even; the page fixes no summation order),
 *      r = fp32(1 / fp32(sqrt(fp32(var + rms_eps)))), x <- fp32(fp32(x*r)*g)
 *      with g = rms_weight (the product is skipped when rms_weight is NULL);
 *      rms_weight is read only with rmsnorm;
 *   2. FWHT (s.1): blockwise, stages h = 1..256, then x <- fp32(x * c) with
 *      c = fp32(1/sqrt(512));
 *   3. the plain quantiser above on the result.
 *   Bit-exact: q and sx.  Inputs whose squares overflow fp32 (|x| >= 2^64)
 *   are outside the contract.
 * Errors: NULL pointers, M < 0, K <= 0, K % 512 != 0 with FWHT, fwht_block
 * not 0 or 512, xdt not F32/BF16, K > 32768 with a prologue (UNSUPPORTED). */
tq_status tq_quant_act_int8(const void* X, tq_dtype xdt, int64_t M, int64_t K,
                            const tq_act_opts* opts, int8_t* q, float* sx,
                            hipStream_t stream);

/* Blockwise fast Walsh-Hadamard transform of length 512 along K
 * (Hetman-2b s.1 fast_walsh_hadamard_transform_512 / blockwise_fwht_forward):
 * nine butterfly stages h = 1, 2, ..., 256 in fp32, pairs (i, i+h) with bit h
 * of i clear becoming (x_i + x_{i+h}, x_i - x_{i+h}); when `normalize` is
 * non-zero the result is multiplied by fp32(1/sqrt(512)) after the last stage.
 *   X [M, K] fp32 or bf16; Y [M, K] fp32 output (may not alias X).
 * Bit-exact against the same expression tree.
 * Errors: NULL pointers, M < 0, K <= 0 or K % 512 != 0, bad dtype. */
tq_status tq_fwht512(const void* X, tq_dtype xdt, int64_t M, int64_t K,
                     int normalize, float* Y, hipStream_t stream);

/* Decode-shaped product for 1 <= M <= 16 tokens (Hetman-2b s.7 GEMV; Foundry
 * "Native Matmul Kernel"; BitRASP additive_ternary_linear_int8):
 *   acc[m, o] = sum_k q[m, k] * w[o, k] (exact int32),
 *   y[m, o]   = acc[m, o] * scale_o * sx[m] in fp32 (TQ_F32), the same rounded
 *               to bf16 (TQ_BF16), or acc itself (TQ_I32).
 *   q [M, K] int8; sx [M] fp32; packed [N, K/4]; scale [1] or [N] fp32 per g;
 *   Y [M, N] of dtype ydt, 4-byte aligned (2 for bf16).
 * The packed weight is streamed from HBM once, 16 bytes per lane, and decoded
 * in registers.  Errors: NULL pointers, M > 16, K <= 0 or K % 4 != 0,
 * N < 0, bad ydt, K > 2^24 / 127 (int32 headroom). */
tq_status tq_ternary_gemv(const int8_t* q, const float* sx, int64_t M,
                          const uint8_t* packed, const float* scale, tq_gran g,
                          int64_t N, int64_t K, void* Y, tq_dtype ydt,
                          hipStream_t stream);

/* Prefill-shaped product for any M >= 0, same contract as tq_ternary_gemv
 * (same inputs, outputs and errors, without the M <= 16 limit).  Packed
 * tiles are decoded to int8 in LDS once per workgroup and contracted with
 * int8 MFMA (v_mfma_i32_32x32x32_i8). */
tq_status tq_ternary_gemm(const int8_t* q, const float* sx, int64_t M,
                          const uint8_t* packed, const float* scale, tq_gran g,
                          int64_t N, int64_t K, void* Y, tq_dtype ydt,
                          hipStream_t stream);

/* Decode step in one call: per-token int8 quantisation of X followed by the
 * decode GEMV (Hetman-2b s.5 BitLinear: quantise, integer contraction, scale
 * fusion; s.7 GEMV).  The results -- q, sx and Y -- are bit for bit those of
 * tq_quant_act_int8(X, xdt, M, K, opts, q, sx) followed by
 * tq_ternary_gemv(q, sx, M, packed, scale, g, N, K, Y, ydt).
 * With the plain quantiser (no RMSNorm / FWHT), 16-byte aligned X and
 * packed, K % 64 == 0, and one token or up to four tokens with M*K <= 16384,
 * this is a single kernel launch: every workgroup quantises the tokens
 * itself into LDS and workgroup 0 writes q and sx.  Otherwise (more token
 * work, a prologue, other shapes) it is the two launches, which are then the
 * faster form.  The results do not depend on which.
 *   X [M, K] fp32/bf16; q [M, K] int8 and sx [M] fp32 are outputs (required);
 *   packed, scale, g, N, K, Y, ydt as for tq_ternary_gemv.
 * Errors: those of the two calls; M > 16 is TQ_ERR_SHAPE. */
tq_status tq_quant_ternary_gemv(const void* X, tq_dtype xdt, int64_t M,
                                const tq_act_opts* opts, const uint8_t* packed,
                                const float* scale, tq_gran g, int64_t N, int64_t K,
                                int8_t* q, float* sx, void* Y, tq_dtype ydt,
                                hipStream_t stream);

/* ---- SwiGLU-clamped decode FFN ---------------------------------------------
 * (Hetman-2b s.6 SwiGLUClamped: gate = SiLU(W_gate x), up = W_up x, the
 * product clamped to [-clamp_val, +clamp_val] (default 10) before W_down.)
 * Here each projection is the ternary layer of this library with the per
 * token int8 quantiser; the FFN workload (up 6912 x 2560, down 2560 x 6912,
 * per-row scales) is this shape with d_model = 2560, d_ffn = 6912. */

/* The gate and up projections of the same tokens and the SwiGLU epilogue:
 * q, sx = tq_quant_act_int8(X, opts); g = tq_ternary_gemv(gate), u =
 * tq_ternary_gemv(up) (fp32, per-row or per-tensor scales of the two
 * matrices); H = clamp(g / (1 + exp(-g)) * u, -clamp_val, clamp_val) in fp32,
 * stored as fp32 or bf16 (hdt).  q and sx are bit-exact; H is within fp32
 * rounding of that formula (a few ulp: expf and the division).
 *   X [M, K] fp32/bf16 (1 <= M <= 16); packed_gate / packed_up [N, K/4] and
 *   their scales as for tq_ternary_gemv; q [M, K], sx [M], H [M, N] outputs.
 * One token, and up to four tokens with K % 256 == 0, run as one launch
 * when X and both packed matrices are 16-byte aligned and the quantiser is
 * plain; otherwise the quantiser runs first.
 * Errors: those of tq_quant_ternary_gemv for either matrix; hdt not
 * F32/BF16 is TQ_ERR_DTYPE; clamp_val not finite and > 0 is
 * TQ_ERR_UNSUPPORTED. */
tq_status tq_swiglu_gemv(const void* X, tq_dtype xdt, int64_t M, const tq_act_opts* opts,
                         const uint8_t* packed_gate, const float* scale_gate,
                         const uint8_t* packed_up, const float* scale_up, tq_gran g,
                         int64_t N, int64_t K, float clamp_val, int8_t* q, float* sx,
                         void* H, tq_dtype hdt, hipStream_t stream);

/* The whole decode FFN as two calls, tq_swiglu_gemv (N = d_ffn,
 * K = d_model, H fp32) and then tq_quant_ternary_gemv(H, TQ_F32, M, plain
 * quantiser, packed_down [d_model, d_ffn/4], scale_down, g, d_model, d_ffn,
 * q_h, sx_h, Y, ydt): two launches where both stages fuse their quantiser
 * (one token), up to four where neither does.  opts applies to X only; H is quantised per token with
 * the plain quantiser (eps 1e-6, no clamp).  Every check of both stages runs
 * before anything is launched.  All buffers are the caller's: q_x [M,
 * d_model], sx_x [M], H [M, d_ffn] fp32, q_h [M, d_ffn], sx_h [M], Y [M,
 * d_model] of ydt. */
tq_status tq_ffn_swiglu_decode(const void* X, tq_dtype xdt, int64_t M, const tq_act_opts* opts,
                               const uint8_t* packed_gate, const float* scale_gate,
                               const uint8_t* packed_up, const float* scale_up,
                               const uint8_t* packed_down, const float* scale_down, tq_gran g,
                               int64_t d_model, int64_t d_ffn, float clamp_val, int8_t* q_x,
                               float* sx_x, float* H, int8_t* q_h, float* sx_h, void* Y,
                               tq_dtype ydt, hipStream_t stream);

/* ---- 1-bit sign-packed binary weights ------------------------------------
 * (qste 0.1.1 project description, "What it costs and what it buys": a
 * binary matrix of +-1 with a per-row scale is deployed as R*C/8 bytes of
 * packed signs plus 4*R bytes of scales.)  The pages give the size, not the
 * bit layout; this library packs eight signs per byte, LSB-first, bit 1 for
 * +1 and bit 0 for -1, rows of K/8 bytes along K. */

/* Bytes of a 1-bit sign-packed tensor of numel values: (numel + 7) / 8
 * (0 for numel <= 0). */
size_t tq_packed1_bytes(int64_t numel);

/* Binarize W (+1 where w >= 0, -0.0 and 0 included, else -1) with the
 * absmean scale of tq_pack_ternary (same exact-mean rule, per tensor or per
 * row) and pack the signs.
 *   W       [N, K] fp32, 4-byte aligned, K % 8 == 0.
 *   packed  [N, K/8] bytes (output).
 *   scale   fp32 output, [1] (TQ_PER_TENSOR) or [N] (TQ_PER_ROW).
 *   ws      as for tq_pack_ternary (tq_pack_workspace_bytes(N, K, g) bytes).
 * Errors: those of tq_pack_ternary; K % 8 != 0 is TQ_ERR_SHAPE. */
tq_status tq_pack_binary1(const float* W, int64_t N, int64_t K, tq_gran g,
                          uint8_t* packed, float* scale, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* tq_ternary_gemv for 1-bit sign-packed weights: acc[m, o] = sum_k q[m, k] *
 * b[o, k] with b = +-1 from packed [N, K/8], exact in int32, then
 * y = acc * gamma_o * sx_m as tq_ternary_gemv.  1 <= M <= 16, K % 8 == 0.
 * One token with K % 64 == 0 (K <= 16384) and 2..16 tokens with
 * K % 256 == 0 run on the fast kernels when q and packed are 16-byte
 * aligned; other shapes on a simple kernel.  Same inputs, outputs and errors
 * as tq_ternary_gemv; K % 8 != 0 is TQ_ERR_SHAPE. */
tq_status tq_binary1_gemv(const int8_t* q, const float* sx, int64_t M,
                          const uint8_t* packed, const float* scale, tq_gran g,
                          int64_t N, int64_t K, void* Y, tq_dtype ydt,
                          hipStream_t stream);

/* ---- backward through the packed weights ---------------------------------
 * (Foundry, docs/quantization.md, "Ternary Training (Backward Pass +
 * Stochastic Flip) / Backward Pass": the input gradient multiplies the
 * output gradient against the packed ternary weights, with the same unpacking
 * as the forward, summing over the N outputs.)  The forward being
 * y[m, o] = gamma_o * sum_k x[m, k] w[o, k], this call takes the scale into
 * the gradient (the page's example uses one scale per tensor; a per-row
 * scale multiplies each output's gradient):
 *     dX[m, k] = sum_n dY[m, n] * gamma_n * w[n, k]
 *   dY       [M, N] fp32 or bf16 (dydt), element-aligned.
 *   packed   [N, K/4] codes of tq_pack_ternary (K % 4 == 0).
 *   scale    fp32, [1] (TQ_PER_TENSOR) or [N] (TQ_PER_ROW).
 *   dX       [M, K] fp32, 4-byte aligned.  accumulate = 0 overwrites dX;
 *            accumulate != 0 adds the result to it (the page's += form).
 * Arithmetic: each product dY * gamma_n * w is formed exactly (w is -1, 0 or
 * +1; with a per-row scale, dY * gamma_n is first rounded to fp32) and the
 * sum over n is accumulated in fp32 (on the matrix cores each step of 32
 * rows rounds within one ulp), so the error is that of an fp32 dot product
 * of length N; a per-tensor gamma multiplies the fp32 sum.  Inputs
 * need |dY * gamma| < 3.3e38 (the bf16 range).  N % 8 == 0 with 16-byte
 * aligned dY, dX (and scale, per row) runs on the matrix cores; other shapes
 * on a simple kernel.  N == 0 writes zeros (or leaves dX, with accumulate).
 * Errors: M, N < 0, K <= 0 or K % 4 != 0 is TQ_ERR_SHAPE; dydt other than
 * F32/BF16 is TQ_ERR_DTYPE; NULL dX, or NULL dY, packed or scale with
 * M, N > 0, is TQ_ERR_NULL. */
tq_status tq_ternary_backward_input(const void* dY, tq_dtype dydt, int64_t M,
                                    const uint8_t* packed, const float* scale, tq_gran g,
                                    int64_t N, int64_t K, float* dX, int accumulate,
                                    hipStream_t stream);

/* The weight gradient of the same page: the float product
 *     dW[n, k] = sum_m dY[m, n] * X[m, k]        (X^T dY, laid out [N, K])
 * with no codes and no scale.
 *   X   [M, K] fp32 or bf16 (xdt), dY [M, N] fp32 or bf16 (dydt),
 *       element-aligned.
 *   dW  [N, K] fp32, 4-byte aligned; accumulate != 0 adds to it.
 * Arithmetic: products of a bf16 operand with anything are formed exactly;
 * with both operands fp32 each product carries an error of at most about
 * 2^-23 |dY X| (three-term bf16 splits, the smallest cross terms dropped).
 * Sums are accumulated in fp32 over M (on the matrix cores each accumulation
 * step rounds within one ulp).  N % 8 == 0, K % 8 == 0 and 16-byte
 * aligned X, dY run on the matrix cores; other shapes on a simple kernel.
 * M == 0 writes zeros (or leaves dW, with accumulate).
 * Errors: M, N, K < 0 is TQ_ERR_SHAPE; xdt or dydt other than F32/BF16 is
 * TQ_ERR_DTYPE; NULL dW with N, K > 0, or NULL X, dY with M, N, K > 0, is
 * TQ_ERR_NULL. */
tq_status tq_ternary_backward_weight(const void* X, tq_dtype xdt, const void* dY, tq_dtype dydt,
                                     int64_t M, int64_t N, int64_t K, float* dW, int accumulate,
                                     hipStream_t stream);

/* ---- quantiser and format options -----------------------------------------
 * Threshold ternarization (Foundry docs/quantization.md "Absmean Thresholding
 * (BitNet b1.58)" and fq_quantize_ternary_threshold; BitRASP core_math.py
 * ternarize_weight): q = +1 where w > h, -1 where w < -h, 0 otherwise, in
 * fp32 with strict comparisons. */
typedef enum tq_thresh {
  TQ_THRESH_RELATIVE = 0, /* h = fp32(value * gamma), gamma the absmean scale of
                             tq_pack_ternary (per tensor or row), scale = gamma;
                             value 1 is Foundry's absmean rule, 0.55 BitRASP's,
                             0.5 reproduces tq_pack_ternary                    */
  TQ_THRESH_ABSOLUTE = 1  /* h = value (> 0), scale[0] = value, per tensor only */
} tq_thresh;

/* tq_pack_ternary with a threshold rule.  value must be finite, >= 0
 * (relative) or > 0 (absolute), else TQ_ERR_UNSUPPORTED; TQ_THRESH_ABSOLUTE
 * with TQ_PER_ROW is TQ_ERR_UNSUPPORTED and needs no workspace.  Other
 * arguments and errors as tq_pack_ternary (ternary codes only). */
tq_status tq_pack_ternary_threshold(const float* W, int64_t N, int64_t K, tq_gran g,
                                    tq_thresh kind, float value, uint8_t* packed, float* scale,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Code formats of packed 2-bit weights, four values per byte LSB-first:
 * this library's (Foundry "Ternary Format / Encoding") and Hetman-2b
 * src/quantization.py section 3's Formats 0 and 1.  Each format's unused
 * code reads as 0. */
typedef enum tq_codes {
  TQ_CODES_NATIVE = 0, /* -1 = 00, 0 = 01, +1 = 10 (11 unused)             */
  TQ_CODES_F0 = 1,     /* 0 = 00, +1 = 01, -1 = 11 (10 reserved)            */
  TQ_CODES_F1 = 2      /* 0 = 00, +1 = 01, -1 = 10 (11 reserved)            */
} tq_codes;

/* Re-encode nbytes packed bytes from src_fmt to dst_fmt, value by value.
 * src == dst (in place) is allowed; other overlaps are not.
 * Errors: nbytes < 0 is TQ_ERR_SHAPE; an unknown format TQ_ERR_UNSUPPORTED;
 * NULL src or dst with nbytes > 0 TQ_ERR_NULL. */
tq_status tq_convert_codes(const uint8_t* src, tq_codes src_fmt, uint8_t* dst, tq_codes dst_fmt,
                           int64_t nbytes, hipStream_t stream);

/* Values of numel packed codes (ceil(numel/4) bytes) as int8 -1/0/+1.
 * Errors as tq_convert_codes. */
tq_status tq_unpack_codes(const uint8_t* packed, tq_codes fmt, int64_t numel, int8_t* out,
                          hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* tq_status_str(tq_status s);

/* Name of the last HIP error seen by this thread inside libtq ("hipSuccess"
 * if none).  Pointer to a static string. */
const char* tq_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
