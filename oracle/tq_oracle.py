"""CPU oracle for the ternary (absmean, 2-bit) linear layer.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
HIP library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library.

Sources (cited by page title and section):

* Foundry, docs/quantization.md -- "Ternary Format / Encoding" (2-bit codes,
  LSB-first byte layout, packed size), "Ternary Quantization (BitNet b1.58) /
  How It Works" (absmean scale, round-and-clamp), "Native Matmul Kernel"
  (add/sub/skip contraction, then the scale).
* Hetman-2b, src/quantization.py -- section 1 (FWHT-512 butterfly and its
  1/sqrt(512) normaliser), section 2 (absmean weight quantizer, symmetric
  int8 activation quantizer), section 4 (RMSNorm), section 5 (BitLinear order
  of operations and its scale fusion), section 6 (SwiGLUClamped: SiLU gate
  times up projection, clamped to +-10 before the down projection),
  section 7 (integer GEMV emulator).
* BitRASP, core_math.py -- ``fake_quant_int`` (per-token absmax int8),
  ``ternarize_weight`` (per-output-row absmean), ``additive_ternary_linear_int8``
  (y[o] = sum of x where W=+1 minus sum of x where W=-1).
* Foundry, docs/quantization.md -- "Ternary Training (Backward Pass +
  Stochastic Flip) / Backward Pass": the input gradient multiplies the output
  gradient against the packed ternary weights, summing over N, accumulated
  with += into a caller-zeroed buffer; the weight gradient is the plain float
  product X^T dY with no ternary part and no scale.
* Foundry, docs/quantization.md -- "Absmean Thresholding (BitNet b1.58)"
  (+1 above the threshold, -1 below its negative, 0 between, the threshold
  being mean|w| or a manual value, and the scale the threshold) and the API
  reference (``fq_quantize_ternary_threshold``).
* BitRASP, core_math.py -- ``ternarize_weight``: per-row absmean scale and
  codes w > 0.55*scale -> +1, w < -0.55*scale -> -1, else 0.
* Hetman-2b, src/quantization.py, section 3 (PackedTernaryStorage): Format 0
  (0 -> 00, +1 -> 01, -1 -> 11, 10 reserved as 0) and Format 1 (0 -> 00,
  +1 -> 01, -1 -> 10, 11 reserved as 0), four codes per byte LSB-first,
  decoded with P = B & 0x55, N = (B >> 1) & 0x55 as P - 2(P & N) (Format 0)
  or P - N (Format 1).
* qste 0.1.1 project description -- "What it costs and what it buys"
  (binary +-1 weights with a per-row scale, deployed as R*C/8 bytes of
  packed signs plus 4*R bytes of scales).

Readings taken where the pages are silent or disagree (each is also listed
in the design notes):

* The absmean scale is the correctly rounded fp32 value of the exact mean of
  |w| over the group, then floored at fp32(1e-6).  The pages compute the mean
  in fp32 without fixing a summation order; the exact mean is the one value
  every order approximates.
* Weights are ternarized by round-half-even of the fp32 quotient w/gamma,
  clamped to [-1, 1] (Foundry "How It Works", Hetman-2b section 2).  The
  "Absmean Thresholding" block of the Foundry page (|w| > gamma) is a
  separate option, ``ternarize_threshold``.
* Binary mode: +1 where w >= 0, else -1, with the same per-row absmean scale.
* Activations: per-token eta = max|x| floored at 1e-6, optional clamp to
  [eta_min, eta_max]; s = fp32(127/eta); q = clamp(rint(fp32(x*s)), -127, 127);
  the dequantisation scale returned is sx = fp32(eta/127).
* RMSNorm's mean of squares is the exact mean of the fp32 squares rounded
  once to fp32 (the page fixes no summation order), and rsqrt is a correctly
  rounded square root followed by a correctly rounded division.
* A partial last byte (only possible when the element count is not a multiple
  of four) is padded with the zero code 0b01.
* 1-bit sign packing of binary weights (qste "What it costs and what it
  buys" gives the size, not the layout): eight signs per byte, LSB-first,
  bit 1 for +1 and bit 0 for -1, rows of K/8 bytes along K.
* Threshold options: the comparisons are strict and taken in fp32 against
  fp32(f * gamma) (a factor of the absmean scale, as BitRASP computes
  threshold * scale in its tensor precision) or against the manual value t,
  whose scale is t itself (Foundry: the scale is the threshold).
* Code formats: this library's own codes (-1 = 00, 0 = 01, +1 = 10) convert
  to and from Hetman-2b's Formats 0 and 1 value by value; the reserved code
  of each format (11 here, 10 in Format 0, 11 in Format 1) reads as 0.
* Backward through the input: the layer computes y = gamma * x w^T (the
  activation quantiser passed straight through, as the pages' straight-
  through estimator does), so dX = (dY * gamma) w; the page does not say
  whether its input gradient applies the scale, and the gradient of y does.
* The BitLinear activation prologue (RMSNorm -> FWHT -> int8) runs the
  page's three steps in order with fp32 intermediates (the page rounds back
  to the input dtype between steps, which is the identity for fp32 input).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32
GAMMA_EPS = F32(1e-6)          # floor on the absmean scale (Hetman-2b s.2, BitRASP)
ACT_EPS = F32(1e-6)            # floor on the activation absmax (Hetman-2b s.2)
QMAX = 127                     # symmetric int8 bound (Hetman-2b s.2)
FWHT_BLOCK = 512               # Hetman-2b s.0
FWHT_NORM = F32(1.0 / np.sqrt(512.0))   # fp32(1/sqrt(512)), Hetman-2b s.0 / s.1
ETA_MIN_BITLINEAR = 0.05       # gain clamp used by BitLinear, Hetman-2b s.0 / s.5
ETA_MAX_BITLINEAR = 40.0
RMS_EPS = F32(1e-6)            # Hetman-2b s.4

# --------------------------------------------------------------------------
# Sizes
# --------------------------------------------------------------------------


def packed_bytes(numel: int) -> int:
    """Bytes of a packed ternary tensor: (numel + 3) / 4, rounded down
    (Foundry, "Ternary Format / Encoding")."""
    return (int(numel) + 3) // 4


# --------------------------------------------------------------------------
# Exact rational arithmetic for the absmean scale
# --------------------------------------------------------------------------


def round_rational_to_f32(num: int, den: int) -> np.float32:
    """Round the non-negative rational num/den to the nearest fp32, ties to
    even (IEEE 754 roundTiesToEven).  Subnormal results use the fixed quantum
    2**-149.  Raises OverflowError past the fp32 range."""
    num, den = int(num), int(den)
    if den <= 0 or num < 0:
        raise ValueError("need num >= 0 and den > 0")
    if num == 0:
        return F32(0.0)
    # exponent e with 2**e <= num/den < 2**(e+1)
    e = num.bit_length() - den.bit_length()
    if (num << max(-e, 0)) < (den << max(e, 0)):
        e -= 1
    e = max(e, -126)                      # below 2**-126 the spacing stays 2**-149
    shift = 23 - e                        # scale so the quantum 2**(e-23) becomes 1
    if shift >= 0:
        n2, d2 = num << shift, den
    else:
        n2, d2 = num, den << (-shift)
    m, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (m & 1)):
        m += 1
    value = m * 2.0 ** (e - 23)           # exact in fp64: m <= 2**24
    if value > float(np.finfo(np.float32).max):
        raise OverflowError("result exceeds the fp32 range")
    return F32(value)


def exact_abs_sum_units(w: np.ndarray) -> int:
    """Exact sum of |w| over a finite fp32 array, as an integer count of the
    smallest fp32 quantum 2**-149.

    Each finite fp32 magnitude is M * 2**(b-150) with b = max(E, 1), E the
    biased exponent and M the 24-bit significand (implicit bit included when
    E > 0), i.e. M << (b-1) quanta.  Significands are summed per exponent in
    uint64 (exact while the group holds fewer than 2**40 elements) and the
    per-exponent totals are combined as Python integers."""
    a = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input")
    bits = a.view(np.uint32) & np.uint32(0x7FFFFFFF)
    expo = (bits >> np.uint32(23)).astype(np.int64)
    mant = (bits & np.uint32(0x7FFFFF)).astype(np.uint64)
    mant = np.where(expo > 0, mant | np.uint64(1 << 23), mant)
    b = np.maximum(expo, 1)
    total = 0
    for e in np.unique(b):
        s = int(mant[b == e].sum(dtype=np.uint64))
        total += s << (int(e) - 1)
    return total


def absmean_scale(w_group: np.ndarray) -> np.float32:
    """gamma = max(fp32(mean |w|), fp32(1e-6)) with the mean taken exactly and
    rounded once (Foundry "How It Works" step 1; Hetman-2b s.2 absmean with
    clamp(min=eps); BitRASP ``ternarize_weight`` per-row variant)."""
    n = int(np.asarray(w_group).size)
    if n == 0:
        raise ValueError("absmean of an empty group is undefined")
    total = exact_abs_sum_units(w_group)
    gamma = round_rational_to_f32(total, n << 149)
    return max(gamma, GAMMA_EPS)


def absmean_scales(W: np.ndarray, granularity: str) -> np.ndarray:
    """Scales for W [N, K]: one for the whole tensor ("tensor") or one per
    output row ("row", Foundry per-channel ternary; BitRASP per-output scale)."""
    W = np.asarray(W, dtype=np.float32)
    if granularity == "tensor":
        return np.array([absmean_scale(W)], dtype=np.float32)
    if granularity == "row":
        return np.array([absmean_scale(W[i]) for i in range(W.shape[0])],
                        dtype=np.float32)
    raise ValueError(granularity)


# --------------------------------------------------------------------------
# Weight codes and packing
# --------------------------------------------------------------------------


def ternarize(W: np.ndarray, gammas: np.ndarray) -> np.ndarray:
    """q = clamp(rint(fp32(w / gamma)), -1, 1), round half to even
    (Foundry "How It Works" step 2; Hetman-2b s.2 forward).  ``gammas`` holds
    one scale, or one per row of W."""
    W = np.asarray(W, dtype=np.float32)
    g = np.asarray(gammas, dtype=np.float32)
    g = g.reshape(-1, 1) if g.size > 1 else g.reshape(1, 1)
    t = W / g                                   # IEEE fp32 division
    return np.clip(np.rint(t), -1, 1).astype(np.int8)


def binarize(W: np.ndarray) -> np.ndarray:
    """Binary (+-1) weights: +1 where w >= 0 (zero and -0.0 included), else -1
    (qste "What it costs and what it buys": a matrix of +-1 and a per-row scale)."""
    W = np.asarray(W, dtype=np.float32)
    return np.where(W >= 0, 1, -1).astype(np.int8)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Pack ternary values along the last axis, four per byte, LSB-first, with
    -1 -> 0b00, 0 -> 0b01, +1 -> 0b10 (Foundry "Ternary Format / Encoding").
    A partial last byte is padded with the zero code 0b01."""
    q = np.asarray(q)
    if q.ndim == 1:
        q = q.reshape(1, -1)
    if q.size and (q.min() < -1 or q.max() > 1):
        raise ValueError("values outside {-1, 0, 1}")
    n, k = q.shape
    nb = packed_bytes(k)
    codes = np.ones((n, nb * 4), dtype=np.uint8)            # 0b01 padding
    codes[:, :k] = (q.astype(np.int16) + 1).astype(np.uint8)
    codes = codes.reshape(n, nb, 4)
    out = np.zeros((n, nb), dtype=np.uint8)
    for slot in range(4):
        out |= codes[:, :, slot] << np.uint8(2 * slot)
    return out


def unpack_codes(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of ``pack_codes`` for rows of k values.  The unused code 0b11
    is rejected."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim == 1:
        packed = packed.reshape(1, -1)
    n, nb = packed.shape
    if nb != packed_bytes(k):
        raise ValueError("row length does not match k")
    codes = np.empty((n, nb, 4), dtype=np.uint8)
    for slot in range(4):
        codes[:, :, slot] = (packed >> np.uint8(2 * slot)) & np.uint8(3)
    if np.any(codes == 3):
        raise ValueError("code 0b11 is not a ternary value")
    codes = codes.reshape(n, nb * 4)[:, :k]
    return (codes.astype(np.int16) - 1).astype(np.int8)


def pack_ternary(W: np.ndarray, granularity: str = "tensor", mode: str = "ternary"):
    """Absmean scale(s) + codes + 2-bit packing of W [N, K] (rows along K).
    Returns (packed uint8 [N, ceil(K/4)], scales fp32 [1] or [N])."""
    W = np.asarray(W, dtype=np.float32)
    gam = absmean_scales(W, granularity)
    if mode == "ternary":
        q = ternarize(W, gam)
    elif mode == "binary":
        q = binarize(W)
    else:
        raise ValueError(mode)
    return pack_codes(q), gam


def ternarize_threshold(W: np.ndarray, granularity: str, kind: str, value: float):
    """Codes and scales by a threshold (Foundry "Absmean Thresholding" and
    ``fq_quantize_ternary_threshold``; BitRASP ``ternarize_weight``).
    kind "relative": gamma = the absmean scale (per tensor or row), threshold
    h = fp32(fp32(value) * gamma), scale gamma; value 1 is Foundry's absmean
    rule, 0.55 BitRASP's.  kind "absolute": h = fp32(value) and the scale is h
    (per tensor).  q = +1 where w > h, -1 where w < -h, else 0."""
    W = np.asarray(W, dtype=np.float32)
    if kind == "relative":
        gam = absmean_scales(W, granularity)
        h = (F32(value) * gam).astype(np.float32)          # fp32 product
        scales = gam
    elif kind == "absolute":
        if granularity != "tensor":
            raise ValueError("a manual threshold is one value for the tensor")
        h = np.array([F32(value)], dtype=np.float32)
        scales = h.copy()
    else:
        raise ValueError(kind)
    hh = h.reshape(-1, 1) if h.size > 1 else h.reshape(1, 1)
    q = np.zeros(W.shape, dtype=np.int8)
    q[W > hh] = 1
    q[W < -hh] = -1
    return q, scales


FORMATS = ("native", "f0", "f1")


def encode_format(q: np.ndarray, fmt: str) -> np.ndarray:
    """Pack ternary values along the last axis, four per byte LSB-first, in
    this library's codes ("native") or Hetman-2b s.3 Format 0 / Format 1.
    Format 0's code is the low two bits of the two's-complement int8 value;
    Format 1 maps -1 to 0b10."""
    q = np.asarray(q).astype(np.int8)
    if q.ndim == 1:
        q = q.reshape(1, -1)
    if q.shape[-1] % 4:
        raise ValueError("rows must hold a multiple of four values")
    if fmt == "native":
        return pack_codes(q)
    if fmt == "f0":
        codes = (q.view(np.uint8) & np.uint8(3))              # w & 3
    elif fmt == "f1":
        codes = np.where(q == -1, 2, np.where(q == 1, 1, 0)).astype(np.uint8)
    else:
        raise ValueError(fmt)
    n, k = q.shape
    c = codes.reshape(n, k // 4, 4)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def decode_format(packed: np.ndarray, fmt: str) -> np.ndarray:
    """Values of packed codes in any format (reserved codes read as 0).
    Formats 0 and 1 by the page's bitmasks: per 2-bit field, p = low bit and
    n = high bit; Format 0 v = p - 2(p & n), Format 1 v = p - n.  Native codes
    c = 0, 1, 2 are v = c - 1, with c = 3 read as 0."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim == 1:
        packed = packed.reshape(1, -1)
    n, nb = packed.shape
    fields = np.stack([(packed >> np.uint8(2 * t)) & np.uint8(3) for t in range(4)], axis=-1)
    p = (fields & 1).astype(np.int8)
    hi = ((fields >> 1) & 1).astype(np.int8)
    if fmt == "f0":
        v = p - 2 * (p & hi)
    elif fmt == "f1":
        v = p - hi
    elif fmt == "native":
        v = np.where(fields == 3, 0, fields.astype(np.int16) - 1).astype(np.int8)
    else:
        raise ValueError(fmt)
    return v.reshape(n, nb * 4).astype(np.int8)


def convert_codes(packed: np.ndarray, src: str, dst: str) -> np.ndarray:
    """Re-encode packed codes from one format to another, value by value."""
    return encode_format(decode_format(packed, src), dst)


def packed1_bytes(numel: int) -> int:
    """Bytes of a 1-bit sign-packed tensor: (numel + 7) / 8, rounded down
    (qste "What it costs and what it buys": R*C/8 bytes of packed signs)."""
    if numel < 0:
        raise ValueError("numel must be >= 0")
    return (numel + 7) // 8


def pack_signs(b: np.ndarray) -> np.ndarray:
    """Pack +-1 values along the last axis, eight per byte, LSB-first, bit 1
    for +1 and bit 0 for -1.  Rows must be a whole number of bytes."""
    b = np.asarray(b)
    if b.ndim == 1:
        b = b.reshape(1, -1)
    n, k = b.shape
    if k % 8:
        raise ValueError("row length must be a multiple of 8")
    if b.size and not np.all((b == 1) | (b == -1)):
        raise ValueError("values outside {-1, +1}")
    bits = (b == 1).astype(np.uint8).reshape(n, k // 8, 8)
    out = np.zeros((n, k // 8), dtype=np.uint8)
    for slot in range(8):
        out |= bits[:, :, slot] << np.uint8(slot)
    return out


def unpack_signs(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of ``pack_signs`` for rows of k values -> int8 +-1."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim == 1:
        packed = packed.reshape(1, -1)
    n, nb = packed.shape
    if k % 8 or nb != k // 8:
        raise ValueError("row length does not match k")
    bits = np.empty((n, nb, 8), dtype=np.int8)
    for slot in range(8):
        bits[:, :, slot] = (packed >> np.uint8(slot)) & np.uint8(1)
    return (2 * bits.reshape(n, k) - 1).astype(np.int8)


def pack_binary1(W: np.ndarray, granularity: str = "row"):
    """Binary weights in 1-bit form: absmean scale(s) (the same rule as the
    ternary scale), signs (+1 where w >= 0) packed eight per byte.  Returns
    (packed uint8 [N, K/8], scales fp32 [1] or [N])."""
    W = np.asarray(W, dtype=np.float32)
    return pack_signs(binarize(W)), absmean_scales(W, granularity)


def contract_signs(q: np.ndarray, packed: np.ndarray, k: int) -> np.ndarray:
    """acc[m, o] = sum_k q[m, k] * b[o, k] over the unpacked +-1 weights,
    exact, int64."""
    return _exact_integer_product(q, unpack_signs(packed, k))


# --------------------------------------------------------------------------
# Activations
# --------------------------------------------------------------------------


def quant_act_int8(X: np.ndarray, eps=ACT_EPS, bounds=None):
    """Per-token symmetric int8 quantisation (Hetman-2b s.2; its code reduces
    over the last axis, and BitRASP ``fake_quant_int`` is per token too).

    For each token (row) x:
        eta = max|x_k|, floored at eps, then clamped to bounds = (lo, hi)
              (the gain clamp; None means no clamp);
        s   = fp32(127 / eta);
        q_k = rint(fp32(x_k * s)) clamped to [-127, 127], halves to even;
        sx  = fp32(eta / 127), the dequantisation scale returned.
    Returns (q int8 [M, K], sx fp32 [M])."""
    x = np.asarray(X, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    lo, hi = (F32(0.0), F32(np.inf)) if bounds is None else (F32(bounds[0]), F32(bounds[1]))
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    for i in range(M):
        amax = np.max(np.abs(x[i])) if K else F32(0.0)
        eta = min(max(max(F32(amax), F32(eps)), lo), hi)     # fp32 throughout
        s = F32(F32(QMAX) / eta)
        q[i] = np.clip(np.rint(x[i] * s), -QMAX, QMAX).astype(np.int8)
        sx[i] = F32(eta / F32(QMAX))
    return q, sx


# --------------------------------------------------------------------------
# Walsh-Hadamard rotation
# --------------------------------------------------------------------------


def fwht_block(x: np.ndarray, normalize: bool) -> np.ndarray:
    """Fast Walsh-Hadamard transform of length-512 rows in fp32
    (Hetman-2b s.1): nine butterfly stages with half-widths h = 1, 2, ..., 256
    in that order; at each stage every index i whose bit h is clear is paired
    with i + h and the pair becomes (x_i + x_{i+h}, x_i - x_{i+h}).  When
    normalising, the result is multiplied by fp32(1/sqrt(512)) after the last
    stage."""
    y = np.array(x, dtype=np.float32, copy=True)
    if y.shape[-1] != FWHT_BLOCK:
        raise ValueError("last axis must be 512")
    idx = np.arange(FWHT_BLOCK)
    h = 1
    while h < FWHT_BLOCK:
        lo = idx[(idx & h) == 0]
        hi = lo + h
        a = y[..., lo].copy()
        b = y[..., hi].copy()
        y[..., lo] = a + b
        y[..., hi] = a - b
        h *= 2
    if normalize:
        y = (y * FWHT_NORM).astype(np.float32)
    return y


def fwht512(X: np.ndarray, normalize: bool = True) -> np.ndarray:
    """Blockwise FWHT over consecutive 512-wide blocks of the last axis, which
    must be a multiple of 512 (Hetman-2b s.1, ``blockwise_fwht_forward``)."""
    x = np.asarray(X, dtype=np.float32)
    d = x.shape[-1]
    if d % FWHT_BLOCK:
        raise ValueError("last axis must be a multiple of 512")
    blocks = x.reshape(*x.shape[:-1], d // FWHT_BLOCK, FWHT_BLOCK)
    return fwht_block(blocks, normalize).reshape(x.shape)


def mean_of_squares(x_row: np.ndarray) -> np.float32:
    """var = the fp32 nearest (ties to even) to the exact mean of the fp32
    squares fp32(x_k * x_k) of one token (Hetman-2b s.4: x.pow(2).mean over
    the last axis, in fp32).  The page fixes no summation order; the exact
    mean rounded once is the value every order approximates (the reading
    taken for the absmean scale as well).  The squares are summed exactly as
    integer counts of 2**-149."""
    x = np.asarray(x_row, dtype=np.float32).ravel()
    if x.size == 0:
        raise ValueError("empty token")
    sq = (x * x).astype(np.float32)
    if not np.all(np.isfinite(sq)):
        raise ValueError("a square is not finite in fp32")
    return round_rational_to_f32(exact_abs_sum_units(sq), x.size << 149)


def rms_factor(x_row: np.ndarray, rms_eps=RMS_EPS) -> np.float32:
    """r = fp32(1 / fp32(sqrt(fp32(var + eps)))) with var = mean_of_squares
    (Hetman-2b s.4: rsqrt(variance + eps) in fp32; the reciprocal square
    root is read as a correctly rounded square root followed by a correctly
    rounded division)."""
    t = F32(mean_of_squares(x_row) + F32(rms_eps))
    return F32(F32(1.0) / np.sqrt(t))


def rmsnorm(X: np.ndarray, weight=None, rms_eps=RMS_EPS) -> np.ndarray:
    """Hetman-2b s.4 SubLayerRMSNorm in fp32: token x becomes
    fp32(fp32(x * r) * g) with r = rms_factor(x) and g the norm weight
    (ones when None, a product that changes nothing)."""
    x = np.asarray(X, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    out = np.empty_like(x)
    for i in range(x.shape[0]):
        y = (x[i] * rms_factor(x[i], rms_eps)).astype(np.float32)
        if weight is not None:
            y = (y * np.asarray(weight, dtype=np.float32)).astype(np.float32)
        out[i] = y
    return out


BITLINEAR_BOUNDS = (ETA_MIN_BITLINEAR, ETA_MAX_BITLINEAR)


def bitlinear_prologue(X: np.ndarray, bounds=BITLINEAR_BOUNDS, rms_weight=None,
                       rmsnorm_on: bool = True, fwht: bool = True, eps=ACT_EPS,
                       rms_eps=RMS_EPS):
    """Activation path of Hetman-2b s.5 BitLinear.forward, steps 1-3, in the
    page's order and in fp32:
        1. RMSNorm (s.4), ``rmsnorm`` above;
        2. blockwise FWHT-512 with the 1/sqrt(512) factor (s.1), ``fwht512``;
        3. the per-token int8 quantiser with eps 1e-6 and the gain clamp
           [0.05, 40] (s.2), ``quant_act_int8``.
    Steps 1 and 2 can be switched off.  The page converts each step's result
    back to the input dtype; here every intermediate stays fp32 (the page's
    own behaviour for an fp32 input; a bf16 input widens to fp32 exactly).
    Returns (q int8 [M, K], sx fp32 [M])."""
    x = np.asarray(X, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if rmsnorm_on:
        x = rmsnorm(x, rms_weight, rms_eps)
    if fwht:
        x = fwht512(x, normalize=True)
    return quant_act_int8(x, eps, bounds)


def bitlinear_prologue_fp64(X: np.ndarray, bounds=BITLINEAR_BOUNDS):
    """The same three steps in fp64, with the Hadamard rotation as a product
    with the Sylvester matrix -- used only to bound how far the fp32 chain's
    roundings move a code (by one, at rounding boundaries)."""
    x = np.asarray(X, dtype=np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    xn = x / np.sqrt(ms + 1e-6)
    H = hadamard_matrix(FWHT_BLOCK).astype(np.float64) / np.sqrt(512.0)
    M, K = x.shape
    xr = (xn.reshape(M, K // FWHT_BLOCK, FWHT_BLOCK) @ H.T).reshape(M, K)
    eta = np.maximum(np.max(np.abs(xr), axis=1), 1e-6)
    if bounds is not None:
        eta = np.clip(eta, bounds[0], bounds[1])
    q = np.clip(np.rint(xr * (127.0 / eta)[:, None]), -127, 127).astype(np.int8)
    return q, eta / 127.0


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix H[i, j] = (-1)**popcount(i & j), int64."""
    i = np.arange(n).reshape(-1, 1)
    j = np.arange(n).reshape(1, -1)
    v = i & j
    pc = np.zeros_like(v)
    while np.any(v):
        pc += v & 1
        v >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


# --------------------------------------------------------------------------
# Contraction and epilogue
# --------------------------------------------------------------------------


def _exact_integer_product(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """q [M, K] times w^T for integer-valued q (|q| <= 128) and w in
    {-1, 0, +1}, as a float64 matrix product: every product and every partial
    sum is an integer of magnitude at most 128 K < 2**53, so each step of the
    library's product is exact in any order and the result is the exact
    integer sum.  Returns int64, checked to fit int32."""
    q = np.asarray(q)
    k = q.shape[-1] if q.ndim else 0
    if 128 * k >= 2**53:
        raise ValueError("K too large for an exact float64 product")
    acc = (q.astype(np.float64) @ np.asarray(w, dtype=np.float64).T).astype(np.int64)
    if acc.size and (acc.max() > 2**31 - 1 or acc.min() < -2**31):
        raise OverflowError("accumulator exceeds int32")
    return acc


def contract(q: np.ndarray, packed: np.ndarray, k: int) -> np.ndarray:
    """acc[m, o] = sum_k q[m, k] * w[o, k] over the unpacked weight codes (the
    add/sub/skip contraction of Foundry "Native Matmul Kernel" and Hetman-2b
    s.7, which is this integer matrix product), exact (see
    ``_exact_integer_product``).  Returns int64."""
    return _exact_integer_product(q, unpack_codes(packed, k))


def contract_rows(q: np.ndarray, packed: np.ndarray, k: int, rows) -> np.ndarray:
    """``contract`` restricted to the output rows ``rows`` -> int64 [M, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    return contract(q, np.asarray(packed)[rows], k)


def epilogue(acc: np.ndarray, gammas: np.ndarray, sx: np.ndarray,
             rows=None) -> np.ndarray:
    """y[m, o] = acc[m, o] * gamma_o * sx_m evaluated in fp64 from the exact
    accumulator (Foundry "How It Works" step 4: scale after the integer loop;
    Hetman-2b s.5/s.7 scale fusion).  ``gammas`` is one scale or one per row;
    ``rows`` selects the per-row scales of a column subset."""
    g = np.asarray(gammas, dtype=np.float64).ravel()
    if g.size > 1 and rows is not None:
        g = g[np.asarray(rows)]
    g = g.reshape(1, -1) if g.size > 1 else g.reshape(1, 1)
    s = np.asarray(sx, dtype=np.float64).reshape(-1, 1)
    return np.asarray(acc, dtype=np.float64) * g * s


def bf16_round_from_f64(y: np.ndarray) -> np.ndarray:
    """fp64 -> nearest fp32 -> nearest bf16 (ties to even), returned as fp32.
    Used only to state the bf16-output tolerance."""
    a = np.asarray(y, dtype=np.float64).astype(np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return bits.astype(np.uint32).view(np.float32)


def ternary_linear(X: np.ndarray, W: np.ndarray, granularity: str = "tensor",
                   mode: str = "ternary", prologue: bool = False):
    """Whole layer: pack W, quantise X (with the BitLinear prologue if asked),
    contract, rescale.  Returns a dict of every intermediate."""
    packed, gam = pack_ternary(W, granularity, mode)
    if prologue:
        q, sx = bitlinear_prologue(X)
    else:
        q, sx = quant_act_int8(X)
    k = np.asarray(W).shape[1]
    acc = contract(q, packed, k)
    y = epilogue(acc, gam, sx)
    return dict(packed=packed, scale=gam, q=q, sx=sx, acc=acc, y=y)


def backward_input(dY: np.ndarray, packed: np.ndarray, gammas: np.ndarray, k: int) -> np.ndarray:
    """dX[m, k] = sum_n dY[m, n] * gamma_n * w[n, k] in fp64 (Foundry
    "Backward Pass", fq_matmul_ternary_backward_input; gamma per tensor or
    per output row n).  The caller adds it to its accumulator."""
    w = unpack_codes(packed, k).astype(np.float64)
    g = np.asarray(gammas, dtype=np.float64)
    dYs = np.asarray(dY, dtype=np.float64) * (g if g.size > 1 else g[0])
    return dYs @ w


def backward_weight(X: np.ndarray, dY: np.ndarray) -> np.ndarray:
    """dW[n, k] = sum_m dY[m, n] * X[m, k] in fp64 (Foundry "Backward Pass",
    fq_matmul_ternary_backward_weight: the float product X^T dY, no scale),
    laid out [N, K] like the weight."""
    return np.asarray(dY, dtype=np.float64).T @ np.asarray(X, dtype=np.float64)


SWIGLU_CLAMP = 10.0           # Hetman-2b s.6 default clamp value


def swiglu_clamped(g: np.ndarray, u: np.ndarray, clamp_val: float = SWIGLU_CLAMP) -> np.ndarray:
    """h = clamp(silu(g) * u, -c, c) with silu(g) = g / (1 + exp(-g)), in fp64
    (Hetman-2b s.6 SwiGLUClamped: gate = SiLU(W_gate x), up = W_up x,
    clamped activation before W_down)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    silu = g / (1.0 + np.exp(-g))
    return np.clip(silu * u, -clamp_val, clamp_val)


def ffn_swiglu_decode(X: np.ndarray, gate, up, down, clamp_val: float = SWIGLU_CLAMP):
    """Decode FFN of ternary layers (Hetman-2b s.6 with the plain quantiser):
    gate, up and down are (packed, scales) pairs.  Returns (h fp64 [M, N_ffn],
    the gate and up outputs g, u, and y fp64 [M, d]) where the down
    projection quantises h per token exactly as ``quant_act_int8`` does."""
    X = np.asarray(X, dtype=np.float32)
    q, sx = quant_act_int8(X)
    k = X.shape[1]
    g = epilogue(contract(q, gate[0], k), gate[1], sx)
    u = epilogue(contract(q, up[0], k), up[1], sx)
    h = swiglu_clamped(g, u, clamp_val)
    hq, hs = quant_act_int8(h.astype(np.float32))
    y = epilogue(contract(hq, down[0], h.shape[1]), down[1], hs)
    return h, g, u, y


def exact_fraction_mean(w: np.ndarray) -> Fraction:
    """Mean of |w| as an exact Fraction (slow; for small arrays in tests)."""
    vals = [Fraction(float(abs(v))) for v in np.asarray(w, dtype=np.float32).ravel()]
    return sum(vals, Fraction(0)) / len(vals)
