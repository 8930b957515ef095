"""Python binding of libtq (argument marshalling only).

Each function has the name of the C entry point it calls and forwards torch
tensors as raw device pointers plus the current HIP stream; every step of the
computation runs in libtq's kernels.  PyTorch supplies device memory and
streams.  Importing this module fails if libtq.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m ternary_quantized_linear_absmean_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

# enums of include/tq.h
TQ_OK = 0
STATUS_NAMES = {0: "TQ_OK", 1: "TQ_ERR_NULL", 2: "TQ_ERR_SHAPE", 3: "TQ_ERR_DTYPE",
                4: "TQ_ERR_ALIGN", 5: "TQ_ERR_WORKSPACE", 6: "TQ_ERR_UNSUPPORTED",
                7: "TQ_ERR_HIP"}
DTYPES = {"f32": 0, "bf16": 1, "i32": 2}
GRANULARITY = {"tensor": 0, "row": 1}
MODES = {"ternary": 0, "binary": 1}
THRESHOLDS = {"relative": 0, "absolute": 1}
CODES = {"native": 0, "f0": 1, "f1": 2}
EXPORTED = ["tq_packed_bytes", "tq_pack_workspace_bytes", "tq_pack_ternary",
            "tq_pack_ternary_noalloc",
            "tq_quant_act_int8", "tq_fwht512", "tq_ternary_gemv", "tq_ternary_gemm",
            "tq_quant_ternary_gemv", "tq_packed1_bytes", "tq_pack_binary1",
            "tq_binary1_gemv", "tq_swiglu_gemv", "tq_ffn_swiglu_decode",
            "tq_ternary_backward_input", "tq_ternary_backward_weight",
            "tq_pack_ternary_threshold", "tq_convert_codes", "tq_unpack_codes", "tq_status_str",
            "tq_last_hip_error", "tq_version"]

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


class TqActOpts(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_float), ("clamp", _int), ("eta_min", ctypes.c_float),
                ("eta_max", ctypes.c_float), ("rmsnorm", _int), ("rms_eps", ctypes.c_float),
                ("rms_weight", _vp), ("fwht_block", _int)]


_lib.tq_packed_bytes.argtypes = [_i64]
_lib.tq_packed_bytes.restype = ctypes.c_size_t
_lib.tq_pack_workspace_bytes.argtypes = [_i64, _i64, _int]
_lib.tq_pack_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_pack_ternary.argtypes = [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.tq_pack_ternary.restype = _int
_lib.tq_pack_ternary_noalloc.argtypes = [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp]
_lib.tq_pack_ternary_noalloc.restype = _int
_lib.tq_quant_act_int8.argtypes = [_vp, _int, _i64, _i64, ctypes.POINTER(TqActOpts), _vp, _vp, _vp]
_lib.tq_quant_act_int8.restype = _int
_lib.tq_fwht512.argtypes = [_vp, _int, _i64, _i64, _int, _vp, _vp]
_lib.tq_fwht512.restype = _int
for _name in ("tq_ternary_gemv", "tq_ternary_gemm"):
    getattr(_lib, _name).argtypes = [_vp, _vp, _i64, _vp, _vp, _int, _i64, _i64, _vp, _int, _vp]
    getattr(_lib, _name).restype = _int
_lib.tq_quant_ternary_gemv.argtypes = [_vp, _int, _i64, ctypes.POINTER(TqActOpts), _vp, _vp,
                                       _int, _i64, _i64, _vp, _vp, _vp, _int, _vp]
_lib.tq_quant_ternary_gemv.restype = _int
_lib.tq_swiglu_gemv.argtypes = [_vp, _int, _i64, ctypes.POINTER(TqActOpts), _vp, _vp, _vp, _vp,
                                _int, _i64, _i64, ctypes.c_float, _vp, _vp, _vp, _int, _vp]
_lib.tq_swiglu_gemv.restype = _int
_lib.tq_ffn_swiglu_decode.argtypes = [_vp, _int, _i64, ctypes.POINTER(TqActOpts), _vp, _vp, _vp,
                                      _vp, _vp, _vp, _int, _i64, _i64, ctypes.c_float, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _int, _vp]
_lib.tq_ffn_swiglu_decode.restype = _int
_lib.tq_packed1_bytes.argtypes = [_i64]
_lib.tq_packed1_bytes.restype = ctypes.c_size_t
_lib.tq_pack_binary1.argtypes = [_vp, _i64, _i64, _int, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.tq_pack_binary1.restype = _int
_lib.tq_binary1_gemv.argtypes = [_vp, _vp, _i64, _vp, _vp, _int, _i64, _i64, _vp, _int, _vp]
_lib.tq_binary1_gemv.restype = _int
_lib.tq_ternary_backward_input.argtypes = [_vp, _int, _i64, _vp, _vp, _int, _i64, _i64, _vp,
                                           _int, _vp]
_lib.tq_ternary_backward_input.restype = _int
_lib.tq_ternary_backward_weight.argtypes = [_vp, _int, _vp, _int, _i64, _i64, _i64, _vp, _int,
                                            _vp]
_lib.tq_ternary_backward_weight.restype = _int
_lib.tq_pack_ternary_threshold.argtypes = [_vp, _i64, _i64, _int, _int, ctypes.c_float, _vp, _vp,
                                           _vp, ctypes.c_size_t, _vp]
_lib.tq_pack_ternary_threshold.restype = _int
_lib.tq_convert_codes.argtypes = [_vp, _int, _vp, _int, _i64, _vp]
_lib.tq_convert_codes.restype = _int
_lib.tq_unpack_codes.argtypes = [_vp, _int, _i64, _vp, _vp]
_lib.tq_unpack_codes.restype = _int
_lib.tq_status_str.argtypes = [_int]
_lib.tq_status_str.restype = ctypes.c_char_p
_lib.tq_last_hip_error.argtypes = []
_lib.tq_last_hip_error.restype = ctypes.c_char_p
_lib.tq_version.argtypes = []
_lib.tq_version.restype = ctypes.c_char_p


class TqError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = f"{call}: {STATUS_NAMES.get(status, status)} ({tq_status_str(status)})"
        if status == 7:
            msg += f" [{tq_last_hip_error()}]"
        super().__init__(msg)


def _check(status: int, call: str) -> None:
    if status != TQ_OK:
        raise TqError(status, call)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _arg(t, name: str, dtypes, shape=None, numel=None, like=None, min_numel=None) -> torch.Tensor:
    """Check one tensor argument before anything is launched: dtype, then
    exact shape or element count (or at least min_numel elements), then
    contiguity (`like` is accepted for symmetry; _devices checks placement).  The C entry points see raw pointers only, so a buffer
    of the wrong size or type would be read or written out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _devices(**tensors) -> None:
    """Every tensor argument is a device tensor, all on one device (checked
    after the dtype and size checks of _arg)."""
    first = None
    for name, t in tensors.items():
        if t is None:
            continue
        _dev(t, name)
        if first is None:
            first = t
        elif t.device != first.device:
            raise ValueError(f"{name} must be on {first.device}, got {t.device}")


def _enum(table: dict, value: str, name: str) -> int:
    if value not in table:
        raise ValueError(f"{name} must be one of {sorted(table)}, got {value!r}")
    return table[value]


def _scale_numel(granularity: str, N: int) -> int:
    return N if _enum(GRANULARITY, granularity, "granularity") == 1 else 1


_ACT_DT = {torch.float32: 0, torch.bfloat16: 1}
_Y_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}


# ------------------------------------------------------------------- sizes

def tq_packed_bytes(numel: int) -> int:
    return int(_lib.tq_packed_bytes(int(numel)))


def tq_pack_workspace_bytes(N: int, K: int, granularity: str = "tensor") -> int:
    return int(_lib.tq_pack_workspace_bytes(int(N), int(K), GRANULARITY[granularity]))


def tq_status_str(status: int) -> str:
    return _lib.tq_status_str(int(status)).decode()


def tq_last_hip_error() -> str:
    return _lib.tq_last_hip_error().decode()


def tq_version() -> str:
    return _lib.tq_version().decode()


# --------------------------------------------------------------- weights

def tq_pack_ternary(W: torch.Tensor, granularity: str = "tensor", mode: str = "ternary",
                    packed: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None):
    """W [N, K] fp32 -> (packed uint8 [N, K/4], scale fp32 [1] or [N])."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [N, K]")
    N, K = W.shape
    _arg(W, "W", torch.float32)
    ns = _scale_numel(granularity, N)
    _enum(MODES, mode, "mode")
    if packed is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((ns,), dtype=torch.float32, device=W.device)
    _arg(packed, "packed", torch.uint8, numel=N * (K // 4), like=W)
    _arg(scale, "scale", torch.float32, numel=ns, like=W)
    need = tq_pack_workspace_bytes(N, K, granularity)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=W.device)
    if workspace is not None:
        _arg(workspace, "workspace", torch.uint8, like=W)
        if workspace.numel() < need:
            raise ValueError(f"workspace must hold at least {need} bytes")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _devices(W=W, packed=packed, scale=scale, workspace=workspace)
    _check(_lib.tq_pack_ternary(W.data_ptr(), N, K, GRANULARITY[granularity], MODES[mode],
                                _ptr(packed), _ptr(scale), _ptr(workspace), ws_bytes,
                                _stream(stream)), "tq_pack_ternary")
    return packed, scale


def tq_pack_ternary_noalloc(W: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
                            granularity: str = "tensor", mode: str = "ternary", stream=None):
    """tq_pack_ternary with the library's static scratch instead of a
    workspace: the caller passes both outputs and nothing is allocated."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [N, K]")
    N, K = W.shape
    _arg(W, "W", torch.float32)
    ns = _scale_numel(granularity, N)
    _enum(MODES, mode, "mode")
    _arg(packed, "packed", torch.uint8, numel=N * (K // 4))
    _arg(scale, "scale", torch.float32, numel=ns)
    _devices(W=W, packed=packed, scale=scale)
    _check(_lib.tq_pack_ternary_noalloc(W.data_ptr(), N, K, GRANULARITY[granularity],
                                        MODES[mode], packed.data_ptr(), scale.data_ptr(),
                                        _stream(stream)), "tq_pack_ternary_noalloc")
    return packed, scale


def tq_packed1_bytes(numel: int) -> int:
    return int(_lib.tq_packed1_bytes(numel))


def tq_pack_binary1(W: torch.Tensor, granularity: str = "row",
                    packed: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None):
    """W [N, K] fp32 -> (packed uint8 [N, K/8] signs, scale fp32 [1] or [N])."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [N, K]")
    N, K = W.shape
    _arg(W, "W", torch.float32)
    ns = _scale_numel(granularity, N)
    if packed is None:
        packed = torch.empty((N, K // 8), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((ns,), dtype=torch.float32, device=W.device)
    _arg(packed, "packed", torch.uint8, numel=N * (K // 8), like=W)
    _arg(scale, "scale", torch.float32, numel=ns, like=W)
    need = tq_pack_workspace_bytes(N, K, granularity)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=W.device)
    if workspace is not None:
        _arg(workspace, "workspace", torch.uint8, like=W)
        if workspace.numel() < need:
            raise ValueError(f"workspace must hold at least {need} bytes")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _devices(W=W, packed=packed, scale=scale, workspace=workspace)
    _check(_lib.tq_pack_binary1(W.data_ptr(), N, K, GRANULARITY[granularity], _ptr(packed),
                                _ptr(scale), _ptr(workspace), ws_bytes, _stream(stream)),
           "tq_pack_binary1")
    return packed, scale


# ------------------------------------------------------------ activations

def _act_in(X, name="X"):
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor [M, K]")
    _arg(X, name, tuple(_ACT_DT))
    return X.shape


def _opts(eps, clamp, rmsnorm, rms_eps, rms_weight, fwht_block, K=None, like=None) -> TqActOpts:
    if rms_weight is not None:
        _arg(rms_weight, "rms_weight", torch.float32, numel=K, like=like)
    return TqActOpts(eps=eps, clamp=1 if clamp else 0,
                     eta_min=clamp[0] if clamp else 0.0, eta_max=clamp[1] if clamp else 0.0,
                     rmsnorm=1 if rmsnorm else 0, rms_eps=rms_eps,
                     rms_weight=_ptr(rms_weight), fwht_block=fwht_block)


def tq_quant_act_int8(X: torch.Tensor, eps: float = 1e-6, clamp=None, rmsnorm: bool = False,
                      rms_eps: float = 1e-6, rms_weight: torch.Tensor | None = None,
                      fwht_block: int = 0, q: torch.Tensor | None = None,
                      sx: torch.Tensor | None = None, stream=None):
    """X [M, K] fp32/bf16 -> (q int8 [M, K], sx fp32 [M]).  ``clamp`` is an
    (eta_min, eta_max) pair or None."""
    M, K = _act_in(X)
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    _arg(q, "q", torch.int8, shape=(M, K), like=X)
    _arg(sx, "sx", torch.float32, numel=M, like=X)
    opts = _opts(eps, clamp, rmsnorm, rms_eps, rms_weight, fwht_block, K, X)
    _devices(X=X, q=q, sx=sx, rms_weight=rms_weight)
    _check(_lib.tq_quant_act_int8(X.data_ptr(), _ACT_DT[X.dtype], M, K, ctypes.byref(opts),
                                  _ptr(q), _ptr(sx), _stream(stream)), "tq_quant_act_int8")
    return q, sx


def tq_fwht512(X: torch.Tensor, normalize: bool = True, Y: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Blockwise FWHT-512 along the last axis of X [M, K] -> fp32 [M, K]."""
    M, K = _act_in(X)
    if Y is None:
        Y = torch.empty((M, K), dtype=torch.float32, device=X.device)
    _arg(Y, "Y", torch.float32, shape=(M, K), like=X)
    _devices(X=X, Y=Y)
    _check(_lib.tq_fwht512(X.data_ptr(), _ACT_DT[X.dtype], M, K, 1 if normalize else 0,
                           _ptr(Y), _stream(stream)), "tq_fwht512")
    return Y


# ------------------------------------------------------------ contraction

def _contract(fn, name, q, sx, packed, scale, N, K, granularity, out_dtype, Y, stream,
              bits=2):
    if not isinstance(q, torch.Tensor) or q.dim() != 2:
        raise ValueError("q must be a 2-D tensor [M, K]")
    M = q.shape[0]
    _arg(q, "q", torch.int8, shape=(M, K))
    _arg(sx, "sx", torch.float32, numel=M, like=q)
    _arg(packed, "packed", torch.uint8, min_numel=N * (K * bits // 8), like=q)
    _arg(scale, "scale", torch.float32, min_numel=_scale_numel(granularity, N), like=q)
    ydt = _enum(DTYPES, out_dtype, "out_dtype")
    if Y is None:
        Y = torch.empty((M, N), dtype=_Y_TORCH[out_dtype], device=q.device)
    _arg(Y, "Y", _Y_TORCH[out_dtype], shape=(M, N), like=q)
    _devices(q=q, sx=sx, packed=packed, scale=scale, Y=Y)
    _check(fn(q.data_ptr(), sx.data_ptr(), M, packed.data_ptr(), scale.data_ptr(),
              GRANULARITY[granularity], N, K, _ptr(Y), ydt, _stream(stream)),
           name)
    return Y


def tq_ternary_gemv(q, sx, packed, scale, N: int, K: int, granularity: str = "tensor",
                    out_dtype: str = "f32", Y=None, stream=None) -> torch.Tensor:
    """y = (q @ W^T) * scale * sx for M <= 16 tokens -> [M, N]."""
    return _contract(_lib.tq_ternary_gemv, "tq_ternary_gemv", q, sx, packed, scale, N, K,
                     granularity, out_dtype, Y, stream)


def tq_binary1_gemv(q, sx, packed, scale, N: int, K: int, granularity: str = "row",
                    out_dtype: str = "f32", Y=None, stream=None) -> torch.Tensor:
    """tq_ternary_gemv with 1-bit sign-packed weights (packed [N, K/8])."""
    return _contract(_lib.tq_binary1_gemv, "tq_binary1_gemv", q, sx, packed, scale, N, K,
                     granularity, out_dtype, Y, stream, bits=1)


def tq_ternary_gemm(q, sx, packed, scale, N: int, K: int, granularity: str = "tensor",
                    out_dtype: str = "f32", Y=None, stream=None) -> torch.Tensor:
    """Same contract as tq_ternary_gemv for any number of tokens."""
    return _contract(_lib.tq_ternary_gemm, "tq_ternary_gemm", q, sx, packed, scale, N, K,
                     granularity, out_dtype, Y, stream)


def tq_quant_ternary_gemv(X: torch.Tensor, packed, scale, N: int, K: int,
                          granularity: str = "tensor", out_dtype: str = "f32", eps: float = 1e-6,
                          clamp=None, rmsnorm: bool = False, rms_eps: float = 1e-6,
                          rms_weight: torch.Tensor | None = None, fwht_block: int = 0,
                          q: torch.Tensor | None = None, sx: torch.Tensor | None = None,
                          Y: torch.Tensor | None = None, stream=None):
    """Quantise X [M, K] (M <= 16) and apply the decode GEMV in one call ->
    (Y [M, N], q int8 [M, K], sx fp32 [M])."""
    M, KX = _act_in(X)
    if KX != K:
        raise ValueError(f"X must have K = {K} columns, got {KX}")
    _arg(packed, "packed", torch.uint8, min_numel=N * (K // 4), like=X)
    _arg(scale, "scale", torch.float32, min_numel=_scale_numel(granularity, N), like=X)
    _enum(DTYPES, out_dtype, "out_dtype")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    if Y is None:
        Y = torch.empty((M, N), dtype=_Y_TORCH[out_dtype], device=X.device)
    _arg(q, "q", torch.int8, shape=(M, K), like=X)
    _arg(sx, "sx", torch.float32, numel=M, like=X)
    _arg(Y, "Y", _Y_TORCH[out_dtype], shape=(M, N), like=X)
    opts = _opts(eps, clamp, rmsnorm, rms_eps, rms_weight, fwht_block, K, X)
    _devices(X=X, packed=packed, scale=scale, q=q, sx=sx, Y=Y, rms_weight=rms_weight)
    _check(_lib.tq_quant_ternary_gemv(X.data_ptr(), _ACT_DT[X.dtype], M, ctypes.byref(opts),
                                      packed.data_ptr(), scale.data_ptr(),
                                      GRANULARITY[granularity], N, K, _ptr(q), _ptr(sx),
                                      _ptr(Y), DTYPES[out_dtype], _stream(stream)),
           "tq_quant_ternary_gemv")
    return Y, q, sx


def tq_swiglu_gemv(X: torch.Tensor, packed_gate, scale_gate, packed_up, scale_up, N: int,
                   K: int, granularity: str = "row", clamp_val: float = 10.0,
                   out_dtype: str = "f32", eps: float = 1e-6, clamp=None, rmsnorm: bool = False,
                   rms_eps: float = 1e-6, rms_weight: torch.Tensor | None = None,
                   fwht_block: int = 0, q: torch.Tensor | None = None,
                   sx: torch.Tensor | None = None, H: torch.Tensor | None = None, stream=None):
    """Gate and up projections of X [M, K] (M <= 16) with the SwiGLU-clamp
    epilogue -> (H [M, N], q int8 [M, K], sx fp32 [M])."""
    M, KX = _act_in(X)
    if KX != K:
        raise ValueError(f"X must have K = {K} columns, got {KX}")
    ns = _scale_numel(granularity, N)
    for t, name in ((packed_gate, "packed_gate"), (packed_up, "packed_up")):
        _arg(t, name, torch.uint8, min_numel=N * (K // 4), like=X)
    for t, name in ((scale_gate, "scale_gate"), (scale_up, "scale_up")):
        _arg(t, name, torch.float32, min_numel=ns, like=X)
    _enum(DTYPES, out_dtype, "out_dtype")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=X.device)
    if H is None:
        H = torch.empty((M, N), dtype=_Y_TORCH[out_dtype], device=X.device)
    _arg(q, "q", torch.int8, shape=(M, K), like=X)
    _arg(sx, "sx", torch.float32, numel=M, like=X)
    _arg(H, "H", _Y_TORCH[out_dtype], shape=(M, N), like=X)
    opts = _opts(eps, clamp, rmsnorm, rms_eps, rms_weight, fwht_block, K, X)
    _devices(X=X, packed_gate=packed_gate, scale_gate=scale_gate, packed_up=packed_up,
             scale_up=scale_up, q=q, sx=sx, H=H, rms_weight=rms_weight)
    _check(_lib.tq_swiglu_gemv(X.data_ptr(), _ACT_DT[X.dtype], M, ctypes.byref(opts),
                               packed_gate.data_ptr(), scale_gate.data_ptr(),
                               packed_up.data_ptr(), scale_up.data_ptr(),
                               GRANULARITY[granularity], N, K, clamp_val, _ptr(q), _ptr(sx),
                               _ptr(H), DTYPES[out_dtype], _stream(stream)), "tq_swiglu_gemv")
    return H, q, sx


def tq_ffn_swiglu_decode(X: torch.Tensor, gate, up, down, d_model: int, d_ffn: int,
                         granularity: str = "row", clamp_val: float = 10.0,
                         out_dtype: str = "f32", eps: float = 1e-6, clamp=None,
                         buffers: dict | None = None, Y: torch.Tensor | None = None,
                         stream=None):
    """Decode FFN: gate, up, down are (packed, scale) pairs.  Returns
    (Y [M, d_model], buffers) where buffers holds q_x, sx_x, H, q_h, sx_h."""
    M, KX = _act_in(X)
    if KX != d_model:
        raise ValueError(f"X must have d_model = {d_model} columns, got {KX}")
    ns_f, ns_m = _scale_numel(granularity, d_ffn), _scale_numel(granularity, d_model)
    for (pk, sc), name, nrow, ncol, ns in ((gate, "gate", d_ffn, d_model, ns_f),
                                           (up, "up", d_ffn, d_model, ns_f),
                                           (down, "down", d_model, d_ffn, ns_m)):
        _arg(pk, f"{name} packed", torch.uint8, min_numel=nrow * (ncol // 4), like=X)
        _arg(sc, f"{name} scale", torch.float32, min_numel=ns, like=X)
    _enum(DTYPES, out_dtype, "out_dtype")
    b = dict(buffers or {})
    dv = X.device
    b.setdefault("q_x", torch.empty((M, d_model), dtype=torch.int8, device=dv))
    b.setdefault("sx_x", torch.empty((M,), dtype=torch.float32, device=dv))
    b.setdefault("H", torch.empty((M, d_ffn), dtype=torch.float32, device=dv))
    b.setdefault("q_h", torch.empty((M, d_ffn), dtype=torch.int8, device=dv))
    b.setdefault("sx_h", torch.empty((M,), dtype=torch.float32, device=dv))
    if Y is None:
        Y = torch.empty((M, d_model), dtype=_Y_TORCH[out_dtype], device=dv)
    for key, dt, shp in (("q_x", torch.int8, (M, d_model)), ("sx_x", torch.float32, (M,)),
                         ("H", torch.float32, (M, d_ffn)), ("q_h", torch.int8, (M, d_ffn)),
                         ("sx_h", torch.float32, (M,))):
        _arg(b[key], key, dt, shape=shp, like=X)
    _arg(Y, "Y", _Y_TORCH[out_dtype], shape=(M, d_model), like=X)
    opts = _opts(eps, clamp, False, 1e-6, None, 0)
    _devices(X=X, gate_packed=gate[0], gate_scale=gate[1], up_packed=up[0], up_scale=up[1],
             down_packed=down[0], down_scale=down[1], Y=Y, **b)
    _check(_lib.tq_ffn_swiglu_decode(
        X.data_ptr(), _ACT_DT[X.dtype], M, ctypes.byref(opts), gate[0].data_ptr(),
        gate[1].data_ptr(), up[0].data_ptr(), up[1].data_ptr(), down[0].data_ptr(),
        down[1].data_ptr(), GRANULARITY[granularity], d_model, d_ffn, clamp_val,
        _ptr(b["q_x"]), _ptr(b["sx_x"]), _ptr(b["H"]), _ptr(b["q_h"]), _ptr(b["sx_h"]),
        _ptr(Y), DTYPES[out_dtype], _stream(stream)), "tq_ffn_swiglu_decode")
    return Y, b


def tq_ternary_backward_input(dY: torch.Tensor, packed, scale, K: int,
                              granularity: str = "tensor", dX: torch.Tensor | None = None,
                              accumulate: bool = False, stream=None) -> torch.Tensor:
    """dX [M, K] fp32 = (dY [M, N] * gamma) contracted with the packed codes
    over N; with accumulate the result is added to the given dX."""
    M, N = _act_in(dY, "dY")
    _arg(packed, "packed", torch.uint8, min_numel=N * (K // 4), like=dY)
    _arg(scale, "scale", torch.float32, min_numel=_scale_numel(granularity, N), like=dY)
    if dX is None:
        if accumulate:
            raise ValueError("accumulate needs dX")
        dX = torch.empty((M, K), dtype=torch.float32, device=dY.device)
    _arg(dX, "dX", torch.float32, shape=(M, K), like=dY)
    _devices(dY=dY, packed=packed, scale=scale, dX=dX)
    _check(_lib.tq_ternary_backward_input(dY.data_ptr(), _ACT_DT[dY.dtype], M,
                                          packed.data_ptr(), scale.data_ptr(),
                                          GRANULARITY[granularity], N, K, dX.data_ptr(),
                                          1 if accumulate else 0, _stream(stream)),
           "tq_ternary_backward_input")
    return dX


def tq_ternary_backward_weight(X: torch.Tensor, dY: torch.Tensor, dW: torch.Tensor | None = None,
                               accumulate: bool = False, stream=None) -> torch.Tensor:
    """dW [N, K] fp32 = dY^T X over the M tokens; with accumulate the result
    is added to the given dW."""
    M, K = _act_in(X)
    MY, N = _act_in(dY, "dY")
    if MY != M:
        raise ValueError("X and dY must have the same number of rows")
    if dW is None:
        if accumulate:
            raise ValueError("accumulate needs dW")
        dW = torch.empty((N, K), dtype=torch.float32, device=X.device)
    _arg(dW, "dW", torch.float32, shape=(N, K), like=X)
    _devices(X=X, dY=dY, dW=dW)
    _check(_lib.tq_ternary_backward_weight(X.data_ptr(), _ACT_DT[X.dtype], dY.data_ptr(),
                                           _ACT_DT[dY.dtype], M, N, K, dW.data_ptr(),
                                           1 if accumulate else 0, _stream(stream)),
           "tq_ternary_backward_weight")
    return dW


def tq_pack_ternary_threshold(W: torch.Tensor, granularity: str = "tensor",
                              kind: str = "relative", value: float = 0.55,
                              packed: torch.Tensor | None = None,
                              scale: torch.Tensor | None = None, stream=None):
    """Threshold ternarization + 2-bit packing of W [N, K] fp32 -> (packed
    uint8 [N, K/4], scale fp32 [1] or [N])."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [N, K]")
    N, K = W.shape
    _arg(W, "W", torch.float32)
    ns = _scale_numel(granularity, N)
    _enum(THRESHOLDS, kind, "kind")
    if packed is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((ns,), dtype=torch.float32, device=W.device)
    _arg(packed, "packed", torch.uint8, numel=N * (K // 4), like=W)
    _arg(scale, "scale", torch.float32, numel=ns, like=W)
    nws = tq_pack_workspace_bytes(N, K, granularity)
    ws = torch.empty((max(nws, 8),), dtype=torch.uint8, device=W.device)
    _devices(W=W, packed=packed, scale=scale)
    _check(_lib.tq_pack_ternary_threshold(W.data_ptr(), N, K, GRANULARITY[granularity],
                                          THRESHOLDS[kind], value, packed.data_ptr(),
                                          scale.data_ptr(), ws.data_ptr(), ws.numel(),
                                          _stream(stream)), "tq_pack_ternary_threshold")
    return packed, scale


def tq_convert_codes(src: torch.Tensor, src_fmt: str, dst_fmt: str,
                     dst: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Re-encode packed codes (uint8, any shape) from one format to another."""
    _dev(src, "src")
    if src.dtype != torch.uint8:
        raise ValueError("src must be uint8")
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, "dst")
    if dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("dst must be uint8 with src's size")
    _enum(CODES, src_fmt, "src_fmt")
    _enum(CODES, dst_fmt, "dst_fmt")
    _check(_lib.tq_convert_codes(src.data_ptr(), CODES[src_fmt], dst.data_ptr(), CODES[dst_fmt],
                                 src.numel(), _stream(stream)), "tq_convert_codes")
    return dst


def tq_unpack_codes(packed: torch.Tensor, fmt: str, numel: int,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Values -1/0/+1 (int8, numel of them) of packed codes in a format."""
    _dev(packed, "packed")
    if packed.dtype != torch.uint8 or packed.numel() * 4 < numel:
        raise ValueError("packed must be uint8 with at least ceil(numel/4) bytes")
    if out is None:
        out = torch.empty((numel,), dtype=torch.int8, device=packed.device)
    _dev(out, "out")
    if out.dtype != torch.int8 or out.numel() != numel:
        raise ValueError("out must be int8 with numel elements")
    _enum(CODES, fmt, "fmt")
    _check(_lib.tq_unpack_codes(packed.data_ptr(), CODES[fmt], numel, out.data_ptr(),
                                _stream(stream)), "tq_unpack_codes")
    return out


def raw_library() -> ctypes.CDLL:
    """The loaded libtq handle (for tests of the C ABI itself)."""
    return _lib
