"""The C ABI on the CPU: the library loads, exports what include/tq.h
declares, and rejects bad arguments before touching HIP.

No call here can reach a kernel launch: each one fails validation or is an
empty (M == 0 / N == 0) call, which returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

tqmod = pytest.importorskip("ternary_quantized_linear_absmean_amd.tq",
                            reason="libtq.so not built")
lib = tqmod.raw_library()

OK, NULL, SHAPE, DTYPE, ALIGN, WS, UNSUP = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(tqmod.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_packed_bytes_and_workspace():
    assert tqmod.tq_packed_bytes(4096 * 4096) == 4194304
    assert tqmod.tq_packed_bytes(256) == 64
    assert [tqmod.tq_packed_bytes(n) for n in range(0, 10)] == [0, 1, 1, 1, 1, 2, 2, 2, 2, 3]
    assert tqmod.tq_packed_bytes(-5) == 0
    assert tqmod.tq_pack_workspace_bytes(4096, 4096, "tensor") > 0
    assert tqmod.tq_pack_workspace_bytes(4096, 4096, "row") == 0
    assert tqmod.tq_pack_workspace_bytes(4, 6, "tensor") == 0


def test_status_strings():
    for s in range(8):
        assert tqmod.tq_status_str(s)
    assert tqmod.tq_status_str(99) == "unknown status"
    assert tqmod.tq_version() == "0.1.0"
    assert tqmod.tq_last_hip_error() == "hipSuccess"


def _gemv(*a):
    return lib.tq_ternary_gemv(*a)


def _gemm(*a):
    return lib.tq_ternary_gemm(*a)


def _gemv1(*a):
    return lib.tq_binary1_gemv(*a)


@pytest.mark.parametrize("fn", [_gemv, _gemm, _gemv1])
def test_contract_validation(fn):
    P = 0x10000  # never dereferenced: every call below fails validation
    # shapes
    assert fn(P, P, -1, P, P, 0, 16, 64, P, 0, None) == SHAPE
    assert fn(P, P, 1, P, P, 0, -1, 64, P, 0, None) == SHAPE
    assert fn(P, P, 1, P, P, 0, 16, 0, P, 0, None) == SHAPE
    assert fn(P, P, 1, P, P, 0, 16, 62, P, 0, None) == SHAPE
    # enums
    assert fn(P, P, 1, P, P, 2, 16, 64, P, 0, None) == UNSUP
    assert fn(P, P, 1, P, P, 0, 16, 64, P, 3, None) == DTYPE
    # K beyond the int32 headroom of 127 * K < 2^24
    assert fn(P, P, 1, P, P, 0, 16, 132112, P, 0, None) == UNSUP
    # NULL pointers with a non-empty problem
    assert fn(None, P, 1, P, P, 0, 16, 64, P, 0, None) == NULL
    assert fn(P, None, 1, P, P, 0, 16, 64, P, 0, None) == NULL
    assert fn(P, P, 1, None, P, 0, 16, 64, P, 0, None) == NULL
    assert fn(P, P, 1, P, None, 0, 16, 64, P, 0, None) == NULL
    assert fn(P, P, 1, P, P, 0, 16, 64, None, 0, None) == NULL
    # misaligned fp32 pointers
    assert fn(P, P + 1, 1, P, P, 0, 16, 64, P, 0, None) == ALIGN
    assert fn(P, P, 1, P, P + 2, 0, 16, 64, P, 0, None) == ALIGN
    assert fn(P, P, 1, P, P, 0, 16, 64, P + 2, 0, None) == ALIGN
    assert fn(P, P, 1, P, P, 0, 16, 64, P + 1, 1, None) == ALIGN
    # empty problems are valid no-ops, even with NULL pointers
    assert fn(None, None, 0, None, None, 0, 16, 64, None, 0, None) == OK
    assert fn(None, None, 1, None, None, 0, 0, 64, None, 0, None) == OK


def test_gemv_token_limit():
    P = 0x10000
    assert _gemv(P, P, 17, P, P, 0, 16, 64, P, 0, None) == SHAPE
    # the GEMM has no such limit: same call fails only on the NULL Y
    assert _gemm(P, P, 17, P, P, 0, 16, 64, None, 0, None) == NULL


def test_binary1_validation():
    P = 0x10000
    # 1-bit rows are whole bytes: K % 8
    assert _gemv1(P, P, 1, P, P, 0, 16, 12, P, 0, None) == SHAPE
    assert _gemv1(P, P, 17, P, P, 0, 16, 64, P, 0, None) == SHAPE
    f = lib.tq_pack_binary1
    assert f(P, 4, 12, 0, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, -1, 64, 0, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, 4, 64, 5, P, P, P, 1 << 20, None) == UNSUP
    assert f(None, 4, 64, 1, P, P, None, 0, None) == NULL
    assert f(P, 4, 64, 0, P, P, None, 1 << 20, None) == WS
    assert f(P + 2, 4, 64, 1, P, P, None, 0, None) == ALIGN
    assert f(None, 0, 64, 1, None, None, None, 0, None) == OK
    assert tqmod.tq_packed1_bytes(0) == 0
    assert tqmod.tq_packed1_bytes(2048 * 2048) == 2048 * 2048 // 8
    assert tqmod.tq_packed1_bytes(9) == 2


def test_backward_input_validation():
    P = 0x10000
    f = lib.tq_ternary_backward_input
    # (dY, dydt, M, packed, scale, g, N, K, dX, accumulate, stream)
    assert f(P, 0, 4, P, P, 0, 8, 6, P, 0, None) == SHAPE          # K % 4
    assert f(P, 0, 4, P, P, 0, 8, 0, P, 0, None) == SHAPE          # K <= 0
    assert f(P, 0, -1, P, P, 0, 8, 64, P, 0, None) == SHAPE
    assert f(P, 0, 4, P, P, 0, -8, 64, P, 0, None) == SHAPE
    assert f(P, 2, 4, P, P, 0, 8, 64, P, 0, None) == DTYPE         # int32 dY
    assert f(P, 0, 4, P, P, 7, 8, 64, P, 0, None) == UNSUP
    assert f(P, 0, 4, P, P, 0, 8, 64, None, 0, None) == NULL
    assert f(None, 0, 4, P, P, 0, 8, 64, P, 0, None) == NULL
    assert f(P, 0, 4, None, P, 1, 8, 64, P, 0, None) == NULL
    assert f(P, 0, 4, P, None, 1, 8, 64, P, 0, None) == NULL
    assert f(P + 2, 0, 4, P, P, 0, 8, 64, P, 0, None) == ALIGN     # fp32 dY
    assert f(P, 0, 4, P, P, 0, 8, 64, P + 2, 0, None) == ALIGN     # dX
    assert f(P, 0, 4, P, P + 1, 0, 8, 64, P, 0, None) == ALIGN     # scale
    assert f(None, 0, 0, None, None, 0, 8, 64, None, 0, None) == OK  # M == 0


def test_backward_weight_validation():
    P = 0x10000
    f = lib.tq_ternary_backward_weight
    # (X, xdt, dY, dydt, M, N, K, dW, accumulate, stream)
    assert f(P, 0, P, 0, -1, 8, 8, P, 0, None) == SHAPE
    assert f(P, 0, P, 0, 4, -8, 8, P, 0, None) == SHAPE
    assert f(P, 0, P, 0, 4, 8, -8, P, 0, None) == SHAPE
    assert f(P, 2, P, 0, 4, 8, 8, P, 0, None) == DTYPE
    assert f(P, 0, P, 2, 4, 8, 8, P, 0, None) == DTYPE
    assert f(P, 0, P, 0, 4, 8, 8, None, 0, None) == NULL
    assert f(None, 0, P, 0, 4, 8, 8, P, 0, None) == NULL
    assert f(P, 0, None, 0, 4, 8, 8, P, 0, None) == NULL
    assert f(P + 2, 0, P, 0, 4, 8, 8, P, 0, None) == ALIGN
    assert f(P, 0, P + 2, 0, 4, 8, 8, P, 0, None) == ALIGN
    assert f(P, 0, P, 0, 4, 8, 8, P + 1, 0, None) == ALIGN
    assert f(None, 0, None, 0, 4, 0, 8, None, 0, None) == OK   # empty dW


def test_threshold_and_format_validation():
    P = 0x10000
    f = lib.tq_pack_ternary_threshold
    # (W, N, K, g, kind, value, packed, scale, ws, ws_bytes, stream)
    assert f(P, 4, 6, 0, 0, 0.55, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, 4, 64, 0, 2, 0.55, P, P, P, 1 << 20, None) == UNSUP       # unknown kind
    assert f(P, 4, 64, 0, 0, -0.1, P, P, P, 1 << 20, None) == UNSUP       # negative factor
    assert f(P, 4, 64, 0, 0, float("nan"), P, P, P, 1 << 20, None) == UNSUP
    assert f(P, 4, 64, 1, 1, 0.05, P, P, None, 0, None) == UNSUP          # manual per row
    assert f(P, 4, 64, 0, 1, 0.0, P, P, None, 0, None) == UNSUP           # manual t = 0
    assert f(P, 4, 64, 0, 0, 0.55, P, P, None, 0, None) == WS             # tensor needs ws
    assert f(None, 4, 64, 1, 0, 0.55, P, P, None, 0, None) == NULL
    assert f(P + 2, 4, 64, 1, 0, 0.55, P, P, None, 0, None) == ALIGN
    assert f(None, 0, 64, 1, 0, 0.55, None, None, None, 0, None) == OK
    g = lib.tq_convert_codes
    assert g(P, 0, P, 1, -1, None) == SHAPE
    assert g(P, 3, P, 1, 16, None) == UNSUP
    assert g(P, 0, P, 7, 16, None) == UNSUP
    assert g(None, 0, P, 1, 16, None) == NULL
    assert g(None, 0, None, 1, 0, None) == OK
    u = lib.tq_unpack_codes
    assert u(P, 0, -4, P, None) == SHAPE
    assert u(P, 5, 4, P, None) == UNSUP
    assert u(P, 1, 4, None, None) == NULL
    assert u(None, 2, 0, None, None) == OK


def test_swiglu_validation():
    P = 0x10000
    f = lib.tq_swiglu_gemv
    opts = None
    # (X, xdt, M, opts, pg, sg, pu, su, g, N, K, clamp, q, sx, H, hdt, stream)
    assert f(P, 1, 17, opts, P, P, P, P, 1, 16, 64, 10.0, P, P, P, 0, None) == SHAPE
    assert f(P, 1, 1, opts, P, P, P, P, 1, 16, 64, 10.0, P, P, P, 2, None) == DTYPE   # int32 H
    assert f(P, 1, 1, opts, P, P, P, P, 1, 16, 64, 0.0, P, P, P, 0, None) == UNSUP
    assert f(P, 1, 1, opts, P, P, P, P, 1, 16, 64, float("inf"), P, P, P, 0, None) == UNSUP
    assert f(P, 1, 1, opts, P, P, None, P, 1, 16, 64, 10.0, P, P, P, 0, None) == NULL
    assert f(P, 1, 1, opts, P, P, P, P + 2, 1, 16, 64, 10.0, P, P, P, 0, None) == ALIGN
    assert f(P, 1, 1, opts, P, P, P, P, 1, 16, 62, 10.0, P, P, P, 0, None) == SHAPE
    assert f(None, 1, 0, opts, None, None, None, None, 1, 16, 64, 10.0, None, None, None, 0,
             None) == OK
    d = lib.tq_ffn_swiglu_decode
    # (X, xdt, M, opts, pg, sg, pu, su, pd, sd, g, d_model, d_ffn, clamp,
    #  q_x, sx_x, H, q_h, sx_h, Y, ydt, stream): a bad down stage fails before launch
    assert d(P, 1, 1, None, P, P, P, P, None, P, 1, 64, 128, 10.0, P, P, P, P, P, P, 0,
             None) == NULL
    assert d(P, 1, 1, None, P, P, P, P, P, P, 1, 64, 128, 10.0, P, P, P, P, P, P, 3,
             None) == DTYPE
    assert d(P, 1, 1, None, P, P, P, P, P, P, 1, 64, 128, 10.0, P, P, P + 2, P, P, P, 0,
             None) == ALIGN


def test_pack_validation():
    P = 0x10000
    f = lib.tq_pack_ternary
    assert f(P, -1, 64, 0, 0, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, 4, 0, 0, 0, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, 4, 6, 0, 0, P, P, P, 1 << 20, None) == SHAPE
    assert f(P, 4, 64, 5, 0, P, P, P, 1 << 20, None) == UNSUP
    assert f(P, 4, 64, 0, 7, P, P, P, 1 << 20, None) == UNSUP
    assert f(P, 1 << 20, 1 << 20, 0, 0, P, P, P, 1 << 20, None) == UNSUP   # 2^40 values
    assert f(None, 4, 64, 0, 0, P, P, P, 1 << 20, None) == NULL
    assert f(P, 4, 64, 0, 0, None, P, P, 1 << 20, None) == NULL
    assert f(P, 4, 64, 0, 0, P, None, P, 1 << 20, None) == NULL
    assert f(P + 2, 4, 64, 0, 0, P, P, P, 1 << 20, None) == ALIGN
    assert f(P, 4, 64, 0, 0, P, P + 1, P, 1 << 20, None) == ALIGN
    assert f(P, 4, 64, 0, 0, P, P, None, 1 << 20, None) == WS
    assert f(P, 4, 64, 0, 0, P, P, P, 16, None) == WS
    assert f(P, 4, 64, 0, 0, P, P, P + 4, 1 << 20, None) == ALIGN
    assert f(None, 0, 64, 0, 0, None, None, None, 0, None) == OK


def test_quant_validation():
    P = 0x10000
    f = lib.tq_quant_act_int8
    O = tqmod.TqActOpts
    assert f(P, 0, -1, 64, None, P, P, None) == SHAPE
    assert f(P, 0, 1, 0, None, P, P, None) == SHAPE
    assert f(P, 2, 1, 64, None, P, P, None) == DTYPE
    assert f(None, 0, 1, 64, None, P, P, None) == NULL
    assert f(P, 0, 1, 64, None, None, P, None) == NULL
    assert f(P, 0, 1, 64, None, P, None, None) == NULL
    assert f(P + 2, 0, 1, 64, None, P, P, None) == ALIGN
    assert f(P + 1, 1, 1, 64, None, P, P, None) == ALIGN
    assert f(P, 0, 1, 64, None, P, P + 2, None) == ALIGN
    assert f(None, 0, 0, 64, None, None, None, None) == OK

    def opts(**kw):
        base = dict(eps=1e-6, clamp=0, eta_min=0.0, eta_max=0.0, rmsnorm=0, rms_eps=1e-6,
                    rms_weight=None, fwht_block=0)
        base.update(kw)
        return O(**base)
    import ctypes
    r = lambda o, K=512: f(P, 0, 1, K, ctypes.byref(o), P, P, None)
    assert r(opts(fwht_block=256)) == UNSUP
    assert r(opts(fwht_block=512), K=1000) == SHAPE
    assert r(opts(eps=0.0)) == UNSUP
    assert r(opts(eps=float("nan"))) == UNSUP
    assert r(opts(clamp=1, eta_min=0.0, eta_max=40.0)) == UNSUP
    assert r(opts(clamp=1, eta_min=50.0, eta_max=40.0)) == UNSUP
    assert r(opts(rmsnorm=1, rms_eps=-1.0)) == UNSUP
    assert r(opts(rmsnorm=1), K=65536) == UNSUP
    assert r(opts(rmsnorm=1, rms_weight=P + 2)) == ALIGN


def test_fwht_validation():
    P = 0x10000
    f = lib.tq_fwht512
    assert f(P, 0, 1, 500, 1, P, None) == SHAPE
    assert f(P, 0, -1, 512, 1, P, None) == SHAPE
    assert f(P, 3, 1, 512, 1, P, None) == DTYPE
    assert f(None, 0, 1, 512, 1, P, None) == NULL
    assert f(P, 0, 1, 512, 1, None, None) == NULL
    assert f(P + 2, 0, 1, 512, 1, P, None) == ALIGN
    assert f(P, 0, 1, 512, 1, P + 2, None) == ALIGN
    assert f(None, 0, 0, 512, 1, None, None) == OK


def test_product_path_has_no_cpu_fallback():
    # nothing in the package imports the oracle or computes on the host
    pkg = os.path.join(ROOT, "ternary_quantized_linear_absmean_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), fn
            assert "numpy" not in src, fn


# ------------------------------------------------ binding argument checks

torch = pytest.importorskip("torch")


def _raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_binding_contraction_checks_every_buffer():
    # host tensors: the shape and dtype checks run first, so each mismatch
    # below is reported before the device check (which a correct host tensor
    # reaches last); nothing is ever launched
    i8, f32, u8 = torch.int8, torch.float32, torch.uint8
    q, sx, pk, sc = _t((2, 64), i8), _t((2,), f32), _t((10, 16), u8), _t((1,), f32)
    for fn in (tqmod.tq_ternary_gemv, tqmod.tq_ternary_gemm):
        _raises("must be a device tensor", fn, q, sx, pk, sc, 10, 64)
        _raises("q must have shape", fn, _t((2, 60), i8), sx, pk, sc, 10, 64)
        _raises("q must have dtype", fn, _t((2, 64), f32), sx, pk, sc, 10, 64)
        _raises("sx must hold 2", fn, q, _t((3,), f32), pk, sc, 10, 64)
        _raises("packed must hold at least 160", fn, q, sx, _t((9, 16), u8), sc, 10, 64)
        _raises("scale must hold at least 10", fn, q, sx, pk, sc, 10, 64, "row")
        _raises("Y must have dtype torch.float32", fn, q, sx, pk, sc, 10, 64, "tensor", "f32",
                Y=_t((2, 10), torch.bfloat16))
        _raises("Y must have shape", fn, q, sx, pk, sc, 10, 64, "tensor", "bf16",
                Y=_t((2, 11), torch.bfloat16))
        _raises("granularity must be one of", fn, q, sx, pk, sc, 10, 64, "rows")
        _raises("out_dtype must be one of", fn, q, sx, pk, sc, 10, 64, "tensor", "f16")
    _raises("packed must hold at least 80", tqmod.tq_binary1_gemv, q, sx, _t((79,), u8),
            _t((10,), f32), 10, 64)


def test_binding_quant_pack_and_fused_checks():
    f32, u8, i8 = torch.float32, torch.uint8, torch.int8
    X = _t((3, 512), f32)
    _raises("must be a device tensor", tqmod.tq_quant_act_int8, X)
    _raises("X must have dtype", tqmod.tq_quant_act_int8, _t((3, 512), torch.float16))
    _raises("q must have shape", tqmod.tq_quant_act_int8, X, q=_t((3, 511), i8))
    _raises("sx must hold 3", tqmod.tq_quant_act_int8, X, sx=_t((2,), f32))
    _raises("rms_weight must hold 512", tqmod.tq_quant_act_int8, X, rmsnorm=True,
            rms_weight=_t((511,), f32))
    _raises("Y must have shape", tqmod.tq_fwht512, X, Y=_t((3, 256), f32))
    W = _t((8, 64), f32)
    _raises("packed must hold 128", tqmod.tq_pack_ternary, W, packed=_t((8, 15), u8))
    _raises("scale must hold 8", tqmod.tq_pack_ternary, W, "row", scale=_t((1,), f32))
    _raises("workspace must hold at least", tqmod.tq_pack_ternary, W, "tensor",
            packed=_t((8, 16), u8), scale=_t((1,), f32), workspace=_t((8,), u8))
    _raises("mode must be one of", tqmod.tq_pack_ternary, W, "tensor", "tern")
    _raises("packed must hold 64", tqmod.tq_pack_binary1, W, packed=_t((8, 16), u8))
    _raises("kind must be one of", tqmod.tq_pack_ternary_threshold, W, "tensor", "rel")
    pk, sc = _t((10, 128), u8), _t((1,), f32)
    _raises("X must have K = 512", tqmod.tq_quant_ternary_gemv, _t((2, 256), f32), pk, sc, 10,
            512)
    _raises("Y must have dtype", tqmod.tq_quant_ternary_gemv, _t((2, 512), f32), pk, sc, 10, 512,
            Y=_t((2, 10), torch.int32))
    _raises("packed_up must hold at least", tqmod.tq_swiglu_gemv, _t((2, 512), f32), pk, sc,
            _t((10, 127), u8), sc, 10, 512, "tensor")
    _raises("H must have shape", tqmod.tq_swiglu_gemv, _t((2, 512), f32), pk, sc, pk, sc, 10, 512,
            "tensor", H=_t((2, 9), f32))
    g, u, d = (_t((16, 8), u8), _t((16,), f32)), (_t((16, 8), u8), _t((16,), f32)), \
        (_t((32, 4), u8), _t((32,), f32))
    _raises("down packed must hold at least", tqmod.tq_ffn_swiglu_decode, _t((1, 32), f32), g, u,
            (_t((32, 3), u8), _t((32,), f32)), 32, 16)
    _raises("sx_h must have shape", tqmod.tq_ffn_swiglu_decode, _t((1, 32), f32), g, u, d, 32, 16,
            buffers={"sx_h": _t((2,), f32)})
    _raises("packed must hold at least", tqmod.tq_ternary_backward_input, _t((4, 10), f32),
            _t((10, 15), u8), sc, 64)


def test_package_exports_every_entry_point():
    import ternary_quantized_linear_absmean_amd as pkg
    for name in declared_functions():
        assert name in pkg.__all__, name
        assert getattr(pkg, name) is getattr(tqmod, name)


def test_noalloc_pack_validation():
    # argument errors return before any HIP call (no device is touched)
    f = lib.tq_pack_ternary_noalloc
    buf = (ctypes.c_float * 64)()
    out = (ctypes.c_uint8 * 16)()
    sc = (ctypes.c_float * 4)()
    p = lambda o: ctypes.cast(o, ctypes.c_void_p)  # noqa: E731
    assert f(p(buf), 4, 6, 0, 0, p(out), p(sc), None) == SHAPE
    assert f(p(buf), -1, 8, 0, 0, p(out), p(sc), None) == SHAPE
    assert f(p(buf), 4, 8, 2, 0, p(out), p(sc), None) == UNSUP
    assert f(p(buf), 4, 8, 0, 5, p(out), p(sc), None) == UNSUP
    assert f(None, 4, 8, 0, 0, p(out), p(sc), None) == NULL
    assert f(p(buf), 0, 8, 0, 0, None, None, None) == OK
    assert f(p(buf), 1 << 21, 1 << 20, 0, 0, p(out), p(sc), None) == UNSUP
