"""The allocation-free pack entry point, tq_pack_ternary_noalloc, called
through the C ABI, against tq_pack_ternary with a workspace: packed bytes
and scales bit for bit, on consecutive calls (the static scratch keeps the
previous call's contents), the second smaller than the first, including
tensors whose absmean sits on an fp32 rounding midpoint (the exact integer
path, which uses the scratch's exponent bins)."""
import ctypes
import sys

import numpy as np
import pytest

import tq_inputs as ti

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("ternary_quantized_linear_absmean_amd.tq")

DEV = "cuda:0"
GRAN = {"tensor": 0, "row": 1}
MODE = {"ternary": 0, "binary": 1}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _inputs():
    big = ti.normal_weights(8101, 4096, 4096)
    tie = np.ones((64, 128), np.float32)
    tie[:, ::2] = _f32(0x3F800001)          # mean 1 + 2^-24: an fp32 midpoint
    small = ti.normal_weights(8102, 257, 68)
    return [("4096x4096", big), ("64x128 midpoint", tie), ("257x68", small)]


def _noalloc(W, gran, mode):
    N, K = W.shape
    packed = torch.full((N, K // 4), 0xA5, dtype=torch.uint8, device=DEV)
    scale = torch.full((N if gran == "row" else 1,), float("nan"), dtype=torch.float32,
                       device=DEV)
    lib = tq.raw_library()
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.tq_pack_ternary_noalloc(ctypes.c_void_p(W.data_ptr()), N, K, GRAN[gran],
                                     MODE[mode], ctypes.c_void_p(packed.data_ptr()),
                                     ctypes.c_void_p(scale.data_ptr()), ctypes.c_void_p(st))
    assert rc == 0, tq.tq_status_str(rc)
    return packed, scale


@pytest.mark.parametrize("gran", ["tensor", "row"])
@pytest.mark.parametrize("mode", ["ternary", "binary"])
def test_noalloc_pack_matches_workspace_pack(gran, mode):
    for name, Wn in _inputs():
        say(f"noalloc pack {name} {gran} {mode}")
        W = torch.from_numpy(np.ascontiguousarray(Wn)).to(DEV)
        p0, s0 = tq.tq_pack_ternary(W, gran, mode)
        p1, s1 = _noalloc(W, gran, mode)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(p1.cpu().numpy(), p0.cpu().numpy())
        np.testing.assert_array_equal(s1.cpu().numpy().view(np.uint32),
                                      s0.cpu().numpy().view(np.uint32))
    # the midpoint tensor's scale is the exact rounding (ties to even: 1.0)
    W = torch.from_numpy(_inputs()[1][1]).to(DEV)
    _, s = _noalloc(W, "tensor", "ternary")
    torch.cuda.synchronize()
    assert s.cpu().numpy()[0] == np.float32(1.0)


def test_noalloc_pack_rejects_bad_arguments_before_launch():
    lib = tq.raw_library()
    st = torch.cuda.current_stream().cuda_stream
    W = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    p = torch.zeros((4, 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((1,), dtype=torch.float32, device=DEV)
    args = lambda K: (ctypes.c_void_p(W.data_ptr()), 4, K, 0, 0, ctypes.c_void_p(p.data_ptr()),
                      ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(st))
    assert lib.tq_pack_ternary_noalloc(*args(6)) == 2          # K % 4 != 0: shape
    assert lib.tq_pack_ternary_noalloc(None, 4, 8, 0, 0, None, None, None) == 1
    assert lib.tq_pack_ternary_noalloc(*args(8)) == 0
