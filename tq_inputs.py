"""Seeded synthetic inputs for the ternary linear layer.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it.  Every array is produced by ``numpy.random.default_rng(seed)``
(PCG64).

Workloads (weights are [N_out, K_in] row-major, activations are [M, K]):

* ``tiny``      W 256x256 ~N(0, 0.02), per-tensor scale; X 4x256 ~N(0, 1) fp32.
* ``decode``    W 4096x4096 ~N(0, 0.02), per-tensor; X 1x4096 ~N(0, 1) bf16.
* ``ffn``       up W 6912x2560 and down W 2560x6912 ~N(0, 0.02), per-row
                scales; X bx2560 / bx6912 ~N(0, 1) bf16, b in {1, 4, 16}.
* ``prefill``   X 2048x4096 ~N(0, 1) bf16; W 11008x4096 ~N(0, 0.02) per-tensor.
* ``bitlinear`` X 512x4096 Student-t(3) bf16, RMSNorm + FWHT-512 prologue;
                W 4096x4096 ~N(0, 0.02) per-row, ternary and binary (sign).

Output gradients for the backward through a workload's matrix are dY [b, N_out]
~N(0, 1) fp32 (bf16-rounded when asked for).

Seeds: weights use ``1000*cfg + j``, activations ``1000*cfg + 100 + j + b`` and
output gradients ``1000*cfg + 500 + j + b``, where ``cfg`` is the workload
number (1..5 in the order above), ``j`` the matrix index (up=0, down=1) and
``b`` the batch size.
"""
from __future__ import annotations

import numpy as np

WEIGHT_SIGMA = np.float32(0.02)

WORKLOADS = {
    "tiny": dict(cfg=1, mats=[(256, 256)], batches=[4], x_dtype="f32",
                 x_dist="normal", gran="tensor", modes=["ternary"], y_dtype="f32"),
    "decode": dict(cfg=2, mats=[(4096, 4096)], batches=[1], x_dtype="bf16",
                   x_dist="normal", gran="tensor", modes=["ternary"], y_dtype="f32"),
    "ffn": dict(cfg=3, mats=[(6912, 2560), (2560, 6912)], batches=[1, 4, 16],
                x_dtype="bf16", x_dist="normal", gran="row", modes=["ternary"],
                y_dtype="f32"),
    "prefill": dict(cfg=4, mats=[(11008, 4096)], batches=[2048], x_dtype="bf16",
                    x_dist="normal", gran="tensor", modes=["ternary"], y_dtype="bf16"),
    "bitlinear": dict(cfg=5, mats=[(4096, 4096)], batches=[512], x_dtype="bf16",
                      x_dist="student_t3", gran="row", modes=["ternary", "binary"],
                      y_dtype="f32", prologue=True),
}


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even), returned as
    fp32 so that the same numbers can be handed to either side exactly.
    Inputs are finite by construction."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return bits.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def weight_seed(cfg: int, j: int = 0) -> int:
    return 1000 * cfg + j


def act_seed(cfg: int, j: int, b: int) -> int:
    return 1000 * cfg + 100 + j + b


def grad_seed(cfg: int, j: int, b: int) -> int:
    return 1000 * cfg + 500 + j + b


def normal_weights(seed: int, n: int, k: int, sigma=WEIGHT_SIGMA) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)


def activations(seed: int, m: int, k: int, dist: str = "normal",
                dtype: str = "bf16") -> np.ndarray:
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((m, k), dtype=np.float32)
    elif dist == "student_t3":
        x = rng.standard_t(3, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    if dtype == "bf16":
        x = to_bf16_values(x)
    return x


def workload_weights(name: str, j: int = 0) -> np.ndarray:
    w = WORKLOADS[name]
    n, k = w["mats"][j]
    return normal_weights(weight_seed(w["cfg"], j), n, k)


def workload_activations(name: str, j: int = 0, b: int | None = None) -> np.ndarray:
    w = WORKLOADS[name]
    n, k = w["mats"][j]
    if b is None:
        b = w["batches"][0]
    return activations(act_seed(w["cfg"], j, b), b, k, w["x_dist"], w["x_dtype"])


def output_grads(seed: int, m: int, n: int, dtype: str = "f32") -> np.ndarray:
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((m, n), dtype=np.float32)
    return to_bf16_values(g) if dtype == "bf16" else g


def workload_output_grads(name: str, j: int = 0, b: int | None = None,
                          dtype: str = "f32") -> np.ndarray:
    w = WORKLOADS[name]
    n, k = w["mats"][j]
    if b is None:
        b = w["batches"][0]
    return output_grads(grad_seed(w["cfg"], j, b), b, n, dtype)


def random_ternary(seed: int, n: int, k: int) -> np.ndarray:
    """Uniform codes in {-1, 0, +1} as int8 (for layout tests)."""
    rng = np.random.default_rng(seed)
    return rng.integers(-1, 2, size=(n, k), dtype=np.int8)


def random_int8(seed: int, m: int, k: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(m, k), dtype=np.int8)
