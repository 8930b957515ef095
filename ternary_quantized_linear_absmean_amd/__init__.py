"""libtq: a ternary (absmean, 2-bit) linear layer for AMD Instinct MI355X.

The C ABI is declared in include/tq.h and implemented by libtq.so (HIP,
gfx950).  ``ternary_quantized_linear_absmean_amd.tq`` is the Python binding;
its names are re-exported here on first use, and importing them fails loudly
when the library has not been built (there is no fallback path).
"""
from __future__ import annotations

__all__ = ["tq_packed_bytes", "tq_pack_workspace_bytes", "tq_pack_ternary",
           "tq_pack_ternary_noalloc",
           "tq_quant_act_int8", "tq_fwht512", "tq_ternary_gemv", "tq_ternary_gemm",
           "tq_quant_ternary_gemv",
           "tq_packed1_bytes", "tq_pack_binary1", "tq_binary1_gemv",
           "tq_swiglu_gemv", "tq_ffn_swiglu_decode",
           "tq_ternary_backward_input", "tq_ternary_backward_weight",
           "tq_pack_ternary_threshold", "tq_convert_codes", "tq_unpack_codes",
           "tq_status_str", "tq_last_hip_error", "tq_version", "TqError"]


def __getattr__(name):
    if name in __all__:
        from . import tq as _tq
        return getattr(_tq, name)
    raise AttributeError(name)
