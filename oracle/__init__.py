"""CPU oracle for the ternary linear layer -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .tq_oracle import *  # noqa: F401,F403
from .tq_oracle import (absmean_scale, absmean_scales, binarize, contract,
                        contract_rows, epilogue, exact_abs_sum_units,
                        exact_fraction_mean, fwht512, fwht_block,
                        hadamard_matrix, pack_codes, pack_ternary,
                        packed_bytes, quant_act_int8, rms_factor,
                        mean_of_squares, rmsnorm, bitlinear_prologue,
                        bitlinear_prologue_fp64, BITLINEAR_BOUNDS,
                        round_rational_to_f32, ternarize, ternary_linear,
                        unpack_codes, bf16_round_from_f64, FWHT_NORM,
                        packed1_bytes, pack_signs, unpack_signs, pack_binary1,
                        contract_signs, swiglu_clamped, ffn_swiglu_decode,
                        SWIGLU_CLAMP, backward_input, backward_weight,
                        ternarize_threshold, encode_format, decode_format,
                        convert_codes, FORMATS)
