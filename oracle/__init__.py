"""CPU fp64 oracle for the W4A16 / ternary / W16A16 / MXFP4 small-M linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.
"""
from .oracle import (build, num_threads, f16_to_f64, bf16_to_f64, w4_dequant, w4_gemv,
                     w2t_dequant, w2t_gemv, w16_gemv, e2m1_to_f64, e8m0_to_f64, mx_dequant,
                     mx_gemv)

__all__ = ["build", "num_threads", "f16_to_f64", "bf16_to_f64", "w4_dequant", "w4_gemv",
           "w2t_dequant", "w2t_gemv", "w16_gemv", "e2m1_to_f64", "e8m0_to_f64", "mx_dequant",
           "mx_gemv"]
