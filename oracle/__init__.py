"""CPU oracle for the OrbitQuant quantized linear layer (float64, plain numpy/scipy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it, and it never calls the HIP library: the two share no code.

What it computes (OrbitQuant summary on picx.dev, "Methodology"):
  rpbh.py       the RPBH rotation as an explicit dense d x d matrix
                ("Randomized Permuted Block-Hadamard (RPBH) Rotation"), its
                composition over several passes and the O(d) flatness statistics
                ("Quantizing With Randomized Hadamard Transforms", gist.science).
  density.py    the sphere-coordinate marginal f_d and its cell integrals
                ("Theoretical Basis", item 1).
  lloyd_max.py  the Lloyd-Max codebook for f_d by plain Lloyd iteration
                ("Theoretical Basis", item 2).
  quantize.py   rotate, normalise, brute-force argmin; the weight fold
                ("Offline Weight Quantization", "Online Activation Quantization").
  linear.py     the dequantised product with the rotation cancelled, and the
                packed code format written out from its documented definition.
  activation.py GELU (erf and tanh forms) applied to the product, the activation
                a fused MLP up-projection produces (Nunchaku / SVDQuant in
                Diffusers, on fusing GELU with the MLP).

Every function cites the passage it follows.  Each is pinned in
tests/test_oracle_*.py against closed forms, printed values or brute force.
"""
from .rpbh import flatness, hadamard, rotate, rpbh_composed, rpbh_matrix
from .density import log_fd, fd, gaussian_limit_pdf, cell_mass, cell_moment, mean_abs_t
from .lloyd_max import lloyd_max, thresholds_midpoint
from .quantize import argmin_codes, rotate_normalize, quantize_activations, fold_weights, bf16_rne
from .activation import ACTIVATIONS, activation, gelu_erf, gelu_tanh, lut_gemm_act
from .linear import (decode_lut_bf16, linear_a16, lut_gemm, orbq_linear, unquantized_fold, to_sign_magnitude,
                     from_sign_magnitude, pack_codes, unpack_codes, codes_row_bytes)

__all__ = [
    "hadamard", "rpbh_matrix", "rotate", "rpbh_composed", "flatness", "log_fd", "fd", "gaussian_limit_pdf", "cell_mass",
    "cell_moment", "mean_abs_t", "lloyd_max", "thresholds_midpoint", "argmin_codes",
    "rotate_normalize", "quantize_activations", "fold_weights", "bf16_rne", "decode_lut_bf16",
    "lut_gemm", "orbq_linear", "unquantized_fold", "to_sign_magnitude", "from_sign_magnitude",
    "pack_codes", "unpack_codes", "codes_row_bytes", "ACTIVATIONS", "activation", "gelu_erf",
    "gelu_tanh", "lut_gemm_act", "linear_a16",
]
