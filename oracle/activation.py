"""GELU after the quantized product (oracle; test infrastructure only).

Nunchaku / SVDQuant in Diffusers (ai-papers.net), section on quantizing one's own model: the
further speed-ups it lists are fusing the Q, K and V projections and fusing GELU with the MLP,
both of which rewrite the model's structure.  The MLP of a diffusion transformer block is
up-projection, GELU, down-projection; the fusion applies GELU to the up-projection's output
where that output is produced, so the down-projection's quantizer reads the activated tensor.

The pages name GELU without a formula.  Both standard forms are defined here, in float64:
  * "erf":  GELU(x) = x Phi(x), Phi the standard normal CDF;
  * "tanh": GELU(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), the tanh form that
            transformer MLPs commonly use.
Phi is evaluated through the complementary error function (scipy.special.erfc), accurate in
both tails.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc

from .linear import lut_gemm

ACTIVATIONS = ("none", "gelu_tanh", "gelu_erf")


def gelu_erf(x) -> np.ndarray:
    """x Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2."""
    x = np.asarray(x, dtype=np.float64)
    return x * 0.5 * erfc(-x / math.sqrt(2.0))


def gelu_tanh(x) -> np.ndarray:
    """x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def activation(y, act: str) -> np.ndarray:
    """The named activation applied elementwise ("none" returns y as float64)."""
    if act == "none":
        return np.asarray(y, dtype=np.float64)
    if act == "gelu_tanh":
        return gelu_tanh(y)
    if act == "gelu_erf":
        return gelu_erf(y)
    raise ValueError(f"unknown activation {act!r}")


def lut_gemm_act(codes_x, s, cent_a, codes_w, r, cent_w, act: str) -> np.ndarray:
    """The quantized product followed by the activation: act(Y), Y as in lut_gemm."""
    return activation(lut_gemm(codes_x, s, cent_a, codes_w, r, cent_w), act)
