"""Seeded synthetic inputs for the OrbitQuant quantized linear layer.

This module only draws random numbers and casts them to bf16.  It holds none
of the method's arithmetic (no rotation, normalisation, codebook or product),
so both the CPU oracle and the HIP path may take their inputs from here.

Every draw uses numpy ``Generator(PCG64(seed))`` in float64 followed by a
round-to-nearest-even cast to bf16.  The shapes follow the diffusion-transformer
linear layers the OrbitQuant summary evaluates (FLUX.1 image DiTs and Wan 2.1
video DiTs, picx.dev summary, "Empirical Validation / Results"); the trained
weights and prompts are not available, so heavy-tailed synthetic activations
with outlier channels stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "bf16_bits_from_f64", "f64_from_bf16_bits", "rotation", "activations",
    "weights", "gelu_input", "Layer", "CONFIGS", "HEADLINE", "layer_inputs",
]


# ---------------------------------------------------------------- bf16 casting
def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return uint16 bits.

    The value is first rounded to float32 (nearest-even), then the float32 bit
    pattern is rounded to its upper 16 bits (nearest-even).  Input tensors are
    defined as whatever this produces, so the double rounding is part of the
    input recipe, not of any computation under test.
    """
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    u = (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------ rotation inputs
def rotation(d: int, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Random permutation pi (int32[d]) and Rademacher signs (int8[d]).

    The pages fix the rotation once per dimension and draw it at random; the
    generator is not specified, so seed = d by default.
    """
    rng = np.random.Generator(np.random.PCG64(d if seed is None else seed))
    perm = rng.permutation(d).astype(np.int32)
    signs = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    return perm, signs


def rotation_passes(d: int, passes: int) -> tuple[np.ndarray, np.ndarray]:
    """`passes` independent (perm, signs) draws back to back (int32[passes d], int8[passes d]):
    pass 0 is rotation(d), pass p > 0 uses seed d + 1000003 p."""
    draws = [rotation(d, None if p == 0 else d + 1000003 * p) for p in range(passes)]
    return (np.concatenate([x[0] for x in draws]), np.concatenate([x[1] for x in draws]))


# ----------------------------------------------------------- activation inputs
def activations(n: int, d: int, seed: int, kind: str = "heavy",
                outlier_frac: float = 0.001, outlier_gain: float = 30.0,
                frames: int | None = None, tokens_per_frame: int | None = None,
                as_float: bool = False) -> np.ndarray:
    """Synthetic DiT activations, returned as bf16 bits [n, d] (or float64).

    kind:
      "gauss"  N(0,1) entries times a per-channel log-normal(0,1) scale.
      "heavy"  Student-t(nu=3) entries times a per-channel log-normal(0,1) scale.
      "video"  "heavy" plus a per-frame drifting mean mu_f = (f/(F-1))*2*g with a
               fixed g ~ N(0,1)^d; frame f = row // tokens_per_frame.
    Outlier channels: round(outlier_frac*d) (at least 1) channels, chosen by
    the same generator, are multiplied by outlier_gain.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = np.exp(rng.standard_normal(d))
    n_out = max(1, int(round(outlier_frac * d))) if outlier_frac > 0 else 0
    out_ch = rng.choice(d, size=n_out, replace=False) if n_out else np.empty(0, np.int64)
    gain = np.ones(d)
    gain[out_ch] = outlier_gain
    col = scale * gain
    x = np.empty((n, d), dtype=np.float64)
    g = rng.standard_normal(d) if kind == "video" else None
    chunk = 2048
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        if kind == "gauss":
            base = rng.standard_normal((r1 - r0, d))
        else:
            base = rng.standard_t(3.0, size=(r1 - r0, d))
        blk = base * col[None, :]
        if kind == "video":
            assert frames and tokens_per_frame
            f = np.arange(r0, r1) // tokens_per_frame
            mu = (f / max(1, frames - 1))[:, None] * 2.0 * g[None, :]
            blk = blk + mu
        x[r0:r1] = blk
    return x if as_float else bf16_bits_from_f64(x)


def weights(m: int, d: int, seed: int, std: float = 0.02, as_float: bool = False) -> np.ndarray:
    """W ~ N(0, std^2), [m, d], as bf16 bits (or float64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal((m, d)) * std
    return w if as_float else bf16_bits_from_f64(w)


def gelu_input(n: int, d: int, seed: int, pre_std: float = 1.0) -> np.ndarray:
    """Stand-in for GELU(up-projection output), the input of an MLP down layer.

    Pre-activations are N(0, pre_std^2) times a per-channel log-normal(0, 0.5)
    scale; GELU (erf form) is applied in float64 and the result cast to bf16.
    """
    from scipy.special import erf
    rng = np.random.Generator(np.random.PCG64(seed))
    col = np.exp(0.5 * rng.standard_normal(d)) * pre_std
    out = np.empty((n, d), dtype=np.uint16)
    chunk = 1024
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        pre = rng.standard_normal((r1 - r0, d)) * col[None, :]
        out[r0:r1] = bf16_bits_from_f64(0.5 * pre * (1.0 + erf(pre / math.sqrt(2.0))))
    return out


# --------------------------------------------------------------- the layers
@dataclasses.dataclass(frozen=True)
class Layer:
    """One quantized linear layer: Y[n, m] = X[n, d] W[m, d]^T at (bits_w, bits_a)."""
    name: str
    n: int
    d: int
    m: int
    bits_w: int
    bits_a: int
    block: int
    x_kind: str
    x_seed: int
    w_seed: int
    outlier_frac: float = 0.001
    outlier_gain: float = 30.0

    @property
    def flops(self) -> float:
        return 2.0 * self.n * self.m * self.d


CONFIGS: dict[str, Layer] = {
    # tiny W4A4: 64x256 -> 256, block 64, Gaussian x log-normal scales, 2 outliers x50
    "tiny": Layer("tiny", 64, 256, 256, 4, 4, 64, "gauss", 101, 102, 2 / 256, 50.0),
    # FLUX fused QKV projection, W4A4
    "flux_qkv": Layer("flux_qkv", 4608, 3072, 9216, 4, 4, 128, "heavy", 201, 202),
    # FLUX MLP pair (CFG batch 2), W4A4
    "flux_mlp_up": Layer("flux_mlp_up", 9216, 3072, 12288, 4, 4, 128, "heavy", 301, 302),
    "flux_mlp_down": Layer("flux_mlp_down", 9216, 12288, 3072, 4, 4, 128, "gelu", 304, 303),
    # headline: the first 4608 tokens of the MLP-up input against the MLP-up weights
    "flux_mlp_up_4608": Layer("flux_mlp_up_4608", 4608, 3072, 12288, 4, 4, 128, "heavy", 301, 302),
    # W2A4 variant of the MLP-up shape, outlier fraction 0.5%
    "flux_mlp_up_w2a4": Layer("flux_mlp_up_w2a4", 4608, 3072, 12288, 2, 4, 128, "heavy", 401, 402,
                              0.005, 30.0),
    # W3A3 variant of the headline layer (same tokens and weights, 8-centroid codebooks)
    "flux_mlp_up_w3a3": Layer("flux_mlp_up_w3a3", 4608, 3072, 12288, 3, 3, 128, "heavy", 301, 302),
    # Wan 2.1 1.3B video FFN, W4A6 (21 frames x 30 x 52 latent tokens)
    "wan_ffn_up": Layer("wan_ffn_up", 32760, 1536, 8960, 4, 6, 128, "video", 501, 502),
    "wan_ffn_down": Layer("wan_ffn_down", 32760, 8960, 1536, 4, 6, 128, "gelu", 504, 503),
}
HEADLINE = "flux_mlp_up_4608"


def layer_inputs(layer: Layer, rows: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(X bits [rows or n, d], W bits [m, d]) for a layer.

    ``rows`` keeps only the first rows of X (the generator is row-sequential,
    so the first rows do not depend on how many are drawn).
    """
    n = layer.n if rows is None else min(rows, layer.n)
    if layer.x_kind == "gelu":
        x = gelu_input(n, layer.d, layer.x_seed)
    elif layer.x_kind == "video":
        x = activations(n, layer.d, layer.x_seed, "video", layer.outlier_frac,
                        layer.outlier_gain, frames=21, tokens_per_frame=30 * 52)
    else:
        x = activations(n, layer.d, layer.x_seed, layer.x_kind, layer.outlier_frac,
                        layer.outlier_gain)
    w = weights(layer.m, layer.d, layer.w_seed)
    return x, w


def random_code_bytes(rows: int, row_bytes: int, seed: int) -> np.ndarray:
    """Uniformly random packed code bytes [rows, row_bytes] (every byte pattern is a valid
    packed code array for 2-, 4- and 6-bit codes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)


def random_norms(rows: int, seed: int, lo: float = 0.5, hi: float = 2.0) -> np.ndarray:
    """Positive per-row scales drawn uniformly from [lo, hi), float64."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(lo, hi, rows)
