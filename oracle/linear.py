"""The quantized product and the packed code format (oracle; test
infrastructure only).

OrbitQuant summary (picx.dev), "Online Activation Quantization": the rotations
cancel, W^' x^' ~= W Pi^T Pi x = W x, so no inverse rotation is applied.  With
x^'_i = s_i C_a[a_i] and w^'_j = r'_j C_w[w_j]:
    Y[i, j] = s_i * r'_j * sum_k C_a[a_ik] * C_w[w_jk].
Reading where the pages are silent: the decoded centroids are rounded to bf16
(round-to-nearest-even) before the product, the precision the product runs in;
the sum itself is exact up to float64 rounding here.

Packed code format (a definition of the library's data layout, written out
here independently of the library's code):
  * code value: sign-magnitude index.  For N = 2^b centroids in ascending
    order, centroid k >= N/2 is stored as k - N/2 (top bit 0, positive) and
    centroid k < N/2 as N/2 + (N/2 - 1 - k) (top bit 1, negative); the low
    b-1 bits rank |centroid| from the smallest magnitude up.
  * row layout: codes of one row in order, rows back to back, d*b/8 bytes per row.
      b = 4: code j in byte j//2, bits 4*(j%2) .. +3
      b = 2: code j in byte j//4, bits 2*(j%4) .. +1
      b = 6: code j in the 3-byte little-endian group j//4, bits 6*(j%4) .. +5
      b = 3: code j in the 3-byte little-endian group j//8, bits 3*(j%8) .. +2
"""
from __future__ import annotations

import numpy as np

from .quantize import argmin_codes, bf16_rne, quantize_activations, rotate_normalize
from .rpbh import rotate


def decode_lut_bf16(centroids) -> np.ndarray:
    """bf16-rounded centroid values (float64) used by the product."""
    return bf16_rne(np.asarray(centroids, dtype=np.float64))


def lut_gemm(codes_x, s, cent_a, codes_w, r, cent_w) -> np.ndarray:
    """Y[i, j] = s_i r_j sum_k C^_a[a_ik] C^_w[w_jk] in float64 (dequantise, then product)."""
    A = decode_lut_bf16(cent_a)[np.asarray(codes_x)]
    B = decode_lut_bf16(cent_w)[np.asarray(codes_w)]
    return (A @ B.T) * np.asarray(s, np.float64)[:, None] * np.asarray(r, np.float64)[None, :]


def orbq_linear(X, Pi, cent_a, codes_w, r, cent_w, eps: float = 1e-8):
    """Online forward: quantize X, then the product with the folded weights."""
    codes_x, s, _ = quantize_activations(X, Pi, cent_a, eps)
    return lut_gemm(codes_x, s, cent_a, codes_w, r, cent_w), codes_x, s


def unquantized_fold(X, W, Pi) -> np.ndarray:
    """(X Pi^T)(W Pi^T)^T: the rotation cancels, so this equals X W^T."""
    return rotate(X, Pi) @ rotate(W, Pi).T


# ------------------------------------------------------------- code format
def to_sign_magnitude(k, bits: int) -> np.ndarray:
    half = 1 << (bits - 1)
    k = np.asarray(k, dtype=np.int64)
    return np.where(k >= half, k - half, half + (half - 1 - k))


def from_sign_magnitude(c, bits: int) -> np.ndarray:
    half = 1 << (bits - 1)
    c = np.asarray(c, dtype=np.int64)
    return np.where(c < half, half + c, (half - 1) - (c - half))


def codes_row_bytes(d: int, bits: int) -> int:
    if (d * bits) % 8:
        raise ValueError("d*bits must be a multiple of 8")
    return d * bits // 8


def pack_codes(k, bits: int) -> np.ndarray:
    """Ascending centroid indices [rows, d] -> packed uint8 [rows, d*bits/8]."""
    k = np.asarray(k, dtype=np.int64)
    rows, d = k.shape
    c = to_sign_magnitude(k, bits).astype(np.uint32)
    if bits == 4:
        c = c.reshape(rows, d // 2, 2)
        return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)
    if bits == 2:
        c = c.reshape(rows, d // 4, 4)
        return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
    if bits == 6:
        c = c.reshape(rows, d // 4, 4)
        g = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
        out = np.stack([g & 0xFF, (g >> 8) & 0xFF, (g >> 16) & 0xFF], axis=-1)
        return out.reshape(rows, d // 4 * 3).astype(np.uint8)
    if bits == 3:
        c = c.reshape(rows, d // 8, 8)
        g = np.zeros((rows, d // 8), dtype=np.uint32)
        for i in range(8):
            g |= c[..., i] << (3 * i)
        out = np.stack([g & 0xFF, (g >> 8) & 0xFF, (g >> 16) & 0xFF], axis=-1)
        return out.reshape(rows, d // 8 * 3).astype(np.uint8)
    raise ValueError("bits must be 2, 3, 4 or 6")


def unpack_codes(packed, bits: int, d: int) -> np.ndarray:
    """Packed uint8 [rows, d*bits/8] -> ascending centroid indices int64 [rows, d]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.uint32)
    rows = p.shape[0]
    if bits == 4:
        c = np.stack([p & 0xF, p >> 4], axis=-1).reshape(rows, d)
    elif bits == 2:
        c = np.stack([(p >> s) & 3 for s in (0, 2, 4, 6)], axis=-1).reshape(rows, d)
    elif bits == 6:
        g3 = p.reshape(rows, d // 4, 3)
        g = g3[..., 0] | (g3[..., 1] << 8) | (g3[..., 2] << 16)
        c = np.stack([(g >> s) & 63 for s in (0, 6, 12, 18)], axis=-1).reshape(rows, d)
    elif bits == 3:
        g3 = p.reshape(rows, d // 8, 3)
        g = g3[..., 0] | (g3[..., 1] << 8) | (g3[..., 2] << 16)
        c = np.stack([(g >> (3 * i)) & 7 for i in range(8)], axis=-1).reshape(rows, d)
    else:
        raise ValueError("bits must be 2, 3, 4 or 6")
    return from_sign_magnitude(c, bits)


def linear_a16(X, Pi, codes_w, r, cent_w) -> np.ndarray:
    """Weight-only product with bf16 activations: Y[i, j] = r_j sum_k bf16((Pi x_i)_k) C^_w[w_jk].

    The OrbitQuant pages keep the AdaLN activations in BF16 while its modulation weights are
    quantized (ai-papers.net article, AdaLN section; picx.dev summary, "AdaLN Bit-Width
    Ablation (Figure 6)").  The weights are the usual folded codes, so the activations are
    rotated by the same Pi (the rotations cancel, "Online Activation Quantization") but not
    normalised or quantized.  Reading: the rotated activations are rounded to bf16 (round to
    nearest even) once, the precision the product takes its operands in.
    """
    A = bf16_rne(rotate(X, Pi))
    B = decode_lut_bf16(cent_w)[np.asarray(codes_w)]
    return (A @ B.T) * np.asarray(r, np.float64)[None, :]
