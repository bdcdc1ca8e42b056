"""OrbitQuant quantized linear layer on AMD Instinct MI355X (gfx950).

Python binding of liborbq, the C-ABI library declared in include/orbq.h.  This module
only marshals arguments: torch provides device memory and the current HIP stream, and
every step of the layer runs in liborbq's HIP kernels.  There is no fallback: if the
library is not built or no GPU is present the calls raise.

    rot = Rotation.create(d, block, perm, signs)        # fixed once per dimension
    cb = Codebook.lloyd_max(d, bits)                    # one per (d, bits), data-free
    w_codes, w_norms = fold_weights(W, rot, cb_w)       # offline
    Y = linear(X, rot, cb_a, w_codes, w_norms, cb_w)    # online
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "OrbqError", "library_path", "load", "Rotation", "Codebook", "codes_row_bytes", "fold_weights",
    "rpbh_quantize", "lut_gemm", "linear_workspace_bytes", "linear", "linear_noalloc", "test_rotate", "test_quantize_t",
    "test_mfma_rate",
    "F32", "BF16",
]

F32, BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    """The in-tree liborbq.so, or the file named by the ORBQ_LIBRARY environment variable."""
    return os.environ.get("ORBQ_LIBRARY") or os.path.join(_HERE, "liborbq.so")


class OrbqError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed with {status}: {detail}")
        self.status = status


class _Rpbh(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("block", ctypes.c_int32), ("perm", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("passes", ctypes.c_int32)]


class _Codebook(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("centroids", ctypes.POINTER(ctypes.c_float))]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SIGS = {
    "orbq_codebook_lloyd_max": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(ctypes.c_float)]),
    "orbq_rpbh_validate": (ctypes.c_int, [_I32, _I32, _P, _P]),
    "orbq_codebook_validate": (ctypes.c_int, [ctypes.POINTER(_Codebook)]),
    "orbq_codes_row_bytes": (ctypes.c_size_t, [_I64, _I32]),
    "orbq_fold_weights": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), ctypes.POINTER(_Codebook),
                                         _F, _P, _P, _P]),
    "orbq_rpbh_quantize": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), ctypes.POINTER(_Codebook),
                                          _F, _P, _P, _P]),
    "orbq_lut_gemm": (ctypes.c_int, [_P, _P, ctypes.POINTER(_Codebook), _P, _P, ctypes.POINTER(_Codebook),
                                     _I64, _I64, _I64, _P, ctypes.c_int, _I64, _P]),
    "orbq_lut_gemm_act": (ctypes.c_int, [_P, _P, ctypes.POINTER(_Codebook), _P, _P, ctypes.POINTER(_Codebook),
                                         _I64, _I64, _I64, ctypes.c_int, _P, ctypes.c_int, _I64, _P]),
    "orbq_linear_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I32]),
    "orbq_linear": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), ctypes.POINTER(_Codebook), _F,
                                   _P, _P, ctypes.POINTER(_Codebook), _I64, _P, ctypes.c_size_t, _P,
                                   ctypes.c_int, _I64, _P]),
    "orbq_linear_act": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), ctypes.POINTER(_Codebook), _F,
                                       _P, _P, ctypes.POINTER(_Codebook), _I64, _P, ctypes.c_size_t, ctypes.c_int,
                                       _P, ctypes.c_int, _I64, _P]),
    "orbq_linear_noalloc": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), ctypes.POINTER(_Codebook), _F,
                                           _P, _P, ctypes.POINTER(_Codebook), _I64, ctypes.c_int, _P, ctypes.c_int, _I64,
                                           _P]),
    "orbq_rpbh_flatness": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "orbq_linear_a16_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "orbq_linear_a16": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), _P, _P, ctypes.POINTER(_Codebook),
                                       _I64, _P, ctypes.c_size_t, _P, ctypes.c_int, _I64, _P]),
    "orbq_rht_passes": (ctypes.c_int32, [ctypes.c_float, ctypes.c_float, _I32, _I32]),
    "orbq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "orbq_last_error": (ctypes.c_char_p, []),
    "orbq_test_rotate": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.POINTER(_Rpbh), _P, _P, _P]),
    "orbq_test_quantize_t": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_Codebook), _P, _P]),
    "orbq_test_mfma_rate": (ctypes.c_int, [_I32, _I32, _P, ctypes.POINTER(ctypes.c_double), _P]),
}


@functools.lru_cache(maxsize=None)
def load() -> ctypes.CDLL:
    """Load liborbq.so (built in-tree by calibration_free_w4a4_amd.build)."""
    path = library_path()
    if not os.path.exists(path):
        raise OrbqError(-5, "load", f"{path} is not built; run python -m calibration_free_w4a4_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _check(status: int, func: str) -> None:
    if status != 0:
        lib = load()
        raise OrbqError(status, func, f"{lib.orbq_status_string(status).decode()}: {lib.orbq_last_error().decode()}")


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise OrbqError(-5, "orbq", "no HIP device is available")
    return torch


def _stream(torch, dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dev_tensor(t, dtype, name):
    if not t.is_cuda:
        raise OrbqError(-1, name, "tensor must be on the GPU")
    if t.dtype != dtype:
        raise OrbqError(-1, name, f"tensor must be {dtype}, got {t.dtype}")
    return t


# ---------------------------------------------------------------- descriptors
@dataclass
class Rotation:
    """RPBH rotation for dimension d: device perm (int32[passes * d], or None for the identity)
    and signs (int8[passes * d]); passes > 1 composes that many RPBH passes."""
    d: int
    block: int
    perm: "object"
    signs: "object"
    passes: int = 1

    @classmethod
    def create(cls, d: int, block: int, perm, signs: np.ndarray, device=None, passes: int = 1) -> "Rotation":
        signs = np.ascontiguousarray(signs, dtype=np.int8)
        if perm is not None:
            perm = np.ascontiguousarray(perm, dtype=np.int32)
        if signs.size != passes * d or (perm is not None and perm.size != passes * d):
            raise OrbqError(-1, "Rotation", f"{passes} passes need perm and signs of {passes * d} entries")
        for p in range(passes):  # each pass is one RPBH rotation
            _check(load().orbq_rpbh_validate(d, block, None if perm is None else perm[p * d:].ctypes.data,
                                             signs[p * d:].ctypes.data), "orbq_rpbh_validate")
        torch = _torch()
        dev = device or torch.device("cuda", torch.cuda.current_device())
        dperm = None if perm is None else torch.from_numpy(perm).to(dev)
        return cls(d, block, dperm, torch.from_numpy(signs).to(dev), passes)

    def struct(self) -> _Rpbh:
        return _Rpbh(self.d, self.block, 0 if self.perm is None else self.perm.data_ptr(), self.signs.data_ptr(),
                     self.passes)


@dataclass
class Codebook:
    """Lloyd-Max codebook (host fp32 centroids) for (d, bits)."""
    d: int
    bits: int
    centroids: np.ndarray

    @classmethod
    def lloyd_max(cls, d: int, bits: int) -> "Codebook":
        return cls(d, bits, _lloyd_max_cached(d, bits).copy())

    @classmethod
    def from_centroids(cls, d: int, bits: int, centroids) -> "Codebook":
        c = np.ascontiguousarray(centroids, dtype=np.float32)
        if c.shape != (1 << bits,):
            raise OrbqError(-1, "Codebook", f"need {1 << bits} centroids")
        return cls(d, bits, c)

    def struct(self) -> _Codebook:
        c = self.centroids
        cached = getattr(self, "_struct", None)
        if cached is not None and self._keep is c and (cached.d, cached.bits) == (self.d, self.bits):
            return cached  # the struct points at the live float32 array itself
        c = np.ascontiguousarray(c, dtype=np.float32)
        self._keep = c
        st = _Codebook(self.d, self.bits, c.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        self._struct = st if c is self.centroids else None
        return st


@functools.lru_cache(maxsize=None)
def _lloyd_max_cached(d: int, bits: int) -> np.ndarray:
    out = np.zeros(1 << bits, dtype=np.float32)
    _check(load().orbq_codebook_lloyd_max(d, bits, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))),
           "orbq_codebook_lloyd_max")
    return out


def codes_row_bytes(d: int, bits: int) -> int:
    return int(load().orbq_codes_row_bytes(d, bits))


def linear_workspace_bytes(n: int, d: int, bits_a: int) -> int:
    """Bytes of orbq_linear's workspace: the token codes and norms (for 6-bit activations,
    room for the codes' bf16 centroids, which the layer keeps when m >= 2048)."""
    return int(load().orbq_linear_workspace_bytes(n, d, bits_a))


# ------------------------------------------------------------------ the calls
def fold_weights(W, rot: Rotation, cb: Codebook, eps: float = 1e-8, out_codes=None, out_norms=None):
    """Offline fold + quantize of bf16 weights [m, d] -> (codes uint8 [m, d*b/8], r' bf16 [m])."""
    torch = _torch()
    _dev_tensor(W, torch.bfloat16, "fold_weights")
    m, d = W.shape
    codes = out_codes if out_codes is not None else torch.empty((m, codes_row_bytes(d, cb.bits)), dtype=torch.uint8,
                                                                device=W.device)
    norms = out_norms if out_norms is not None else torch.empty((m,), dtype=torch.bfloat16, device=W.device)
    r, c = rot.struct(), cb.struct()
    _check(load().orbq_fold_weights(W.data_ptr(), m, d, W.stride(0), ctypes.byref(r), ctypes.byref(c), eps,
                                    codes.data_ptr(), norms.data_ptr(), _stream(torch, W.device)), "orbq_fold_weights")
    return codes, norms


def rpbh_quantize(X, rot: Rotation, cb: Codebook, eps: float = 1e-8, out_codes=None, out_norms=None):
    """Online activation quantization of bf16 tokens [n, d] -> (codes uint8 [n, d*b/8], s fp32 [n])."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "rpbh_quantize")
    n, d = X.shape
    codes = out_codes if out_codes is not None else torch.empty((n, codes_row_bytes(d, cb.bits)), dtype=torch.uint8,
                                                                device=X.device)
    norms = out_norms if out_norms is not None else torch.empty((n,), dtype=torch.float32, device=X.device)
    r, c = rot.struct(), cb.struct()
    _check(load().orbq_rpbh_quantize(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), ctypes.byref(c), eps,
                                     codes.data_ptr(), norms.data_ptr(), _stream(torch, X.device)),
           "orbq_rpbh_quantize")
    return codes, norms


ACTIVATIONS = {"none": 0, "gelu_tanh": 1, "gelu_erf": 2}   # orbq_activation


def _act(act: str) -> int:
    if act not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}, not {act!r}")
    return ACTIVATIONS[act]


def lut_gemm(x_codes, x_norms, cb_a: Codebook, w_codes, w_norms, cb_w: Codebook, d: int, out_dtype=None, out=None,
             act: str = "none"):
    """Y [n, m] = act(diag(s) C_a[x_codes] C_w[w_codes]^T diag(r')); act "none" calls
    orbq_lut_gemm, "gelu_tanh" / "gelu_erf" orbq_lut_gemm_act."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    n, m = x_codes.shape[0], w_codes.shape[0]
    Y = out if out is not None else torch.empty((n, m), dtype=out_dtype, device=x_codes.device)
    a, w = cb_a.struct(), cb_w.struct()
    yt = BF16 if Y.dtype == torch.bfloat16 else F32
    code = _act(act)
    if code == 0:
        _check(load().orbq_lut_gemm(x_codes.data_ptr(), x_norms.data_ptr(), ctypes.byref(a), w_codes.data_ptr(),
                                    w_norms.data_ptr(), ctypes.byref(w), n, m, d, Y.data_ptr(), yt, Y.stride(0),
                                    _stream(torch, x_codes.device)), "orbq_lut_gemm")
    else:
        _check(load().orbq_lut_gemm_act(x_codes.data_ptr(), x_norms.data_ptr(), ctypes.byref(a), w_codes.data_ptr(),
                                        w_norms.data_ptr(), ctypes.byref(w), n, m, d, code, Y.data_ptr(), yt,
                                        Y.stride(0), _stream(torch, x_codes.device)), "orbq_lut_gemm_act")
    return Y


def linear(X, rot: Rotation, cb_a: Codebook, w_codes, w_norms, cb_w: Codebook, eps: float = 1e-8, out_dtype=None,
           workspace=None, out=None, act: str = "none"):
    """The online layer: Y [n, m] from bf16 tokens X [n, d] and folded weights (act as in
    lut_gemm: "none" calls orbq_linear, a GELU form orbq_linear_act)."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "linear")
    out_dtype = out_dtype or torch.float32
    n, d = X.shape
    m = w_codes.shape[0]
    need = linear_workspace_bytes(n, d, cb_a.bits)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    Y = out if out is not None else torch.empty((n, m), dtype=out_dtype, device=X.device)
    r, a, w = rot.struct(), cb_a.struct(), cb_w.struct()
    yt = BF16 if Y.dtype == torch.bfloat16 else F32
    ws_bytes = workspace.numel() * workspace.element_size()
    code = _act(act)
    if code == 0:
        _check(load().orbq_linear(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), ctypes.byref(a), eps,
                                  w_codes.data_ptr(), w_norms.data_ptr(), ctypes.byref(w), m, workspace.data_ptr(),
                                  ws_bytes, Y.data_ptr(), yt, Y.stride(0), _stream(torch, X.device)), "orbq_linear")
    else:
        _check(load().orbq_linear_act(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), ctypes.byref(a), eps,
                                      w_codes.data_ptr(), w_norms.data_ptr(), ctypes.byref(w), m, workspace.data_ptr(),
                                      ws_bytes, code, Y.data_ptr(), yt, Y.stride(0), _stream(torch, X.device)),
               "orbq_linear_act")
    return Y


NOALLOC_SCRATCH_BYTES = 16 << 20   # ORBQ_NOALLOC_SCRATCH_BYTES


def linear_noalloc(X, rot: Rotation, cb_a: Codebook, w_codes, w_norms, cb_w: Codebook, eps: float = 1e-8,
                   out_dtype=None, out=None, act: str = "none"):
    """The online layer without a caller workspace (orbq_linear_noalloc): the token codes go to
    the library's fixed per-device scratch array, so the call allocates nothing on the device
    when `out` is given.  Calls on one GPU that overlap in time race on that array."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "linear_noalloc")
    out_dtype = out_dtype or torch.float32
    n, d = X.shape
    m = w_codes.shape[0]
    Y = out if out is not None else torch.empty((n, m), dtype=out_dtype, device=X.device)
    r, a, w = rot.struct(), cb_a.struct(), cb_w.struct()
    yt = BF16 if Y.dtype == torch.bfloat16 else F32
    _check(load().orbq_linear_noalloc(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), ctypes.byref(a), eps,
                                      w_codes.data_ptr(), w_norms.data_ptr(), ctypes.byref(w), m, _act(act),
                                      Y.data_ptr(), yt, Y.stride(0), _stream(torch, X.device)), "orbq_linear_noalloc")
    return Y


def linear_a16_workspace_bytes(n: int, d: int, m: int) -> int:
    """Bytes of orbq_linear_a16's workspace: one 16-token chunk of rotated bf16 tokens and
    their norms."""
    return int(load().orbq_linear_a16_workspace_bytes(n, d, m))


def linear_a16(X, rot: Rotation, w_codes, w_norms, cb_w: Codebook, out_dtype=None, workspace=None, out=None):
    """Weight-only product: Y [n, m] from bf16 tokens X [n, d] (rotated, not quantized) and
    folded weight codes (orbq_linear_a16)."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "linear_a16")
    out_dtype = out_dtype or torch.float32
    n, d = X.shape
    m = w_codes.shape[0]
    need = linear_a16_workspace_bytes(n, d, m)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    Y = out if out is not None else torch.empty((n, m), dtype=out_dtype, device=X.device)
    r, w = rot.struct(), cb_w.struct()
    _check(load().orbq_linear_a16(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), w_codes.data_ptr(),
                                  w_norms.data_ptr(), ctypes.byref(w), m, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), Y.data_ptr(),
                                  BF16 if Y.dtype == torch.bfloat16 else F32, Y.stride(0), _stream(torch, X.device)),
           "orbq_linear_a16")
    return Y


def flatness(X):
    """(rho3, rhoinf) fp32 [n] of bf16 rows X [n, d]: sqrt(d) ||x||_3^3 / ||x||_2^3 and
    sqrt(d) ||x||_inf / ||x||_2 (orbq_rpbh_flatness)."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "flatness")
    n, d = X.shape
    rho3 = torch.empty((n,), dtype=torch.float32, device=X.device)
    rhoinf = torch.empty((n,), dtype=torch.float32, device=X.device)
    _check(load().orbq_rpbh_flatness(X.data_ptr(), n, d, X.stride(0), rho3.data_ptr(), rhoinf.data_ptr(),
                                     _stream(torch, X.device)), "orbq_rpbh_flatness")
    return rho3, rhoinf


def rht_passes(rho3: float, rhoinf: float, d: int, vector_quantization: bool = False) -> int:
    """Composed passes the adaptive check asks for (orbq_rht_passes)."""
    r = load().orbq_rht_passes(float(rho3), float(rhoinf), d, int(vector_quantization))
    if r < 0:
        _check(r, "orbq_rht_passes")
    return r


def test_rotate(X, rot: Rotation):
    """Test-only: x' = Pi x (fp32 [n, d]) and s (fp32 [n]) as the quantize kernel computes them."""
    torch = _torch()
    _dev_tensor(X, torch.bfloat16, "test_rotate")
    n, d = X.shape
    xr = torch.empty((n, d), dtype=torch.float32, device=X.device)
    s = torch.empty((n,), dtype=torch.float32, device=X.device)
    r = rot.struct()
    _check(load().orbq_test_rotate(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), xr.data_ptr(), s.data_ptr(),
                                   _stream(torch, X.device)), "orbq_test_rotate")
    return xr, s


def test_quantize_t(t, cb: Codebook):
    """Test-only: the kernels' decision on given normalised values t (fp32) -> sign-magnitude codes."""
    torch = _torch()
    _dev_tensor(t, torch.float32, "test_quantize_t")
    out = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    c = cb.struct()
    _check(load().orbq_test_quantize_t(t.data_ptr(), t.numel(), ctypes.byref(c), out.data_ptr(),
                                       _stream(torch, t.device)), "orbq_test_quantize_t")
    return out


def test_mfma_rate(workgroups: int, iters: int, sink=None, device=None) -> float:
    """Test-only: launches the matrix-core rate probe (orbq_test_mfma_rate) on the current stream
    and returns the floating-point operations of the launch; time it with events."""
    torch = _torch()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if sink is None:
        sink = torch.empty((workgroups * 512,), dtype=torch.float32, device=dev)
    flops = ctypes.c_double(0.0)
    _check(load().orbq_test_mfma_rate(workgroups, iters, sink.data_ptr(), ctypes.byref(flops), _stream(torch, dev)),
           "orbq_test_mfma_rate")
    return flops.value
