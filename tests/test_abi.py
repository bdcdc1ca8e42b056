"""CPU tests of the C-ABI library: it loads, exports what include/orbq.h declares, its
host-only calls work, and every argument error is caught before anything is launched.
No GPU is needed: no call here reaches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import calibration_free_w4a4_amd as orbq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orbq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(orbq.library_path()), reason="liborbq.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(orbq_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(orbq.library_path())
    names = declared_functions()
    assert len(names) >= 13
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(orbq._SIGS), "binding signatures out of sync with the header"


@pytest.mark.parametrize("d,bits", [(256, 4), (3072, 4), (3072, 2), (12288, 4), (1536, 6), (8960, 6),
                                    (1536, 4), (8960, 4), (3072, 3), (256, 3)])
def test_library_codebook_matches_oracle(d, bits, cb):
    lib_c = orbq.Codebook.lloyd_max(d, bits).centroids
    ref = oracle.lloyd_max(d, bits)
    assert np.max(np.abs(lib_c.astype(np.float64) - ref) / np.abs(ref)) < 1e-6   # fp32 rounding
    # both converge to the unique optimum (f_d is log-concave): the fp32 codebooks coincide
    assert np.array_equal(lib_c, cb(d, bits))


def test_library_codebook_float64_agreement():
    """The library's float64 iterate agrees with the oracle's far below fp32 resolution:
    checked through the fp32 result of a 1-bit codebook, whose value has a closed form."""
    c = orbq.Codebook.lloyd_max(3072, 1).centroids
    assert c[1] == np.float32(oracle.mean_abs_t(3072)) and c[0] == -c[1]


def test_rpbh_validate():
    lib = orbq.load()
    d = 256
    perm = np.random.default_rng(0).permutation(d).astype(np.int32)
    signs = np.ones(d, np.int8)
    assert lib.orbq_rpbh_validate(d, 64, perm.ctypes.data, signs.ctypes.data) == 0
    bad = perm.copy(); bad[3] = bad[4]
    assert lib.orbq_rpbh_validate(d, 64, bad.ctypes.data, signs.ctypes.data) == -1
    bad = perm.copy(); bad[0] = d
    assert lib.orbq_rpbh_validate(d, 64, bad.ctypes.data, signs.ctypes.data) == -1
    s2 = signs.copy(); s2[7] = 0
    assert lib.orbq_rpbh_validate(d, 64, perm.ctypes.data, s2.ctypes.data) == -1
    assert lib.orbq_rpbh_validate(d, 32, perm.ctypes.data, signs.ctypes.data) == -2
    assert lib.orbq_rpbh_validate(192, 128, perm.ctypes.data, signs.ctypes.data) == -1
    # Hadamard blocks: powers of two in [64, 4096] dividing d; perm NULL = identity
    p2 = np.random.default_rng(1).permutation(8192).astype(np.int32)
    s2 = np.ones(8192, np.int8)
    for blk, want in ((64, 0), (256, 0), (1024, 0), (2048, 0), (4096, 0), (8192, -2), (96, -2), (32, -2)):
        assert lib.orbq_rpbh_validate(8192, blk, p2.ctypes.data, s2.ctypes.data) == want, blk
    assert lib.orbq_rpbh_validate(12288, 4096, None, np.ones(12288, np.int8).ctypes.data) == 0
    assert lib.orbq_rpbh_validate(12288, 8192, None, np.ones(12288, np.int8).ctypes.data) == -2
    assert lib.orbq_rpbh_validate(6144, 4096, None, np.ones(6144, np.int8).ctypes.data) == -1  # 4096 does not divide d
    assert lib.orbq_rpbh_validate(8192, 512, None, s2.ctypes.data) == 0
    assert lib.orbq_rpbh_validate(8192, 512, p2.ctypes.data, None) == -1


def _cb_struct(c, d, bits):
    c = np.ascontiguousarray(c, np.float32)
    return orbq._Codebook(d, bits, c.ctypes.data_as(ctypes.POINTER(ctypes.c_float))), c


def test_codebook_validate(cb):
    lib = orbq.load()
    good = cb(256, 4)
    s, keep = _cb_struct(good, 256, 4)
    assert lib.orbq_codebook_validate(ctypes.byref(s)) == 0
    for broken in (good[::-1].copy(), np.where(np.arange(16) == 3, good * 1.0001, good)):
        s, keep = _cb_struct(broken, 256, 4)
        assert lib.orbq_codebook_validate(ctypes.byref(s)) == -6
    nan = good.copy(); nan[5] = np.nan
    s, keep = _cb_struct(nan, 256, 4)
    assert lib.orbq_codebook_validate(ctypes.byref(s)) == -6
    s, keep = _cb_struct(np.linspace(-1, 1, 32), 256, 5)
    assert lib.orbq_codebook_validate(ctypes.byref(s)) == -2


def test_sizes():
    lib = orbq.load()
    assert lib.orbq_codes_row_bytes(3072, 4) == 1536
    assert lib.orbq_codes_row_bytes(3072, 2) == 768
    assert lib.orbq_codes_row_bytes(8960, 6) == 6720
    assert lib.orbq_codes_row_bytes(3, 2) == 0
    ws = lib.orbq_linear_workspace_bytes(4608, 3072, 4)
    assert ws == ((4608 * 1536 + 255) // 256) * 256 + 4608 * 4
    assert lib.orbq_linear_workspace_bytes(10, 3072, 5) == 0
    assert lib.orbq_linear_workspace_bytes(10, 3072, 3) == ((10 * 1152 + 255) // 256) * 256 + 40
    # 6-bit activations: the layer keeps their bf16 centroids, 2 d bytes per token
    assert lib.orbq_linear_workspace_bytes(10, 1536, 6) == ((10 * 3072 + 255) // 256) * 256 + 40


def test_status_strings():
    lib = orbq.load()
    for code, name in ((0, b"ORBQ_OK"), (-1, b"ORBQ_ERR_INVALID_ARG"), (-4, b"ORBQ_ERR_WORKSPACE"),
                       (-6, b"ORBQ_ERR_CODEBOOK")):
        assert lib.orbq_status_string(code) == name


def test_argument_errors_return_before_launch(cb):
    """Every argument error is reported synchronously with its status; none needs a GPU."""
    lib = orbq.load()
    d = 256
    c4, keep4 = _cb_struct(cb(d, 4), d, 4)
    rot = orbq._Rpbh(d, 64, 0x1000, 0x2000)     # device arrays are never dereferenced on the host
    P = 0x10000                                  # a 16-byte aligned dummy device address
    q = lib.orbq_rpbh_quantize
    # bad shapes / arguments
    assert q(P, 8, d, d - 1, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, None) == -1      # ld < d
    assert q(P, -1, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, None) == -1         # n < 0
    assert q(None, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, None) == -1       # NULL X
    assert q(P + 2, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, None) == -3      # misaligned
    assert q(P, 8, d, d + 4, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, None) == -3      # pitch
    assert q(P, 8, d, d, None, ctypes.byref(c4), 1e-8, P, P, None) == -1                       # no rotation
    assert q(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), float("nan"), P, P, None) == -1  # eps
    rot32 = orbq._Rpbh(d, 32, 0x1000, 0x2000)
    assert q(P, 8, d, d, ctypes.byref(rot32), ctypes.byref(c4), 1e-8, P, P, None) == -2        # block
    dd = 8192
    cdd, keepdd = _cb_struct(cb(dd, 4), dd, 4)
    rot4k2 = orbq._Rpbh(dd, 4096, 0x1000, 0x2000, 2)
    assert q(P, 8, dd, dd, ctypes.byref(rot4k2), ctypes.byref(cdd), 1e-8, P, P, None) == -2    # passes, block 4096
    rot_mis = orbq._Rpbh(d, 64, 0x1004, 0x2000)
    assert q(P, 8, d, d, ctypes.byref(rot_mis), ctypes.byref(c4), 1e-8, P, P, None) == -3      # perm alignment
    c4d, keep = _cb_struct(cb(d, 4), 512, 4)
    assert q(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4d), 1e-8, P, P, None) == -1         # codebook d
    c5, keep5 = _cb_struct(np.linspace(-1, 1, 32), d, 5)
    assert q(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c5), 1e-8, P, P, None) == -2          # bits
    c3, keep3 = _cb_struct(cb(d, 3), d, 3)
    g0 = lib.orbq_lut_gemm
    assert g0(P, P, ctypes.byref(c3), P, P, ctypes.byref(c4), 8, 8, d, P, 0, 8, None) == -2      # 3-bit with 4-bit
    assert "ld" in lib.orbq_last_error().decode() or lib.orbq_last_error()
    # n == 0 is a no-op that succeeds without touching the device
    assert q(None, 0, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, None, None, None) == 0
    # gemm
    g = lib.orbq_lut_gemm
    assert g(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 8, d, P, 0, 4, None) == -1       # ldy < m
    assert g(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 8, d, P + 4, 0, 8, None) == -3   # Y misaligned
    assert g(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 4, d, P, 0, 6, None) == -3       # fp32 pitch
    assert g(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 8, d, P, 7, 8, None) == -1       # y_type
    assert g(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 0, 8, d, P, 0, 8, None) == 0        # empty
    # linear workspace
    ln = lib.orbq_linear
    need = lib.orbq_linear_workspace_bytes(8, d, 4)
    assert ln(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, ctypes.byref(c4), 8, P, need - 1,
              P, 0, 8, None) == -4
    assert ln(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, ctypes.byref(c4), 8, None, need,
              P, 0, 8, None) == -4
    assert ln(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, ctypes.byref(c4), 8, P + 16, need,
              P, 0, 8, None) == -3
    # composed passes: 0..3 accepted, others unsupported (checked before any launch)
    rot4 = orbq._Rpbh(d, 64, 0x1000, 0x2000, 4)
    assert q(P, 8, d, d, ctypes.byref(rot4), ctypes.byref(c4), 1e-8, P, P, None) == -2
    rotm = orbq._Rpbh(d, 64, 0x1000, 0x2000, -1)
    assert q(P, 8, d, d, ctypes.byref(rotm), ctypes.byref(c4), 1e-8, P, P, None) == -2
    assert q(None, 0, d, d, ctypes.byref(orbq._Rpbh(d, 64, 0x1000, 0x2000, 3)), ctypes.byref(c4), 1e-8,
             None, None, None) == 0
    # activation entry points
    ga = lib.orbq_lut_gemm_act
    assert ga(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 8, d, 3, P, 0, 8, None) == -1   # activation
    assert ga(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 8, 8, d, 1, P, 0, 4, None) == -1   # ldy < m
    assert ga(P, P, ctypes.byref(c4), P, P, ctypes.byref(c4), 0, 8, d, 2, P, 0, 8, None) == 0    # empty
    la = lib.orbq_linear_act
    assert la(P, 8, d, d, ctypes.byref(rot), ctypes.byref(c4), 1e-8, P, P, ctypes.byref(c4), 8, P, need,
              -1, P, 0, 8, None) == -1
    # weight-only product
    a16 = lib.orbq_linear_a16
    wsa = lib.orbq_linear_a16_workspace_bytes(8, d, 8)
    assert wsa > 0 and lib.orbq_linear_a16_workspace_bytes(8, 192, 8) == 0
    assert a16(P, 8, d, d, ctypes.byref(rot), P, P + 1, ctypes.byref(c4), 8, P, wsa, P, 0, 8, None) == -3  # w_norms
    assert a16(P, 8, d, d, ctypes.byref(rot), P + 8, P, ctypes.byref(c4), 8, P, wsa, P, 0, 8, None) == -3  # codes
    assert a16(P, 8, d, d, ctypes.byref(rot), P, P + 2, ctypes.byref(c4), 8, P, wsa - 1, P, 0, 8, None) == -4
    assert a16(P, 8, d, d, ctypes.byref(rot), P, P + 2, ctypes.byref(c4), 8, P + 16, wsa, P, 0, 8, None) == -3
    assert a16(P, 8, d, d, ctypes.byref(rot), P, P + 2, ctypes.byref(c4), 8, P, wsa, P, 0, 4, None) == -1  # ldy
    assert a16(P, 8, d, d, ctypes.byref(rot), P, P + 2, ctypes.byref(c4), 8, P, wsa, P, 5, 8, None) == -1  # y_type
    assert a16(P, 0, d, d, ctypes.byref(rot), P, P, ctypes.byref(c4), 8, None, 0, P, 0, 8, None) == 0
    rot192 = orbq._Rpbh(192, 64, 0x1000, 0x2000)
    c192, keep192 = _cb_struct(cb(192, 4), 192, 4)
    assert a16(P, 8, 192, 192, ctypes.byref(rot192), P, P, ctypes.byref(c192), 8, P, 1 << 20, P, 0, 8, None) == -2
    # flatness
    fl = lib.orbq_rpbh_flatness
    assert fl(P, 8, d, d - 8, P, P, None) == -1          # ldx < d
    assert fl(P, 8, 252, 256, P, P, None) == -2          # d not a multiple of 8
    assert fl(P + 2, 8, d, d, P, P, None) == -3          # misaligned rows
    assert fl(None, 0, d, d, None, None, None) == 0      # empty
    # quantize_t
    assert lib.orbq_test_quantize_t(P, -1, ctypes.byref(c4), P, None) == -1
    assert lib.orbq_test_quantize_t(P, 0, ctypes.byref(c4), P, None) == 0
    # matrix-core probe: range and pointer checks before any launch
    fl_out = ctypes.c_double(-1.0)
    probe = lib.orbq_test_mfma_rate
    assert probe(0, 400, P, ctypes.byref(fl_out), None) == -1           # no workgroups
    assert probe(65537, 400, P, ctypes.byref(fl_out), None) == -1       # too many
    assert probe(256, 402, P, ctypes.byref(fl_out), None) == -1         # iters not a multiple of 4
    assert probe(256, 0, P, ctypes.byref(fl_out), None) == -1
    assert probe(256, (1 << 24) + 4, P, ctypes.byref(fl_out), None) == -1
    assert probe(256, 400, None, ctypes.byref(fl_out), None) == -1      # NULL sink
    assert probe(256, 400, P, None, None) == -1                         # NULL flops
    assert probe(256, 400, P + 2, ctypes.byref(fl_out), None) == -3     # misaligned sink
    assert fl_out.value == -1.0                                        # nothing written on error


def test_rht_passes_rule():
    """Host rule of the adaptive check: against a Gaussian row's statistics."""
    import math
    lib = orbq.load()
    d = 3072
    g3 = 2 * math.sqrt(2 / math.pi)
    ginf = math.sqrt(2 * math.log(2 * d))
    assert lib.orbq_rht_passes(1.0, 1.0, d, 0) == 1               # constant row
    assert lib.orbq_rht_passes(g3, 4.0, d, 0) == 1                # Gaussian-like
    assert lib.orbq_rht_passes(math.sqrt(d), math.sqrt(d), d, 0) == 2   # one-hot
    assert lib.orbq_rht_passes(math.sqrt(d), math.sqrt(d), d, 1) == 3
    assert lib.orbq_rht_passes(1.0, ginf * 0.99, d, 1) == 1
    assert lib.orbq_rht_passes(1.0, ginf * 1.5, d, 1) == 2
    assert lib.orbq_rht_passes(-1.0, 1.0, d, 0) == -1
    assert lib.orbq_rht_passes(float("nan"), 1.0, d, 0) == -1
