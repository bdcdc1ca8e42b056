"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Tolerances (the layer's stated parity bar):
  * codes bit-exact except coordinates within 1e-5 (t units) of a decision boundary,
    counted, at most 1e-5 of all coordinates;
  * product from identical codes within 2e-3 max error relative to s_i r'_j sum|C_a C_w|
    (fp32 accumulation gives ~1e-6);
  * s within 1e-6 relative; r' equal to the oracle's bf16 or one bf16 ulp away when the
    exact norm sits within 1e-6 (relative) of a bf16 rounding midpoint.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import oracle_codebook
from tests.gpu_common import (check_codes, check_rprime, dense_pi, dev_bf16, gemm_error, host_bits, log,
                              torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orbq():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import calibration_free_w4a4_amd as m
    m.load()
    return m


def gpu_codebook(orbq, d, bits):
    cb = orbq.Codebook.lloyd_max(d, bits)
    ref = oracle_codebook(d, bits)
    assert np.array_equal(cb.centroids, ref), "library and oracle codebooks differ"
    return cb, ref


def gpu_rotation(orbq, d, h):
    perm, signs = workloads.rotation(d)
    return orbq.Rotation.create(d, h, perm, signs)


# ----------------------------------------------------------------- decision rule
@pytest.mark.parametrize("d,bits", [(256, 4), (3072, 4), (3072, 2), (1536, 6), (8960, 6), (12288, 4), (3072, 3),
                                    (256, 3)])
def test_quantize_t_exact(orbq, d, bits):
    """The kernels' decision on given fp32 t equals the oracle's exact argmin, bit for bit,
    including every boundary, its fp32 neighbours, zeros, denormals and far tails."""
    torch = torch_mod()
    log(f"quantize_t d={d} bits={bits}")
    cb, c = gpu_codebook(orbq, d, bits)
    m = oracle.thresholds_midpoint(c)
    probes = [np.float32(x) for x in (0.0, -0.0, 1e-45, -1e-45, 1e-38, -1e-38, 1.0, -1.0, 0.999, -0.999)]
    for mid in m:
        f = np.float32(mid)
        for k in range(-3, 4):
            probes.append(np.float32(f + k * np.spacing(f)) if k else f)
    t = np.concatenate([np.array(probes, np.float32), c,
                        (np.random.default_rng(d).standard_normal(200000) / math.sqrt(d)).astype(np.float32),
                        np.linspace(-2 * c[-1], 2 * c[-1], 100001, dtype=np.float32)])
    got = orbq.test_quantize_t(torch.from_numpy(t).cuda(), cb).cpu().numpy().astype(np.int64)
    ref = oracle.to_sign_magnitude(oracle.argmin_codes(t.astype(np.float64), c), bits)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} decisions differ, first t={t[bad[:5]]} gpu={got[bad[:5]]} ref={ref[bad[:5]]}"


# ----------------------------------------------------------------- rotation
@pytest.mark.parametrize("d,h,n", [(256, 64, 64), (3072, 128, 19), (1536, 128, 9), (8960, 128, 5),
                                   (12288, 128, 3), (384, 128, 7)])
def test_rotation_matches_dense_matrix(orbq, d, h, n):
    log(f"rotate d={d} h={h} n={n}")
    rot = gpu_rotation(orbq, d, h)
    X = workloads.activations(n, d, seed=1000 + d, kind="heavy", outlier_frac=0.002)
    xr, s = orbq.test_rotate(dev_bf16(X), rot)
    xr, s = xr.cpu().numpy().astype(np.float64), s.cpu().numpy().astype(np.float64)
    Xf = workloads.f64_from_bf16_bits(X)
    ref = oracle.rotate(Xf, dense_pi(d, h))
    nrm = np.linalg.norm(Xf, axis=1)
    err = np.abs(xr - ref) / nrm[:, None]
    assert err.max() < 1e-5, err.max()
    assert np.sqrt(np.mean(err ** 2)) < 1e-6
    assert np.max(np.abs(s - nrm) / nrm) < 1e-6


@pytest.mark.parametrize("d,h,ident", [(3072, 256, False), (3072, 512, False), (3072, 1024, False),
                                        (1024, 1024, False), (3072, 128, True), (3072, 1024, True),
                                        (512, 64, True), (8192, 2048, False), (8192, 4096, False),
                                        (12288, 4096, False), (12288, 4096, True), (4096, 4096, True)])
def test_rotation_large_blocks_and_identity(orbq, d, h, ident):
    """Hadamard blocks of 256..4096 (cross-lane stages by DPP row mirrors, swizzle and lane
    exchange; the stages of 2048- and 4096-wide blocks that cross waves through LDS) and the
    identity permutation (perm = NULL), against the dense matrix."""
    log(f"rotate d={d} h={h} identity={ident}")
    perm, signs = workloads.rotation(d)
    rot = orbq.Rotation.create(d, h, None if ident else perm, signs)
    X = workloads.activations(9, d, seed=2000 + d + h, kind="heavy", outlier_frac=0.002)
    xr, s = orbq.test_rotate(dev_bf16(X), rot)
    xr, s = xr.cpu().numpy().astype(np.float64), s.cpu().numpy().astype(np.float64)
    Xf = workloads.f64_from_bf16_bits(X)
    Pi = oracle.rpbh_matrix(d, h, np.arange(d) if ident else perm, signs)
    ref = oracle.rotate(Xf, Pi)
    nrm = np.linalg.norm(Xf, axis=1)
    err = np.abs(xr - ref) / nrm[:, None]
    assert err.max() < 1e-5, err.max()
    assert np.max(np.abs(s - nrm) / nrm) < 1e-6


@pytest.mark.parametrize("d,h,ident,weights", [(3072, 1024, False, False), (3072, 128, True, False),
                                                (3072, 512, True, True), (12288, 4096, False, False),
                                                (12288, 4096, True, False), (8192, 2048, False, True)])
def test_quantize_large_blocks_and_identity(orbq, d, h, ident, weights):
    """Codes and norms with the larger blocks (up to 4096, the largest power of two dividing the
    FLUX hidden width 12288) and without the permutation, against the oracle."""
    n = 131 if d <= 3072 else 37
    perm, signs = workloads.rotation(d)
    rot = orbq.Rotation.create(d, h, None if ident else perm, signs)
    cb, c = gpu_codebook(orbq, d, 4)
    src = workloads.activations(n, d, seed=3000 + h, kind="heavy") if not weights else workloads.weights(n, d, 3001)
    if weights:
        codes, norms = orbq.fold_weights(dev_bf16(src), rot, cb)
        norms = norms.float()
    else:
        codes, norms = orbq.rpbh_quantize(dev_bf16(src), rot, cb)
    Pi = oracle.rpbh_matrix(d, h, np.arange(d) if ident else perm, signs)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(src), Pi, c)
    check_codes(oracle.unpack_codes(codes.cpu().numpy(), 4, d), k_ref, T_ref, c, f"h={h} identity={ident}")
    got = norms.cpu().numpy().astype(np.float64)
    if weights:
        check_rprime(got, s_ref, "r'")
    else:
        assert np.max(np.abs(got - s_ref) / s_ref) < 1e-6


@pytest.mark.parametrize("d,h,passes,ident", [(3072, 128, 2, False), (3072, 128, 3, False), (256, 64, 3, False),
                                               (1024, 1024, 2, True), (3072, 256, 2, True), (1536, 512, 2, False)])
def test_rotation_composed_passes(orbq, d, h, passes, ident):
    """Composed RPBH passes (each with its own permutation and signs; identity permutations
    keep the later passes in registers) against the oracle's dense product of the passes."""
    log(f"rotate d={d} h={h} passes={passes} identity={ident}")
    perm, signs = workloads.rotation_passes(d, passes)
    rot = orbq.Rotation.create(d, h, None if ident else perm, signs, passes=passes)
    X = workloads.activations(11, d, seed=4000 + d + passes, kind="heavy", outlier_frac=0.002)
    xr, s = orbq.test_rotate(dev_bf16(X), rot)
    xr, s = xr.cpu().numpy().astype(np.float64), s.cpu().numpy().astype(np.float64)
    Xf = workloads.f64_from_bf16_bits(X)
    ref = oracle.rotate(Xf, oracle.rpbh_composed(d, h, None if ident else perm, signs, passes))
    nrm = np.linalg.norm(Xf, axis=1)
    err = np.abs(xr - ref) / nrm[:, None]
    assert err.max() < 1e-5, err.max()
    assert np.max(np.abs(s - nrm) / nrm) < 1e-6


@pytest.mark.parametrize("passes,weights,kind", [(2, False, "heavy"), (2, True, "weights"), (3, False, "spikes")])
def test_quantize_composed_passes(orbq, passes, weights, kind):
    """Codes and norms through composed passes against the oracle, including one-hot tokens
    (the inputs a single pass handles worst)."""
    d, h, n = 3072, 128, 77
    perm, signs = workloads.rotation_passes(d, passes)
    rot = orbq.Rotation.create(d, h, perm, signs, passes=passes)
    cb, c = gpu_codebook(orbq, d, 4)
    if kind == "spikes":
        # a spike per token plus a little noise (exact one-hot rows rotate onto a lattice of
        # t values, which may sit within the boundary tolerance of a threshold)
        f = workloads.f64_from_bf16_bits(workloads.activations(n, d, seed=6)) * 1e-2
        f[np.arange(n), np.random.default_rng(5).integers(0, d, n)] += 3.0
        src = workloads.bf16_bits_from_f64(f)
    elif kind == "weights":
        src = workloads.weights(n, d, 3101)
    else:
        src = workloads.activations(n, d, seed=3100, kind="heavy")
    if weights:
        codes, norms = orbq.fold_weights(dev_bf16(src), rot, cb)
        norms = norms.float()
    else:
        codes, norms = orbq.rpbh_quantize(dev_bf16(src), rot, cb)
    Pi = oracle.rpbh_composed(d, h, perm, signs, passes)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(src), Pi, c)
    check_codes(oracle.unpack_codes(codes.cpu().numpy(), 4, d), k_ref, T_ref, c, f"passes={passes} {kind}")
    got = norms.cpu().numpy().astype(np.float64)
    if weights:
        check_rprime(got, s_ref, "r'")
    else:
        assert np.max(np.abs(got - s_ref) / s_ref) < 1e-6


def test_flatness_statistics(orbq):
    """orbq_rpbh_flatness against the oracle on heavy-tailed tokens plus a zero, a constant and
    a one-hot row (ragged row count); orbq_rht_passes on their statistics."""
    torch = torch_mod()
    d, n = 3072, 1003
    X = workloads.activations(n, d, seed=77, kind="heavy")
    X[5] = 0
    X[6] = workloads.bf16_bits_from_f64(np.full(d, 0.75))
    X[7] = 0; X[7, 123] = workloads.bf16_bits_from_f64(np.array([-2.0]))[0]
    r3, ri = orbq.flatness(dev_bf16(X))
    torch.cuda.synchronize()
    r3, ri = r3.cpu().numpy().astype(np.float64), ri.cpu().numpy().astype(np.float64)
    e3, ei = oracle.flatness(workloads.f64_from_bf16_bits(X))
    assert np.max(np.abs(r3 - e3) / np.maximum(e3, 1e-30)) < 2e-5
    assert np.max(np.abs(ri - ei) / np.maximum(ei, 1e-30)) < 2e-5
    assert r3[5] == 0 and ri[5] == 0
    assert abs(r3[6] - 1) < 1e-5 and abs(ri[6] - 1) < 1e-5
    assert abs(r3[7] - math.sqrt(d)) < 1e-3 and abs(ri[7] - math.sqrt(d)) < 1e-3
    assert orbq.rht_passes(r3[7], ri[7], d) == 2 and orbq.rht_passes(r3[7], ri[7], d, True) == 3
    assert orbq.rht_passes(r3[6], ri[6], d) == 1 and orbq.rht_passes(r3[6], ri[6], d, True) == 1
    assert orbq.flatness(dev_bf16(X[:0]))[0].numel() == 0


# ----------------------------------------------------------------- quantize / fold
def _quant_case(orbq, name, rows=None, sample=None, weights=False):
    torch = torch_mod()
    L = workloads.CONFIGS[name]
    bits = L.bits_w if weights else L.bits_a
    X, W = workloads.layer_inputs(L, rows=rows)
    src = W if weights else X
    log(f"quantize {name} weights={weights} shape={src.shape} bits={bits}")
    rot = gpu_rotation(orbq, L.d, L.block)
    cb, c = gpu_codebook(orbq, L.d, bits)
    dsrc = dev_bf16(src)
    if weights:
        codes, norms = orbq.fold_weights(dsrc, rot, cb)
    else:
        codes, norms = orbq.rpbh_quantize(dsrc, rot, cb)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    norms = (norms.float() if weights else norms).cpu().numpy().astype(np.float64)
    idx = np.arange(src.shape[0]) if sample is None else sample(src.shape[0])
    Sf = workloads.f64_from_bf16_bits(src[idx])
    Pi = dense_pi(L.d, L.block)
    k_ref, s_ref, T_ref = oracle.quantize_activations(Sf, Pi, c)
    k_gpu = oracle.unpack_codes(codes[idx], bits, L.d)
    check_codes(k_gpu, k_ref, T_ref, c, f"{name} codes")
    if weights:
        check_rprime(norms[idx], s_ref, f"{name} r'")
    else:
        assert np.max(np.abs(norms[idx] - s_ref) / s_ref) < 1e-6
    return codes, norms


def _sample_rows(n, k=48, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1, n // 2], rng.choice(n, size=min(k, n), replace=False)]))


def test_quantize_tiny_full(orbq):
    _quant_case(orbq, "tiny")


def test_fold_tiny_full(orbq):
    _quant_case(orbq, "tiny", weights=True)


@pytest.mark.parametrize("name,rows", [("flux_qkv", 515), ("flux_mlp_up_w2a4", 130), ("wan_ffn_up", 257),
                                       ("wan_ffn_down", 67), ("flux_mlp_down", 33)])
def test_quantize_ragged_full_compare(orbq, name, rows):
    """Several workgroups and a ragged last group, every coordinate compared."""
    _quant_case(orbq, name, rows=rows)


@pytest.mark.parametrize("name", ["flux_qkv", "flux_mlp_up_w2a4", "wan_ffn_up"])
def test_fold_weights_sampled(orbq, name):
    _quant_case(orbq, name, weights=True, sample=lambda n: _sample_rows(n, 40, 1))


@pytest.mark.parametrize("d,h,bits,n,weights", [(256, 64, 3, 37, False), (1536, 128, 6, 35, False),
                                                (3072, 128, 2, 19, True), (8960, 128, 6, 7, False),
                                                (256, 64, 4, 70, True), (3072, 128, 3, 5, True),
                                                (12288, 128, 4, 3, False), (1536, 128, 4, 1, True)])
def test_quantize_outputs_every_byte_written(orbq, d, h, bits, n, weights):
    """Code and norm buffers filled with 0xFF before the call come out byte-identical to a run
    into zero-filled buffers: every byte of every row is written, the 3- and 6-bit row tails and
    the ragged last token group included, and nothing past the outputs (a 0xFF guard row after
    them stays untouched)."""
    torch = torch_mod()
    log(f"poisoned outputs d={d} h={h} bits={bits} n={n} weights={weights}")
    rot = gpu_rotation(orbq, d, h)
    cb, _ = gpu_codebook(orbq, d, bits)
    src = workloads.weights(n, d, 700 + d) if weights else workloads.activations(n, d, 701 + d, kind="heavy")
    dsrc = dev_bf16(src)
    rb = orbq.codes_row_bytes(d, bits)
    ndt = torch.bfloat16 if weights else torch.float32
    outs = []
    for fill in (0xFF, 0x00):
        codes = torch.full((n + 1, rb), fill, dtype=torch.uint8, device="cuda")
        norms = torch.empty((n + 1,), dtype=ndt, device="cuda")
        norms.view(torch.int16 if weights else torch.int32).fill_(-1 if fill else 0)
        f = orbq.fold_weights if weights else orbq.rpbh_quantize
        f(dsrc, rot, cb, out_codes=codes[:n], out_norms=norms[:n])
        torch.cuda.synchronize()
        outs.append((codes.cpu().numpy(), norms.view(torch.uint8).cpu().numpy()))
    (c1, n1), (c0, n0) = outs
    assert np.array_equal(c1[:n], c0[:n]), "a code byte kept its fill value"
    esz = 2 if weights else 4
    assert np.array_equal(n1[:n * esz], n0[:n * esz]), "a norm byte kept its fill value"
    assert (c1[n] == 0xFF).all() and (c0[n] == 0).all(), "codes written past the last row"
    assert (n1[n * esz:] == 0xFF).all() and (n0[n * esz:] == 0).all(), "norms written past the last row"


@pytest.mark.parametrize("d,h,n,weights", [(3072, 128, 333, False), (3072, 128, 97, True), (256, 64, 70, False)])
def test_quantize_3bit(orbq, d, h, n, weights):
    """3-bit codes (W3A3): 16 codes per lane in 6 bytes (three 16-bit stores at 2-byte aligned
    offsets), every coordinate against the oracle; ragged last group."""
    log(f"quantize 3-bit d={d} n={n} weights={weights}")
    rot = gpu_rotation(orbq, d, h)
    cb, c = gpu_codebook(orbq, d, 3)
    src = workloads.weights(n, d, 1301) if weights else workloads.activations(n, d, seed=1300, kind="heavy")
    if weights:
        codes, norms = orbq.fold_weights(dev_bf16(src), rot, cb)
        norms = norms.float()
    else:
        codes, norms = orbq.rpbh_quantize(dev_bf16(src), rot, cb)
    assert codes.shape == (n, d * 3 // 8)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(src), dense_pi(d, h), c)
    check_codes(oracle.unpack_codes(codes.cpu().numpy(), 3, d), k_ref, T_ref, c, "3-bit")
    got = norms.cpu().numpy().astype(np.float64)
    if weights:
        check_rprime(got, s_ref, "r'")
    else:
        assert np.max(np.abs(got - s_ref) / s_ref) < 1e-6


# ----------------------------------------------------------------- product
def _gemm_case(orbq, n, m, d, ba, bw, out_bf16=False, seed=7, sample=None):
    torch = torch_mod()
    log(f"gemm n={n} m={m} d={d} A{ba} W{bw} bf16={out_bf16}")
    ca_cb, ca = gpu_codebook(orbq, d, ba)
    cw_cb, cw = gpu_codebook(orbq, d, bw)
    xb = workloads.random_code_bytes(n, d * ba // 8, seed)
    wb = workloads.random_code_bytes(m, d * bw // 8, seed + 1)
    s = workloads.random_norms(n, seed + 2).astype(np.float32)
    r_bits = workloads.bf16_bits_from_f64(workloads.random_norms(m, seed + 3, 0.01, 0.1))
    Y = orbq.lut_gemm(torch.from_numpy(xb).cuda(), torch.from_numpy(s).cuda(), ca_cb,
                      torch.from_numpy(wb).cuda(), dev_bf16(r_bits), cw_cb, d,
                      out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    Yh = (Y.float() if out_bf16 else Y).cpu().numpy().astype(np.float64)
    r = workloads.f64_from_bf16_bits(r_bits)
    la, lw = oracle.decode_lut_bf16(ca), oracle.decode_lut_bf16(cw)
    if sample is None:
        A = la[oracle.unpack_codes(xb, ba, d)]
        B = lw[oracle.unpack_codes(wb, bw, d)]
        e = gemm_error(Yh, A, B, s.astype(np.float64), r)
    else:
        ii, jj = sample
        A = la[oracle.unpack_codes(xb[ii], ba, d)]
        B = lw[oracle.unpack_codes(wb[jj], bw, d)]
        e = gemm_error(Yh[np.ix_(ii, jj)], A, B, s[ii].astype(np.float64), r[jj])
    log(f"  max relative error {e:.3g}")
    tol = 2e-3 + (2.0 ** -8 if out_bf16 else 0.0)
    assert e <= tol
    return e


@pytest.mark.parametrize("n,m,d,out_bf16", [(1920, 12288, 256, True), (1000, 4096, 192, False),
                                             (4608, 12288, 128, True)])
def test_lut_gemm_grouped_tile_order(orbq, n, m, d, out_bf16):
    """Column-tile counts that divide by 8 take the grouped XCD order (groups of token tiles x an
    XCD's column tiles): 8 token tiles in groups of 5 (a short last group), 4 ragged token tiles in
    one short group with an odd K-tile count, and the headline's 12 token tiles in 3 groups of 4.
    Every output element against the oracle."""
    _gemm_case(orbq, n, m, d, 4, 4, out_bf16=out_bf16, seed=41)


@pytest.mark.parametrize("ba,bw", [(4, 4), (4, 2), (6, 4), (2, 2), (6, 6), (2, 6), (3, 3)])
def test_lut_gemm_tiny_all_bit_pairs(orbq, ba, bw):
    assert _gemm_case(orbq, 64, 256, 256, ba, bw) < 1e-5


@pytest.mark.parametrize("out_bf16", [False, True])
def test_lut_gemm_ragged(orbq, out_bf16):
    """Ragged n and m (partial tiles on both axes), several K tiles."""
    _gemm_case(orbq, 300, 520, 3072, 4, 4, out_bf16=out_bf16)


@pytest.mark.parametrize("n,m,d", [(300, 520, 3072), (70, 200, 192), (1000, 2100, 1536)])
def test_lut_gemm_w3a3(orbq, n, m, d):
    """3-bit x 3-bit: units of 8 codes at 3-byte offsets (8-byte loads from the aligned word
    below), ragged tiles, odd K-tile counts."""
    _gemm_case(orbq, n, m, d, 3, 3)


@pytest.mark.parametrize("ba,bw", [(4, 4), (6, 4), (2, 6)])
@pytest.mark.parametrize("d", [192, 320, 64])
def test_lut_gemm_odd_k_tile_count(orbq, ba, bw, d):
    """d / 64 odd: the kernel pads the K loop with a leading all-zero tile."""
    assert _gemm_case(orbq, 70, 200, d, ba, bw) < 1e-5


@pytest.mark.parametrize("ba,bw,out_bf16,d", [(4, 4, True, 512), (4, 4, False, 576), (6, 4, True, 512),
                                               (4, 2, True, 576), (3, 3, True, 576)])
def test_lut_gemm_wide_tiles_ragged(orbq, ba, bw, out_bf16, d):
    """Shapes for which the host picks 384 x 192 workgroup tiles, with partial tiles on both axes
    (last token tile 284 of 384 rows, last weight tile 136 of 192 rows) and even or odd K-tile
    counts; sampled outputs include the ragged borders."""
    n, m = 4508, 12232  # Y rows stay 16-byte aligned (m multiple of 8)
    ii = np.unique(np.concatenate([np.arange(0, 40), np.arange(4224 - 8, 4224 + 8), np.arange(n - 40, n)]))
    jj = np.unique(np.concatenate([np.arange(0, 40), np.arange(12096 - 8, 12096 + 8), np.arange(m - 40, m)]))
    _gemm_case(orbq, n, m, d, ba, bw, out_bf16=out_bf16, sample=(ii, jj))


def test_lut_gemm_from_oracle_codes(orbq):
    """The product of codes the oracle produced from real activations and weights."""
    torch = torch_mod()
    L = workloads.CONFIGS["tiny"]
    X, W = workloads.layer_inputs(L)
    Pi = dense_pi(L.d, L.block)
    cb, c = gpu_codebook(orbq, L.d, 4)
    kx, s, _ = oracle.quantize_activations(workloads.f64_from_bf16_bits(X), Pi, c)
    kw, r, _, _ = oracle.fold_weights(workloads.f64_from_bf16_bits(W), Pi, c)
    Y = orbq.lut_gemm(torch.from_numpy(oracle.pack_codes(kx, 4)).cuda(),
                      torch.from_numpy(s.astype(np.float32)).cuda(), cb,
                      torch.from_numpy(oracle.pack_codes(kw, 4)).cuda(),
                      dev_bf16(workloads.bf16_bits_from_f64(r)), cb, L.d)
    lut = oracle.decode_lut_bf16(c)
    e = gemm_error(Y.cpu().numpy().astype(np.float64), lut[kx], lut[kw],
                   s.astype(np.float32).astype(np.float64), r)
    assert e < 1e-5


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf"])
@pytest.mark.parametrize("out_bf16", [False, True])
@pytest.mark.parametrize("n,m", [(300, 520), (800, 400)])
def test_lut_gemm_activation(orbq, act, out_bf16, n, m):
    """GELU in the epilogue (orbq_lut_gemm_act) against the oracle's float64 GELU of the float64
    product.  Norms are scaled so that the outputs span the whole GELU (|Y| up to ~50: the
    curved middle and both tails); full and edge tiles."""
    torch = torch_mod()
    d, ba, bw, seed = 1536, 4, 4, 31
    log(f"gemm+{act} n={n} m={m} d={d} bf16={out_bf16}")
    ca_cb, ca = gpu_codebook(orbq, d, ba)
    cw_cb, cw = gpu_codebook(orbq, d, bw)
    xb = workloads.random_code_bytes(n, d * ba // 8, seed)
    wb = workloads.random_code_bytes(m, d * bw // 8, seed + 1)
    s = workloads.random_norms(n, seed + 2, 5.0, 20.0).astype(np.float32)
    s[::17] *= 20.0  # some rows far into the tails
    r_bits = workloads.bf16_bits_from_f64(workloads.random_norms(m, seed + 3, 1.0, 4.0))
    Y = orbq.lut_gemm(torch.from_numpy(xb).cuda(), torch.from_numpy(s).cuda(), ca_cb,
                      torch.from_numpy(wb).cuda(), dev_bf16(r_bits), cw_cb, d,
                      out_dtype=torch.bfloat16 if out_bf16 else torch.float32, act=act)
    torch.cuda.synchronize()
    G = (Y.float() if out_bf16 else Y).cpu().numpy().astype(np.float64)
    r = workloads.f64_from_bf16_bits(r_bits)
    A = oracle.decode_lut_bf16(ca)[oracle.unpack_codes(xb, ba, d)]
    B = oracle.decode_lut_bf16(cw)[oracle.unpack_codes(wb, bw, d)]
    Yref = oracle.lut_gemm(oracle.unpack_codes(xb, ba, d), s.astype(np.float64), ca,
                           oracle.unpack_codes(wb, bw, d), r, cw)
    Gref = oracle.activation(Yref, act)
    den = (np.abs(A) @ np.abs(B).T) * s.astype(np.float64)[:, None] * r[None, :]
    e = float(np.max(np.abs(G - Gref) / den))
    big = np.abs(Yref) > 0.5
    fe = float(np.max(np.abs(G - Gref)[big] / np.maximum(np.abs(Gref[big]), 1e-3)))
    log(f"  |Y| max {np.abs(Yref).max():.1f}; error / |dot| scale {e:.3g}; relative to |GELU(Y)| where |Y| > 0.5: {fe:.3g}")
    assert np.abs(Yref).max() > 20 and (Yref < -3).any() and (Yref > 3).any()
    # fp32: accumulation order and the fp32 GELU (< 1e-6 of |Y|); bf16 adds one rounding (2^-8)
    assert e <= (2.0 ** -8 + 1e-5 if out_bf16 else 1e-5)
    assert np.isfinite(G).all()


def test_lut_gemm_act_none_and_linear_act(orbq):
    """ACT_NONE through orbq_lut_gemm_act gives orbq_lut_gemm's bits; orbq_linear_act gives
    rpbh_quantize then lut_gemm_act's bits."""
    import ctypes
    torch = torch_mod()
    L = workloads.CONFIGS["tiny"]
    X, W = workloads.layer_inputs(L)
    rot = gpu_rotation(orbq, L.d, L.block)
    cb, _ = gpu_codebook(orbq, L.d, 4)
    dX, dW = dev_bf16(X), dev_bf16(W)
    wc, wn = orbq.fold_weights(dW, rot, cb)
    xc, xs = orbq.rpbh_quantize(dX, rot, cb)
    Y0 = orbq.lut_gemm(xc, xs, cb, wc, wn, cb, L.d)
    Y1 = torch.empty_like(Y0)
    a = cb.struct()
    st = orbq.load().orbq_lut_gemm_act(xc.data_ptr(), xs.data_ptr(), ctypes.byref(a), wc.data_ptr(), wn.data_ptr(),
                                       ctypes.byref(a), L.n, L.m, L.d, 0, Y1.data_ptr(), 0, Y1.stride(0),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0
    st = orbq.load().orbq_lut_gemm_act(xc.data_ptr(), xs.data_ptr(), ctypes.byref(a), wc.data_ptr(), wn.data_ptr(),
                                       ctypes.byref(a), L.n, L.m, L.d, 7, Y1.data_ptr(), 0, Y1.stride(0),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == -1  # unknown activation
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)
    for act in ("gelu_tanh", "gelu_erf"):
        for dt in (torch.float32, torch.bfloat16):
            G1 = orbq.linear(dX, rot, cb, wc, wn, cb, act=act, out_dtype=dt)
            G2 = orbq.lut_gemm(xc, xs, cb, wc, wn, cb, L.d, act=act, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(G1, G2), (act, dt)


@pytest.mark.parametrize("n,d,m,bw,out_bf16,passes", [
    (2, 3072, 18432, 4, False, 1), (1, 256, 100, 4, False, 1), (3, 3072, 777, 3, True, 1),
    (1, 12288, 3072, 4, False, 1), (5, 3072, 1000, 6, True, 1), (16, 1536, 1000, 6, True, 1),
    (37, 3072, 700, 2, False, 1), (5, 12288, 3072, 4, True, 1), (2, 3072, 600, 4, False, 2),
    (2, 3072, 16384, 4, True, 1), (3, 3072, 24576, 4, False, 1), (16, 3072, 12288, 4, True, 1),
    (16, 3072, 18432, 4, False, 1)])
def test_linear_a16_weight_only(orbq, n, d, m, bw, out_bf16, passes):
    """orbq_linear_a16 (bf16 activations rotated, weight codes decoded) against the oracle's
    weight-only product: 16-token chunks, a composed rotation, ragged m, 2/3/4/6-bit weights, the
    AdaLN modulation shape (2 x 3072 -> 18432), and workgroups of 2 to 5 16-row column blocks
    (on 256 compute units: m = 24576 takes 2, 12288 with 16 tokens 3, 16384 4, 18432 5, the last
    also with 16 tokens and the largest partial-sum buffer, 60 KB of LDS)."""
    torch = torch_mod()
    log(f"linear_a16 n={n} d={d} m={m} W{bw} bf16={out_bf16} passes={passes}")
    h = 64 if d == 256 else 128
    if passes == 1:
        rot = gpu_rotation(orbq, d, h)
    else:
        pp, sp = workloads.rotation_passes(d, passes)
        rot = orbq.Rotation.create(d, h, pp, sp, passes=passes)
    cb, c = gpu_codebook(orbq, d, bw)
    X = workloads.activations(n, d, seed=900 + n, kind="heavy")
    W = workloads.weights(m, d, 901)
    wc, wn = orbq.fold_weights(dev_bf16(W), rot, cb)
    Y = orbq.linear_a16(dev_bf16(X), rot, wc, wn, cb, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    Yg = Y.float().cpu().numpy().astype(np.float64)
    codes = oracle.unpack_codes(wc.cpu().numpy(), bw, d)
    r = wn.float().cpu().numpy().astype(np.float64)
    Pi = dense_pi(d, h) if passes == 1 else oracle.rpbh_composed(d, h, pp, sp, passes)
    Xf = workloads.f64_from_bf16_bits(X)
    Yo = oracle.linear_a16(Xf, Pi, codes, r, c)
    A = oracle.bf16_rne(oracle.rotate(Xf, Pi))
    den = (np.abs(A) @ np.abs(oracle.decode_lut_bf16(c)[codes]).T) * r[None, :]
    e = float(np.max(np.abs(Yg - Yo) / den))
    log(f"  max error / |dot| scale {e:.3g}")
    assert e <= 2e-3 + (2.0 ** -8 if out_bf16 else 0.0)
    # against the unquantized product: the weight quantization error only, within the
    # codebook's distortion bound (sqrt(3) pi / 2) 4^-b per coordinate, with 20 % slack
    ref = Xf @ workloads.f64_from_bf16_bits(W).T
    rel = np.linalg.norm(Yg - ref) / np.linalg.norm(ref)
    log(f"  ||Y - XW^T|| / ||XW^T|| = {rel:.4f}")
    assert rel < 1.2 * math.sqrt(math.sqrt(3) * math.pi / 2 * 4.0 ** -bw)


def test_linear_a16_workspace_reuse(orbq):
    """The weight-only product keeps rotated tokens and K-split partial sums in the caller's
    workspace: a workspace filled with 0xFF bytes, reused over calls of different shapes (3
    chunks of 16 tokens, then 2 tokens, then the first shape again), gives the same outputs as
    fresh zeroed workspaces, bit for bit (no call depends on what the workspace held)."""
    torch = torch_mod()
    d, h = 3072, 128
    rot = gpu_rotation(orbq, d, h)
    cb, c = gpu_codebook(orbq, d, 4)
    W = workloads.weights(1000, d, 911)
    wc, wn = orbq.fold_weights(dev_bf16(W), rot, cb)
    need = max(orbq.linear_a16_workspace_bytes(n, d, 1000) for n in (37, 2))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for n in (37, 2, 37):
        log(f"linear_a16 reused workspace: n={n}")
        X = dev_bf16(workloads.activations(n, d, seed=912 + n, kind="heavy"))
        Y = orbq.linear_a16(X, rot, wc, wn, cb, out_dtype=torch.bfloat16, workspace=ws)
        fresh = torch.zeros((orbq.linear_a16_workspace_bytes(n, d, 1000),), dtype=torch.uint8, device="cuda")
        Y0 = orbq.linear_a16(X, rot, wc, wn, cb, out_dtype=torch.bfloat16, workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))


@pytest.mark.parametrize("d,h,m,bw", [(3072, 128, 1000, 4), (1536, 64, 530, 2), (3072, 128, 700, 6)])
def test_linear_a16_rotation_inside_the_product(orbq, d, h, m, bw):
    """Chunks of a few tokens rotate inside the product (one launch); a 16-token chunk rotates in a
    launch of its own first.  Token rows are independent, so rows taken one or two at a time
    (the one-launch form) equal the same rows of a 16-token call (the two-launch form) bit for
    bit.  test_linear_a16_weight_only checks both forms against the oracle."""
    torch = torch_mod()
    rot = gpu_rotation(orbq, d, h)
    cb, c = gpu_codebook(orbq, d, bw)
    W = workloads.weights(m, d, 931 + bw)
    wc, wn = orbq.fold_weights(dev_bf16(W), rot, cb)
    Xb = workloads.activations(16, d, seed=932, kind="heavy")
    X = dev_bf16(Xb)
    log(f"linear_a16 one- and two-launch forms: d={d} h={h} m={m} bw={bw}")
    Y16 = orbq.linear_a16(X, rot, wc, wn, cb, out_dtype=torch.bfloat16)
    for t0, k in ((0, 1), (5, 2), (15, 1)):
        Yk = orbq.linear_a16(X[t0:t0 + k].contiguous(), rot, wc, wn, cb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(Yk.view(torch.int16), Y16[t0:t0 + k].view(torch.int16)), (t0, k)
    # rows with a pitch above d (ldx = d + 64) through the one-launch form
    wide = torch.zeros((2, d + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :d] = X[3:5]
    Yw = orbq.linear_a16(wide[:, :d], rot, wc, wn, cb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(Yw.view(torch.int16), Y16[3:5].view(torch.int16))


# ----------------------------------------------------------------- the layer
def test_linear_equals_quantize_then_gemm(orbq):
    torch = torch_mod()
    L = workloads.CONFIGS["tiny"]
    X, W = workloads.layer_inputs(L)
    rot = gpu_rotation(orbq, L.d, L.block)
    cb, c = gpu_codebook(orbq, L.d, 4)
    dX, dW = dev_bf16(X), dev_bf16(W)
    wc, wn = orbq.fold_weights(dW, rot, cb)
    Y = orbq.linear(dX, rot, cb, wc, wn, cb)
    xc, xs = orbq.rpbh_quantize(dX, rot, cb)
    Y2 = orbq.lut_gemm(xc, xs, cb, wc, wn, cb, L.d)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    # against the oracle chain end to end (codes may flip at boundaries)
    Pi = dense_pi(L.d, L.block)
    kw, r, _, _ = oracle.fold_weights(workloads.f64_from_bf16_bits(W), Pi, c)
    Yo, kx, s = oracle.orbq_linear(workloads.f64_from_bf16_bits(X), Pi, c, kw, r, c)
    lut = oracle.decode_lut_bf16(c)
    den = (np.abs(lut[kx]) @ np.abs(lut[kw]).T) * s[:, None] * r[None, :]
    e = np.max(np.abs(Y.cpu().numpy() - Yo) / den)
    log(f"  linear vs oracle chain: {e:.3g}")
    assert e < 2e-3
    # quantization error of the whole layer against the unquantized product (informational bound)
    ref = workloads.f64_from_bf16_bits(X) @ workloads.f64_from_bf16_bits(W).T
    rel = np.linalg.norm(Y.cpu().numpy() - ref) / np.linalg.norm(ref)
    log(f"  ||Y - XW^T|| / ||XW^T|| = {rel:.4f}")
    assert rel < 0.3


def test_linear_w3a3_end_to_end(orbq):
    """W3A3 layer: orbq_linear equals quantize-then-gemm bit for bit, and matches the oracle
    chain (codes may flip at boundaries) within 2e-3 of the |dot| scale."""
    torch = torch_mod()
    d, h, n, m = 3072, 128, 130, 400
    rot = gpu_rotation(orbq, d, h)
    cb, c = gpu_codebook(orbq, d, 3)
    X = workloads.activations(n, d, seed=1400, kind="heavy")
    W = workloads.weights(m, d, 1401)
    dX = dev_bf16(X)
    wc, wn = orbq.fold_weights(dev_bf16(W), rot, cb)
    Y = orbq.linear(dX, rot, cb, wc, wn, cb)
    xc, xs = orbq.rpbh_quantize(dX, rot, cb)
    Y2 = orbq.lut_gemm(xc, xs, cb, wc, wn, cb, d)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    Pi = dense_pi(d, h)
    kw, r, _, _ = oracle.fold_weights(workloads.f64_from_bf16_bits(W), Pi, c)
    Yo, kx, s = oracle.orbq_linear(workloads.f64_from_bf16_bits(X), Pi, c, kw, r, c)
    lut = oracle.decode_lut_bf16(c)
    den = (np.abs(lut[kx]) @ np.abs(lut[kw]).T) * s[:, None] * r[None, :]
    e = np.max(np.abs(Y.cpu().numpy() - Yo) / den)
    log(f"  W3A3 linear vs oracle chain: {e:.3g}")
    assert e < 2e-3


@pytest.mark.parametrize("n,d,h,m,bw,passes,act,out_bf16", [
    (130, 1536, 128, 2116, 4, 1, "none", False),      # ragged token and weight tiles
    (777, 320, 64, 2056, 4, 1, "gelu_tanh", True),    # an odd K-tile count (5), GELU epilogue
    (64, 3072, 128, 2048, 2, 2, "none", True),        # 2-bit weights, two composed RPBH passes
    (400, 512, 128, 2300, 6, 1, "gelu_erf", False),   # 6-bit weights (their pair table)
    (1, 1536, 128, 4096, 4, 1, "none", True),         # a single token
    (300, 1536, 128, 400, 4, 1, "none", False),       # m < 2048: the layer keeps the packed codes
])
def test_linear_a6_decoded_equals_codes_path(orbq, n, d, h, m, bw, passes, act, out_bf16):
    """6-bit activations: with m >= 2048 orbq_linear keeps the codes' bf16 centroids in its
    workspace and its product stages them without decoding.  Its output equals rpbh_quantize
    then lut_gemm on the packed codes bit for bit (the same bf16 products summed in the same
    order), and the first case also matches the oracle chain within 2e-3 of the |dot| scale."""
    torch = torch_mod()
    log(f"linear A6 decoded: n={n} d={d} h={h} m={m} W{bw} passes={passes} act={act} bf16={out_bf16}")
    perm, signs = workloads.rotation_passes(d, passes)
    rot = orbq.Rotation.create(d, h, perm, signs, passes=passes)
    cba, ca = gpu_codebook(orbq, d, 6)
    cbw, cw = gpu_codebook(orbq, d, bw)
    X = workloads.activations(n, d, seed=1500 + n, kind="heavy", outlier_frac=0.002)
    W = workloads.weights(m, d, 1501 + m)
    dX = dev_bf16(X)
    wc, wn = orbq.fold_weights(dev_bf16(W), rot, cbw)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    assert orbq.linear_workspace_bytes(n, d, 6) == -(-n * d * 2 // 256) * 256 + 4 * n
    Y = orbq.linear(dX, rot, cba, wc, wn, cbw, act=act, out_dtype=dt)
    xc, xs = orbq.rpbh_quantize(dX, rot, cba)
    Y2 = orbq.lut_gemm(xc, xs, cba, wc, wn, cbw, d, act=act, out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16) if out_bf16 else Y.view(torch.int32),
                       Y2.view(torch.int16) if out_bf16 else Y2.view(torch.int32))
    if n == 130:
        Pi = oracle.rpbh_composed(d, h, perm, signs, passes)
        kw, r, _, _ = oracle.fold_weights(workloads.f64_from_bf16_bits(W), Pi, cw)
        Yo, kx, s = oracle.orbq_linear(workloads.f64_from_bf16_bits(X), Pi, ca, kw, r, cw)
        den = (np.abs(oracle.decode_lut_bf16(ca)[kx]) @ np.abs(oracle.decode_lut_bf16(cw)[kw]).T) * s[:, None] * r[None, :]
        e = np.max(np.abs(Y.cpu().numpy() - Yo) / den)
        log(f"  W{bw}A6 linear vs oracle chain: {e:.3g}")
        assert e < 2e-3


# ----------------------------------------------------------------- edge cases
def test_edge_cases(orbq):
    torch = torch_mod()
    d, h = 256, 64
    rot = gpu_rotation(orbq, d, h)
    cb, c = gpu_codebook(orbq, d, 4)
    # zero rows, a constant row, a single outlier, and n = 1
    X = np.zeros((5, d))
    X[1] = 1.0
    X[2, 17] = 1000.0
    X[3] = np.linspace(-1, 1, d)
    X[4] = -0.0
    bits = workloads.bf16_bits_from_f64(X)
    bits[4] = 0x8000                       # -0.0 everywhere
    codes, s = orbq.rpbh_quantize(dev_bf16(bits), rot, cb)
    k = oracle.unpack_codes(codes.cpu().numpy(), 4, d)
    k_ref, s_ref, T = oracle.quantize_activations(workloads.f64_from_bf16_bits(bits), dense_pi(d, h), c)
    check_codes(k, k_ref, T, c, "edge rows", max_frac=2.0 / k.size)
    assert np.all(k[0] == 7) and np.all(k[4] == 7) and s.cpu()[0] == 0 and s.cpu()[4] == 0
    one, _ = orbq.rpbh_quantize(dev_bf16(bits[2:3]), rot, cb)
    assert torch.equal(one.cpu(), codes.cpu()[2:3])
    # strided input (ldx > d) and padded output (ldy > m)
    big = np.zeros((5, d + 64), np.uint16)
    big[:, :d] = bits
    dbig = dev_bf16(big)
    c2, _ = orbq.rpbh_quantize(dbig[:, :d], rot, cb)
    assert torch.equal(c2.cpu(), codes.cpu())
    wc, wn = orbq.fold_weights(dev_bf16(bits), rot, cb)
    Yp = torch.full((5, 12), float("nan"), device="cuda")
    orbq.lut_gemm(codes, s, cb, wc, wn, cb, d, out=Yp[:, :5])
    assert torch.isnan(Yp[:, 5:]).all() and not torch.isnan(Yp[:, :5]).any()
    # n = 0 and m = 0 are no-ops
    e0, s0 = orbq.rpbh_quantize(dev_bf16(bits[:0]), rot, cb)
    assert e0.numel() == 0
