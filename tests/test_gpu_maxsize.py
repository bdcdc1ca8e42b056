"""GPU tests at sizes past 2^31 bytes per buffer: the launch chunking of rpbh_quantize (token
rows) and lut_gemm (token rows and weight rows), which keeps every buffer extent addressable with
32-bit offsets.

The large inputs repeat a small block (device-side tiling of seeded workloads data), so every
repeat must reproduce the block's result bit for bit: a property that holds at any size, checked
on the device.  The block itself is checked against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import oracle_codebook
from tests.gpu_common import check_codes, dense_pi, dev_bf16, gemm_error, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orbq():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import calibration_free_w4a4_amd as m
    m.load()
    return m


def test_quantize_rows_past_2_31_bytes(orbq):
    """4096-wide tokens, 2 x 131072 + 1234 rows (2.16 GB of bf16 input): three launches."""
    torch = torch_mod()
    d, h, blk = 4096, 128, 1024
    n = 2 * 131072 + 1234
    reps = -(-n // blk)
    log(f"quantize n={n} d={d} ({n * d * 2 / 2**30:.2f} GiB input)")
    perm, signs = workloads.rotation(d)
    rot = orbq.Rotation.create(d, h, perm, signs)
    cb = orbq.Codebook.lloyd_max(d, 4)
    B = workloads.activations(blk, d, seed=7001, kind="heavy")
    X = dev_bf16(B).repeat(reps, 1)[:n].contiguous()
    codes, norms = orbq.rpbh_quantize(X, rot, cb)
    del X
    torch.cuda.synchronize()
    cb0, nb0 = codes[:blk], norms[:blk]
    for r in range(1, reps):
        rows = min(blk, n - r * blk)
        assert torch.equal(codes[r * blk:r * blk + rows], cb0[:rows]), f"repeat {r} codes differ"
        assert torch.equal(norms[r * blk:r * blk + rows], nb0[:rows]), f"repeat {r} norms differ"
    # the block against the oracle (a sample of its rows)
    idx = np.arange(0, blk, 37)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(B[idx]), dense_pi(d, h),
                                                      oracle_codebook(d, 4))
    check_codes(oracle.unpack_codes(cb0.cpu().numpy()[idx], 4, d), k_ref, T_ref, oracle_codebook(d, 4), "block")
    assert np.max(np.abs(nb0.cpu().numpy()[idx] - s_ref) / s_ref) < 1e-6


@pytest.mark.parametrize("side", ["weights", "tokens"])
def test_lut_gemm_codes_past_2_31_bytes(orbq, side):
    """lut_gemm with 2.15 GB of weight codes (1,051,512 rows x 4096 at 4 bits: two launches
    over weight-row blocks) or of token codes (same count of token rows)."""
    torch = torch_mod()
    d, blk = 4096, 4096
    big = 1048512 + 3000
    small = 64 if side == "weights" else 192
    n, m = (small, big) if side == "weights" else (big, small)
    log(f"lut_gemm {side}: n={n} m={m} d={d}")
    cb = orbq.Codebook.lloyd_max(d, 4)
    c = oracle_codebook(d, 4)
    rb = d // 2
    big_codes_blk = workloads.random_code_bytes(blk, rb, 7101)
    small_codes = workloads.random_code_bytes(small, rb, 7102)
    big_norm_blk = workloads.random_norms(blk, 7103, 0.5, 2.0)
    small_norm = workloads.random_norms(small, 7104, 0.5, 2.0)
    reps = -(-big // blk)
    big_codes = torch.from_numpy(big_codes_blk).cuda().repeat(reps, 1)[:big].contiguous()
    if side == "weights":
        xc, xs = torch.from_numpy(small_codes).cuda(), torch.from_numpy(small_norm.astype(np.float32)).cuda()
        r_bits = workloads.bf16_bits_from_f64(big_norm_blk)
        wc = big_codes
        wn = dev_bf16(r_bits).repeat(reps)[:big].contiguous()
    else:
        xc = big_codes
        xs = torch.from_numpy(big_norm_blk.astype(np.float32)).cuda().repeat(reps)[:big].contiguous()
        r_bits = workloads.bf16_bits_from_f64(small_norm)
        wc, wn = torch.from_numpy(small_codes).cuda(), dev_bf16(r_bits)
    Y = orbq.lut_gemm(xc, xs, cb, wc, wn, cb, d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del big_codes, xc, wc
    Yb = Y if side == "weights" else Y.t()        # the big axis last
    first = Yb[:, :blk]
    for r in range(1, reps):
        cols = min(blk, big - r * blk)
        assert torch.equal(Yb[:, r * blk:r * blk + cols], first[:, :cols]), f"repeat {r} differs"
    # the first block against the oracle from the codes (sampled rows of the small side)
    lut = oracle.decode_lut_bf16(c)
    ii = np.arange(0, small, 5)
    jj = np.arange(0, blk, 11)
    Asm = lut[oracle.unpack_codes(small_codes[ii], 4, d)]
    Abg = lut[oracle.unpack_codes(big_codes_blk[jj], 4, d)]
    Ysub = first.float().cpu().numpy().astype(np.float64)[np.ix_(ii, jj)]
    r_small = small_norm.astype(np.float32).astype(np.float64) if side == "weights" else \
        workloads.f64_from_bf16_bits(r_bits)
    r_big = workloads.f64_from_bf16_bits(workloads.bf16_bits_from_f64(big_norm_blk)) if side == "weights" else \
        big_norm_blk.astype(np.float32).astype(np.float64)
    e = gemm_error(Ysub, Asm, Abg, r_small[ii], r_big[jj])
    log(f"  max relative error {e:.3g}")
    assert e <= 2e-3 + 2.0 ** -8


def test_linear_a6_centroids_past_2_31_bytes(orbq):
    """The layer's path for 6-bit activations keeps the codes' bf16 centroids (2 d bytes per
    token): 352525 tokens of 3072 make 2.17 GB of them (and of input), so rpbh_quantize and the
    product both split their launches.  Every repeat of the 1024-token block gives the block's
    output bit for bit, and the block equals rpbh_quantize then lut_gemm on its packed codes."""
    torch = torch_mod()
    d, h, blk, m = 3072, 128, 1024, 2048
    n = 349525 + 3000
    reps = -(-n // blk)
    log(f"linear A6 centroids n={n} d={d} m={m} ({n * d * 2 / 2**30:.2f} GiB of centroids)")
    perm, signs = workloads.rotation(d)
    rot = orbq.Rotation.create(d, h, perm, signs)
    cba, cbw = orbq.Codebook.lloyd_max(d, 6), orbq.Codebook.lloyd_max(d, 4)
    wc, wn = orbq.fold_weights(dev_bf16(workloads.weights(m, d, 7201)), rot, cbw)
    B = dev_bf16(workloads.activations(blk, d, seed=7202, kind="heavy"))
    X = B.repeat(reps, 1)[:n].contiguous()
    Y = orbq.linear(X, rot, cba, wc, wn, cbw, out_dtype=torch.bfloat16)
    del X
    torch.cuda.synchronize()
    first = Y[:blk]
    for r in range(1, reps):
        rows = min(blk, n - r * blk)
        assert torch.equal(Y[r * blk:r * blk + rows], first[:rows]), f"repeat {r} differs"
    xc, xs = orbq.rpbh_quantize(B, rot, cba)
    Y2 = orbq.lut_gemm(xc, xs, cba, wc, wn, cbw, d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), Y2.view(torch.int16))
