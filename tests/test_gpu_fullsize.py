"""GPU parity at the layers' full sizes, in the launch configuration bench.py times.

Each case generates the layer's full seeded inputs, folds the weights, runs rpbh_quantize and
lut_gemm with bf16 output (exactly the calls the benchmark step makes), and checks the result
against the CPU oracle:
  * the FLUX MLP-up headline (4608 x 3072 -> 12288, W4A4): every token code, every weight code
    and every output element;
  * the other layers: sampled token rows, weight rows and output blocks (the first, middle and
    last rows, the largest-norm row and seeded random rows), since the oracle's dense rotation of
    a whole 12288- or 8960-wide layer takes minutes;
  * orbq_linear (workspace entry point) gives the same bits as the two calls.
Tolerances as in test_gpu_parity.py; bf16 output adds one bf16 ulp (2^-8 relative) to 2e-3.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import oracle_codebook
from tests.gpu_common import check_codes, dense_pi, dev_bf16, gemm_error, log, torch_mod

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3 + 2.0 ** -8


@pytest.fixture(scope="module")
def orbq():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import calibration_free_w4a4_amd as m
    m.load()
    return m


def _sample(n: int, X_bits: np.ndarray | None, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = [0, n // 2, n - 1]
    if X_bits is not None:
        nrm = np.concatenate([np.einsum("ij,ij->i", *(2 * [workloads.f64_from_bf16_bits(X_bits[r:r + 2048])]))
                              for r in range(0, n, 2048)])
        pick.append(int(np.argmax(nrm)))
    return np.unique(np.concatenate([pick, rng.choice(n, size=min(k, n), replace=False)]))


def _run_layer(orbq, L):
    """Fold, then the benchmark step (rpbh_quantize into preallocated buffers, lut_gemm to bf16)."""
    torch = torch_mod()
    X, W = workloads.layer_inputs(L)
    perm, signs = workloads.rotation(L.d)
    rot = orbq.Rotation.create(L.d, L.block, perm, signs)
    cb_a, cb_w = orbq.Codebook.lloyd_max(L.d, L.bits_a), orbq.Codebook.lloyd_max(L.d, L.bits_w)
    dX, dW = dev_bf16(X), dev_bf16(W)
    w_codes, w_norms = orbq.fold_weights(dW, rot, cb_w)
    x_codes = torch.empty((L.n, orbq.codes_row_bytes(L.d, L.bits_a)), dtype=torch.uint8, device="cuda")
    x_norms = torch.empty((L.n,), dtype=torch.float32, device="cuda")
    Y = torch.empty((L.n, L.m), dtype=torch.bfloat16, device="cuda")
    orbq.rpbh_quantize(dX, rot, cb_a, out_codes=x_codes, out_norms=x_norms)
    orbq.lut_gemm(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, L.d, out=Y)
    ws = torch.empty((orbq.linear_workspace_bytes(L.n, L.d, L.bits_a),), dtype=torch.uint8, device="cuda")
    Y2 = torch.empty_like(Y)
    orbq.linear(dX, rot, cb_a, w_codes, w_norms, cb_w, workspace=ws, out=Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "orbq_linear differs from the two calls"
    del dX, dW, Y2, ws
    return (X, W, x_codes.cpu().numpy(), x_norms.cpu().numpy().astype(np.float64),
            w_codes.cpu().numpy(), w_norms.float().cpu().numpy().astype(np.float64), Y.float().cpu().numpy())


def _check_rows(name, src_bits, codes, norms, idx, L, bits, weights):
    c = oracle_codebook(L.d, bits)
    Pi = dense_pi(L.d, L.block)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(src_bits[idx]), Pi, c)
    check_codes(oracle.unpack_codes(codes[idx], bits, L.d), k_ref, T_ref, c, name)
    if weights:
        r_ref = oracle.bf16_rne(s_ref)
        ulp = 2.0 ** (np.floor(np.log2(r_ref)) - 7)
        assert np.all(np.abs(norms[idx] - r_ref) <= ulp), f"{name}: r' more than one bf16 ulp off"
    else:
        assert np.max(np.abs(norms[idx] - s_ref) / s_ref) < 1e-6, f"{name}: s off"


def _check_gemm(name, L, x_codes, x_norms, w_codes, w_norms, Y, ii, jj):
    la = oracle.decode_lut_bf16(oracle_codebook(L.d, L.bits_a))
    lw = oracle.decode_lut_bf16(oracle_codebook(L.d, L.bits_w))
    A = la[oracle.unpack_codes(x_codes[ii], L.bits_a, L.d)]
    B = lw[oracle.unpack_codes(w_codes[jj], L.bits_w, L.d)]
    e = gemm_error(Y[np.ix_(ii, jj)].astype(np.float64), A, B, x_norms[ii], w_norms[jj])
    log(f"  {name}: {len(ii)} x {len(jj)} outputs, max relative error {e:.3g}")
    assert e <= BF16_TOL
    assert np.isfinite(Y).all()


def test_headline_every_element(orbq):
    """flux_mlp_up_4608 at full size: all 14.2M token codes, 37.7M weight codes, 56.6M outputs."""
    L = workloads.CONFIGS[workloads.HEADLINE]
    log(f"full size {L.name}: n={L.n} d={L.d} m={L.m} W{L.bits_w}A{L.bits_a}")
    X, W, xc, xs, wc, wn, Y = _run_layer(orbq, L)
    _check_rows("token codes (all)", X, xc, xs, np.arange(L.n), L, L.bits_a, False)
    for r0 in range(0, L.m, 4096):  # the weight rows in slices (memory)
        _check_rows(f"weight codes rows {r0}..", W, wc, wn, np.arange(r0, min(L.m, r0 + 4096)), L, L.bits_w, True)
    for r0 in range(0, L.n, 1536):  # every output, in row blocks
        _check_gemm(f"Y rows {r0}..", L, xc, xs, wc, wn, Y, np.arange(r0, min(L.n, r0 + 1536)), np.arange(L.m))


@pytest.mark.parametrize("name", ["flux_qkv", "flux_mlp_up", "flux_mlp_down", "flux_mlp_up_w2a4",
                                  "flux_mlp_up_w3a3", "wan_ffn_up", "wan_ffn_down"])
def test_layer_full_size_sampled(orbq, name):
    L = workloads.CONFIGS[name]
    log(f"full size {name}: n={L.n} d={L.d} m={L.m} W{L.bits_w}A{L.bits_a}")
    X, W, xc, xs, wc, wn, Y = _run_layer(orbq, L)
    k = 24 if L.d > 4096 else 64
    ii = _sample(L.n, X, k, 11)
    jj = _sample(L.m, None, k, 12)
    _check_rows("token codes (sampled rows)", X, xc, xs, ii, L, L.bits_a, False)
    _check_rows("weight codes (sampled rows)", W, wc, wn, jj, L, L.bits_w, True)
    _check_gemm("Y (sampled block)", L, xc, xs, wc, wn, Y, ii, jj)
    # a second, independent sample of outputs from rows not in ii (any (i, j) is checkable from codes)
    i2 = _sample(L.n, None, 256, 13)
    j2 = _sample(L.m, None, 256, 14)
    _check_gemm("Y (second sampled block)", L, xc, xs, wc, wn, Y, i2, j2)
