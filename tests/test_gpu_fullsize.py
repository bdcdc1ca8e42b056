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
from tests.gpu_common import check_codes, check_rprime, dense_pi, dev_bf16, gemm_error, log, torch_mod

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
        check_rprime(norms[idx], s_ref, f"{name} r'")
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


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf"])
def test_flux_mlp_pair_chain(orbq, act):
    """The FLUX MLP pair (9216 tokens, 3072 -> 12288 -> 3072, W4A4, block 128) chained as a model
    runs it: the up layer through orbq_linear_act with GELU in the epilogue and bf16 output, and
    that exact bf16 hidden tensor fed to the down layer (rpbh_quantize on d = 12288, then
    lut_gemm to bf16).  Checked against the oracle on sampled rows:
      * the hidden tensor: the oracle's float64 GELU of the product of the up layer's own codes;
      * the down layer's token codes and s: the oracle's quantizer on the identical bf16 tensor;
      * the down layer's weight codes and r';
      * the down layer's outputs from identical codes."""
    torch = torch_mod()
    Lu, Ld = workloads.CONFIGS["flux_mlp_up"], workloads.CONFIGS["flux_mlp_down"]
    n = Lu.n
    log(f"MLP pair {act}: {n} x {Lu.d} -> {Lu.m} -> {Ld.m}")
    X, Wu = workloads.layer_inputs(Lu)
    Wd = workloads.weights(Ld.m, Ld.d, Ld.w_seed)
    rot_u = orbq.Rotation.create(Lu.d, Lu.block, *workloads.rotation(Lu.d))
    rot_d = orbq.Rotation.create(Ld.d, Ld.block, *workloads.rotation(Ld.d))
    cb_u, cb_d = orbq.Codebook.lloyd_max(Lu.d, 4), orbq.Codebook.lloyd_max(Ld.d, 4)
    dX = dev_bf16(X)
    wcu, wnu = orbq.fold_weights(dev_bf16(Wu), rot_u, cb_u)
    wcd, wnd = orbq.fold_weights(dev_bf16(Wd), rot_d, cb_d)
    H = torch.empty((n, Lu.m), dtype=torch.bfloat16, device="cuda")
    orbq.linear(dX, rot_u, cb_u, wcu, wnu, cb_u, out=H, act=act)
    xcu, xsu = orbq.rpbh_quantize(dX, rot_u, cb_u)  # the up layer's token codes, for the check
    xcd = torch.empty((n, orbq.codes_row_bytes(Ld.d, 4)), dtype=torch.uint8, device="cuda")
    xsd = torch.empty((n,), dtype=torch.float32, device="cuda")
    orbq.rpbh_quantize(H, rot_d, cb_d, out_codes=xcd, out_norms=xsd)
    Y = torch.empty((n, Ld.m), dtype=torch.bfloat16, device="cuda")
    orbq.lut_gemm(xcd, xsd, cb_d, wcd, wnd, cb_d, Ld.d, out=Y)
    torch.cuda.synchronize()
    ii = _sample(n, X, 24, 21)
    jj = _sample(Lu.m, None, 64, 22)
    # hidden tensor on sampled rows and columns
    Hs = H[torch.from_numpy(ii).cuda()].float().cpu().numpy().astype(np.float64)
    xcu_h, xsu_h = xcu.cpu().numpy(), xsu.cpu().numpy().astype(np.float64)
    wcu_h, wnu_h = wcu.cpu().numpy(), wnu.float().cpu().numpy().astype(np.float64)
    cu = oracle_codebook(Lu.d, 4)
    ku_x, ku_w = oracle.unpack_codes(xcu_h[ii], 4, Lu.d), oracle.unpack_codes(wcu_h[jj], 4, Lu.d)
    Gref = oracle.lut_gemm_act(ku_x, xsu_h[ii], cu, ku_w, wnu_h[jj], cu, act)
    lut = oracle.decode_lut_bf16(cu)
    den = (np.abs(lut[ku_x]) @ np.abs(lut[ku_w]).T) * xsu_h[ii][:, None] * wnu_h[jj][None, :]
    e = float(np.max(np.abs(Hs[:, jj] - Gref) / den))
    log(f"  hidden {act}(Y_up): {len(ii)} x {len(jj)} outputs, error / |dot| scale {e:.3g}")
    assert e <= 2.0 ** -8 + 1e-5
    assert np.isfinite(Hs).all()
    # the down layer on the identical bf16 hidden tensor
    H_bits = Hs.astype(np.float32).view(np.uint32) >> 16  # bf16 values are exact in fp32
    H_bits = H_bits.astype(np.uint16)
    xcd_h, xsd_h = xcd.cpu().numpy(), xsd.cpu().numpy().astype(np.float64)
    cd = oracle_codebook(Ld.d, 4)
    Pi = dense_pi(Ld.d, Ld.block)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(H_bits), Pi, cd)
    check_codes(oracle.unpack_codes(xcd_h[ii], 4, Ld.d), k_ref, T_ref, cd, "down token codes (sampled rows)")
    assert np.max(np.abs(xsd_h[ii] - s_ref) / s_ref) < 1e-6, "down s off"
    wcd_h, wnd_h = wcd.cpu().numpy(), wnd.float().cpu().numpy().astype(np.float64)
    jd = _sample(Ld.m, None, 24, 23)
    _check_rows("down weight codes (sampled rows)", Wd, wcd_h, wnd_h, jd, Ld, 4, True)
    Yh = Y.float().cpu().numpy()
    _check_gemm("down Y (sampled block)", Ld, xcd_h, xsd_h, wcd_h, wnd_h, Yh, ii, _sample(Ld.m, None, 256, 24))
    _check_gemm("down Y (second sample)", Ld, xcd_h, xsd_h, wcd_h, wnd_h, Yh, _sample(n, None, 256, 25),
                _sample(Ld.m, None, 256, 26))


# launch forms of rpbh_quantize on MI355X (256 CUs): 12288 (12 waves, 512 resident workgroups)
# x 4200 rows: pipelined loop + full-range table; 8960 (9 waves, 512) x 1500 rows: pipelined,
# clamped table (and 6-bit codes); 3072 (3 waves, 2048) x 17000 rows: full-range table, two-barrier loop
@pytest.mark.parametrize("d,n,bits,weights", [(12288, 4200, 2, False), (12288, 4200, 3, False), (12288, 4200, 4, False),
                                              (12288, 4200, 4, True), (8960, 1500, 4, False), (8960, 1500, 6, True),
                                              (8960, 1500, 6, False), (3072, 17000, 4, False)])
def test_quantize_loop_and_table_forms(orbq, d, n, bits, weights):
    """rpbh_quantize / fold_weights in the launch forms chosen by the number of token groups per
    workgroup: the full-range decision table (no clamp of the bucket index) and the software-
    pipelined loop (double-buffered staging and norm partials), alone and together.  Sampled
    rows' codes and norms against the oracle, and the poisoned-output check (every byte of every
    row written, the same bits on a second call)."""
    torch = torch_mod()
    h = 128
    log(f"launch forms: d={d} n={n} bits={bits} weights={weights}")
    src = workloads.weights(n, d, 811) if weights else workloads.activations(n, d, 812 + bits, kind="heavy")
    rot = orbq.Rotation.create(d, h, *workloads.rotation(d))
    cb = orbq.Codebook.lloyd_max(d, bits)
    c = oracle_codebook(d, bits)
    dsrc = dev_bf16(src)
    rb = orbq.codes_row_bytes(d, bits)
    codes = torch.full((n, rb), 0xFF, dtype=torch.uint8, device="cuda")
    norms = torch.full((n,), -1.0, dtype=torch.bfloat16 if weights else torch.float32, device="cuda")
    (orbq.fold_weights if weights else orbq.rpbh_quantize)(dsrc, rot, cb, out_codes=codes, out_norms=norms)
    codes0 = torch.zeros_like(codes)
    norms0 = torch.zeros_like(norms)
    (orbq.fold_weights if weights else orbq.rpbh_quantize)(dsrc, rot, cb, out_codes=codes0, out_norms=norms0)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes0) and torch.equal(norms.view(torch.uint8), norms0.view(torch.uint8))
    idx = _sample(n, None if weights else src, 20, 31)
    k_ref, s_ref, T_ref = oracle.quantize_activations(workloads.f64_from_bf16_bits(src[idx]), dense_pi(d, h), c)
    check_codes(oracle.unpack_codes(codes.cpu().numpy()[idx], bits, d), k_ref, T_ref, c, f"{bits}-bit codes")
    got = norms.float().cpu().numpy().astype(np.float64)[idx]
    if weights:
        check_rprime(got, s_ref, "r'")
    else:
        assert np.max(np.abs(got - s_ref) / s_ref) < 1e-6


def test_flux_mlp_pair_permutation_folded(orbq):
    """The down layer's permutation folded into the up layer (FLUX MLP pair, 9216 tokens, GELU
    tanh form): with the up layer's weight rows stored in pi_down order (row j = original row
    pi_down[j]), the up layer's output arrives permuted, H_f[:, j] = H[:, pi_down[j]] bit for bit
    (GELU is elementwise), and the down quantizer without a permutation (same signs and block)
    gives the unfolded chain's down codes, norms and outputs bit for bit."""
    torch = torch_mod()
    Lu, Ld = workloads.CONFIGS["flux_mlp_up"], workloads.CONFIGS["flux_mlp_down"]
    n = Lu.n
    X, Wu = workloads.layer_inputs(Lu)
    Wd = workloads.weights(Ld.m, Ld.d, Ld.w_seed)
    perm_d, signs_d = workloads.rotation(Ld.d)
    rot_u = orbq.Rotation.create(Lu.d, Lu.block, *workloads.rotation(Lu.d))
    rot_d = orbq.Rotation.create(Ld.d, Ld.block, perm_d, signs_d)
    rot_d_f = orbq.Rotation.create(Ld.d, Ld.block, None, signs_d)
    cb_u, cb_d = orbq.Codebook.lloyd_max(Lu.d, 4), orbq.Codebook.lloyd_max(Ld.d, 4)
    dX, dWu = dev_bf16(X), dev_bf16(Wu)
    pd = torch.from_numpy(perm_d.astype(np.int64)).cuda()
    wcu, wnu = orbq.fold_weights(dWu, rot_u, cb_u)
    wcu_f, wnu_f = orbq.fold_weights(dWu[pd].contiguous(), rot_u, cb_u)
    wcd, wnd = orbq.fold_weights(dev_bf16(Wd), rot_d, cb_d)
    assert torch.equal(wcu_f, wcu[pd]) and torch.equal(wnu_f.view(torch.int16), wnu[pd].view(torch.int16))
    outs = []
    for wc, wn, rot in ((wcu, wnu, rot_d), (wcu_f, wnu_f, rot_d_f)):
        H = orbq.linear(dX, rot_u, cb_u, wc, wn, cb_u, out_dtype=torch.bfloat16, act="gelu_tanh")
        xc, xs = orbq.rpbh_quantize(H, rot, cb_d)
        Y = orbq.lut_gemm(xc, xs, cb_d, wcd, wnd, cb_d, Ld.d, out_dtype=torch.bfloat16)
        outs.append((H, xc, xs, Y))
    torch.cuda.synchronize()
    (H, xc, xs, Y), (Hf, xcf, xsf, Yf) = outs
    assert torch.equal(Hf.view(torch.int16), H[:, pd].view(torch.int16)), "permuted hidden tensor differs"
    assert torch.equal(xcf, xc), "down codes differ"
    assert torch.equal(xsf.view(torch.int32), xs.view(torch.int32)), "down norms differ"
    assert torch.equal(Yf.view(torch.int16), Y.view(torch.int16)), "down outputs differ"
    log(f"  folded chain: {n} tokens, hidden, down codes, norms and outputs bit-identical")
