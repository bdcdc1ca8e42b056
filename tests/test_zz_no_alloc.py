"""orbq_linear_noalloc (the entry point without a caller workspace) against orbq_linear_act
(the same layer with a caller workspace), through the C ABI: two calls in a row, the second
with a smaller input, each bit-identical to the workspace entry point; and a call whose
workspace would exceed the fixed scratch array is refused without touching the output."""
import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_common import dev_bf16, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orbq():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import calibration_free_w4a4_amd as m
    m.load()
    return m


def _layer(orbq, n, d, m, bits_a, bits_w, seed):
    X = dev_bf16(workloads.activations(n, d, seed, kind="heavy"))
    W = dev_bf16(workloads.weights(m, d, seed + 1))
    rot = orbq.Rotation.create(d, 128, *workloads.rotation(d))
    cb_a, cb_w = orbq.Codebook.lloyd_max(d, bits_a), orbq.Codebook.lloyd_max(d, bits_w)
    wc, wn = orbq.fold_weights(W, rot, cb_w)
    return X, rot, cb_a, cb_w, wc, wn


def _call_noalloc(orbq, X, rot, cb_a, wc, wn, cb_w, act, Y):
    torch = torch_mod()
    lib = orbq.load()
    r, a, w = rot.struct(), cb_a.struct(), cb_w.struct()
    n, d = X.shape
    return lib.orbq_linear_noalloc(X.data_ptr(), n, d, X.stride(0), ctypes.byref(r), ctypes.byref(a), 1e-8,
                                   wc.data_ptr(), wn.data_ptr(), ctypes.byref(w), wc.shape[0],
                                   orbq.ACTIVATIONS[act], Y.data_ptr(), orbq.BF16 if Y.dtype == torch.bfloat16
                                   else orbq.F32, Y.stride(0), torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_workspace_entry_point(orbq):
    torch = torch_mod()
    cases = [  # (n, d, m, bits_a, bits_w, act, out dtype): the headline layer, then a smaller ragged W4A6 one
        (4608, 3072, 12288, 4, 4, "none", torch.bfloat16),
        (515, 1536, 2100, 6, 4, "gelu_tanh", torch.float32),
    ]
    for k, (n, d, m, ba, bw, act, dt) in enumerate(cases):
        log(f"noalloc call {k}: {n} x {d} -> {m} W{bw}A{ba} act={act} {dt}")
        X, rot, cb_a, cb_w, wc, wn = _layer(orbq, n, d, m, ba, bw, 900 + k)
        assert orbq.linear_workspace_bytes(n, d, ba) <= orbq.NOALLOC_SCRATCH_BYTES
        Y = torch.full((n, m), float("nan"), dtype=dt, device="cuda")
        st = _call_noalloc(orbq, X, rot, cb_a, wc, wn, cb_w, act, Y)
        assert st == 0, orbq.load().orbq_last_error().decode()
        Yref = orbq.linear(X, rot, cb_a, wc, wn, cb_w, out_dtype=dt, act=act)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yref), f"call {k}: differs from orbq_linear_act"
        assert torch.isfinite(Y.float()).all()


def test_noalloc_refuses_beyond_scratch(orbq):
    torch = torch_mod()
    n, d, m = 8192, 4096, 256  # 16 MiB + norms of 4-bit codes: one byte too many
    X, rot, cb_a, cb_w, wc, wn = _layer(orbq, n, d, m, 4, 4, 950)
    assert orbq.linear_workspace_bytes(n, d, 4) > orbq.NOALLOC_SCRATCH_BYTES
    Y = torch.full((n, m), 7.0, dtype=torch.float32, device="cuda")
    st = _call_noalloc(orbq, X, rot, cb_a, wc, wn, cb_w, "none", Y)
    torch.cuda.synchronize()
    assert st == -4, st  # ORBQ_ERR_WORKSPACE
    assert "scratch" in orbq.load().orbq_last_error().decode()
    assert bool((Y == 7.0).all())
    # the binding raises the same error
    with pytest.raises(orbq.OrbqError):
        orbq.linear_noalloc(X, rot, cb_a, wc, wn, cb_w, out=Y)
