"""The matrix-core rate probe (orbq_test_mfma_rate) that bench.py reports as context: it runs,
returns the operation count its launch shape implies, and leaves finite sums in every slot of
its sink (each slot is the sum of one lane's accumulators, so a lane that skipped its MFMAs or
overflowed would show)."""
import math

import pytest

from tests.gpu_common import log, torch_mod

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_counts():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import calibration_free_w4a4_amd as orbq
    orbq.load()
    for wg, iters in ((1, 4), (3, 400), (512, 2000)):
        log(f"mfma probe workgroups={wg} iters={iters}")
        sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda")
        flops = orbq.test_mfma_rate(wg, iters, sink)
        torch.cuda.synchronize()
        assert flops == 2.0 * 32 * 32 * 16 * 9 * iters * 8 * wg
        s = sink.cpu()
        assert torch.isfinite(s).all(), "a sink slot was not written or overflowed"
        # random signs: the sums are spread around zero, not all equal
        assert s.abs().max().item() > 0 and len(set(s[:64].tolist())) > 1
