#!/usr/bin/env python3
"""Benchmark of the OrbitQuant quantized linear layer on one MI355X.

Workload (default): the FLUX MLP-up layer, 4608 tokens x 3072 -> 12288, W4A4, RPBH block 128,
16-level Lloyd-Max codebooks for f_3072 on both operands; synthetic heavy-tailed activations
(Student-t(3) x per-channel log-normal scales, 0.1% outlier channels x30) and N(0, 0.02^2)
weights (workloads.py).  The weights are folded once, untimed (the offline pass).

One step = the whole online hot path on one batch: rpbh_quantize (rotate, normalise, quantize,
pack the activations) then lut_gemm (decode, MFMA, rescale), both through the C ABI on the
current stream, inputs already resident in HBM.  The JSON line reports orbq_linear TFLOP/s
(2 n m d / step time, K steps back to back with nothing else enqueued) as `value`; a second
pass of K steps with HIP events between the launches gives the per-kernel durations (mean and
p10 / p50 / p90), the rpbh_quantize GB/s and the MFMA roofline of the dominant kernel
(lut_gemm); a loop of lut_gemm alone, against the step loop, gives rpbh_quantize's event-free cost
in the step; the CPU oracle is timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20       # Infinity Cache
SETTLE_S = 1.0               # untimed steady-state work before the warmup steps
CPU_SECONDS = 10.0           # the oracle's CPU leg repeats its sample until this much time


CSRC = os.path.join(ROOT, "calibration_free_w4a4_amd", "csrc")
# every source a kernel's code or its launch shape (grid, tiles, LDS layout) depends on
KERNEL_SOURCES = {
    "lut_gemm": ["lut_gemm_kernel.h", "lut_gemm.hip", "lut_gemm_a2.hip", "lut_gemm_a3.hip", "lut_gemm_a4.hip",
                 "lut_gemm_a6.hip", "lut_gemm_abf.hip", "internal.h"],
    "rpbh_quantize": ["rpbh_quantize_kernel.h", "rpbh_quantize.hip", "rpbh_quantize_b64.hip",
                      "rpbh_quantize_b128.hip", "rpbh_quantize_b256.hip", "rpbh_quantize_b512.hip",
                      "rpbh_quantize_b1024.hip", "rpbh_quantize_b2048.hip", "rpbh_quantize_b4096.hip",
                      "internal.h"],
}


def source_digest(kernel: str) -> str:
    """sha256 over the kernel's sources (KERNEL_SOURCES, in that order, each file's name and
    bytes): the tag a committed counter or trace summary carries."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(f.encode() + b"\0")
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def _summary(kernel: str, suffix: str, workload: str):
    """The `key: value` lines of a committed profiles/ summary, or None when it is missing or
    the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.{suffix}")
    if not os.path.exists(path):
        return None
    rec = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith(("#", " ")):
            k, v = ln.split(":", 1)
            rec[k.strip()] = v.strip()
    return rec if rec.get("source_sha256") == source_digest(kernel) else None


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None."""
    rec = _summary(kernel, "pmc.txt", workload)
    return float(rec["hbm_bytes_per_launch"]) if rec and "hbm_bytes_per_launch" in rec else None


def _trace_us(kernel: str, workload: str):
    """Average launch duration from the committed rocprofv3 --kernel-trace summary, or None."""
    rec = _summary(kernel, "trace.txt", workload)
    return float(rec["average_us"]) if rec and "average_us" in rec else None


def _pct(xs, q: float) -> float:
    xs = sorted(xs)
    i = (len(xs) - 1) * q
    lo = int(i)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)


def _r(v: float, nd: int):
    """round(), with NaN (a leg that did not run) reported as null."""
    return None if v != v else round(v, nd)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> int:
    """A plain device-to-device copy of known size, the yardstick that scales the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of the layer's kernels."""
    import torch

    src = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the hot path (skip the orbq_linear cross-check, the cold-cache "
                         "rpbh_quantize run and the torch context); for profiler runs")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warmup steps (clock settle)")
    ap.add_argument("--source-digest", action="store_true",
                    help="print the source digests that profiles/ summaries are tagged with, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--rotation-ablation", action="store_true",
                    help="time rpbh_quantize under the rotation variants of the rotation ablation "
                         "(RPBH, block RHT without permutation, RHT over the widest power-of-two blocks, dense Haar "
                         "rotation as a bf16 GEMM) on the workload's activations; prints its own line")
    ap.add_argument("--mlp", action="store_true",
                    help="time the FLUX MLP pair (up-projection, GELU, down-projection; 9216 tokens, "
                         "3072 -> 12288 -> 3072, W4A4) with GELU fused into the up-projection's "
                         "epilogue against GELU as a separate pass; prints its own line")
    ap.add_argument("--a16", action="store_true",
                    help="time the weight-only product (bf16 activations, 4-bit weight codes) on the FLUX "
                         "AdaLN modulation shape (2 x 3072 -> 18432) against torch's bf16 GEMM of the dense "
                         "weights; prints its own line")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle sample tokens (default: all)")
    ap.add_argument("--cpu-weights", type=int, default=None, help="oracle sample weight rows (default: all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is data-parallel "
              "over tokens and the multi-GPU sharding is not built.", file=sys.stderr)
        return 2

    if args.source_digest:
        print(json.dumps({k: source_digest(k) for k in KERNEL_SOURCES}))
        return 0
    if args.copy_calibration:
        return copy_calibration()

    import numpy as np
    import torch

    import calibration_free_w4a4_amd as orbq
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    name = args.workload or workloads.HEADLINE
    L = workloads.CONFIGS[name]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.mlp:
        return mlp_pair(orbq, workloads, args)
    if args.a16:
        return a16_modulation(orbq, workloads, args)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    X_bits, W_bits = workloads.layer_inputs(L)
    X, W = to_dev(X_bits), to_dev(W_bits)
    perm, signs = workloads.rotation(L.d)
    rot = orbq.Rotation.create(L.d, L.block, perm, signs)
    cb_a = orbq.Codebook.lloyd_max(L.d, L.bits_a)
    cb_w = orbq.Codebook.lloyd_max(L.d, L.bits_w)
    w_codes, w_norms = orbq.fold_weights(W, rot, cb_w)           # offline, untimed
    x_codes = torch.empty((L.n, orbq.codes_row_bytes(L.d, L.bits_a)), dtype=torch.uint8, device=dev)
    x_norms = torch.empty((L.n,), dtype=torch.float32, device=dev)
    Y = torch.empty((L.n, L.m), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((orbq.linear_workspace_bytes(L.n, L.d, L.bits_a),), dtype=torch.uint8, device=dev)

    if args.rotation_ablation:
        return rotation_ablation(orbq, L, name, X, perm, signs, cb_a, args)

    def quantize(Xin=X):
        orbq.rpbh_quantize(Xin, rot, cb_a, out_codes=x_codes, out_norms=x_norms)

    def gemm():
        orbq.lut_gemm(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, L.d, out=Y)

    # The GPU leaves its idle power state over the first tens of milliseconds of work: run the
    # step for at least --settle seconds of wall time before the W warmup steps so that the timed steps
    # see the steady-state clocks a serving loop runs at.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            quantize()
            gemm()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        quantize()
        gemm()
    torch.cuda.synchronize()

    # ---- timed region: K steps back to back on the launch stream, nothing else enqueued
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        quantize()
        gemm()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # ---- per-kernel durations: K more steps with HIP events on the launch stream before each
    # kernel (a step's first event also ends the previous step's lut_gemm), one after the last
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    for k in range(args.steps):
        ev[2 * k].record()
        quantize()
        ev[2 * k + 1].record()
        gemm()
    ev[2 * args.steps].record()
    torch.cuda.synchronize()
    q_all = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]
    g_all = [ev[2 * k + 1].elapsed_time(ev[2 * k + 2]) for k in range(args.steps)]
    q_ms, g_ms = statistics.mean(q_all), statistics.mean(g_all)

    # ---- rpbh_quantize's event-free cost in the step: the step loop against the same loop of
    # lut_gemm alone (which the GPU, not the host, bounds); the difference is what K1 adds to a
    # step, its duration and the gap it brings, with no event records between launches
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        gemm()
    torch.cuda.synchronize()
    g_only_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    q_marginal_ms = ms_step - g_only_ms

    flops = L.flops
    q_bytes = L.n * (2 * L.d + L.d * L.bits_a // 8 + 4)
    value = flops / (ms_step * 1e-3) / 1e12

    linear_ms = q_cold_ms = ref_gemm_tflops = copy_gbps = copy_same_us = copy_same_step_us = float("nan")
    mfma_tflops = float("nan")
    if not args.no_extras:
        # ---- the same layer through the single orbq_linear entry point (cross-check)
        for _ in range(3):
            orbq.linear(X, rot, cb_a, w_codes, w_norms, cb_w, workspace=ws, out=Y)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            orbq.linear(X, rot, cb_a, w_codes, w_norms, cb_w, workspace=ws, out=Y)
        torch.cuda.synchronize()
        linear_ms = (time.perf_counter() - t2) * 1e3 / args.steps

        # ---- rpbh_quantize with inputs rotated over > 2x the 256 MB Infinity Cache
        nbuf = max(2, -(-2 * MALL_BYTES // (L.n * L.d * 2)))
        bufs = [X] + [X.roll(k + 1, dims=0).contiguous() for k in range(nbuf - 1)]
        reps = max(2, args.steps // nbuf) * nbuf
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for b in bufs:
            quantize(b)
        torch.cuda.synchronize()
        e0.record()
        for k in range(reps):
            quantize(bufs[k % nbuf])
        e1.record()
        torch.cuda.synchronize()
        q_cold_ms = e0.elapsed_time(e1) / reps
        del bufs

        # ---- context: torch's bf16 GEMM of the same shape and a same-size copy
        A = torch.randn((L.n, L.d), dtype=torch.bfloat16, device=dev)
        B = torch.randn((L.d, L.m), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(A, B, out=Y)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            torch.matmul(A, B, out=Y)
        e1.record()
        torch.cuda.synchronize()
        ref_gemm_tflops = flops / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * src.numel() / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
        # a device copy that moves the bytes rpbh_quantize moves (q_bytes / 2 read, as many
        # written), timed the same ways: back to back, and between GEMM launches
        half = q_bytes // 2
        csrc, cdst = src[:half], dst[:half]
        e0.record()
        for _ in range(100):
            cdst.copy_(csrc)
        e1.record()
        torch.cuda.synchronize()
        copy_same_us = e0.elapsed_time(e1) / 100 * 1e3
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for ea, eb in cev:
            gemm()
            ea.record()
            cdst.copy_(csrc)
            eb.record()
        torch.cuda.synchronize()
        copy_same_step_us = statistics.mean(ea.elapsed_time(eb) for ea, eb in cev) * 1e3
        del src, dst, A, B, csrc, cdst
        # the matrix cores' sustained bf16 rate on register operands with random bits, two
        # workgroups per compute unit (orbq_test_mfma_rate): the rate a bf16 contraction on real
        # data can be held against once the chip's power limit sets its clock
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.empty((2 * cus * 512,), dtype=torch.float32, device=dev)
        orbq.test_mfma_rate(2 * cus, 400, sink)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0.record()
            mfma_flops = orbq.test_mfma_rate(2 * cus, 20000, sink)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        mfma_tflops = mfma_flops / (best * 1e-3) / 1e12
        del sink

    g_tflops = flops / (g_ms * 1e-3) / 1e12
    q_gbps = q_bytes / (q_ms * 1e-3) / 1e9
    q_trace_us = _trace_us("rpbh_quantize", name)
    g_trace_us = _trace_us("lut_gemm", name)

    def pcts(xs):
        return {p: round(_pct(xs, q) * 1e3, 2) for p, q in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))}
    line = {
        "metric": "orbq_linear TFLOP/s + rpbh_quantize GB/s, FLUX-shaped 4608x3072->12288 W4A4",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "tokens": L.n, "d": L.d, "m": L.m, "bits_w": L.bits_w,
                   "bits_a": L.bits_a, "block": L.block, "y_dtype": "bf16"},
        "rpbh_quantize_GBps": round(q_gbps, 1),
        "rpbh_quantize_cold_GBps": _r(q_bytes / (q_cold_ms * 1e-3) / 1e9, 1),
        "kernel_ms": {"rpbh_quantize": round(q_ms, 5), "lut_gemm": round(g_ms, 5),
                      "rpbh_quantize_cold": _r(q_cold_ms, 5), "orbq_linear_call": _r(linear_ms, 5)},
        # per-launch event durations over the K timed steps
        "kernel_us_pct": {"rpbh_quantize": pcts(q_all), "lut_gemm": pcts(g_all), "launches": args.steps},
        # the same kernels' average durations in the committed rocprofv3 kernel trace of this
        # workload's step (null when the kernel sources changed since): no event records between
        # launches
        "trace_us": {"rpbh_quantize": q_trace_us, "lut_gemm": g_trace_us,
                     "rpbh_quantize_GBps": _r(q_bytes / (q_trace_us * 1e-6) / 1e9, 1) if q_trace_us else None},
        # K1's cost in the step without events: step time less the time of lut_gemm alone
        "rpbh_quantize_in_step_marginal": {
            "us": round(q_marginal_ms * 1e3, 2),
            "GBps": _r(q_bytes / (q_marginal_ms * 1e-3) / 1e9, 1) if q_marginal_ms > 0 else None},
        "roofline": {"bound": "mfma", "achieved": round(g_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(g_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": _traffic("lut_gemm", name)},
        "rpbh_roofline": {"bound": "hbm", "achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(q_gbps / HBM_PEAK_GBPS, 4),
                          "traffic": _traffic("rpbh_quantize", name)},
        "context": {"torch_bf16_matmul_TFLOPs": _r(ref_gemm_tflops, 1),
                    "torch_copy_GBps": _r(copy_gbps, 1),
                    "copy_of_rpbh_bytes_us": _r(copy_same_us, 2),
                    "copy_of_rpbh_bytes_in_step_us": _r(copy_same_step_us, 2),
                    "mfma_sustained_TFLOPs": _r(mfma_tflops, 1),
                    "mfma_sustained_frac_of_peak": _r(mfma_tflops / BF16_PEAK_TFLOPS, 4),
                    "lut_gemm_frac_of_sustained": _r(g_tflops / mfma_tflops, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(L, X_bits, W_bits, perm, signs, args.cpu_tokens, args.cpu_weights)
    print(json.dumps(line), flush=True)
    return 0


def _event_ms(fn, reps: int) -> float:
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def rotation_ablation(orbq, L, name, X, perm, signs, cb_a, args) -> int:
    """The rotation ablation on one layer's activations: rpbh_quantize (rotate, normalise,
    quantize, pack) under each rotation, back to back on the same resident input.
      rpbh          block h = L.block with the random permutation (the method)
      block_rht     block h = L.block, permutation = identity
      rht_<h>       h = the largest power of two dividing d (1024 at d = 3072, 4096 at d = 12288,
                    the whole vector when d is a power of two), with and without the permutation
      rpbh_2pass, rpbh_3pass  two / three composed RPBH passes, each with its own permutation and
                    signs (composed randomized Hadamard transforms)
      haar_dense    a dense d x d orthogonal rotation applied as a bf16 GEMM (torch / hipBLASLt);
                    the rotation alone, without normalisation or quantization: a lower bound
                    on a dense rotation's cost"""
    import torch

    import workloads

    dev = X.device
    x_codes = torch.empty((L.n, orbq.codes_row_bytes(L.d, L.bits_a)), dtype=torch.uint8, device=dev)
    x_norms = torch.empty((L.n,), dtype=torch.float32, device=dev)
    wide = 1  # the largest power of two dividing d (the pages' default block), up to 4096
    while wide < 4096 and L.d % (2 * wide) == 0:
        wide *= 2
    p3, s3 = workloads.rotation_passes(L.d, 3)
    variants = [("rpbh", L.block, perm, signs, 1), ("block_rht", L.block, None, signs, 1),
                (f"rht_{wide}_perm", wide, perm, signs, 1), (f"rht_{wide}", wide, None, signs, 1),
                ("rpbh_2pass", L.block, p3[:2 * L.d], s3[:2 * L.d], 2), ("rpbh_3pass", L.block, p3, s3, 3)]
    reps = max(50, args.steps)
    t_settle = time.perf_counter()
    rot0 = orbq.Rotation.create(L.d, L.block, perm, signs)
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(50):
            orbq.rpbh_quantize(X, rot0, cb_a, out_codes=x_codes, out_norms=x_norms)
        torch.cuda.synchronize()
    res = {}
    for vname, h, p, sg, k in variants:
        rot = orbq.Rotation.create(L.d, h, p, sg, passes=k)
        ms = _event_ms(lambda: orbq.rpbh_quantize(X, rot, cb_a, out_codes=x_codes, out_norms=x_norms), reps)
        res[vname] = {"block": h, "permutation": p is not None, "passes": k, "us": round(ms * 1e3, 2)}
    # dense orthogonal d x d rotation (QR of a Gaussian matrix; its exact distribution does not
    # matter for the cost) applied to the bf16 activations
    g = torch.Generator(device="cpu").manual_seed(5)
    Q, _ = torch.linalg.qr(torch.randn((L.d, L.d), generator=g, dtype=torch.float32))
    Phi_t = Q.t().contiguous().to(device=dev, dtype=torch.bfloat16)
    Xr = torch.empty((L.n, L.d), dtype=torch.bfloat16, device=dev)
    ms = _event_ms(lambda: torch.matmul(X, Phi_t, out=Xr), reps)
    res["haar_dense_gemm"] = {"block": L.d, "permutation": False, "us": round(ms * 1e3, 2),
                              "note": "rotation only (bf16 GEMM), no normalisation or quantization"}
    base = res["rpbh"]["us"]
    for v in res.values():
        v["vs_rpbh"] = round(v["us"] / base, 3)
    q_bytes = L.n * (2 * L.d + L.d * L.bits_a // 8 + 4)
    for vname, *_ in variants:
        res[vname]["GBps"] = round(q_bytes / (res[vname]["us"] * 1e-6) / 1e9, 1)
    print(json.dumps({"metric": "rotation ablation: rpbh_quantize time per rotation", "unit": "us",
                      "higher_is_better": False, "n_gpus": 1, "reps": reps, "data": "synthetic",
                      "config": {"workload": name, "tokens": L.n, "d": L.d, "bits_a": L.bits_a},
                      "variants": res}), flush=True)
    del Phi_t, Xr
    return 0


def mlp_pair(orbq, workloads, args) -> int:
    """The FLUX MLP pair on one batch: rpbh_quantize, lut_gemm (up) -> GELU -> rpbh_quantize,
    lut_gemm (down), all bf16 between the layers.  Fused: GELU (tanh form) in the
    up-projection's epilogue.  Fused, folded: in addition the down layer's permutation is folded
    into the up layer's weight-row order, so the down quantizer runs without a permutation (its
    codes, norms and outputs are the same bits).  Unfused: the up-projection stores its raw
    product and torch's GELU runs as a separate pass.  Each kernel is timed with HIP events over
    `reps` repetitions of the whole pair, after the settle phase."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    dev = torch.device("cuda", 0)
    Lu, Ld = workloads.CONFIGS["flux_mlp_up"], workloads.CONFIGS["flux_mlp_down"]
    n = Lu.n

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    X_bits, Wu_bits = workloads.layer_inputs(Lu)
    X, Wu, Wd = to_dev(X_bits), to_dev(Wu_bits), to_dev(workloads.weights(Ld.m, Ld.d, Ld.w_seed))
    rot_u = orbq.Rotation.create(Lu.d, Lu.block, *workloads.rotation(Lu.d))
    perm_d, signs_d = workloads.rotation(Ld.d)
    rot_d = orbq.Rotation.create(Ld.d, Ld.block, perm_d, signs_d)
    cb_u, cb_d = orbq.Codebook.lloyd_max(Lu.d, 4), orbq.Codebook.lloyd_max(Ld.d, 4)
    wcu, wnu = orbq.fold_weights(Wu, rot_u, cb_u)
    wcd, wnd = orbq.fold_weights(Wd, rot_d, cb_d)
    # The down layer's permutation folded into the up layer: the up layer's weight rows stored in
    # pi_down order (row j holds original row pi_down[j], an offline re-indexing), so that its
    # GELU output arrives already permuted and the down quantizer applies signs and blocks only
    # (perm = NULL, same signs and block).  GELU is elementwise, so it commutes with the permutation.
    wcu_f, wnu_f = orbq.fold_weights(Wu[torch.from_numpy(perm_d.astype(np.int64)).to(dev)].contiguous(), rot_u, cb_u)
    rot_d_f = orbq.Rotation.create(Ld.d, Ld.block, None, signs_d)
    xcu = torch.empty((n, orbq.codes_row_bytes(Lu.d, 4)), dtype=torch.uint8, device=dev)
    xsu = torch.empty((n,), dtype=torch.float32, device=dev)
    xcd = torch.empty((n, orbq.codes_row_bytes(Ld.d, 4)), dtype=torch.uint8, device=dev)
    xsd = torch.empty((n,), dtype=torch.float32, device=dev)
    H = torch.empty((n, Lu.m), dtype=torch.bfloat16, device=dev)
    H2 = torch.empty_like(H)
    Y = torch.empty((n, Ld.m), dtype=torch.bfloat16, device=dev)

    def stages(variant: str):
        st = [lambda: orbq.rpbh_quantize(X, rot_u, cb_u, out_codes=xcu, out_norms=xsu)]
        if variant == "fused":
            st.append(lambda: orbq.lut_gemm(xcu, xsu, cb_u, wcu, wnu, cb_u, Lu.d, out=H, act="gelu_tanh"))
            st.append(lambda: orbq.rpbh_quantize(H, rot_d, cb_d, out_codes=xcd, out_norms=xsd))
        elif variant == "fused_folded":
            st.append(lambda: orbq.lut_gemm(xcu, xsu, cb_u, wcu_f, wnu_f, cb_u, Lu.d, out=H, act="gelu_tanh"))
            st.append(lambda: orbq.rpbh_quantize(H, rot_d_f, cb_d, out_codes=xcd, out_norms=xsd))
        else:
            st.append(lambda: orbq.lut_gemm(xcu, xsu, cb_u, wcu, wnu, cb_u, Lu.d, out=H2))
            st.append(lambda: torch.ops.aten.gelu.out(H2, approximate="tanh", out=H))
            st.append(lambda: orbq.rpbh_quantize(H, rot_d, cb_d, out_codes=xcd, out_norms=xsd))
        st.append(lambda: orbq.lut_gemm(xcd, xsd, cb_d, wcd, wnd, cb_d, Ld.d, out=Y))
        return st

    names = {"fused": ["rpbh_quantize_up", "lut_gemm_up_gelu", "rpbh_quantize_down", "lut_gemm_down"],
             "fused_folded": ["rpbh_quantize_up", "lut_gemm_up_gelu", "rpbh_quantize_down_noperm", "lut_gemm_down"],
             "unfused": ["rpbh_quantize_up", "lut_gemm_up", "gelu_pass", "rpbh_quantize_down", "lut_gemm_down"]}
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle:
        for _ in range(5):
            for f in stages("fused"):
                f()
        torch.cuda.synchronize()
    reps = max(10, args.steps // 4)
    out = {}
    for variant in ("fused", "fused_folded", "unfused"):
        st = stages(variant)
        for _ in range(3):
            for f in st:
                f()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(st) + 1)] for _ in range(reps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for k in range(reps):
            for i, f in enumerate(st):
                ev[k][i].record()
                f()
            ev[k][len(st)].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / reps
        per = {nm: round(statistics.mean(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(reps)) * 1e3, 2)
               for i, nm in enumerate(names[variant])}
        out[variant] = {"us_per_kernel": per, "ms_per_pair": round(wall, 4)}
    flops = 2.0 * n * Lu.d * Lu.m + 2.0 * n * Ld.d * Ld.m
    torch.cuda.synchronize()
    # the fused up-projection equals torch's GELU of the unfused one (to bf16 rounding)
    Hf = torch.empty_like(H)
    orbq.lut_gemm(xcu, xsu, cb_u, wcu, wnu, cb_u, Lu.d, out=Hf, act="gelu_tanh")
    ref = F.gelu(H2.float(), approximate="tanh")
    agree = float(((Hf.float() - ref).abs() / ref.abs().clamp_min(1e-2)).max())
    for k in out:
        out[k]["TFLOPs"] = round(flops / (out[k]["ms_per_pair"] * 1e-3) / 1e12, 1)
    print(json.dumps({"metric": "FLUX MLP pair (up, GELU, down) time per batch, GELU fused vs separate",
                      "unit": "ms", "higher_is_better": False, "n_gpus": 1, "reps": reps, "data": "synthetic",
                      "dtype": "bf16",
                      "config": {"workload": "flux_mlp_pair", "tokens": n, "d": Lu.d, "hidden": Lu.m,
                                 "bits_w": 4, "bits_a": 4, "block": Lu.block, "gelu": "tanh"},
                      "fused": out["fused"], "fused_folded": out["fused_folded"], "unfused": out["unfused"],
                      "saving_ms": round(out["unfused"]["ms_per_pair"] - out["fused"]["ms_per_pair"], 4),
                      "folded_saving_ms": round(out["fused"]["ms_per_pair"] - out["fused_folded"]["ms_per_pair"], 4),
                      "fused_vs_torch_gelu_max_rel_diff": round(agree, 5)}), flush=True)
    return 0


def a16_modulation(orbq, workloads, args) -> int:
    """Weight-only product on the FLUX AdaLN modulation shape: 2 tokens (a CFG pair of
    conditioning vectors) x 3072 -> 18432 (six modulation vectors), 4-bit weight codes, bf16
    activations and output.  One call = rotate the tokens, stream the codes, add the K splits.
    Bytes per call: the codes, r', X in and Y out; `achieved` is those bytes over the mean call
    time (HIP events around 200 back-to-back calls)."""
    import numpy as np
    import torch

    n, d, m, bw = 2, 3072, 18432, 4
    dev = torch.device("cuda", 0)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    X = to_dev(workloads.activations(n, d, seed=602, kind="heavy"))
    W = to_dev(workloads.weights(m, d, 601))
    rot = orbq.Rotation.create(d, 128, *workloads.rotation(d))
    cb = orbq.Codebook.lloyd_max(d, bw)
    wc, wn = orbq.fold_weights(W, rot, cb)
    ws = torch.empty((orbq.linear_a16_workspace_bytes(n, d, m),), dtype=torch.uint8, device=dev)
    Y = torch.empty((n, m), dtype=torch.bfloat16, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle:
        for _ in range(200):
            orbq.linear_a16(X, rot, wc, wn, cb, workspace=ws, out=Y)
        torch.cuda.synchronize()
    reps = 200
    ms = _event_ms(lambda: orbq.linear_a16(X, rot, wc, wn, cb, workspace=ws, out=Y), reps)
    Yd = torch.empty_like(Y)
    ms_dense = _event_ms(lambda: torch.matmul(X, W.t(), out=Yd), reps)
    nbytes = m * d * bw // 8 + 2 * m + 2 * n * d + 2 * n * m
    gbps = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "weight-only (A16) product, FLUX AdaLN modulation shape", "unit": "GB/s",
                      "value": round(gbps, 1), "higher_is_better": True, "n_gpus": 1, "reps": reps,
                      "data": "synthetic", "dtype": "bf16",
                      "config": {"workload": "flux_adaln_a16", "tokens": n, "d": d, "m": m, "bits_w": bw,
                                 "block": 128},
                      "us_per_call": round(ms * 1e3, 2), "bytes_per_call": nbytes,
                      "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                   "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
                      "context": {"torch_bf16_dense_gemm_us": round(ms_dense * 1e3, 2),
                                  "dense_weight_bytes": 2 * m * d}}), flush=True)
    return 0


def cpu_baseline(L, X_bits, W_bits, perm, signs, n_tok, n_w):
    """The oracle as it stands (numpy float64) on a bounded sample of the same layer: the first
    n_tok tokens against the first n_w weight rows (default: the whole layer; weights folded
    untimed), repeated until CPU_SECONDS have passed; throughput over all repetitions."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import workloads

    n_tok = L.n if n_tok is None else min(n_tok, L.n)
    n_w = L.m if n_w is None else min(n_w, L.m)
    Pi = oracle.rpbh_matrix(L.d, L.block, perm, signs)
    c_a = oracle.lloyd_max(L.d, L.bits_a).astype(np.float32)
    c_w = oracle.lloyd_max(L.d, L.bits_w).astype(np.float32)
    kw, r, _, _ = oracle.fold_weights(workloads.f64_from_bf16_bits(W_bits[:n_w]), Pi, c_w)
    Xs = workloads.f64_from_bf16_bits(X_bits[:n_tok])
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < CPU_SECONDS:
        oracle.orbq_linear(Xs, Pi, c_a, kw, r, c_w)
        reps += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(2.0 * n_tok * n_w * L.d * reps / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2), "repetitions": reps,
            "sample": f"{n_tok} tokens x {n_w} weight rows of {L.name} (d={L.d}), the online layer "
                      "(rotate + quantize + float64 dequantised product) repeated for at least "
                      f"{CPU_SECONDS:.0f} s"}


if __name__ == "__main__":
    sys.exit(main())
