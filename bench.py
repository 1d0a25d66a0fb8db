#!/usr/bin/env python3
"""HelixLinear forward throughput on one MI355X.

Workload (default): the Qwen2.5-3B-shaped u8 layer set (q, k, v, o, gate, up,
down; 7 HelixLinear layers with their own 256-entry codebooks and 0.1%
sidecars), decode with one token (M = 1), fp32 activations.  A step is one
forward through all 7 layers.  Inputs are seeded synthetic data resident in HBM
before timing; the compressed weights rotate over enough copies (>= 512 MB)
that no layer is served from the 256 MB Infinity Cache.

Reported value: algorithmic GB/s of the step (compressed bytes the method must
move: indices, codebook, sidecar triplets, x, bias, y) over the GPU time of the
timed steps.  Extra fields carry the M = 8 decode set and the bf16 prefill
GEMM at M = 2048 (TFLOP/s), the roofline of the dominant kernel and the CPU
oracle baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6   # MI355X dense bf16 matrix (256 CU x 2.4 GHz x 4096 flop/clk)
MALL_BYTES = 256 << 20
ROTATE_BYTES = 2 * MALL_BYTES


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(fmt, N, K, nnz, M, x_bytes, bias=True):
    """Bytes the forward must move for one layer: index storage, codebook,
    sidecar triplets (12 B each), activations, bias and the fp32 output."""
    if fmt == "u8":
        idx, cb = N * K, 256 * 4
    else:
        idx, cb = N * 3 * ((K + 3) // 4), 4096 * 8
    return idx + cb + 12 * nnz + M * K * x_bytes + (4 * N if bias else 0) + 4 * M * N


def source_digest():
    h = hashlib.sha256()
    for f in ("hxq_device.h", "hxq_gemv.hip", "hxq_gemm.hip", "hxq_launch.h", "hxq_api.cpp"):
        with open(os.path.join(ROOT, "vq_compressed_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


class Launcher:
    """Pre-marshalled C-ABI calls for one layer copy (keeps host overhead low)."""

    def __init__(self, L, fmt, d, x, y, M, N, K, stream):
        import vq_compressed_linear_amd as hx

        self.fn = L.hxq_linear_fwd_u8 if fmt == "u8" else L.hxq_linear_fwd_pk12
        self.args = (d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                     d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(),
                     x.data_ptr(), hx.HXQ_BF16 if x.dtype.is_floating_point and x.element_size() == 2
                     else hx.HXQ_F32, d["bias"].data_ptr(), y.data_ptr(), M, N, K, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("libhxq call failed with status %d" % st)


def to_dev(lay, torch):
    import numpy as np

    def t(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()

    return dict(codebook=t(lay.codebook), indices=t(lay.indices), rows=t(lay.rows, np.int32),
                cols=t(lay.cols, np.int32), deltas=t(lay.deltas, np.float32), bias=t(lay.bias, np.float32))


def hold_gpu(torch, ms):
    """Keep the GPU busy for about `ms` so the host can queue a timed region
    ahead of execution (launch latency then stays out of the event times)."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 2.0e6))
        return
    a = torch.randn(4096, 4096, device="cuda")
    for _ in range(max(1, int(ms / 0.5))):
        a = a @ a
        a = a / a.norm()


def time_steps(torch, launchers, steps, warmup, per_kernel=True):
    """launchers[r][i]: copy r, layer i.  Returns (total_ms, [per-launch ms by layer])."""
    R = len(launchers)
    nl = len(launchers[0])
    for s in range(warmup):
        for f in launchers[s % R]:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nl)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    hold_gpu(torch, 20 + steps * nl * 0.05)
    t0.record()
    for s in range(steps):
        row = launchers[s % R]
        for i in range(nl):
            if per_kernel:
                ev[s][i][0].record()
            row[i]()
            if per_kernel:
                ev[s][i][1].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)] for i in range(nl)] if per_kernel else None
    return total, per


def build_set(torch, L, layers, M, xdt, cfg_x, copies, stream):
    import numpy as np

    from hxq_synth import gen

    launch = [[] for _ in range(copies)]
    devs = [[to_dev(l, torch) for l in layers] for _ in range(copies)]
    xs, ys = [], []
    for i, lay in enumerate(layers):
        xf = gen.synth_x(cfg_x, i, M, lay.K)
        if xdt == "bf16":
            x = torch.from_numpy(gen.to_bf16_bits(xf).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            x = torch.from_numpy(xf).cuda()
        xs.append(x)
        ys.append(torch.empty((M, lay.N), dtype=torch.float32, device="cuda"))
    for r in range(copies):
        for i, lay in enumerate(layers):
            launch[r].append(Launcher(L, lay.fmt, devs[r][i], xs[i], ys[i], M, lay.N, lay.K, stream))
    return launch, devs, xs, ys


def cpu_baseline(layers, M, budget_s=15.0):
    """The CPU oracle over the same layer set, as many whole steps as fit in
    about `budget_s` seconds (at least one)."""
    import numpy as np

    import oracle
    from hxq_synth import gen

    xs = [gen.synth_x(1, i, M, l.K) for i, l in enumerate(layers)]
    steps, t0 = 0, time.perf_counter()
    while True:
        for lay, x in zip(layers, xs):
            oracle.hxq_linear_fwd_u8(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, x,
                                     "f32", lay.bias, want_bound=False)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 500:
            break
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    byts = sum(algorithmic_bytes(l.fmt, l.N, l.K, l.nnz, M, 4) for l in layers)
    return dict(value=round(byts * steps / el / 1e9, 4), unit="GB/s", cores=int(cores), kind="oracle",
                sample="%d full step(s) of the 7-layer set at M=%d (fp64 numpy oracle), %.1f s"
                       % (steps, M, el))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import vq_compressed_linear_amd as hx
    from hxq_synth import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 10}))
        return 0
    L = hx.lib()
    stream = torch.cuda.current_stream().cuda_stream
    props = torch.cuda.get_device_properties(0)
    log("device", props.name, "CUs", props.multi_processor_count)

    log("generating the Qwen2.5-3B-shaped u8 layer set")
    t0 = time.perf_counter()
    layers = gen.config_layers(1)
    log("generated in %.1f s" % (time.perf_counter() - t0))
    set_bytes = sum(l.compressed_bytes() for l in layers)
    copies = max(1, -(-ROTATE_BYTES // set_bytes))
    log("set %.1f MB compressed, %d rotating copies" % (set_bytes / 1e6, copies))

    results = {}
    for M in (1, 8):
        launch, devs, xs, ys = build_set(torch, L, layers, M, "f32", 1, copies, stream)
        # pass 1: the step as it runs (no per-kernel events); pass 2: per-launch events
        total_ms, _ = time_steps(torch, launch, args.steps, args.warmup, per_kernel=False)
        _, per = time_steps(torch, launch, args.steps, 2, per_kernel=True)
        byts = [algorithmic_bytes(l.fmt, l.N, l.K, l.nnz, M, 4) for l in layers]
        step_ms = total_ms / args.steps
        med = [float(np.median(p)) for p in per]
        results[M] = dict(step_ms=step_ms, bytes=sum(byts), per_layer=[
            dict(layer=l.name, N=l.N, K=l.K, bytes=b, median_us=round(m * 1e3, 3),
                 gbs=round(b / (m * 1e-3) / 1e9, 1)) for l, b, m in zip(layers, byts, med)],
            kernel_total_ms=sum(sum(p) for p in per), launches=args.steps * len(layers),
            kernel_bytes=sum(byts) * args.steps)
        log("M=%d step %.2f us, %.1f GB/s" % (M, step_ms * 1e3, sum(byts) / (step_ms * 1e-3) / 1e9))
        del launch, devs, xs, ys
        torch.cuda.empty_cache()

    prefill = None
    if not args.no_prefill:
        M = 2048
        launch, devs, xs, ys = build_set(torch, L, layers, M, "bf16", 4, 1, stream)
        steps = max(3, args.steps // 5)
        total_ms, per = time_steps(torch, launch, steps, max(1, args.warmup // 5))
        flops = sum(2.0 * M * l.N * l.K for l in layers)
        tfs = flops / (total_ms / steps * 1e-3) / 1e12
        prefill = dict(workload="Qwen2.5-3B-shaped u8 layer set, prefill M=2048, bf16 x", M=M,
                       step_ms=round(total_ms / steps, 4), tflops=round(tfs, 2),
                       frac_of_mfma_peak=round(tfs / MFMA_BF16_PEAK_TFS, 4),
                       per_layer_median_us=[round(float(np.median(p)) * 1e3, 2) for p in per])
        log("prefill M=2048 step %.1f us, %.1f TFLOP/s" % (total_ms / steps * 1e3, tfs))
        del launch, devs, xs, ys
        torch.cuda.empty_cache()

    r1 = results[1]
    value = r1["bytes"] / (r1["step_ms"] * 1e-3) / 1e9
    avg_launch_s = r1["kernel_total_ms"] * 1e-3 / r1["launches"]
    avg_bytes = r1["kernel_bytes"] / r1["launches"]
    achieved = avg_bytes / avg_launch_s / 1e9
    traffic = load_traffic("gemv_u8_valu_m1")
    out = {
        "metric": "HelixLinear decode GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; k-means codebooks fit on N(0, 0.02^2) weights with 0.1% outliers)",
        "config": {"workload": "Qwen2.5-3B-shaped HelixLinear layer set (q,k,v,o,gate,up,down), "
                               "u8 1D VQ + 0.1% sidecar, decode M=1, fp32 x",
                   "M": 1, "layers": len(layers), "bytes_per_step": r1["bytes"],
                   "rotating_copies": copies},
        "roofline": {"bound": "hbm", "kernel": "gemv_u8_valu<MT=1,R=4>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(avg_bytes)},
        "decode_m8": {"step_ms": round(results[8]["step_ms"], 5),
                      "gbs": round(results[8]["bytes"] / (results[8]["step_ms"] * 1e-3) / 1e9, 1),
                      "per_layer": results[8]["per_layer"]},
        "per_layer_m1": r1["per_layer"],
        "prefill": prefill,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(layers, 1)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
