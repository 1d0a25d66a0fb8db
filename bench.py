#!/usr/bin/env python3
"""HelixLinear forward throughput on one MI355X.

Workload: the Qwen2.5-3B-shaped u8 layer set (q, k, v, o, gate, up, down:
seven HelixLinear layers, each with its own 256-entry codebook and a 0.1%
sidecar), decode with one token (M = 1), fp32 activations.  A step is one
forward through all seven layers, issued the way a decoder layer issues them:
the projections that read the same activations share a launch
(hxq_linear_fwd_grouped for q|k|v and gate|up; o and down alone), four
launches in all.  Inputs are seeded synthetic data resident in HBM before
timing; the compressed weights rotate over enough copies (>= 512 MB) that no
step is served from the 256 MB Infinity Cache.

value: algorithmic GB/s of the step (the compressed bytes the method must
move: indices, codebooks, sidecar triplets, x once per launch, bias, y) over
the GPU time of the timed steps.  Also reported: the same step issued as seven
single-layer calls, the M = 8 step, the bf16 prefill GEMM at M = 2048
(TFLOP/s; u8 layer set and two pk12 layers), the input gradient dx = dy W of
the layer set (M = 1 fp32 in GB/s, M = 2048 bf16 in TFLOP/s), the read
bandwidth of a plain streaming kernel over the same rotated buffers, the
roofline of the dominant launch (gate|up) and the CPU oracle baseline.

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
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
DOMINANT = 2                  # gate|up: the largest launch of the step


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_bytes(fmt, N, K, nnz, M, x_bytes, bias=True, with_x=True):
    """Bytes one layer's forward must move: index storage, codebook, sidecar
    triplets (12 B each), activations (unless another layer of the same
    launch reads them), bias and the fp32 output."""
    if fmt == "u8":
        idx, cb = N * K, 256 * 4
    else:
        idx, cb = N * 3 * ((K + 3) // 4), 4096 * 8
    return idx + cb + 12 * nnz + (M * K * x_bytes if with_x else 0) + (4 * N if bias else 0) + 4 * M * N


def group_bytes(layers, M, x_bytes):
    return sum(layer_bytes(l.fmt, l.N, l.K, l.nnz, M, x_bytes, with_x=(i == 0)) for i, l in enumerate(layers))


# the decode kernel's source and the headers it includes: the counters in
# profiles/traffic.json are that kernel's and stay valid while these are unchanged
DECODE_SOURCES = ("hxq_decode1.hip", "hxq_decode.hip", "hxq_device.h", "hxq_launch.h")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vq_compressed_linear_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
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


def to_dev(lay, torch):
    import numpy as np

    def t(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()

    return dict(codebook=t(lay.codebook), indices=t(lay.indices), rows=t(lay.rows, np.int32),
                cols=t(lay.cols, np.int32), deltas=t(lay.deltas, np.float32), bias=t(lay.bias, np.float32))


class GroupCall:
    """One pre-marshalled hxq_linear_fwd_grouped call (keeps host overhead low)."""

    def __init__(self, L, B, devs, ys, x, M, K, stream):
        arr = (B.HxqLayer * len(devs))()
        for i, (d, y) in enumerate(zip(devs, ys)):
            arr[i] = B.HxqLayer(d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                                d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(),
                                d["bias"].data_ptr(), y.data_ptr(), y.shape[1])
        self.fn = L.hxq_linear_fwd_grouped
        xdt = B.HXQ_BF16 if x.element_size() == 2 else B.HXQ_F32
        self.args = (B.HXQ_FMT_U8, arr, len(devs), x.data_ptr(), xdt, M, K, stream)
        self.keep = arr

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("hxq_linear_fwd_grouped failed with status %d" % st)


class LayerCall:
    """One pre-marshalled single-layer call."""

    def __init__(self, L, B, d, y, x, M, N, K, stream, pk12=False):
        self.fn = L.hxq_linear_fwd_pk12 if pk12 else L.hxq_linear_fwd_u8
        xdt = B.HXQ_BF16 if x.element_size() == 2 else B.HXQ_F32
        self.args = (d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(), d["cols"].data_ptr(),
                     d["deltas"].data_ptr(), d["rows"].numel(), x.data_ptr(), xdt, d["bias"].data_ptr(),
                     y.data_ptr(), M, N, K, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("HelixLinear forward failed with status %d" % st)


class BwdCall:
    """One pre-marshalled hxq_linear_bwd_x call (dx = dy W, the input gradient)."""

    def __init__(self, L, B, d, dy, dx, M, N, K, stream, ws):
        self.fn = L.hxq_linear_bwd_x
        dyt = B.HXQ_BF16 if dy.element_size() == 2 else B.HXQ_F32
        self.args = (B.HXQ_FMT_U8, d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                     d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(), dy.data_ptr(), dyt,
                     dx.data_ptr(), M, N, K, ws.data_ptr(), ws.numel(), stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("hxq_linear_bwd_x failed with status %d" % st)


def bwd_bytes(l, M, dy_bytes):
    """Bytes the input gradient of one u8 layer must move: index storage,
    codebook, sidecar triplets, dy once and the fp32 dx."""
    return l.N * l.K + 256 * 4 + 12 * l.nnz + M * l.N * dy_bytes + 4 * M * l.K


def input_gradient(torch, L, B, layers, devs, M, dtype, steps, warmup, stream):
    """dx = dy W for every layer of the set, one call per layer (devs[r][i]:
    copy r of layer i).  Returns per-layer averages and the seven-layer step."""
    import numpy as np

    rng = np.random.Generator(np.random.PCG64(77))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dys = [torch.from_numpy(rng.standard_normal((M, l.N)).astype(np.float32)).cuda().to(tdt) for l in layers]
    dxs = [torch.empty((M, l.K), dtype=torch.float32, device="cuda") for l in layers]
    need = max(L.hxq_linear_bwd_x_workspace(B.HXQ_FMT_U8, B.HXQ_F32 if dtype == "f32" else B.HXQ_BF16, M, l.N,
                                            l.K, l.nnz) for l in layers)
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device="cuda")
    calls = [[BwdCall(L, B, row[i], dys[i], dxs[i], M, l.N, l.K, stream, ws) for i, l in enumerate(layers)]
             for row in devs]
    total = time_steps(torch, calls, steps, warmup)
    avg = []
    for i in range(len(layers)):
        ti = time_steps(torch, [[row[i]] for row in calls], steps, 1)
        avg.append(ti / steps)
    xb = 4 if dtype == "f32" else 2
    rows = []
    for l, m in zip(layers, avg):
        r = dict(layer=l.name, N=l.N, K=l.K, avg_us=round(m * 1e3, 3))
        if M == 1:
            r["gbs"] = round(bwd_bytes(l, M, xb) / (m * 1e-3) / 1e9, 1)
        else:
            r["tflops"] = round(2.0 * M * l.N * l.K / (m * 1e-3) / 1e12, 1)
        rows.append(r)
    step_us = total / steps * 1e3
    out = dict(M=M, dy_dtype=dtype, step_us=round(step_us, 2), layers=rows, workspace_bytes=int(need))
    if M == 1:
        gbs = sum(bwd_bytes(l, M, xb) for l in layers) / (step_us * 1e-6) / 1e9
        out.update(workload="input gradient dx = dy W of the Qwen2.5-3B-shaped u8 layer set, M=1, fp32 dy, "
                            "one call per layer, rotating copies", gbs=round(gbs, 1),
                   frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
    else:
        tfs = sum(2.0 * M * l.N * l.K for l in layers) / (step_us * 1e-6) / 1e12
        out.update(workload="input gradient dx = dy W of the Qwen2.5-3B-shaped u8 layer set, M=%d, bf16 dy "
                            "(bf16 matrix cores), one call per layer" % M, tflops=round(tfs, 1),
                   frac_of_mfma_peak=round(tfs / MFMA_BF16_PEAK_TFS, 4))
    del dys, dxs, ws
    return out


def hold_gpu(torch, ms):
    """Keep the GPU busy for about `ms` so the host can queue a timed region
    ahead of execution (launch latency then stays out of the event times)."""
    torch.cuda._sleep(int(ms * 2.0e6))


def time_steps(torch, calls, steps, warmup):
    """calls[r][i]: copy r, launch i.  Times `steps` steps (copy s % R at step
    s) between two events on the launch stream, with nothing between the
    launches.  Returns the total in ms."""
    R = len(calls)
    for s in range(warmup):
        for f in calls[s % R]:
            f()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    hold_gpu(torch, 20 + steps * len(calls[0]) * 0.05)
    t0.record()
    for s in range(steps):
        for f in calls[s % R]:
            f()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


class LayerSet:
    """Device copies of the layer set, activations and outputs for one M."""

    def __init__(self, torch, L, B, layers, M, xdt, cfg_x, copies, stream):
        import numpy as np

        from hxq_synth import gen

        self.layers = layers
        self.by_name = {l.name: i for i, l in enumerate(layers)}
        self.devs = [[to_dev(l, torch) for l in layers] for _ in range(copies)]
        self.xs, self.ys = [], []
        for i, lay in enumerate(layers):
            xf = gen.synth_x(cfg_x, i, M, lay.K)
            if xdt == "bf16":
                x = torch.from_numpy(gen.to_bf16_bits(xf).view(np.int16)).cuda().view(torch.bfloat16)
            else:
                x = torch.from_numpy(xf).cuda()
            self.xs.append(x)
            self.ys.append(torch.empty((M, lay.N), dtype=torch.float32, device="cuda"))
        self.grouped = []
        self.single = []
        for r in range(copies):
            row = []
            for g in GROUPS:
                idx = [self.by_name[n] for n in g]
                row.append(GroupCall(L, B, [self.devs[r][i] for i in idx], [self.ys[i] for i in idx],
                                     self.xs[idx[0]], M, layers[idx[0]].K, stream))
            self.grouped.append(row)
            self.single.append([LayerCall(L, B, self.devs[r][i], self.ys[i], self.xs[i], M, l.N, l.K, stream)
                                for i, l in enumerate(layers)])
        xb = 2 if xdt == "bf16" else 4
        self.group_bytes = [group_bytes([layers[self.by_name[n]] for n in g], M, xb) for g in GROUPS]
        self.layer_bytes = [layer_bytes(l.fmt, l.N, l.K, l.nnz, M, xb) for l in layers]


def stream_ceiling(torch, L, sets, steps):
    """GB/s of hxq_stream_read over the gate and up index buffers of every
    rotating copy (each launch reads one of them: the same bytes the
    dominant launch streams, in the same rotation)."""
    import numpy as np

    bufs = []
    for devs in sets.devs:
        for n in GROUPS[DOMINANT]:
            bufs.append(devs[sets.by_name[n]]["indices"])
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def reader(b):
        def f():
            st = L.hxq_stream_read(b.data_ptr(), b.numel(), sink.data_ptr(), 4096, stream)
            if st != 0:
                raise RuntimeError("hxq_stream_read failed with status %d" % st)
        return f

    calls = [[reader(b)] for b in bufs]
    n = max(steps, len(bufs))
    total = time_steps(torch, calls, n, 2)
    avg = total / n
    nbytes = bufs[0].numel()
    return dict(kernel="stream_read_kernel (hxq_stream_read)", bytes_per_launch=nbytes,
                avg_us=round(avg * 1e3, 3), gbs=round(nbytes / (avg * 1e-3) / 1e9, 1))


def prefill_pk12(torch, L, B, stream, M, steps):
    """The bf16 matrix-core GEMM on 2D-VQ (pk12) layers of the pk12
    configuration's shapes (seeded random pair indices and codebook, 0.05%
    sidecar: the kernel's speed does not depend on how the codebook was fit),
    one single-layer call per layer at M tokens of bf16 x."""
    import numpy as np

    from hxq_synth import gen

    rows = []
    for i, (name, N, K) in enumerate(gen.CONFIGS[3]["layers"]):
        lay = gen.random_layer(9000 + i, N, K, "pk12", nnz=N * K // 2000)
        d = to_dev(lay, torch)
        xf = gen.synth_x(3, i, M, K)
        x = torch.from_numpy(gen.to_bf16_bits(xf).view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        call = LayerCall(L, B, d, y, x, M, N, K, stream, pk12=True)
        t = time_steps(torch, [[call]], steps, 1) / steps
        rows.append(dict(layer=name, N=N, K=K, avg_us=round(t * 1e3, 2),
                         tflops=round(2.0 * M * N * K / (t * 1e-3) / 1e12, 1)))
        del d, x, y
    return dict(workload="2D-VQ (pk12) gate/down-shaped layers (11008x2048, 2048x11008), prefill M=%d, "
                         "bf16 x, one call per layer" % M, M=M, layers=rows)


def buffered_baseline(torch, L, B, layers, stream, M, steps, fused_step_us):
    """The buffered design the pages describe, for comparison only (the
    library never forms the weight): per layer, the dense bf16 weight into
    one shared buffer sized to the largest layer (hxq_dequant_bf16), then the
    library bf16 matmul (torch.mm, hipBLASLt), bias added; bf16 x at M tokens."""
    import numpy as np

    from hxq_synth import gen

    devs = [to_dev(l, torch) for l in layers]
    big = max(l.N * l.K for l in layers)
    wbuf = torch.empty(big, dtype=torch.bfloat16, device="cuda")
    xs = [torch.from_numpy(gen.to_bf16_bits(gen.synth_x(4, i, M, l.K)).view(np.int16)).cuda().view(torch.bfloat16)
          for i, l in enumerate(layers)]
    deq_args = []
    for d, l in zip(devs, layers):
        deq_args.append((B.HXQ_FMT_U8, d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                         d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(), wbuf.data_ptr(), l.N, l.K,
                         stream))
    biases = [d["bias"].to(torch.bfloat16) for d in devs]

    def deq(i):
        def f():
            st = L.hxq_dequant_bf16(*deq_args[i])
            if st != 0:
                raise RuntimeError("hxq_dequant_bf16 failed with status %d" % st)
        return f

    def mm(i):
        w = wbuf[: layers[i].N * layers[i].K].view(layers[i].N, layers[i].K)

        def f():
            torch.addmm(biases[i], xs[i], w.t())
        return f

    per = []
    for i, l in enumerate(layers):
        td = time_steps(torch, [[deq(i)]], steps, 1) / steps
        tm = time_steps(torch, [[mm(i)]], steps, 1) / steps
        per.append(dict(layer=l.name, dequant_us=round(td * 1e3, 2), matmul_us=round(tm * 1e3, 2)))
    step = time_steps(torch, [[f for i in range(len(layers)) for f in (deq(i), mm(i))]], steps, 1) / steps
    flops = sum(2.0 * M * l.N * l.K for l in layers)
    return dict(workload="the same u8 layer set at M=%d, bf16 x: per layer the bf16 weight into one shared buffer, "
                         "then torch.addmm (hipBLASLt, bf16 output)" % M,
                step_us=round(step * 1e3, 2), tflops=round(flops / (step * 1e-3) / 1e12, 1),
                fused_step_us=fused_step_us, layers=per)


def cpu_baseline(layers, M, budget_s=15.0):
    """The CPU oracle over the same layer set, as many whole steps as fit in
    about `budget_s` seconds (at least one)."""
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
    byts = sum(layer_bytes(l.fmt, l.N, l.K, l.nnz, M, 4) for l in layers)
    return dict(value=round(byts * steps / el / 1e9, 4), unit="GB/s", cores=int(cores), kind="oracle",
                sample="%d full step(s) of the 7-layer set at M=%d (fp64 numpy oracle), %.1f s"
                       % (steps, M, el))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline step (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import vq_compressed_linear_amd as hx
    from hxq_synth import gen
    from vq_compressed_linear_amd import _binding as B

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

    # ---- headline: M = 1, grouped launches
    s1 = LayerSet(torch, L, B, layers, 1, "f32", 1, copies, stream)
    total_ms = time_steps(torch, s1.grouped, args.steps, args.warmup)
    step_ms = total_ms / args.steps
    bytes_step = sum(s1.group_bytes)
    value = bytes_step / (step_ms * 1e-3) / 1e9
    log("M=1 grouped step %.2f us, %.1f GB/s" % (step_ms * 1e3, value))
    # each launch type timed on its own, back to back over the rotating copies
    # (events around the whole run, so no event sits between two launches)
    avg = []
    for g in range(len(GROUPS)):
        tg = time_steps(torch, [[row[g]] for row in s1.grouped], args.steps, 2)
        avg.append(tg / args.steps)
    per_group = [dict(launch="|".join(g), bytes=b, avg_us=round(m * 1e3, 3),
                      gbs=round(b / (m * 1e-3) / 1e9, 1)) for g, b, m in zip(GROUPS, s1.group_bytes, avg)]
    dom_avg_s = avg[DOMINANT] * 1e-3
    dom_bytes = s1.group_bytes[DOMINANT]
    achieved = dom_bytes / dom_avg_s / 1e9

    extras = {}
    if not args.no_extras:
        total1 = time_steps(torch, s1.single, args.steps, args.warmup)
        avg1 = []
        for i in range(len(layers)):
            ti = time_steps(torch, [[row[i]] for row in s1.single], args.steps, 2)
            avg1.append(ti / args.steps)
        extras["per_layer_step_m1"] = dict(
            step_us=round(total1 / args.steps * 1e3, 3),
            gbs=round(sum(s1.layer_bytes) / (total1 / args.steps * 1e-3) / 1e9, 1),
            layers=[dict(layer=l.name, N=l.N, K=l.K, bytes=b, avg_us=round(m * 1e3, 3),
                         gbs=round(b / (m * 1e-3) / 1e9, 1))
                    for l, b, m in zip(layers, s1.layer_bytes, avg1)])
        extras["stream_ceiling"] = stream_ceiling(torch, L, s1, args.steps)
        log("stream ceiling %.1f GB/s" % extras["stream_ceiling"]["gbs"])
        extras["input_gradient_m1"] = input_gradient(torch, L, B, layers, s1.devs, 1, "f32", args.steps,
                                                     args.warmup, stream)
        log("input gradient M=1 step %.1f us, %.1f GB/s" % (extras["input_gradient_m1"]["step_us"],
                                                            extras["input_gradient_m1"]["gbs"]))
    del s1
    torch.cuda.empty_cache()

    if not args.no_extras:
        s8 = LayerSet(torch, L, B, layers, 8, "f32", 1, copies, stream)
        total8 = time_steps(torch, s8.grouped, args.steps, args.warmup)
        avg8 = []
        for g in range(len(GROUPS)):
            tg = time_steps(torch, [[row[g]] for row in s8.grouped], args.steps, 2)
            avg8.append(tg / args.steps)
        extras["decode_m8"] = dict(
            step_us=round(total8 / args.steps * 1e3, 3),
            gbs=round(sum(s8.group_bytes) / (total8 / args.steps * 1e-3) / 1e9, 1),
            launches=[dict(launch="|".join(g), avg_us=round(m * 1e3, 3)) for g, m in zip(GROUPS, avg8)])
        log("M=8 grouped step %.2f us" % (total8 / args.steps * 1e3))
        del s8
        torch.cuda.empty_cache()

    if not args.no_extras and not args.no_prefill:
        M = 2048
        sp = LayerSet(torch, L, B, layers, M, "bf16", 4, 1, stream)
        steps = max(3, args.steps // 10)
        # the step as launches that share x (q|k|v, o, gate|up, down), like the decode step
        total_p = time_steps(torch, sp.grouped, steps, max(1, args.warmup // 5))
        avg_g = []
        for g in range(len(GROUPS)):
            tg = time_steps(torch, [[row[g]] for row in sp.grouped], steps, 1)
            avg_g.append(tg / steps)
        avgp = []
        for i in range(len(layers)):
            ti = time_steps(torch, [[row[i]] for row in sp.single], steps, 1)
            avgp.append(ti / steps)
        flops = sum(2.0 * M * l.N * l.K for l in layers)
        tfs = flops / (total_p / steps * 1e-3) / 1e12
        gfl = [sum(2.0 * M * layers[sp.by_name[n]].N * layers[sp.by_name[n]].K for n in g) for g in GROUPS]
        extras["prefill"] = dict(workload="Qwen2.5-3B-shaped u8 layer set, prefill M=2048, bf16 x; launches "
                                          "q|k|v, o, gate|up, down", M=M,
                                 step_us=round(total_p / steps * 1e3, 2), tflops=round(tfs, 2),
                                 frac_of_mfma_peak=round(tfs / MFMA_BF16_PEAK_TFS, 4),
                                 launches=[dict(launch="|".join(g), avg_us=round(m * 1e3, 2),
                                                tflops=round(f / (m * 1e-3) / 1e12, 1))
                                           for g, m, f in zip(GROUPS, avg_g, gfl)],
                                 single_layer_calls=[dict(layer=l.name, avg_us=round(m * 1e3, 2),
                                                          tflops=round(2.0 * M * l.N * l.K / (m * 1e-3) / 1e12, 1))
                                                     for l, m in zip(layers, avgp)])
        log("prefill M=2048 step %.1f us, %.1f TFLOP/s" % (total_p / steps * 1e3, tfs))
        extras["input_gradient_m2048"] = input_gradient(torch, L, B, layers, sp.devs, M, "bf16", steps,
                                                        max(1, args.warmup // 5), stream)
        log("input gradient M=2048 step %.1f us, %.1f TFLOP/s" % (extras["input_gradient_m2048"]["step_us"],
                                                                  extras["input_gradient_m2048"]["tflops"]))
        del sp
        torch.cuda.empty_cache()
        extras["prefill_pk12"] = prefill_pk12(torch, L, B, stream, M, steps)
        extras["buffered_baseline"] = buffered_baseline(torch, L, B, layers, stream, M, steps,
                                                        extras["prefill"]["step_us"])
        log("buffered (dequant + library matmul) M=2048 step %.1f us"
            % extras["buffered_baseline"]["step_us"])
        log("pk12 prefill M=2048: %s" % ", ".join("%s %.1f us" % (r["layer"], r["avg_us"])
                                                  for r in extras["prefill_pk12"]["layers"]))

    out = {
        "metric": "HelixLinear decode GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; k-means codebooks fit on N(0, 0.02^2) weights with 0.1% outliers)",
        "config": {"workload": "Qwen2.5-3B-shaped HelixLinear layer set (q,k,v,o,gate,up,down), "
                               "u8 1D VQ + 0.1% sidecar, decode M=1, fp32 x; launches q|k|v, o, gate|up, down",
                   "M": 1, "layers": len(layers), "launches_per_step": len(GROUPS),
                   "bytes_per_step": bytes_step, "rotating_copies": copies},
        "roofline": {"bound": "hbm", "kernel": "decode1_gemv (gate|up launch)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("decode_gemv_gate_up_m1"),
                     "avg_launch_us": round(dom_avg_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(dom_bytes)},
        "per_launch_m1": per_group,
        "cpu_baseline": None,
    }
    out.update(extras)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(layers, 1)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
