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
the layer set, one grouped call per shared input like the forward (M = 1
fp32 in GB/s, M = 2048 bf16 in TFLOP/s), the read
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
FP32_PEAK_TFS = 157.3         # MI355X fp32 vector / matrix-core rate (the fp32-arithmetic paths)
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


class WsCall:
    """One pre-marshalled hxq_linear_fwd_ws call: a single layer with a
    workspace for its k split (the prefill steps' o and down launches)."""

    def __init__(self, L, B, d, y, x, M, N, K, stream, ws):
        self.fn = L.hxq_linear_fwd_ws
        xdt = B.HXQ_BF16 if x.element_size() == 2 else B.HXQ_F32
        self.args = (B.HXQ_FMT_U8, d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                     d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(), x.data_ptr(), xdt,
                     d["bias"].data_ptr(), y.data_ptr(), M, N, K,
                     ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("hxq_linear_fwd_ws failed with status %d" % st)


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


class BwdGroupCall:
    """One pre-marshalled hxq_linear_bwd_x_grouped call: dx = sum_i dy_i W_i
    over layers that share their input."""

    def __init__(self, L, B, ds, dys, dx, M, K, stream, ws):
        self.fn = L.hxq_linear_bwd_x_grouped
        self.arr = (B.HxqBwdLayer * len(ds))()
        for i, (d, dy) in enumerate(zip(ds, dys)):
            self.arr[i] = B.HxqBwdLayer(d["codebook"].data_ptr(), d["indices"].data_ptr(), d["rows"].data_ptr(),
                                        d["cols"].data_ptr(), d["deltas"].data_ptr(), d["rows"].numel(),
                                        dy.data_ptr(), d["indices"].shape[0])
        self.dyt = B.HXQ_BF16 if dys[0].element_size() == 2 else B.HXQ_F32
        self.need = L.hxq_linear_bwd_x_grouped_workspace(B.HXQ_FMT_U8, self.dyt, self.arr, len(ds), M, K)
        self.args = (B.HXQ_FMT_U8, self.arr, len(ds), self.dyt, dx.data_ptr(), M, K,
                     ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("hxq_linear_bwd_x_grouped failed with status %d" % st)


def bwd_bytes(l, M, dy_bytes):
    """Bytes the input gradient of one u8 layer must move: index storage,
    codebook, sidecar triplets, dy once and the fp32 dx."""
    return l.N * l.K + 256 * 4 + 12 * l.nnz + M * l.N * dy_bytes + 4 * M * l.K


def bwd_group_bytes(ls, M, dy_bytes):
    """The same for layers sharing their input: one dx for the group."""
    return sum(bwd_bytes(l, M, dy_bytes) - 4 * M * l.K for l in ls) + 4 * M * ls[0].K


def input_gradient(torch, L, B, layers, devs, M, dtype, steps, warmup, stream):
    """dx = dy W through the layer set (devs[r][i]: copy r of layer i): the
    step is one grouped call per input the layers share (q|k|v, o, gate|up,
    down: each input's gradient summed over its layers); per-layer averages
    come from single-layer calls."""
    import numpy as np

    rng = np.random.Generator(np.random.PCG64(77))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dys = [torch.from_numpy(rng.standard_normal((M, l.N)).astype(np.float32)).cuda().to(tdt) for l in layers]
    dxs = [torch.empty((M, l.K), dtype=torch.float32, device="cuda") for l in layers]
    by_name = {l.name: i for i, l in enumerate(layers)}
    gidx = [[by_name[n] for n in g] for g in GROUPS]
    gdx = [torch.empty((M, layers[ix[0]].K), dtype=torch.float32, device="cuda") for ix in gidx]
    need = max(L.hxq_linear_bwd_x_workspace(B.HXQ_FMT_U8, B.HXQ_F32 if dtype == "f32" else B.HXQ_BF16, M, l.N,
                                            l.K, l.nnz) for l in layers)
    for ix, dx in zip(gidx, gdx):
        probe = BwdGroupCall(L, B, [devs[0][i] for i in ix], [dys[i] for i in ix], dx, M, layers[ix[0]].K,
                             stream, None)
        if probe.need < 0:
            raise RuntimeError("hxq_linear_bwd_x_grouped_workspace failed with status %d" % probe.need)
        need = max(need, probe.need)
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device="cuda")
    calls = [[BwdCall(L, B, row[i], dys[i], dxs[i], M, l.N, l.K, stream, ws) for i, l in enumerate(layers)]
             for row in devs]
    gcalls = [[BwdGroupCall(L, B, [row[i] for i in ix], [dys[i] for i in ix], dx, M, layers[ix[0]].K, stream, ws)
               for ix, dx in zip(gidx, gdx)] for row in devs]
    total = time_steps(torch, gcalls, steps, warmup)
    per_group = []
    for g in range(len(GROUPS)):
        tg = time_steps(torch, [[row[g]] for row in gcalls], steps, 1)
        per_group.append(round(tg / steps * 1e3, 2))
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
    out = dict(M=M, dy_dtype=dtype, step_us=round(step_us, 2), layers=rows, workspace_bytes=int(need),
               launches=dict(zip(["qkv", "o", "gateup", "down"], per_group)))
    if M == 1:
        gbs = sum(bwd_group_bytes([layers[i] for i in ix], M, xb) for ix in gidx) / (step_us * 1e-6) / 1e9
        out.update(workload="input gradient of the Qwen2.5-3B-shaped u8 layer set, M=1, fp32 dy: one grouped "
                            "call per shared input (q|k|v, o, gate|up, down; dx = sum of dy_i W_i), rotating copies",
                   gbs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
    else:
        tfs = sum(2.0 * M * l.N * l.K for l in layers) / (step_us * 1e-6) / 1e12
        out.update(workload="input gradient of the Qwen2.5-3B-shaped u8 layer set, M=%d, bf16 dy (bf16 matrix "
                            "cores): one grouped call per shared input (q|k|v, o, gate|up, down)" % M,
                   tflops=round(tfs, 1), frac_of_mfma_peak=round(tfs / MFMA_BF16_PEAK_TFS, 4))
    del dys, dxs, gdx, ws
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
        """Launches that share x go through hxq_linear_fwd_grouped; with bf16
        x (the prefill steps) a layer alone goes through hxq_linear_fwd_ws
        with a workspace for its k split."""
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
        self.ws = None
        if xdt == "bf16":
            need = max(L.hxq_linear_fwd_workspace(B.HXQ_FMT_U8, B.HXQ_BF16, M, l.N, l.K) for l in layers)
            if need < 0:
                raise RuntimeError("hxq_linear_fwd_workspace failed with status %d" % need)
            if need > 0:
                self.ws = torch.empty(int(need), dtype=torch.uint8, device="cuda")
        for r in range(copies):
            row = []
            for g in GROUPS:
                idx = [self.by_name[n] for n in g]
                if len(idx) == 1 and xdt == "bf16":
                    i = idx[0]
                    row.append(WsCall(L, B, self.devs[r][i], self.ys[i], self.xs[i], M, layers[i].N, layers[i].K,
                                      stream, self.ws))
                else:
                    row.append(GroupCall(L, B, [self.devs[r][i] for i in idx], [self.ys[i] for i in idx],
                                         self.xs[idx[0]], M, layers[idx[0]].K, stream))
            self.grouped.append(row)
            self.single.append([LayerCall(L, B, self.devs[r][i], self.ys[i], self.xs[i], M, l.N, l.K, stream)
                                for i, l in enumerate(layers)])
        xb = 2 if xdt == "bf16" else 4
        self.group_bytes = [group_bytes([layers[self.by_name[n]] for n in g], M, xb) for g in GROUPS]
        self.layer_bytes = [layer_bytes(l.fmt, l.N, l.K, l.nnz, M, xb) for l in layers]


def stream_ceiling(torch, L, nbytes, steps):
    """Attainable read bandwidth at the dominant launch's size: hxq_stream_read
    (ordinary loads) and hxq_stream_read_nt (non-temporal loads) over
    contiguous buffers of `nbytes` (as many rotating copies as exceed twice the
    Infinity Cache), for a sweep of grid sizes; the best is the ceiling the
    decode kernels are compared against."""
    nb = nbytes // 16 * 16
    copies = max(2, -(-ROTATE_BYTES // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(i & 255) for i in range(copies)]
    stream = torch.cuda.current_stream().cuda_stream
    sweep = []
    for loads, fn in (("ordinary", L.hxq_stream_read), ("non-temporal", L.hxq_stream_read_nt)):
        for wgs in (256, 512, 1024, 2048, 4096, 8192):
            words = 8 * wgs  # a word per wave
            sink = torch.zeros(words, dtype=torch.int32, device="cuda")

            def reader(b, sink=sink, words=words, fn=fn):
                def f():
                    st = fn(b.data_ptr(), nb, sink.data_ptr(), words, stream)
                    if st != 0:
                        raise RuntimeError("stream read failed with status %d" % st)
                return f

            calls = [[reader(b)] for b in bufs]
            n = max(steps, len(bufs))
            avg = time_steps(torch, calls, n, 2) / n
            sweep.append(dict(loads=loads, workgroups=wgs, avg_us=round(avg * 1e3, 3),
                              gbs=round(nb / (avg * 1e-3) / 1e9, 1)))
    best = max(sweep, key=lambda r: r["gbs"])
    del bufs
    torch.cuda.empty_cache()
    return dict(kernel="stream_read_kernel (hxq_stream_read, hxq_stream_read_nt)", bytes_per_launch=nb,
                rotating_copies=copies, best_loads=best["loads"], best_workgroups=best["workgroups"],
                avg_us=best["avg_us"], gbs=best["gbs"], sweep=sweep)


def percentiles(torch, calls, n):
    """p10 / p50 / p90 of single launch durations (an event pair around each
    launch, copies rotating; the first launches are warm-up)."""
    import numpy as np

    R = len(calls)
    for s in range(4):
        for f in calls[s % R]:
            f()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    hold_gpu(torch, 20 + n * 0.05)
    for s in range(n):
        evs[s][0].record()
        for f in calls[s % R]:
            f()
        evs[s][1].record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return dict(p10_us=round(float(np.percentile(d, 10)), 3), p50_us=round(float(np.percentile(d, 50)), 3),
                p90_us=round(float(np.percentile(d, 90)), 3), launches=n)


def roof(bytes_, flops, t_us, arith):
    """GB/s and TFLOP/s of one measurement and its fraction of the binding
    roof: HBM, or the compute rate of its arithmetic (fp32 vector / matrix
    cores at 157.3 TFLOP/s, bf16 matrix cores at 2516.6), whichever would take
    longer at 100%."""
    t = t_us * 1e-6
    peak = FP32_PEAK_TFS if arith == "f32" else MFMA_BF16_PEAK_TFS
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_cmp = flops / (peak * 1e12)
    bound = "hbm" if t_hbm >= t_cmp else ("fp32_alu" if arith == "f32" else "mfma_bf16")
    return dict(gbs=round(bytes_ / t / 1e9, 1), tflops=round(flops / t / 1e12, 2),
                frac_hbm=round(bytes_ / t / 1e9 / HBM_PEAK_GBS, 4),
                frac_compute=round(flops / t / 1e12 / peak, 4), bound=bound,
                frac_of_binding=round(max(t_hbm, t_cmp) / t, 4))


def measure_layers(torch, L, B, layers, cases, steps, warmup, stream, cfg_x):
    """Single-layer forwards of `layers` for each (M, x dtype) in `cases`, over
    rotating copies of the layers (>= 512 MB in all), timed back to back.
    Returns one record per (layer, M, dtype) with its binding-roof fraction."""
    import numpy as np

    from hxq_synth import gen

    nbytes = sum(l.compressed_bytes() for l in layers)
    copies = max(1, -(-ROTATE_BYTES // nbytes))
    devs = [[to_dev(l, torch) for l in layers] for _ in range(copies)]
    rows = []
    for M, xdt in cases:
        for i, lay in enumerate(layers):
            xf = gen.synth_x(cfg_x, i, M, lay.K)
            if xdt == "bf16":
                x = torch.from_numpy(gen.to_bf16_bits(xf).view(np.int16)).cuda().view(torch.bfloat16)
            else:
                x = torch.from_numpy(xf).cuda()
            y = torch.empty((M, lay.N), dtype=torch.float32, device="cuda")
            calls = [[LayerCall(L, B, row[i], y, x, M, lay.N, lay.K, stream, pk12=lay.fmt == "pk12")]
                     for row in devs]
            n = max(steps, copies)
            t_us = time_steps(torch, calls, n, warmup) / n * 1e3
            xb = 2 if xdt == "bf16" else 4
            arith = "bf16" if (xdt == "bf16" and M > 16) else "f32"
            r = dict(layer=lay.name, fmt=lay.fmt, N=lay.N, K=lay.K, M=M, x=xdt, avg_us=round(t_us, 3))
            r.update(roof(layer_bytes(lay.fmt, lay.N, lay.K, lay.nnz, M, xb), 2.0 * M * lay.N * lay.K, t_us, arith))
            rows.append(r)
            del x, y
    del devs
    torch.cuda.empty_cache()
    return dict(rotating_copies=copies, layers=rows)


def config_blocks(torch, L, B, stream, steps, warmup):
    """The single-layer configuration (0), the Mamba2-shaped projections at
    1, 16 and 64 tokens in fp32 and bf16 (2) and the pk12 gate/down shapes at
    1 and 16 tokens (3), each with its binding roof."""
    from hxq_synth import gen

    out = {}
    out["config0"] = measure_layers(torch, L, B, gen.config_layers(0), [(1, "f32")], steps, warmup, stream, 0)
    out["config0"]["workload"] = "single 256x256 u8 layer, M=1, fp32 x (latency-bound: 70 KB)"
    log("config 0: %.2f us" % out["config0"]["layers"][0]["avg_us"])
    out["config2"] = measure_layers(torch, L, B, gen.config_layers(2),
                                    [(m, d) for d in ("f32", "bf16") for m in (1, 16, 64)], steps, warmup, stream, 2)
    out["config2"]["workload"] = ("Mamba2-1.3B-shaped u8 projections (in_proj 8512x2048, out_proj 2048x4096), "
                                  "0.1% sidecar, M = 1, 16, 64, fp32 and bf16 x")
    log("config 2: " + ", ".join("%s M=%d %s %.1f us" % (r["layer"], r["M"], r["x"], r["avg_us"])
                                 for r in out["config2"]["layers"]))
    pk = [gen.random_layer(9100 + i, N, K, "pk12", nnz=N * K // 2000) for i, (_, N, K) in enumerate(gen.PK12_LAYERS)]
    for l, (name, _, _) in zip(pk, gen.PK12_LAYERS):
        l.name = name
    out["config3"] = measure_layers(torch, L, B, pk, [(1, "f32"), (16, "f32")], steps, warmup, stream, 3)
    out["config3"]["workload"] = ("2D-VQ pk12 gate/down shapes (11008x2048, 2048x11008), 0.05% sidecar, "
                                  "M = 1 and 16, fp32 x; seeded random pair indices and codebook (the "
                                  "kernels' speed does not depend on how the codebook was fit)")
    log("config 3: " + ", ".join("%s M=%d %.1f us" % (r["layer"], r["M"], r["avg_us"])
                                 for r in out["config3"]["layers"]))
    return out


def prefill_big(torch, L, B, layers, stream, steps):
    """Config 4 at M = 25600 (50 chunks of 512 tokens, bf16 x): gate|up as one
    launch sharing x, then down, as a prefill step issues them."""
    import numpy as np

    from hxq_synth import gen

    M = 25600
    by = {l.name: l for l in layers}
    sel = [by["gate"], by["up"], by["down"]]
    devs = [to_dev(l, torch) for l in sel]
    x_gu = torch.from_numpy(gen.to_bf16_bits(gen.synth_x(4, 4, M, 2048)).view(np.int16)).cuda().view(torch.bfloat16)
    x_dn = torch.from_numpy(gen.to_bf16_bits(gen.synth_x(4, 6, M, 11008)).view(np.int16)).cuda().view(torch.bfloat16)
    ys = [torch.empty((M, l.N), dtype=torch.float32, device="cuda") for l in sel]
    gu = GroupCall(L, B, devs[:2], ys[:2], x_gu, M, 2048, stream)
    need = L.hxq_linear_fwd_workspace(B.HXQ_FMT_U8, B.HXQ_BF16, M, sel[2].N, sel[2].K)
    ws = torch.empty(int(need), dtype=torch.uint8, device="cuda") if need > 0 else None
    dn = WsCall(L, B, devs[2], ys[2], x_dn, M, sel[2].N, sel[2].K, stream, ws)
    t_gu = time_steps(torch, [[gu]], steps, 1) / steps * 1e3
    t_dn = time_steps(torch, [[dn]], steps, 1) / steps * 1e3
    f_gu = 2.0 * 2.0 * M * 11008 * 2048
    f_dn = 2.0 * M * 2048 * 11008
    b_gu = group_bytes(sel[:2], M, 2)
    b_dn = layer_bytes("u8", sel[2].N, sel[2].K, sel[2].nnz, M, 2)
    r_gu = dict(launch="gate|up", avg_us=round(t_gu, 2))
    r_gu.update(roof(b_gu, f_gu, t_gu, "bf16"))
    r_dn = dict(launch="down", avg_us=round(t_dn, 2))
    r_dn.update(roof(b_dn, f_dn, t_dn, "bf16"))
    tf = (f_gu + f_dn) / ((t_gu + t_dn) * 1e-6) / 1e12
    del devs, x_gu, x_dn, ys, ws
    torch.cuda.empty_cache()
    return dict(workload="gate|up and down of the Qwen2.5-3B-shaped u8 set at M=25600 (50 x 512 tokens), bf16 x",
                M=M, step_us=round(t_gu + t_dn, 2), tflops=round(tf, 1),
                frac_of_mfma_peak=round(tf / MFMA_BF16_PEAK_TFS, 4), launches=[r_gu, r_dn])


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
    """The CPU oracle (fp64 numpy) over the same layer set: three runs, each
    as many whole steps as fit in a third of `budget_s` (at least one), the
    median reported; BLAS threads as numpy has them (normally one per core the
    process may run on)."""
    import numpy as np

    import oracle
    from hxq_synth import gen

    xs = [gen.synth_x(1, i, M, l.K) for i, l in enumerate(layers)]
    byts = sum(layer_bytes(l.fmt, l.N, l.K, l.nnz, M, 4) for l in layers)
    rates, total_steps, total_s = [], 0, 0.0
    for _ in range(3):
        steps, t0 = 0, time.perf_counter()
        while True:
            for lay, x in zip(layers, xs):
                oracle.hxq_linear_fwd_u8(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, x,
                                         "f32", lay.bias, want_bound=False)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s / 3 or steps >= 200:
                break
        rates.append(byts * steps / el / 1e9)
        total_steps += steps
        total_s += el
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = None
    return dict(value=round(float(np.median(rates)), 4), unit="GB/s", cores=len(os.sched_getaffinity(0)),
                blas_threads=blas, kind="oracle", runs=[round(r, 4) for r in rates],
                sample="3 runs (median reported) of whole steps of the 7-layer Qwen2.5-3B-shaped u8 set at M=%d "
                       "(fp64 numpy oracle); %d steps in %.1f s" % (M, total_steps, total_s))


def cpu_single_thread(layer_sets):
    """The CPU oracle on one thread: one forward per layer of each
    configuration at one token (configs 0-3), median of three."""
    import numpy as np

    import oracle
    from hxq_synth import gen

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    out = {}
    with threadpool_limits(limits=1):
        for name, cfg, lays in layer_sets:
            byts = sum(layer_bytes(l.fmt, l.N, l.K, l.nnz, 1, 4) for l in lays)
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                for i, lay in enumerate(lays):
                    x = gen.synth_x(cfg, i, 1, lay.K)
                    if lay.fmt == "u8":
                        oracle.hxq_linear_fwd_u8(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, x,
                                                 "f32", lay.bias, want_bound=False)
                    else:
                        oracle.hxq_linear_fwd_pk12(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, x,
                                                   "f32", lay.bias, lay.N, lay.K, want_bound=False)
                times.append(time.perf_counter() - t0)
            t = float(np.median(times))
            out[name] = dict(step_ms=round(t * 1e3, 2), gbs=round(byts / t / 1e9, 4))
    return out


def receipt(torch, props, layers):
    """What the numbers were measured on and with: hardware, software
    versions, and the SHA-256 of the seeded inputs (per layer, over its
    codebook, indices, sidecar and bias arrays)."""
    import hashlib
    import platform

    import numpy as np

    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    inputs = {}
    for l in layers:
        h = hashlib.sha256()
        for k, v in sorted(l.sha256().items()):
            h.update((k + v).encode())
        inputs[l.name] = h.hexdigest()[:16]
    return dict(gpu=props.name, arch=getattr(props, "gcnArchName", None), cus=props.multi_processor_count,
                gpu_mem_gib=round(props.total_memory / 2 ** 30, 1), host_cpu=cpu,
                host_cores=len(os.sched_getaffinity(0)), rocm=rocm, torch=torch.__version__,
                torch_hip=getattr(torch.version, "hip", None), numpy=np.__version__,
                python=platform.python_version(), inputs_sha256=inputs,
                input_seeds="SeedSequence([20260403, cfg, layer, stream]) (hxq_synth)")


# ---- summaries of rocprofv3 databases (host only: sqlite3, no GPU)

def _db(path):
    """The rocpd database at `path`, or the one file *_results.db under it."""
    import glob
    import sqlite3
    if os.path.isdir(path):
        found = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
        if len(found) != 1:
            raise SystemExit("expected one *_results.db under %s, found %d" % (path, len(found)))
        path = found[0]
    return sqlite3.connect(path)


def summarise_trace(path):
    """Per kernel and grid size: calls, mean, median, p10, p90, min, max
    duration (us)."""
    rows = _db(path).execute("select name, grid_x, workgroup_x, duration from kernels order by start").fetchall()
    by = {}
    for name, gx, wx, d in rows:
        by.setdefault("%s [%d wg]" % (name, gx // max(wx, 1)), []).append(d / 1e3)
    out = ["%-90s %6s %9s %9s %9s %9s %9s %9s" % ("kernel", "calls", "avg_us", "median", "p10", "p90", "min",
                                                  "max")]
    for name, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(ds)
        q = lambda f: v[min(len(v) - 1, int(f * len(v)))]
        out.append("%-90s %6d %9.3f %9.3f %9.3f %9.3f %9.3f %9.3f" % (name[:90], len(v), sum(v) / len(v), q(0.5),
                                                                     q(0.1), q(0.9), v[0], v[-1]))
    return "\n".join(out)


def counters_by_kernel(path):
    """{"kernel [workgroups wg]": {counter: [value per dispatch, in dispatch order]}}."""
    rows = _db(path).execute("select kernel_name, grid_size_x, workgroup_size_x, counter_name, value, dispatch_id "
                             "from counters_collection order by dispatch_id").fetchall()
    by = {}
    for k, gx, wx, c, v, _ in rows:
        by.setdefault("%s [%d wg]" % (k, gx // max(wx, 1)), {}).setdefault(c, []).append(v)
    return by


def summarise_counters(path, match, cycle=None, cycles=0):
    """Per kernel (and grid) mean counter values per dispatch; with `cycle`
    (launch names) the first `cycles` rounds of matching dispatches are taken
    as that repeating sequence of launches and summarised per launch."""
    if cycle:
        rows = _db(path).execute("select dispatch_id, kernel_name, counter_name, value from counters_collection "
                                 "order by dispatch_id").fetchall()
        disp = {}
        for did, k, c, v in rows:
            if match in k:
                disp.setdefault(did, {})[c] = v
        order = sorted(disp)[:len(cycle) * cycles]
        out = []
        for i, name in enumerate(cycle):
            sel = [disp[did] for did in order[i::len(cycle)]]
            out.append("%s (%d dispatches)" % (name, len(sel)))
            for c in sorted(sel[0]) if sel else []:
                vs = [d[c] for d in sel if c in d]
                out.append("   %-28s %16.1f per dispatch" % (c, sum(vs) / len(vs)))
        return "\n".join(out)
    out = []
    for k, cs in counters_by_kernel(path).items():
        if match not in k:
            continue
        out.append(k)
        for c in sorted(cs):
            vs = cs[c]
            out.append("   %-28s %16.1f per dispatch (%d dispatches)" % (c, sum(vs) / len(vs), len(vs)))
    return "\n".join(out)


def summarise_traffic(d, steps=10, warmup=10):
    """FETCH_SIZE / WRITE_SIZE of the M = 1 decode launches (the bench run with
    --no-extras, `steps` timed steps after `warmup`: its first decode
    dispatches are whole steps, q|k|v, o, gate|up, down in turn), scaled by
    what the counters read for the plain device copy of --copy-calibration.
    Writes profiles/traffic.json and returns a text summary."""
    def series(sub, counter, match):
        # values of the matching dispatches in dispatch order
        rows = _db(os.path.join(d, sub)).execute(
            "select dispatch_id, kernel_name, value from counters_collection where counter_name = ? "
            "order by dispatch_id", (counter,)).fetchall()
        return [v for _, k, v in rows if match in k]
    copy_kib = (64 << 20) * 4 / 1024
    cf = series("copyf", "FETCH_SIZE", "copyBuffer")
    cw = series("copyw", "WRITE_SIZE", "copyBuffer")
    fscale = copy_kib / (sum(cf) / len(cf))
    wscale = copy_kib / (sum(cw) / len(cw))
    fe = series("fetch", "FETCH_SIZE", "decode1_gemv")
    wr = series("write", "WRITE_SIZE", "decode1_gemv")
    n = len(GROUPS)
    lo, hi = warmup * n, (warmup + steps) * n
    if len(fe) < hi or len(wr) < hi:
        raise SystemExit("fewer decode dispatches than %d steps" % (warmup + steps))
    import numpy as np
    from hxq_synth import gen
    layers = gen.config_layers(1)
    algo = []
    for grp in GROUPS:
        sel = [l for l in layers if l.name in grp]
        algo.append(group_bytes(sel, 1, 4))
    rec = {}
    lines = ["launch     FETCH_SIZE KiB  WRITE_SIZE KiB    HBM bytes  algorithmic bytes  ratio"]
    for g in range(n):
        f = float(np.mean(fe[lo + g:hi:n]))
        w = float(np.mean(wr[lo + g:hi:n]))
        hbm = int(round((f * fscale + w * wscale) * 1024))
        name = "|".join(GROUPS[g])
        rec[name] = dict(fetch_kib=f, write_kib=w, hbm_bytes_per_launch=hbm, algorithmic_bytes=algo[g],
                         ratio=round(hbm / algo[g], 4))
        lines.append("%-9s %15.1f %15.1f %12d %18d %6.3f" % (name, f, w, hbm, algo[g], hbm / algo[g]))
    dom = "|".join(GROUPS[DOMINANT])
    out = {"decode_gemv_gate_up_m1": dict(rec[dom], source_digest=source_digest(), fetch_scale=round(fscale, 4),
                                          write_scale=round(wscale, 4),
                                          counters="FETCH_SIZE, WRITE_SIZE (KiB per dispatch, mean over the "
                                                   "%d timed steps)" % steps),
           "all_launches_m1": rec}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    head = ["calibration (plain 256 MiB device copy):",
            "  FETCH_SIZE reads %.0f KiB per copy -> scale %.4f" % (sum(cf) / len(cf), fscale),
            "  WRITE_SIZE reads %.0f KiB per copy -> scale %.4f" % (sum(cw) / len(cw), wscale), "",
            "decode launches of the %d timed steps (mean per dispatch), scaled:" % steps]
    tail = ["", "digest of the decode kernels' sources and headers (%s) when taken: %s"
            % (", ".join(DECODE_SOURCES), source_digest())]
    return "\n".join(head + lines + tail)


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
    ap.add_argument("--profile-decode", type=int, default=0, metavar="M",
                    help="only run --steps grouped decode steps at M tokens (fp32 x) and print their "
                         "per-launch times (for profiler runs at other token counts)")
    ap.add_argument("--profile-prefill", type=int, default=0, metavar="M",
                    help="only run --steps grouped prefill steps at M tokens (bf16 x) and print their "
                         "per-launch times (for profiler runs)")
    ap.add_argument("--profile-bwd", type=int, default=0, metavar="M",
                    help="only run --steps input-gradient steps at M tokens (fp32 dy below 16 tokens, bf16 "
                         "from 16) and print their per-layer times (for profiler runs)")
    ap.add_argument("--summarise-trace", metavar="DB", help="print a kernel-trace summary of a rocprofv3 database")
    ap.add_argument("--summarise-counters", metavar="DB", help="print per-kernel counter means of a rocprofv3 "
                                                              "database (kernels whose name holds --match)")
    ap.add_argument("--match", default="hxq", help="kernel-name filter for --summarise-counters")
    ap.add_argument("--launch-cycle", default="", help="with --summarise-counters: comma-separated names of the "
                                                       "launches the matching dispatches repeat in turn")
    ap.add_argument("--cycles", type=int, default=0, help="with --launch-cycle: rounds of launches to take")
    ap.add_argument("--summarise-traffic", metavar="DIR",
                    help="DIR/{fetch,write,copyf,copyw}: write profiles/traffic.json from those counter runs")
    args = ap.parse_args(argv)
    if args.summarise_trace:
        print(summarise_trace(args.summarise_trace))
        return 0
    if args.summarise_counters:
        cyc = [c for c in args.launch_cycle.split(",") if c]
        print(summarise_counters(args.summarise_counters, args.match, cyc, args.cycles))
        return 0
    if args.summarise_traffic:
        print(summarise_traffic(args.summarise_traffic))
        return 0
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

    if args.profile_prefill > 0:
        sp = LayerSet(torch, L, B, layers, args.profile_prefill, "bf16", 4, 1, stream)
        total = time_steps(torch, sp.grouped, args.steps, args.warmup)
        per = []
        for g in range(len(GROUPS)):
            tg = time_steps(torch, [[row[g]] for row in sp.grouped], args.steps, 1)
            per.append(dict(launch="|".join(GROUPS[g]), avg_us=round(tg / args.steps * 1e3, 3)))
        print(json.dumps(dict(profile_prefill_m=args.profile_prefill, steps=args.steps,
                              step_us=round(total / args.steps * 1e3, 3), launches=per)))
        return 0
    if args.profile_decode > 0:
        sp = LayerSet(torch, L, B, layers, args.profile_decode, "f32", 1, copies, stream)
        total = time_steps(torch, sp.grouped, args.steps, args.warmup)
        per = []
        for g in range(len(GROUPS)):
            tg = time_steps(torch, [[row[g]] for row in sp.grouped], args.steps, 2)
            per.append(dict(launch="|".join(GROUPS[g]), avg_us=round(tg / args.steps * 1e3, 3)))
        print(json.dumps(dict(profile_decode_m=args.profile_decode, steps=args.steps,
                              step_us=round(total / args.steps * 1e3, 3), launches=per)))
        return 0

    if args.profile_bwd > 0:
        sp = LayerSet(torch, L, B, layers, 1, "f32", 1, copies, stream)
        out = input_gradient(torch, L, B, layers, sp.devs, args.profile_bwd,
                             "f32" if args.profile_bwd < 16 else "bf16", args.steps, args.warmup, stream)
        print(json.dumps(dict(profile_bwd_m=args.profile_bwd, steps=args.steps, **out)))
        return 0

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
        extras["dominant_launch_percentiles"] = percentiles(torch, [[row[DOMINANT]] for row in s1.grouped], 200)
        extras["input_gradient_m1"] = input_gradient(torch, L, B, layers, s1.devs, 1, "f32", args.steps,
                                                     args.warmup, stream)
        log("input gradient M=1 step %.1f us, %.1f GB/s" % (extras["input_gradient_m1"]["step_us"],
                                                            extras["input_gradient_m1"]["gbs"]))
    del s1
    torch.cuda.empty_cache()
    if not args.no_extras:
        extras["stream_ceiling"] = stream_ceiling(torch, L, dom_bytes, args.steps)
        log("stream ceiling %.1f GB/s (%d workgroups)" % (extras["stream_ceiling"]["gbs"],
                                                          extras["stream_ceiling"]["best_workgroups"]))

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
        m8_bytes = sum(s8.group_bytes)
        extras["decode_m8"].update(roof(m8_bytes, sum(2.0 * 8 * l.N * l.K for l in layers),
                                        total8 / args.steps * 1e3, "f32"))
        del s8
        torch.cuda.empty_cache()
        extras.update(config_blocks(torch, L, B, stream, args.steps, args.warmup))

    if not args.no_extras and not args.no_prefill:
        # config 4 at 512 tokens: the grouped step
        s5 = LayerSet(torch, L, B, layers, 512, "bf16", 4, 1, stream)
        st5 = max(5, args.steps // 5)
        t5 = time_steps(torch, s5.grouped, st5, 2) / st5
        avg5 = []
        for g in range(len(GROUPS)):
            avg5.append(time_steps(torch, [[row[g]] for row in s5.grouped], st5, 1) / st5)
        fl5 = sum(2.0 * 512 * l.N * l.K for l in layers)
        tf5 = fl5 / (t5 * 1e-3) / 1e12
        gfl5 = [sum(2.0 * 512 * layers[s5.by_name[n]].N * layers[s5.by_name[n]].K for n in g) for g in GROUPS]
        extras["prefill_m512"] = dict(
            workload="Qwen2.5-3B-shaped u8 layer set, M=512, bf16 x; launches q|k|v, o, gate|up, down", M=512,
            step_us=round(t5 * 1e3, 2), tflops=round(tf5, 2), frac_of_mfma_peak=round(tf5 / MFMA_BF16_PEAK_TFS, 4),
            launches=[dict(launch="|".join(g), avg_us=round(m * 1e3, 2), **roof(b, f, m * 1e3, "bf16"))
                      for g, m, f, b in zip(GROUPS, avg5, gfl5, s5.group_bytes)])
        log("prefill M=512 step %.1f us, %.1f TFLOP/s" % (t5 * 1e3, tf5))
        del s5
        torch.cuda.empty_cache()
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
        extras["prefill_m25600"] = prefill_big(torch, L, B, layers, stream, 3)
        log("prefill M=25600 gate|up + down %.1f us, %.1f TFLOP/s" % (extras["prefill_m25600"]["step_us"],
                                                                      extras["prefill_m25600"]["tflops"]))

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
                     "algorithmic_bytes_per_launch": int(dom_bytes),
                     "frac_of_stream_ceiling": (round(achieved / extras["stream_ceiling"]["gbs"], 4)
                                                if "stream_ceiling" in extras else None)},
        "per_launch_m1": per_group,
        "cpu_baseline": None,
    }
    out.update(extras)
    out["receipt"] = receipt(torch, props, layers)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(layers, 1)
        if not args.no_extras:
            pk = [gen.random_layer(9100 + i, N, K, "pk12", nnz=N * K // 2000)
                  for i, (_, N, K) in enumerate(gen.PK12_LAYERS)]
            out["cpu_baseline"]["single_thread_m1"] = cpu_single_thread(
                [("config0", 0, gen.config_layers(0)), ("config1", 1, layers), ("config2", 2, gen.config_layers(2)),
                 ("config3", 3, pk)])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
