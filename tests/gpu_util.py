"""Helpers for the GPU parity tests: move a synthetic layer to the device,
run the library through its C ABI, and compare with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import vq_compressed_linear_amd as hx

TOL_FP32 = 1e-5   # fp32-arithmetic paths: |y - Y| <= 1e-5 * (|X| |W|^T)
TOL_BF16 = 8e-3   # bf16 matrix-core path


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t

    return t


def dev_layer(lay, device="cuda"):
    t = torch()
    return dict(
        codebook=t.from_numpy(np.ascontiguousarray(lay.codebook)).to(device),
        indices=t.from_numpy(np.ascontiguousarray(lay.indices)).to(device),
        rows=t.from_numpy(np.ascontiguousarray(lay.rows, dtype=np.int32)).to(device),
        cols=t.from_numpy(np.ascontiguousarray(lay.cols, dtype=np.int32)).to(device),
        deltas=t.from_numpy(np.ascontiguousarray(lay.deltas, dtype=np.float32)).to(device),
        bias=t.from_numpy(np.ascontiguousarray(lay.bias, dtype=np.float32)).to(device),
    )


def dev_x(x_np, x_dtype, device="cuda"):
    """fp32 numpy -> device tensor; for bf16 the numpy array holds uint16 bits."""
    t = torch()
    if x_dtype == "f32":
        return t.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(device)
    return t.from_numpy(np.ascontiguousarray(x_np, dtype=np.uint16).view(np.int16)).to(device).view(t.bfloat16)


def run(lay, d, xd, variant=hx.HXQ_VARIANT_AUTO, bias=True, sidecar=True, y=None):
    t = torch()
    M = xd.shape[0]
    if y is None:
        y = t.full((M, lay.N), float("nan"), dtype=t.float32, device=xd.device)
    fn = hx.hxq_linear_fwd_u8 if lay.fmt == "u8" else hx.hxq_linear_fwd_pk12
    r, c, dl = (d["rows"], d["cols"], d["deltas"]) if sidecar else (None, None, None)
    fn(d["codebook"], d["indices"], r, c, dl, xd, d["bias"] if bias else None, y, variant=variant)
    return y


def oracle_fwd(lay, x_np, x_dtype, bias=True, sidecar=True, m_rows=None):
    rows, cols, deltas = (lay.rows, lay.cols, lay.deltas) if sidecar else ([], [], [])
    b = lay.bias if bias else None
    if lay.fmt == "u8":
        return oracle.hxq_linear_fwd_u8(lay.codebook, lay.indices, rows, cols, deltas, x_np,
                                        x_dtype, b, m_rows=m_rows)
    return oracle.hxq_linear_fwd_pk12(lay.codebook, lay.indices, rows, cols, deltas, x_np,
                                      x_dtype, b, lay.N, lay.K, m_rows=m_rows)


def check(y_dev, Y, Bnd, tol, what="", m_rows=None):
    y = y_dev.float().cpu().numpy().astype(np.float64)
    if m_rows is not None:
        y = y[np.asarray(m_rows)]
    assert y.shape == Y.shape, (y.shape, Y.shape)
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    err = np.abs(y - Y)
    ok = err <= tol * Bnd
    ratio = oracle.max_err_ratio(y, Y, Bnd)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d elements out of tolerance (max err/B = %.3g, tol %.1e); first %s"
                             % (what, int((~ok).sum()), ratio, tol, bad.tolist()))
    return ratio


def sample_rows(M, k=64, seed=0):
    if M <= k:
        return np.arange(M)
    rng = np.random.Generator(np.random.PCG64(seed))
    mid = rng.choice(np.arange(1, M - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate(([0, M - 1], mid)))


def tile_rows(M, seed=0):
    """Token rows to compare for a large M: 64 random rows, one random row in
    every 128-token block and the last row of every 256-token block, so every
    tile of the prefill kernels (128 or 256 tokens tall) is looked at."""
    rng = np.random.Generator(np.random.PCG64(seed + 17))
    per128 = np.arange(0, M, 128) + rng.integers(0, 128, size=(M + 127) // 128)
    last256 = np.arange(255, M + 255, 256)
    rows = np.concatenate([sample_rows(M, 64, seed), per128, last256])
    return np.unique(rows[rows < M])
