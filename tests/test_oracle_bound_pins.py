"""Pins of the oracle's tolerance scale B, checked against something other
than the oracle itself.

Every parity check passes when |y - Y| <= tol * B elementwise, so a wrong B
(scaled, shifted by the bias, transposed, or with an absolute value dropped or
taken too early) would loosen or break every GPU comparison at once.  The
scale is the one the tolerance statement fixes: B = |X| |W|^T for the forward
and B = |dY| |W| for the input gradient, with W the dequantised weight whose
repeated sidecar coordinates are summed before the absolute value (HXQ
whitepaper, "Method": sidecar (row, col, delta) corrections; model cards,
"What is HelixCode?": codebook[indices] @ x).  For the sidecar term alone
(y += S x) the scale is the sum of the absolute terms the library adds,
|delta| |x[m][c]| per triplet.

Pins: a pure-Python brute force with correctly rounded (fsum) sums on tiny
non-square and square shapes, u8, pk12 and bf16 activations; and a
hand-worked example with exact binary values (tests/golden/bound_tiny.txt).
"""

import math
import os

import numpy as np
import pytest

import oracle
from hxq_synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _weights_with_sidecar(W, rows, cols, deltas):
    """W (python lists) with every delta added at its (row, col): each entry is
    the correctly rounded sum of its codebook value and its deltas."""
    extra = {}
    for r, c, d in zip(rows, cols, deltas):
        extra.setdefault((int(r), int(c)), []).append(float(d))
    out = [list(map(float, row)) for row in W]
    for (r, c), ds in extra.items():
        out[r][c] = math.fsum([out[r][c]] + ds)
    return out


def _brute_bound_fwd(W, X):
    """B[m][n] = sum_k |x[m][k]| |W[n][k]|, each sum correctly rounded."""
    return np.array([[math.fsum(abs(float(xv)) * abs(w) for xv, w in zip(xr, wr)) for wr in W] for xr in X])


def _brute_bound_bwd(W, DY):
    """B[m][k] = sum_n |dy[m][n]| |W[n][k]|."""
    K = len(W[0])
    return np.array([[math.fsum(abs(float(g)) * abs(W[n][k]) for n, g in enumerate(dr)) for k in range(K)]
                     for dr in DY])


def _sidecar(rng, N, K, nnz):
    pos = np.sort(rng.integers(0, N * K, size=nnz))
    pos[1] = pos[0]  # a repeated coordinate
    pos = np.sort(pos)
    return ((pos // K).astype(np.int32), (pos % K).astype(np.int32),
            (0.3 * rng.standard_normal(nnz)).astype(np.float32))


def _close(B, ref, terms):
    """Both sides sum non-negative terms: they agree to a relative
    terms * 2^-52 (numpy's fp64 matmul rounds each partial sum)."""
    return np.all(np.abs(B - ref) <= (terms + 2) * 2.0 ** -52 * ref)


# ------------------------------------------------------------ forward bound

@pytest.mark.parametrize("N,K,M", [(7, 12, 3), (5, 33, 2), (6, 6, 4)])
def test_bound_u8_bruteforce(N, K, M):
    rng = _rng(5000 + N * K + M)
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _sidecar(rng, N, K, 9)
    # a pair of deltas that cancels its codebook value: |C + d1 + d2| is small
    # while |C| + |d1| + |d2| is not
    deltas[0] = np.float32(-float(cb[int(idx[rows[0], cols[0]])]) - 0.25)
    deltas[1] = np.float32(0.25)
    X = rng.standard_normal((M, K)).astype(np.float32)
    bias = (0.5 + rng.random(N)).astype(np.float32)
    _, B = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
    W = _weights_with_sidecar([[float(cb[i]) for i in r] for r in idx.tolist()], rows, cols, deltas)
    ref = _brute_bound_fwd(W, X.tolist())
    assert B.shape == (M, N)
    assert _close(B, ref, K)


@pytest.mark.parametrize("N,K,M", [(6, 16, 3), (3, 10, 2), (8, 8, 5)])
def test_bound_pk12_bruteforce(N, K, M):
    rng = _rng(6000 + N * K + M)
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    idx2 = rng.integers(0, 4096, size=(N, K // 2))
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _sidecar(rng, N, K, 7)
    X = rng.standard_normal((M, K)).astype(np.float32)
    bias = (0.5 + rng.random(N)).astype(np.float32)
    _, B = oracle.hxq_linear_fwd_pk12(cb2, packed, rows, cols, deltas, X, "f32", bias, N, K)
    W0 = [[float(cb2[int(e)][s]) for e in r for s in (0, 1)] for r in idx2.tolist()]
    W = _weights_with_sidecar(W0, rows, cols, deltas)
    ref = _brute_bound_fwd(W, X.tolist())
    assert B.shape == (M, N)
    assert _close(B, ref, K)


def test_bound_bf16_activations_bruteforce():
    rng = _rng(6100)
    N, K, M = 5, 9, 3
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    bits = (xf.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do
    xb = [[float(np.uint32(int(b) << 16).view(np.float32)) for b in row] for row in bits]
    _, B = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], bits, "bf16", None)
    ref = _brute_bound_fwd([[float(cb[i]) for i in r] for r in idx.tolist()], xb)
    assert _close(B, ref, K)


# ------------------------------------------------------ input-gradient bound

@pytest.mark.parametrize("N,K,M", [(7, 12, 3), (5, 33, 2), (6, 6, 4)])
def test_bound_bwd_u8_bruteforce(N, K, M):
    rng = _rng(7000 + N * K + M)
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _sidecar(rng, N, K, 9)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    _, B = oracle.hxq_linear_bwd_x_u8(cb, idx, rows, cols, deltas, DY, "f32")
    W = _weights_with_sidecar([[float(cb[i]) for i in r] for r in idx.tolist()], rows, cols, deltas)
    ref = _brute_bound_bwd(W, DY.tolist())
    assert B.shape == (M, K)
    assert _close(B, ref, N)


@pytest.mark.parametrize("N,K,M", [(6, 16, 3), (8, 8, 2)])
def test_bound_bwd_pk12_bruteforce(N, K, M):
    rng = _rng(7100 + N * K + M)
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    idx2 = rng.integers(0, 4096, size=(N, K // 2))
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _sidecar(rng, N, K, 7)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    _, B = oracle.hxq_linear_bwd_x_pk12(cb2, packed, rows, cols, deltas, DY, "f32", N, K)
    W0 = [[float(cb2[int(e)][s]) for e in r for s in (0, 1)] for r in idx2.tolist()]
    ref = _brute_bound_bwd(_weights_with_sidecar(W0, rows, cols, deltas), DY.tolist())
    assert B.shape == (M, K)
    assert _close(B, ref, N)


# ------------------------------------------------------- sidecar-only bound

def test_bound_sidecar_add_bruteforce():
    rng = _rng(7200)
    N, K, M = 6, 11, 3
    rows, cols, deltas = _sidecar(rng, N, K, 10)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Z, B = oracle.hxq_sidecar_add(rows, cols, deltas, X, "f32", N)
    zref = np.zeros((M, N))
    bref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            ts = [float(d) * float(X[m][c]) for r, c, d in zip(rows, cols, deltas) if r == n]
            zref[m, n] = math.fsum(ts)
            bref[m, n] = math.fsum(abs(t) for t in ts)
    assert np.all(np.abs(Z - zref) <= 12 * 2.0 ** -52 * bref)
    assert _close(B, bref, 10)


# ------------------------------------------------------------ hand-worked

def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "bound_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, *rest = line.split()
                vals[name] = [float(v) for v in rest]
    return vals


def _golden_layer(g):
    cb = np.full(256, 0.25, np.float32)
    cb[:4] = [0.0, 1.0, -2.0, 0.5]
    idx = np.array(g["indices"], np.uint8).reshape(2, 3)
    rows = np.array(g["sc_rows"], np.int32)
    cols = np.array(g["sc_cols"], np.int32)
    deltas = np.array(g["sc_deltas"], np.float32)
    return cb, idx, rows, cols, deltas


def test_bound_golden_hand_example():
    g = _golden()
    cb, idx, rows, cols, deltas = _golden_layer(g)
    X = np.array(g["x"], np.float32).reshape(2, 3)
    bias = np.array(g["bias"], np.float32)
    Y, B = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
    assert np.array_equal(Y, np.array(g["y"]).reshape(2, 2))
    assert np.array_equal(B, np.array(g["bound"]).reshape(2, 2))


def test_bound_bwd_golden_hand_example():
    g = _golden()
    cb, idx, rows, cols, deltas = _golden_layer(g)
    DY = np.array(g["dy"], np.float32).reshape(2, 2)
    dX, B = oracle.hxq_linear_bwd_x_u8(cb, idx, rows, cols, deltas, DY, "f32")
    assert np.array_equal(dX, np.array(g["dx"]).reshape(2, 3))
    assert np.array_equal(B, np.array(g["bound_bwd"]).reshape(2, 3))


def test_bound_sidecar_golden_hand_example():
    g = _golden()
    _, _, rows, cols, deltas = _golden_layer(g)
    X = np.array(g["x"], np.float32).reshape(2, 3)
    Z, B = oracle.hxq_sidecar_add(rows, cols, deltas, X, "f32", 2)
    assert np.array_equal(Z, np.array(g["z"]).reshape(2, 2))
    assert np.array_equal(B, np.array(g["bound_sidecar"]).reshape(2, 2))
