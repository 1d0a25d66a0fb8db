"""Pins of the CPU oracle against what the pages and plain arithmetic fix.

Each test checks the oracle against something other than itself: a
pure-Python brute force with correctly rounded sums, a closed form, the golden
bytes of the stated 12-bit layout, an exhaustive round trip, or a library
routine.  Shapes are non-square and M > 1 so that a transposed operand, a
swapped row/col or a dropped term shows up.
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


def _bf16_bits_from_float(v):
    return int(np.float32(v).view(np.uint32)) >> 16


# ------------------------------------------------------------ brute force

def _brute_u8(cb, idx, rows, cols, deltas, X, bias):
    """y[m][n] = fsum over k of x[m][k] * (C[idx[n][k]] + sum of deltas at (n, k)) + b[n].
    fp32 x fp32 products are exact in fp64 and fsum rounds the sum once."""
    M = len(X)
    N, K = len(idx), len(idx[0])
    extra = {}
    for r, c, d in zip(rows, cols, deltas):
        extra.setdefault((int(r), int(c)), []).append(float(d))
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                xv = float(X[m][k])
                terms.append(xv * float(cb[int(idx[n][k])]))
                for d in extra.get((n, k), []):
                    terms.append(xv * d)
            if bias is not None:
                terms.append(float(bias[n]))
            out[m][n] = math.fsum(terms)
    return np.array(out)


def _brute_pk12_weights(cb2, packed, N, K):
    """Weights from the packed bytes, one 3-byte group at a time, with Python ints."""
    W = [[0.0] * K for _ in range(N)]
    stride = 3 * ((K + 3) // 4)
    for n in range(N):
        for t in range((K + 3) // 4):
            b0, b1, b2 = (int(packed[n][3 * t + i]) for i in range(3))
            assert 3 * t + 2 < stride
            first = b0 + 256 * (b1 % 16)
            second = (b1 // 16) + 16 * b2
            for pair, e in ((0, first), (1, second)):
                k0 = 4 * t + 2 * pair
                if k0 < K:
                    W[n][k0] = float(cb2[e][0])
                    W[n][k0 + 1] = float(cb2[e][1])
    return W


def _brute_from_W(W, rows, cols, deltas, X, bias):
    M, N, K = len(X), len(W), len(W[0])
    extra = {}
    for r, c, d in zip(rows, cols, deltas):
        extra.setdefault((int(r), int(c)), []).append(float(d))
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            terms = [float(X[m][k]) * W[n][k] for k in range(K)]
            for (r, c), ds in extra.items():
                if r == n:
                    terms += [float(X[m][c]) * d for d in ds]
            if bias is not None:
                terms.append(float(bias[n]))
            out[m, n] = math.fsum(terms)
    return out


def _tiny_sidecar(rng, N, K, nnz):
    pos = np.sort(rng.integers(0, N * K, size=nnz))
    pos[1] = pos[0]  # at least one repeated coordinate
    pos = np.sort(pos)
    return ((pos // K).astype(np.int32), (pos % K).astype(np.int32),
            (0.3 * rng.standard_normal(nnz)).astype(np.float32))


@pytest.mark.parametrize("N,K,M", [(7, 12, 3), (5, 33, 2), (16, 8, 4)])
def test_u8_matches_bruteforce(N, K, M):
    rng = _rng(1000 + N * K + M)
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 9)
    X = rng.standard_normal((M, K)).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    Y, B = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
    ref = _brute_u8(cb, idx.tolist(), rows, cols, deltas, X.tolist(), bias)
    scale = B + np.abs(bias)[None, :]
    assert Y.shape == (M, N)
    assert np.all(np.abs(Y - ref) <= (K + 4) * 2.0 ** -52 * scale)


@pytest.mark.parametrize("N,K,M", [(6, 16, 3), (3, 10, 2), (9, 4, 5)])
def test_pk12_matches_bruteforce(N, K, M):
    rng = _rng(2000 + N * K + M)
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    idx2 = rng.integers(0, 4096, size=(N, K // 2))
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 7)
    X = rng.standard_normal((M, K)).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    Y, B = oracle.hxq_linear_fwd_pk12(cb2, packed, rows, cols, deltas, X, "f32", bias, N, K)
    W = _brute_pk12_weights(cb2, packed.tolist(), N, K)
    ref = _brute_from_W(W, rows, cols, deltas, X.tolist(), bias)
    scale = B + np.abs(bias)[None, :]
    assert np.all(np.abs(Y - ref) <= (K + 4) * 2.0 ** -52 * scale)


def test_bf16_activations_bruteforce():
    rng = _rng(7)
    N, K, M = 5, 9, 3
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    bits = np.array([[_bf16_bits_from_float(v) for v in row] for row in xf], dtype=np.uint16)
    xb = [[float(np.uint32(int(b) << 16).view(np.float32)) for b in row] for row in bits]
    Y, B = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], bits, "bf16", None)
    ref = _brute_u8(cb, idx.tolist(), [], [], [], xb, None)
    assert np.all(np.abs(Y - ref) <= (K + 4) * 2.0 ** -52 * B)


def test_full_config0_fsum():
    """The whole 256 x 256 config-0 layer against the correctly rounded sum."""
    lay = gen.config_layers(0)[0]
    x = gen.synth_x(0, 0, 1, lay.K)
    Y, B = oracle.hxq_linear_fwd_u8(lay.codebook, lay.indices, lay.rows, lay.cols,
                                    lay.deltas, x, "f32", lay.bias)
    W = lay.codebook.astype(np.float64)[lay.indices.astype(np.int64)]
    ref = np.empty(lay.N)
    side = {}
    for r, c, d in zip(lay.rows, lay.cols, lay.deltas):
        side.setdefault(int(r), []).append((int(c), float(d)))
    xs = x[0].astype(np.float64)
    for n in range(lay.N):
        terms = list(W[n] * xs) + [xs[c] * d for c, d in side.get(n, [])] + [float(lay.bias[n])]
        ref[n] = math.fsum(terms)
    assert lay.nnz == 65
    assert np.all(np.abs(Y[0] - ref) <= (lay.K + 4) * 2.0 ** -52 * (B[0] + np.abs(lay.bias)))


# ----------------------------------------------------------- closed forms

def test_constant_index_closed_form():
    """idx == j everywhere, no sidecar: y[m, n] = C[j] * sum_k x[m, k] + b[n].
    With C[j] = 0.375 and small integer x every partial sum is exact."""
    rng = _rng(11)
    N, K, M = 13, 40, 4
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    j = 77
    cb[j] = 0.375
    idx = np.full((N, K), j, dtype=np.uint8)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    bias = rng.integers(-8, 9, size=N).astype(np.float32) / 8
    Y, _ = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], X, "f32", bias)
    expect = 0.375 * X.astype(np.float64).sum(axis=1)[:, None] + bias[None, :]
    assert np.array_equal(Y, expect)


def test_constant_index_pk12_closed_form():
    rng = _rng(12)
    N, K, M = 6, 20, 3
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    e = 3001
    cb2[e] = (0.25, -1.5)
    packed = gen.pack12_rows(np.full((N, K // 2), e))
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    Y, _ = oracle.hxq_linear_fwd_pk12(cb2, packed, [], [], [], X, "f32", None, N, K)
    Xd = X.astype(np.float64)
    expect = 0.25 * Xd[:, 0::2].sum(axis=1) - 1.5 * Xd[:, 1::2].sum(axis=1)
    assert np.array_equal(Y, np.repeat(expect[:, None], N, axis=1))


def test_empty_sidecar_difference():
    """y(S) - y(no sidecar) is the sparse term alone, computed triplet by triplet."""
    rng = _rng(13)
    N, K, M = 11, 24, 3
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 15)
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    y_s, _ = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", None)
    y_0, _ = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], X, "f32", None)
    Z, _ = oracle.hxq_sidecar_add(rows, cols, deltas, X, "f32", N)
    ref = np.zeros((M, N))
    for r, c, d in zip(rows, cols, deltas):
        for m in range(M):
            ref[m, r] = math.fsum([ref[m, r], float(d) * float(X[m, c])])
    assert np.allclose(Z, ref, rtol=0, atol=1e-14)
    assert np.allclose(y_s - y_0, ref, rtol=0, atol=1e-12)


def test_one_hot_reconstructs_columns():
    """x = e_k picks column k of W: y[k, n] = C[idx[n, k]] + deltas at (n, k) + b[n]."""
    rng = _rng(14)
    N, K = 9, 14
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 6)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    X = np.eye(K, dtype=np.float32)
    Y, _ = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
    for k in range(K):
        for n in range(N):
            terms = [float(cb[idx[n, k]]), float(bias[n])]
            terms += [float(d) for r, c, d in zip(rows, cols, deltas) if r == n and c == k]
            assert Y[k, n] == pytest.approx(math.fsum(terms), abs=1e-15)


def test_cross_format_special_case():
    """A 64-entry scalar codebook c makes C2[e] = (c[e >> 6], c[e & 63]); pk12 and
    u8 then describe the same weights and the oracle gives identical outputs."""
    rng = _rng(15)
    N, K, M = 7, 18, 3
    c64 = (0.05 * rng.standard_normal(64)).astype(np.float32)
    cb = np.zeros(256, dtype=np.float32)
    cb[:64] = c64
    idx = rng.integers(0, 64, size=(N, K)).astype(np.uint8)
    e = np.arange(4096)
    cb2 = np.stack([c64[e >> 6], c64[e & 63]], axis=1)
    idx2 = 64 * idx[:, 0::2].astype(np.int64) + idx[:, 1::2]
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 5)
    X = rng.standard_normal((M, K)).astype(np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    y8, _ = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
    y12, _ = oracle.hxq_linear_fwd_pk12(cb2, packed, rows, cols, deltas, X, "f32", bias, N, K)
    assert np.array_equal(y8, y12)


def test_linearity_in_x():
    rng = _rng(16)
    N, K = 10, 32
    cb = rng.integers(-8, 9, size=256).astype(np.float32) / 16
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    a = rng.integers(-4, 5, size=(2, K)).astype(np.float32)
    b = rng.integers(-4, 5, size=(2, K)).astype(np.float32)
    ya, _ = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], a, "f32", None)
    yb, _ = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], b, "f32", None)
    yab, _ = oracle.hxq_linear_fwd_u8(cb, idx, [], [], [], a + 2 * b, "f32", None)
    assert np.array_equal(yab, ya + 2 * yb)


# ---------------------------------------------------------------- 12-bit

def _golden_layout():
    out = []
    with open(os.path.join(GOLDEN, "pk12_layout.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b, b0, b1, b2 = line.split()
                out.append((int(a, 16), int(b, 16), [int(b0, 16), int(b1, 16), int(b2, 16)]))
    return out


def test_pk12_golden_bytes():
    cases = _golden_layout()
    assert cases[0] == (0xABC, 0x123, [0xBC, 0x3A, 0x12])
    for a, b, want in cases:
        packed = gen.pack12_rows(np.array([[a, b]]))
        assert packed.tolist() == [want]
        assert oracle.unpack_pk12(np.array([want], dtype=np.uint8), 1, 4).tolist() == [[a, b]]


def test_pk12_round_trip_exhaustive():
    """Every pair (a, b) in [0, 4096)^2 survives pack -> unpack."""
    b = np.arange(4096)
    for a0 in range(0, 4096, 512):
        a = np.arange(a0, a0 + 512)
        idx2 = np.empty((512, 8192), dtype=np.int64)
        idx2[:, 0::2] = a[:, None]
        idx2[:, 1::2] = b[None, :]
        packed = gen.pack12_rows(idx2)
        assert packed.shape == (512, 3 * 4096)
        back = oracle.unpack_pk12(packed, 512, 2 * 8192)
        assert np.array_equal(back, idx2)


def test_pk12_odd_pair_count_tail():
    """K = 2 (mod 4): the last 3-byte group holds one index and a zero pad."""
    idx2 = np.array([[0x123, 0x456, 0xFED]])
    packed = gen.pack12_rows(idx2)
    assert packed.shape == (1, 6)
    assert packed[0, 3:].tolist() == [0xED, 0x0F, 0x00]
    assert oracle.unpack_pk12(packed, 1, 6).tolist() == idx2.tolist()


# -------------------------------------------------------------- bf16 / bytes

def test_bf16_round_matches_library_cast():
    import torch

    rng = _rng(17)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    ties = (rng.integers(0, 2 ** 16, size=5000).astype(np.uint32) << 16) | 0x8000
    v = np.concatenate([v, ties.view(np.float32), np.array(
        [0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1e-40, -1e-40, 1.0, 1.00390625], np.float32)])
    v = v[np.isfinite(v) | np.isinf(v)]
    ours = oracle.bf16_round_f32(v)
    lib = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), lib.view(np.uint32))


def test_bf16_upcast_matches_library():
    import torch

    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()


def _page_constants():
    out = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


def test_page_byte_counts():
    """Storage closed forms: u8 = N K + 1024 + 12 nnz, pk12 = 3 N ceil(K/4) + 32768 + 12 nnz."""
    pc = _page_constants()
    for fmt, N, K in (("u8", 37, 52), ("pk12", 37, 52), ("pk12", 5, 6)):
        lay = gen.random_layer(5, N, K, fmt, nnz=40)
        if fmt == "u8":
            assert lay.codebook.size == pc["u8_codebook_entries"]
            assert lay.indices.nbytes * 8 == pc["u8_index_bits_per_weight"] * N * K
            expect = N * K + 4 * 256 + 12 * lay.nnz
        else:
            assert lay.codebook.nbytes == pc["pk12_codebook_bytes"]
            assert lay.codebook.shape[0] == pc["pk12_codebook_entries"]
            expect = N * 3 * ((K + 3) // 4) + 32768 + 12 * lay.nnz
            if K % 4 == 0:
                assert lay.indices.nbytes * 8 == pc["pk12_bits_per_weight"] * N * K
                assert lay.indices.nbytes == pc["pk12_bytes_per_index_pair"] * N * K // 4
                assert 100 * (2 * N * K // 2 - lay.indices.nbytes) == \
                    pc["pk12_saving_vs_uint16_percent"] * (2 * N * K // 2)
        assert lay.compressed_bytes() == expect
        assert pc["sidecar_fields_per_entry"] * 4 == 12


# ------------------------------------------- input gradient dX = dY @ W

def _brute_bwd_from_W(W, rows, cols, deltas, DY):
    """dX[m][k] = fsum over n of dy[m][n] * (W[n][k] + deltas at (n, k))."""
    M, N, K = len(DY), len(W), len(W[0])
    extra = {}
    for r, c, d in zip(rows, cols, deltas):
        extra.setdefault((int(r), int(c)), []).append(float(d))
    out = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            terms = []
            for n in range(N):
                g = float(DY[m][n])
                terms.append(g * W[n][k])
                terms += [g * d for d in extra.get((n, k), [])]
            out[m, k] = math.fsum(terms)
    return out


@pytest.mark.parametrize("N,K,M", [(7, 12, 3), (5, 33, 2), (16, 8, 4)])
def test_bwd_u8_matches_bruteforce(N, K, M):
    rng = _rng(3000 + N * K + M)
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 9)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    dX, B = oracle.hxq_linear_bwd_x_u8(cb, idx, rows, cols, deltas, DY, "f32")
    W = [[float(cb[int(i)]) for i in r] for r in idx.tolist()]
    ref = _brute_bwd_from_W(W, rows, cols, deltas, DY.tolist())
    assert dX.shape == (M, K)
    assert np.all(np.abs(dX - ref) <= (N + 4) * 2.0 ** -52 * B)


@pytest.mark.parametrize("N,K,M", [(6, 16, 3), (3, 10, 2), (9, 4, 5)])
def test_bwd_pk12_matches_bruteforce(N, K, M):
    rng = _rng(4000 + N * K + M)
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    idx2 = rng.integers(0, 4096, size=(N, K // 2))
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 7)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    dX, B = oracle.hxq_linear_bwd_x_pk12(cb2, packed, rows, cols, deltas, DY, "f32", N, K)
    W = _brute_pk12_weights(cb2, packed.tolist(), N, K)
    ref = _brute_bwd_from_W(W, rows, cols, deltas, DY.tolist())
    assert dX.shape == (M, K)
    assert np.all(np.abs(dX - ref) <= (N + 4) * 2.0 ** -52 * B)


def _golden_bwd():
    vals = {}
    with open(os.path.join(GOLDEN, "bwd_x_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, *rest = line.split()
                vals[name] = rest
    return vals


def test_bwd_golden_hand_example():
    g = _golden_bwd()
    cb = np.full(256, 0.5, np.float32)
    cb[:4] = [0.0, 1.0, 2.0, -1.0]
    idx = np.array([int(v) for v in g["indices"]], np.uint8).reshape(2, 3)
    rows = np.array([int(v) for v in g["sc_rows"]], np.int32)
    cols = np.array([int(v) for v in g["sc_cols"]], np.int32)
    deltas = np.array([float(v) for v in g["sc_deltas"]], np.float32)
    DY = np.array([float(v) for v in g["dy"]], np.float32).reshape(2, 2)
    want = np.array([float(v) for v in g["dx"]]).reshape(2, 3)
    dX, _ = oracle.hxq_linear_bwd_x_u8(cb, idx, rows, cols, deltas, DY, "f32")
    assert np.array_equal(dX, want)


def test_bwd_constant_index_closed_form():
    # every index e, no sidecar: W = C[e] everywhere, dX[m][k] = C[e] * sum_n dy[m][n]
    rng = _rng(31)
    N, K, M = 13, 10, 3
    cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
    idx = np.full((N, K), 77, np.uint8)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    dX, _ = oracle.hxq_linear_bwd_x_u8(cb, idx, [], [], [], DY, "f32")
    want = float(cb[77]) * np.array([math.fsum(map(float, r)) for r in DY])
    assert np.allclose(dX, np.repeat(want[:, None], K, axis=1), rtol=0, atol=1e-14)


def test_bwd_one_hot_rows_give_weight_rows():
    # dy row m = unit vector at n  ->  dX row m = W[n] (pk12 weights built from bytes)
    rng = _rng(32)
    N, K = 5, 12
    cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
    idx2 = rng.integers(0, 4096, size=(N, K // 2))
    packed = gen.pack12_rows(idx2)
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 5)
    DY = np.eye(N, dtype=np.float32)[[3, 0, 4]]
    dX, _ = oracle.hxq_linear_bwd_x_pk12(cb2, packed, rows, cols, deltas, DY, "f32", N, K)
    W = np.array(_brute_pk12_weights(cb2, packed.tolist(), N, K))
    for r, c, d in zip(rows, cols, deltas):
        W[int(r), int(c)] += float(d)
    assert np.array_equal(dX, W[[3, 0, 4]])


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_adjoint_of_forward(fmt):
    # <dY, X W^T> = <dY W, X>: the input gradient is the adjoint of the pinned
    # forward (bias subtracted), for non-square W and M > 1
    rng = _rng(33 if fmt == "u8" else 34)
    N, K, M = 11, 14, 4
    rows, cols, deltas = _tiny_sidecar(rng, N, K, 8)
    X = rng.standard_normal((M, K)).astype(np.float32)
    DY = rng.standard_normal((M, N)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    if fmt == "u8":
        cb = (0.05 * rng.standard_normal(256)).astype(np.float32)
        idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        Y, _ = oracle.hxq_linear_fwd_u8(cb, idx, rows, cols, deltas, X, "f32", bias)
        dX, _ = oracle.hxq_linear_bwd_x_u8(cb, idx, rows, cols, deltas, DY, "f32")
    else:
        cb2 = (0.05 * rng.standard_normal((4096, 2))).astype(np.float32)
        packed = gen.pack12_rows(rng.integers(0, 4096, size=(N, K // 2)))
        Y, _ = oracle.hxq_linear_fwd_pk12(cb2, packed, rows, cols, deltas, X, "f32", bias, N, K)
        dX, _ = oracle.hxq_linear_bwd_x_pk12(cb2, packed, rows, cols, deltas, DY, "f32", N, K)
    lhs = math.fsum((DY.astype(np.float64) * (Y - bias.astype(np.float64)[None, :])).ravel())
    rhs = math.fsum((dX * X.astype(np.float64)).ravel())
    scale = math.fsum((np.abs(dX) * np.abs(X.astype(np.float64))).ravel()) + 1.0
    assert abs(lhs - rhs) <= 1e-12 * scale
