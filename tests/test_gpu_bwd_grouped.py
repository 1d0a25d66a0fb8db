"""Grouped input gradient dx = sum_i dy_i W_i (layers that share their input,
such as q|k|v or gate|up) through the C ABI, against the CPU oracle: the sum
of each layer's fp64 dY_i @ W_i, with the bound the sum of the layers' bounds.

Cases: the Qwen2.5-3B decode shapes (q|k|v, gate|up at one token), token
tails, the byte-load path, a group with an empty layer, both kernel families
(fp32 vector products; bf16 matrix cores from 16 tokens on shapes they
take, a launch per layer, or from 128 tokens (u8) one 256 x 256 tile
launch for the whole group, also with a dense sidecar in one layer only),
a single active layer (the single-layer call, bitwise), repeat determinism
without a sidecar, and a workspace that is too small.
Tolerances as for the single-layer input gradient.
"""

import numpy as np
import pytest

import gpu_util as G
import oracle
import vq_compressed_linear_amd as hx
from hxq_synth import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("needs a GPU")
    hx.lib()
    yield
    t.cuda.synchronize()


def _fmtc(fmt):
    return hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12


def _dy(seed, M, N, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal((M, N)).astype(np.float32)
    return v if dtype == "f32" else gen.to_bf16_bits(v)


def _oracle_one(lay, dy_np, dtype, sidecar=True):
    rows, cols, deltas = (lay.rows, lay.cols, lay.deltas) if sidecar else ([], [], [])
    if lay.fmt == "u8":
        return oracle.hxq_linear_bwd_x_u8(lay.codebook, lay.indices, rows, cols, deltas, dy_np, dtype)
    return oracle.hxq_linear_bwd_x_pk12(lay.codebook, lay.indices, rows, cols, deltas, dy_np, dtype,
                                        lay.N, lay.K)


def _group(fmt, Ns, K, M, dtype, seed, den=1000):
    lays, devs, dys, dy_nps = [], [], [], []
    for i, N in enumerate(Ns):
        lay = gen.random_layer(seed * 13 + i, N, K, fmt, nnz=max(1, N * K // den) if N else 0,
                               duplicates=True)
        dy_np = _dy(seed * 17 + i, M, N, dtype)
        lays.append(lay)
        devs.append(G.dev_layer(lay))
        dy_nps.append(dy_np)
        dys.append(G.dev_x(dy_np, dtype))
    return lays, devs, dys, dy_nps


def _descs(devs, dys, sidecar=True):
    return [dict(codebook=d["codebook"], indices=d["indices"], sc_rows=d["rows"] if sidecar else None,
                 sc_cols=d["cols"] if sidecar else None, sc_deltas=d["deltas"] if sidecar else None, dy=dy)
            for d, dy in zip(devs, dys)]


def _run(fmt, devs, dys, M, K, sidecar=True, workspace=None):
    t = G.torch()
    dx = t.full((M, K), float("nan"), dtype=t.float32, device="cuda")
    hx.hxq_linear_bwd_x_grouped(_fmtc(fmt), _descs(devs, dys, sidecar), dx, workspace=workspace)
    return dx


def _oracle(lays, dy_nps, dtype, K, sidecar=True):
    M = dy_nps[0].shape[0]
    Y = np.zeros((M, K))
    B = np.zeros((M, K))
    for lay, dy_np in zip(lays, dy_nps):
        if lay.N == 0:
            continue
        y, b = _oracle_one(lay, dy_np, dtype, sidecar)
        Y += y
        B += b
    return Y, B


CASES = [
    # (Ns, K, M)
    ([2048, 256, 256], 2048, 1),   # q|k|v at one token
    ([11008, 11008], 2048, 1),     # gate|up at one token
    ([1000, 64, 300], 1024, 3),
    ([300, 97, 5], 522, 2),        # byte-load path, ragged column tile
    ([700, 300], 2048, 8),
    ([700, 300, 5], 1024, 37),
    ([2048, 256, 256], 2048, 64),  # bf16: matrix cores, a launch per layer
    ([512, 1024], 1024, 300),      # bf16 (u8): one 256 x 256 tile launch for both
    ([2048, 256, 256], 2048, 256),
]


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Ns,K,M", CASES)
def test_bwd_x_grouped_matches_oracle(fmt, dtype, Ns, K, M):
    G.say("bwd_x grouped %s dy=%s Ns=%s K=%d M=%d" % (fmt, dtype, Ns, K, M))
    seed = sum(Ns) + 3 * K + 7 * M
    lays, devs, dys, dy_nps = _group(fmt, Ns, K, M, dtype, seed)
    dx = _run(fmt, devs, dys, M, K)
    Y, B = _oracle(lays, dy_nps, dtype, K)
    tol = G.TOL_BF16 if dtype == "bf16" and M >= 16 else G.TOL_FP32
    G.check(dx, Y, B, tol, "bwd_x grouped %s %s Ns=%s K=%d M=%d" % (fmt, dtype, Ns, K, M))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_x_grouped_skips_empty_layers(fmt):
    K, M = 256, 4
    lays, devs, dys, dy_nps = _group(fmt, [300, 0, 200], K, M, "f32", 31)
    dx = _run(fmt, devs, dys, M, K)
    Y, B = _oracle(lays, dy_nps, "f32", K)
    G.check(dx, Y, B, G.TOL_FP32, "bwd_x grouped %s with an empty layer" % fmt)
    # every layer empty: dx = 0
    t = G.torch()
    _, devs0, dys0, _ = _group(fmt, [0, 0], K, M, "f32", 32)
    dx0 = _run(fmt, devs0, dys0, M, K)
    assert t.equal(dx0, t.zeros_like(dx0))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("dtype,M", [("f32", 2), ("bf16", 64)])
def test_bwd_x_grouped_one_active_layer_is_the_single_call(fmt, dtype, M):
    # without a sidecar both calls are deterministic: the same bits
    t = G.torch()
    K = 1024
    lays, devs, dys, _ = _group(fmt, [0, 704], K, M, dtype, 33)
    dx = _run(fmt, devs, dys, M, K, sidecar=False)
    lay, d = lays[1], devs[1]
    dx1 = t.full((M, K), float("nan"), dtype=t.float32, device="cuda")
    hx.hxq_linear_bwd_x(_fmtc(fmt), d["codebook"], d["indices"], None, None, None, dys[1], dx1, K)
    assert t.equal(dx, dx1)


@pytest.mark.parametrize("dtype,M", [("f32", 1), ("bf16", 64)])
def test_bwd_x_grouped_repeats_bitwise(dtype, M):
    t = G.torch()
    K = 2048
    _, devs, dys, _ = _group("u8", [2048, 256, 256], K, M, dtype, 34)
    a = _run("u8", devs, dys, M, K, sidecar=False)
    b = _run("u8", devs, dys, M, K, sidecar=False)
    assert t.equal(a, b)


def test_bwd_x_grouped_needs_its_workspace():
    t = G.torch()
    K, M = 1024, 2
    _, devs, dys, _ = _group("u8", [300, 200], K, M, "f32", 35)
    dx = t.full((M, K), float("nan"), dtype=t.float32, device="cuda")
    with pytest.raises(hx.HxqError):
        hx.hxq_linear_bwd_x_grouped(hx.HXQ_FMT_U8, _descs(devs, dys), dx,
                                    workspace=t.zeros(16, dtype=t.uint8, device="cuda"))
    t.cuda.synchronize()
    assert bool(t.isnan(dx).all())


def test_bwd_x_grouped_256_tiles_dense_sidecar():
    # one 256 x 256 tile launch for the group with stages of several hundred
    # patch words in one layer and none in the other
    K, M = 1024, 256
    lays, devs, dys, dy_nps = _group("u8", [96, 128], K, M, "bf16", 36, den=8)
    lays[1].rows = lays[1].rows[:0]
    lays[1].cols = lays[1].cols[:0]
    lays[1].deltas = lays[1].deltas[:0]
    devs[1] = G.dev_layer(lays[1])
    dx = _run("u8", devs, dys, M, K)
    Y, B = _oracle(lays, dy_nps, "bf16", K)
    G.check(dx, Y, B, G.TOL_BF16, "bwd_x grouped 256 tiles dense sidecar")


@pytest.mark.parametrize("names", [("q", "k", "v"), ("gate", "up"), ("o",), ("down",)])
def test_bwd_x_grouped_workload_2048_tokens_sampled(names):
    # the bench's input-gradient step at 2048 tokens (bf16 dy), each shared
    # input's grouped call on the Qwen2.5-3B-shaped layers of the workload:
    # every column of dx for one token row in every 128-token block, the last
    # of every 256-token block and 64 more
    by = {l.name: l for l in gen.config_layers(1)}
    lays = [by[n] for n in names]
    M, K = 2048, lays[0].K
    G.say("bwd_x grouped workload %s M=%d" % ("|".join(names), M))
    devs = [G.dev_layer(l) for l in lays]
    dy_nps = [_dy(900 + i, M, l.N, "bf16") for i, l in enumerate(lays)]
    dys = [G.dev_x(d, "bf16") for d in dy_nps]
    dx = _run("u8", devs, dys, M, K)
    rows = G.tile_rows(M)
    Y = np.zeros((len(rows), K))
    B = np.zeros((len(rows), K))
    for lay, dy_np in zip(lays, dy_nps):
        y, b = oracle.hxq_linear_bwd_x_u8(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, dy_np,
                                          "bf16", m_rows=rows)
        Y += y
        B += b
    G.check(dx, Y, B, G.TOL_BF16, "bwd_x grouped workload %s" % "|".join(names), m_rows=rows)
