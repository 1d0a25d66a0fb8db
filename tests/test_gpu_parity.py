"""GPU parity of libhxq against the CPU oracle on small and medium shapes,
edge cases and invariants.  Every call goes through the C ABI."""

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
    hx.lib()  # raises if the library is not built
    yield
    t.cuda.synchronize()


def _x(seed, M, K, x_dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    xf = rng.standard_normal((M, K)).astype(np.float32)
    return gen.to_bf16_bits(xf) if x_dtype == "bf16" else xf


def _case(lay, M, x_dtype, variant, tol, seed=0, what=""):
    x_np = _x(seed, M, lay.K, x_dtype)
    d = G.dev_layer(lay)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype), variant=variant)
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    return G.check(y, Y, B, tol, what)


# ------------------------------------------------------------ fp32 GEMV, u8

U8_SHAPES = [(1000, 2048), (37, 4096), (513, 272), (4, 16), (1, 1040), (300, 11008 // 8 * 8 - 16)]


@pytest.mark.parametrize("N,K", U8_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 9, 16, 17, 40])
def test_u8_gemv_valu(N, K, M):
    G.say("u8 gemv_valu N=%d K=%d M=%d" % (N, K, M))
    lay = gen.random_layer(N * 7 + K, N, K, "u8", nnz=max(1, N * K // 1000), duplicates=True)
    _case(lay, M, "f32", hx.HXQ_VARIANT_GEMV_VALU, G.TOL_FP32, seed=M, what="u8 valu")


@pytest.mark.parametrize("M", [1, 7, 16])
def test_u8_gemv_bf16_x(M):
    lay = gen.random_layer(3, 700, 2048, "u8", nnz=1400)
    _case(lay, M, "bf16", hx.HXQ_VARIANT_AUTO, G.TOL_FP32, seed=M, what="u8 bf16 gemv")


# ----------------------------------------------------------- fp32 GEMV, pk12

@pytest.mark.parametrize("N,K", [(1000, 2048), (333, 1040), (5, 16), (64, 4096)])
@pytest.mark.parametrize("M", [1, 3, 8, 16, 20])
def test_pk12_gemv_valu(N, K, M):
    G.say("pk12 gemv_valu N=%d K=%d M=%d" % (N, K, M))
    lay = gen.random_layer(N + 3 * K, N, K, "pk12", nnz=max(1, N * K // 2000), duplicates=True)
    _case(lay, M, "f32", hx.HXQ_VARIANT_GEMV_VALU, G.TOL_FP32, seed=M, what="pk12 valu")


@pytest.mark.parametrize("M", [1, 16, 40])
def test_pk12_bf16_x(M):
    # up to 16 tokens the fp32 path, beyond it the bf16 matrix-core GEMM
    lay = gen.random_layer(4, 400, 1024, "pk12", nnz=300)
    tol = G.TOL_BF16 if M > 16 else G.TOL_FP32
    _case(lay, M, "bf16", hx.HXQ_VARIANT_AUTO, tol, seed=M, what="pk12 bf16")


# ------------------------------------------------------------------ generic

@pytest.mark.parametrize("fmt,N,K", [("u8", 77, 100), ("u8", 10, 7), ("u8", 3, 1),
                                     ("pk12", 77, 98), ("pk12", 9, 6), ("pk12", 4, 2),
                                     ("u8", 130, 2048), ("pk12", 130, 2048)])
@pytest.mark.parametrize("M", [1, 5])
def test_generic(fmt, N, K, M):
    G.say("generic %s N=%d K=%d M=%d" % (fmt, N, K, M))
    lay = gen.random_layer(11 + N + K, N, K, fmt, nnz=max(1, N * K // 50), duplicates=True)
    variant = hx.HXQ_VARIANT_GENERIC if K % 16 == 0 else hx.HXQ_VARIANT_AUTO
    _case(lay, M, "f32", variant, G.TOL_FP32, seed=M, what="generic")


# ---------------------------------------------------------------- bf16 GEMM

GEMMS = [hx.HXQ_VARIANT_GEMM_BF16, hx.HXQ_VARIANT_GEMM_BF16_T256]  # the automatic choice, and the 256 x 256 tile kernel forced

@pytest.mark.parametrize("N,K", [(1000, 2048), (300, 96), (129, 32), (256, 11008 // 32 * 32)])
@pytest.mark.parametrize("M", [17, 128, 200, 513])
@pytest.mark.parametrize("variant", GEMMS)
def test_u8_gemm_bf16(N, K, M, variant):
    G.say("u8 gemm N=%d K=%d M=%d variant=%d" % (N, K, M, variant))
    lay = gen.random_layer(N + K + 5, N, K, "u8", nnz=max(1, N * K // 1000), duplicates=True)
    _case(lay, M, "bf16", variant, G.TOL_BF16, seed=M, what="gemm")


@pytest.mark.parametrize("N,K", [(1000, 2048), (300, 64), (2048, 4096 + 64), (11008, 2048)])
@pytest.mark.parametrize("M", [17, 130, 300])
@pytest.mark.parametrize("variant", GEMMS)
def test_pk12_gemm_bf16(N, K, M, variant):
    # 2D pairs on the matrix cores: 12-byte index groups, the bf16 pair table
    G.say("pk12 gemm N=%d K=%d M=%d variant=%d" % (N, K, M, variant))
    lay = gen.random_layer(N + K + 9, N, K, "pk12", nnz=max(1, N * K // 2000), duplicates=True)
    _case(lay, M, "bf16", variant, G.TOL_BF16, seed=M, what="pk12 gemm")


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("variant", GEMMS)
def test_gemm_small_m_forced(M, variant):
    lay = gen.random_layer(21, 260, 64, "u8", nnz=40)
    _case(lay, M, "bf16", variant, G.TOL_BF16, seed=M, what="gemm small m")


@pytest.mark.parametrize("N,K,nnz,M", [
    (64, 1024, 8192, 150),    # more triplets in one tile than the patch area holds
    (96, 33024, 3000, 130),   # more stages than the patch bins cover
    (300, 4096, 12000, 200)])  # dense sidecar, patch path in some tiles and walk path in others
@pytest.mark.parametrize("variant", GEMMS)
@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_gemm_sidecar_paths(N, K, nnz, M, variant, fmt):
    G.say("gemm sidecar paths %s N=%d K=%d nnz=%d variant=%d" % (fmt, N, K, nnz, variant))
    lay = gen.random_layer(N + K, N, K, fmt, nnz=nnz, duplicates=True)
    _case(lay, M, "bf16", variant, G.TOL_BF16, seed=M, what="gemm sidecar paths")


def test_gemm_rejects_fp32_x():
    lay = gen.random_layer(22, 64, 64, "u8")
    d = G.dev_layer(lay)
    xd = G.dev_x(_x(0, 32, 64, "f32"), "f32")
    with pytest.raises(hx.HxqError):
        G.run(lay, d, xd, variant=hx.HXQ_VARIANT_GEMM_BF16)


# ---------------------------------------------------------------- edge cases

def test_m_zero_and_n_zero_are_no_ops():
    t = G.torch()
    lay = gen.random_layer(30, 8, 32, "u8", nnz=4)
    d = G.dev_layer(lay)
    xd = t.zeros((0, 32), device="cuda")
    y = t.zeros((0, 8), device="cuda")
    G.run(lay, d, xd, y=y)
    lay0 = gen.random_layer(31, 0, 32, "u8")
    d0 = G.dev_layer(lay0)
    y0 = t.zeros((3, 0), device="cuda")
    hx.hxq_linear_fwd_u8(d0["codebook"], d0["indices"], None, None, None,
                         G.dev_x(_x(0, 3, 32, "f32"), "f32"), None, y0)
    t.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_k_zero_gives_bias(fmt):
    t = G.torch()
    N = 50
    cb = t.zeros(256 if fmt == "u8" else 8192, device="cuda")
    idx = t.zeros((N, 0), dtype=t.uint8, device="cuda")
    bias = t.arange(N, dtype=t.float32, device="cuda")
    x = t.zeros((3, 0), device="cuda")
    y = t.full((3, N), float("nan"), device="cuda")
    fn = hx.hxq_linear_fwd_u8 if fmt == "u8" else hx.hxq_linear_fwd_pk12
    fn(cb, idx, None, None, None, x, bias, y)
    assert t.equal(y.cpu(), bias.cpu().expand(3, N))
    fn(cb, idx, None, None, None, x, None, y)
    assert t.equal(y.cpu(), t.zeros(3, N))


@pytest.mark.parametrize("variant", [hx.HXQ_VARIANT_GEMV_VALU, hx.HXQ_VARIANT_GENERIC])
@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_no_bias_no_sidecar(fmt, variant):
    lay = gen.random_layer(32, 300, 512, fmt, nnz=300)
    x_np = _x(1, 4, 512, "f32")
    d = G.dev_layer(lay)
    for bias in (True, False):
        for sc in (True, False):
            y = G.run(lay, d, G.dev_x(x_np, "f32"), variant=variant, bias=bias, sidecar=sc)
            Y, B = G.oracle_fwd(lay, x_np, "f32", bias=bias, sidecar=sc)
            G.check(y, Y, B, G.TOL_FP32, "bias=%s sidecar=%s" % (bias, sc))


def _heavy_sidecar_layer(fmt, N, K):
    """Many triplets in a few rows (more than one 64-wide batch), on the first
    and last rows and columns."""
    lay = gen.random_layer(33, N, K, fmt)
    rng = np.random.Generator(np.random.PCG64(5))
    rows = np.concatenate([np.full(300, 3), np.zeros(5, int), np.full(5, N - 1),
                           rng.integers(0, N, 100)])
    cols = np.concatenate([rng.integers(0, K, 300), [0, K - 1, 0, 5, 5], [0, K - 1, 1, 1, K - 1],
                           rng.integers(0, K, 100)])
    order = np.lexsort((cols, rows))
    lay.rows = rows[order].astype(np.int32)
    lay.cols = cols[order].astype(np.int32)
    lay.deltas = rng.standard_normal(rows.size).astype(np.float32)
    return lay


@pytest.mark.parametrize("fmt,variant,M,xdt", [
    ("u8", hx.HXQ_VARIANT_GEMV_VALU, 1, "f32"), ("u8", hx.HXQ_VARIANT_GEMV_VALU, 16, "f32"),
    ("pk12", hx.HXQ_VARIANT_GEMV_VALU, 3, "f32"), ("u8", hx.HXQ_VARIANT_GENERIC, 2, "f32"),
    ("pk12", hx.HXQ_VARIANT_GENERIC, 2, "f32"), ("u8", hx.HXQ_VARIANT_GEMM_BF16, 150, "bf16"),
    ("u8", hx.HXQ_VARIANT_GEMM_BF16_T256, 150, "bf16"), ("pk12", hx.HXQ_VARIANT_GEMM_BF16_T256, 150, "bf16")])
def test_dense_sidecar_rows(fmt, variant, M, xdt):
    lay = _heavy_sidecar_layer(fmt, 200, 1024)
    _case(lay, M, xdt, variant, G.TOL_BF16 if variant in GEMMS else G.TOL_FP32,
          what="heavy sidecar")


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_gemm_wide_tiles_ragged(fmt):
    """2000 tokens x 5124 outputs: 168 tiles of 256 x 256 fill most of a
    round over the CUs, so the wide tiles run, with a 4-output last tile and
    an 80-token last tile row."""
    N, K, M = 5124, 128, 2000
    G.say("gemm wide tiles ragged %s" % fmt)
    lay = gen.random_layer(57, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    for variant in GEMMS:
        _case(lay, M, "bf16", variant, G.TOL_BF16, seed=5, what="wide tiles ragged")


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_gemm_full_sidecar_block(fmt):
    """Every weight of a 16-row x 64-column block in the sidecar (1024 triplets
    in one stage of one wave, far past 64) plus a second dense block and
    scattered entries, within the tile's patch area."""
    N, K = 64, 256
    lay = gen.random_layer(41, N, K, fmt)
    rng = np.random.Generator(np.random.PCG64(9))
    r0, c0 = np.meshgrid(np.arange(16), np.arange(64), indexing="ij")
    r1, c1 = np.meshgrid(np.arange(16, 32), np.arange(64, 128), indexing="ij")
    rows = np.concatenate([r0.ravel(), r1.ravel(), rng.integers(0, N, 200)])
    cols = np.concatenate([c0.ravel(), c1.ravel(), rng.integers(0, K, 200)])
    order = np.lexsort((cols, rows))
    lay.rows = rows[order].astype(np.int32)
    lay.cols = cols[order].astype(np.int32)
    lay.deltas = (0.05 * rng.standard_normal(rows.size)).astype(np.float32)
    G.say("gemm full sidecar block %s nnz=%d" % (fmt, rows.size))
    for variant in GEMMS:
        _case(lay, 150, "bf16", variant, G.TOL_BF16, seed=3, what="full sidecar block")


@pytest.mark.parametrize("fmt,variant,M,xdt", [
    ("u8", hx.HXQ_VARIANT_GEMV_VALU, 8, "f32"), ("pk12", hx.HXQ_VARIANT_GEMV_VALU, 16, "f32"),
    ("u8", hx.HXQ_VARIANT_GEMM_BF16, 300, "bf16"), ("u8", hx.HXQ_VARIANT_GENERIC, 3, "f32"),
    ("pk12", hx.HXQ_VARIANT_GEMM_BF16_T256, 300, "bf16")])
def test_canary_and_determinism(fmt, variant, M, xdt):
    """No writes outside y, and two runs give the same bits."""
    t = G.torch()
    lay = gen.random_layer(34, 333, 2048, fmt, nnz=700)
    d = G.dev_layer(lay)
    xd = G.dev_x(_x(2, M, lay.K, xdt), xdt)
    guard = 4096
    outs = []
    for _ in range(2):
        buf = t.full((M * lay.N + 2 * guard,), -7.25, dtype=t.float32, device="cuda")
        y = buf[guard:guard + M * lay.N].view(M, lay.N)
        G.run(lay, d, xd, variant=variant, y=y)
        host = buf.cpu()
        assert bool((host[:guard] == -7.25).all()) and bool((host[-guard:] == -7.25).all())
        outs.append(y.cpu())
    assert t.equal(outs[0], outs[1])


@pytest.mark.parametrize("variant,xdt,M", [(hx.HXQ_VARIANT_GEMV_VALU, "f32", 1),
                                           (hx.HXQ_VARIANT_GEMV_VALU, "f32", 9),
                                           (hx.HXQ_VARIANT_GEMM_BF16, "bf16", 140),
                                           (hx.HXQ_VARIANT_GEMM_BF16_T256, "bf16", 140)])
def test_codebook_permutation_invariance(variant, xdt, M):
    """Permuting the codebook and remapping the indices leaves y unchanged, bit for bit."""
    t = G.torch()
    lay = gen.random_layer(35, 500, 1024, "u8", nnz=500)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(256)
    inv = np.argsort(perm)
    lay2 = gen.Layer(lay.name, -1, 0, lay.N, lay.K, "u8", lay.codebook[perm],
                     inv[lay.indices].astype(np.uint8), lay.rows, lay.cols, lay.deltas, lay.bias)
    xd = G.dev_x(_x(3, M, lay.K, xdt), xdt)
    y1 = G.run(lay, G.dev_layer(lay), xd, variant=variant).cpu()
    y2 = G.run(lay2, G.dev_layer(lay2), xd, variant=variant).cpu()
    assert t.equal(y1, y2)


# ------------------------------------------------------------- exact results

@pytest.mark.parametrize("fmt,variant,xdt,M", [
    ("u8", hx.HXQ_VARIANT_GEMV_VALU, "f32", 1), ("u8", hx.HXQ_VARIANT_GEMV_VALU, "f32", 16),
    ("pk12", hx.HXQ_VARIANT_GEMV_VALU, "f32", 4), ("u8", hx.HXQ_VARIANT_GEMM_BF16, "bf16", 130),
    ("u8", hx.HXQ_VARIANT_GEMM_BF16_T256, "bf16", 130), ("pk12", hx.HXQ_VARIANT_GEMM_BF16_T256, "bf16", 130),
    ("u8", hx.HXQ_VARIANT_GENERIC, "f32", 3)])
def test_constant_index_bit_exact(fmt, variant, xdt, M):
    """idx == j, no sidecar, C[j] = 0.375, integer x: every partial sum is exact,
    so y = C[j] * sum_k x + b exactly."""
    N, K = 300, 2048
    lay = gen.random_layer(36, N, K, fmt)
    if fmt == "u8":
        lay.codebook[17] = 0.375
        lay.indices[:] = 17
        half = (lay.codebook[17], lay.codebook[17])
    else:
        lay.codebook[1234] = (0.375, 0.375)
        lay.indices = gen.pack12_rows(np.full((N, K // 2), 1234))
        half = tuple(lay.codebook[1234])
    lay.bias = (np.arange(N) % 7 - 3).astype(np.float32) / 4
    rng = np.random.Generator(np.random.PCG64(4))
    xf = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    x_np = gen.to_bf16_bits(xf) if xdt == "bf16" else xf
    d = G.dev_layer(lay)
    y = G.run(lay, d, G.dev_x(x_np, xdt), variant=variant, sidecar=False).cpu().numpy()
    expect = (np.float64(half[0]) * xf[:, 0::2].astype(np.float64).sum(1)
              + np.float64(half[1]) * xf[:, 1::2].astype(np.float64).sum(1))
    expect = expect[:, None] + lay.bias[None, :].astype(np.float64)
    assert np.array_equal(y.astype(np.float64), expect)


@pytest.mark.parametrize("fmt,variant", [("u8", hx.HXQ_VARIANT_GEMV_VALU),
                                         ("pk12", hx.HXQ_VARIANT_GEMV_VALU),
                                         ("u8", hx.HXQ_VARIANT_GEMM_BF16),
                                         ("u8", hx.HXQ_VARIANT_GEMM_BF16_T256),
                                         ("pk12", hx.HXQ_VARIANT_GEMM_BF16_T256),
                                         ("u8", hx.HXQ_VARIANT_GENERIC)])
def test_one_hot_dequant_bit_exact(fmt, variant):
    """x = e_k reads column k of the weight: y[k][n] = fp32(C[idx] + delta) on the
    fp32 paths and bf16(fp32(C[idx] + delta)) on the matrix-core path."""
    _one_hot_case(fmt, variant, 260, 96, 200)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("N,K,nnz", [(260, 128, 300), (40, 256, 6000)])
def test_one_hot_gemm_k64(fmt, N, K, nnz):
    """The same probe on the 256-token matrix-core kernel: sidecar patches
    (few triplets) and the per-row walk (more triplets than the patch area)."""
    for variant in GEMMS:
        _one_hot_case(fmt, variant, N, K, nnz)


def _one_hot_case(fmt, variant, N, K, nnz):
    lay = gen.random_layer(37, N, K, fmt, nnz=nnz)  # unique coordinates
    W = (oracle.dequant_u8(lay.codebook, oracle.unpack_u8(lay.indices)) if fmt == "u8" else
         oracle.dequant_pk12(lay.codebook, oracle.unpack_pk12(lay.indices, N, K), K)).astype(np.float32)
    Wf = W.copy()
    Wf[lay.rows, lay.cols] = W[lay.rows, lay.cols] + lay.deltas  # fp32 add, one rounding
    xdt = "bf16" if variant in GEMMS else "f32"
    if variant in GEMMS:
        Wf = oracle.bf16_round_f32(Wf)
    eye = np.eye(K, dtype=np.float32)
    x_np = gen.to_bf16_bits(eye) if xdt == "bf16" else eye
    d = G.dev_layer(lay)
    y = G.run(lay, d, G.dev_x(x_np, xdt), variant=variant, bias=False).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), Wf.T.copy().view(np.uint32))


def test_cross_format_agreement():
    """A pk12 layer built from a 64-entry scalar codebook equals the u8 layer."""
    N, K, M = 400, 1024, 5
    rng = np.random.Generator(np.random.PCG64(8))
    c64 = (0.05 * rng.standard_normal(64)).astype(np.float32)
    cb = np.zeros(256, np.float32)
    cb[:64] = c64
    idx = rng.integers(0, 64, size=(N, K)).astype(np.uint8)
    e = np.arange(4096)
    cb2 = np.stack([c64[e >> 6], c64[e & 63]], 1).astype(np.float32)
    packed = gen.pack12_rows(64 * idx[:, 0::2].astype(np.int64) + idx[:, 1::2])
    base = gen.random_layer(38, N, K, "u8", nnz=400)
    l8 = gen.Layer("a", -1, 0, N, K, "u8", cb, idx, base.rows, base.cols, base.deltas, base.bias)
    l12 = gen.Layer("b", -1, 0, N, K, "pk12", cb2, packed, base.rows, base.cols, base.deltas, base.bias)
    x_np = _x(5, M, K, "f32")
    xd = G.dev_x(x_np, "f32")
    y8 = G.run(l8, G.dev_layer(l8), xd)
    y12 = G.run(l12, G.dev_layer(l12), xd)
    Y, B = G.oracle_fwd(l8, x_np, "f32")
    G.check(y8, Y, B, G.TOL_FP32, "u8")
    G.check(y12, Y, B, G.TOL_FP32, "pk12")
    G.check(y12, y8.cpu().numpy().astype(np.float64), B, 2 * G.TOL_FP32, "u8 vs pk12")


def test_m_prefix_rule():
    lay = gen.random_layer(39, 600, 2048, "u8", nnz=1200)
    x_np = _x(6, 8, 2048, "f32")
    d = G.dev_layer(lay)
    y8 = G.run(lay, d, G.dev_x(x_np, "f32")).cpu().numpy()
    y1 = G.run(lay, d, G.dev_x(x_np[:1], "f32")).cpu().numpy()
    Y, B = G.oracle_fwd(lay, x_np[:1], "f32")
    assert np.all(np.abs(y1[0] - y8[0]) <= 2 * G.TOL_FP32 * B[0])


# ------------------------------------------------------------- sidecar add

@pytest.mark.parametrize("xdt,M", [("f32", 1), ("f32", 8), ("bf16", 200)])
def test_sidecar_add_matches_oracle(xdt, M):
    t = G.torch()
    lay = _heavy_sidecar_layer("u8", 200, 1024)
    x_np = _x(7, M, lay.K, xdt)
    d = G.dev_layer(lay)
    y = t.zeros((M, lay.N), dtype=t.float32, device="cuda")
    hx.hxq_sidecar_add(d["rows"], d["cols"], d["deltas"], G.dev_x(x_np, xdt), y)
    Z, B = oracle.hxq_sidecar_add(lay.rows, lay.cols, lay.deltas, x_np, xdt, lay.N)
    G.check(y, Z, B, G.TOL_FP32, "sidecar add")


@pytest.mark.parametrize("fmt,variant,xdt,M,tol", [
    ("u8", hx.HXQ_VARIANT_GEMV_VALU, "f32", 8, G.TOL_FP32),
    ("pk12", hx.HXQ_VARIANT_GEMV_VALU, "f32", 16, G.TOL_FP32),
    ("u8", hx.HXQ_VARIANT_GEMM_BF16, "bf16", 256, G.TOL_BF16)])
def test_forward_then_sidecar_add(fmt, variant, xdt, M, tol):
    """fwd(no sidecar) followed by hxq_sidecar_add equals fwd(sidecar)."""
    lay = gen.random_layer(40, 512, 2048, fmt, nnz=2000, duplicates=True)
    x_np = _x(8, M, lay.K, xdt)
    d = G.dev_layer(lay)
    xd = G.dev_x(x_np, xdt)
    y = G.run(lay, d, xd, variant=variant, sidecar=False)
    hx.hxq_sidecar_add(d["rows"], d["cols"], d["deltas"], xd, y)
    Y, B = G.oracle_fwd(lay, x_np, xdt)
    G.check(y, Y, B, tol, "fwd + sidecar_add")


def test_side_stream():
    t = G.torch()
    lay = gen.random_layer(41, 700, 2048, "u8", nnz=1400)
    x_np = _x(9, 3, lay.K, "f32")
    d = G.dev_layer(lay)
    xd = G.dev_x(x_np, "f32")
    s = t.cuda.Stream()
    t.cuda.synchronize()
    with t.cuda.stream(s):
        y = t.empty((3, lay.N), device="cuda")
        hx.hxq_linear_fwd_u8(d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], xd,
                             d["bias"], y, stream=s)
    s.synchronize()
    Y, B = G.oracle_fwd(lay, x_np, "f32")
    G.check(y, Y, B, G.TOL_FP32, "side stream")


def test_helix_linear_layer_object():
    lay = gen.random_layer(42, 128, 256, "pk12", nnz=30)
    m = hx.HelixLinear.from_layer(lay)
    x_np = _x(10, 6, 256, "f32")
    y = m(G.dev_x(x_np, "f32").view(2, 3, 256))
    assert tuple(y.shape) == (2, 3, 128)
    Y, B = G.oracle_fwd(lay, x_np, "f32")
    G.check(y.reshape(6, 128), Y, B, G.TOL_FP32, "layer object")


def test_helix_linear_layer_bf16_split():
    # bf16 activations on a down-shaped layer: the layer object's forward
    # takes the workspace entry point, which splits the sum over k here
    lay = gen.random_layer(43, 2048, 11008, "u8", nnz=2048 * 11008 // 1000)
    m = hx.HelixLinear.from_layer(lay)
    assert hx.lib().hxq_linear_fwd_workspace(hx.HXQ_FMT_U8, hx.HXQ_BF16, 512, 2048, 11008) > 0
    x_np = _x(11, 512, 11008, "bf16")
    y = m(G.dev_x(x_np, "bf16").view(2, 256, 11008))
    assert tuple(y.shape) == (2, 256, 2048)
    Y, B = G.oracle_fwd(lay, x_np, "bf16")
    G.check(y.reshape(512, 2048), Y, B, G.TOL_BF16, "layer object bf16 split")
