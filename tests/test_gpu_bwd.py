"""Input gradient dx = dy W of a frozen layer through the C ABI, element by
element against the CPU oracle (fp64 dY @ W, W dequantised with its sidecar).

Shapes cover M = 1 at the full attention and MLP widths of the Qwen2.5-3B
workload (K and N of 2048 and 11008), ragged column tails (K not a multiple
of the 512-column tile), the byte-load path (u8 K % 8 != 0, pk12 K % 16 != 0),
token tails past the 8-token tile, a launch with a single row split (plain
stores) and the empty cases.  Tolerance: 1e-5 * (|dY| |W|) for the fp32 path,
8e-3 * (|dY| |W|) for the bf16 matrix-core kernel (bf16 dy from 16 tokens),
which is also run forced on its own shapes: the MLP widths, K not a multiple
of its 512-column workgroup tile, token tails, the smallest and largest K, and
sidecar bins longer than a wave; likewise the 256 x 256 tile kernel (u8).
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


def _fmt(lay):
    return hx.HXQ_FMT_U8 if lay.fmt == "u8" else hx.HXQ_FMT_PK12


def _dy(seed, M, N, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal((M, N)).astype(np.float32)
    return v if dtype == "f32" else gen.to_bf16_bits(v)


def _oracle(lay, dy_np, dtype, sidecar=True):
    rows, cols, deltas = (lay.rows, lay.cols, lay.deltas) if sidecar else ([], [], [])
    if lay.fmt == "u8":
        return oracle.hxq_linear_bwd_x_u8(lay.codebook, lay.indices, rows, cols, deltas, dy_np, dtype)
    return oracle.hxq_linear_bwd_x_pk12(lay.codebook, lay.indices, rows, cols, deltas, dy_np, dtype,
                                        lay.N, lay.K)


def _run(lay, d, dyd, sidecar=True, variant=hx.HXQ_VARIANT_AUTO, workspace=None):
    t = G.torch()
    M = dyd.shape[0]
    dx = t.full((M, lay.K), float("nan"), dtype=t.float32, device="cuda")
    r, c, dl = (d["rows"], d["cols"], d["deltas"]) if sidecar else (None, None, None)
    hx.hxq_linear_bwd_x(_fmt(lay), d["codebook"], d["indices"], r, c, dl, dyd, dx, lay.K, variant=variant,
                        workspace=workspace)
    return dx


CASES = [
    # (N, K, M): full-width decode shapes, tails, byte path, token tails, one split
    (11008, 2048, 1),
    (2048, 11008, 1),
    (256, 2048, 1),
    (2048, 2048, 2),
    (300, 1024, 4),
    (257, 520, 3),
    (97, 4096 + 16, 5),
    (33, 30, 2),
    (1000, 2048, 8),
    (700, 1024, 37),
    (5, 16, 64),
    (1, 64, 1),
    (256, 4096, 512),
]


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K,M", CASES)
def test_bwd_x_matches_oracle(fmt, dtype, N, K, M):
    if fmt == "pk12" and K % 2:
        pytest.skip("pk12 needs an even K")
    G.say("bwd_x %s dy=%s N=%d K=%d M=%d" % (fmt, dtype, N, K, M))
    lay = gen.random_layer(5000 + N + 3 * K + 7 * M, N, K, fmt, nnz=max(1, N * K // 1000), duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(6000 + N + K + M, M, N, dtype)
    dx = _run(lay, d, G.dev_x(dy_np, dtype))
    G.torch().cuda.synchronize()
    Y, B = _oracle(lay, dy_np, dtype)
    # bf16 dy from 16 tokens may take the bf16 matrix-core kernel
    tol = G.TOL_BF16 if dtype == "bf16" and M >= 16 else G.TOL_FP32
    G.check(dx, Y, B, tol, "bwd_x %s %s N=%d K=%d M=%d" % (fmt, dtype, N, K, M))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_x_without_sidecar(fmt):
    N, K, M = 600, 1536, 3
    G.say("bwd_x %s no sidecar" % fmt)
    lay = gen.random_layer(91, N, K, fmt)
    d = G.dev_layer(lay)
    dy_np = _dy(92, M, N, "f32")
    dx = _run(lay, d, G.dev_x(dy_np, "f32"), sidecar=False)
    Y, B = _oracle(lay, dy_np, "f32", sidecar=False)
    G.check(dx, Y, B, G.TOL_FP32, "bwd_x %s no sidecar" % fmt)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_x_dense_sidecar_rows(fmt):
    # many triplets per row and per column tile, repeated coordinates
    N, K, M = 64, 1024, 2
    G.say("bwd_x %s dense sidecar" % fmt)
    lay = gen.random_layer(93, N, K, fmt, nnz=N * K // 8, duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(94, M, N, "f32")
    dx = _run(lay, d, G.dev_x(dy_np, "f32"), variant=hx.HXQ_VARIANT_GEMV_VALU)
    Y, B = _oracle(lay, dy_np, "f32")
    G.check(dx, Y, B, G.TOL_FP32, "bwd_x %s dense sidecar" % fmt)


def test_bwd_x_empty_rows_give_zero():
    # N == 0: the sum over rows is empty, dx = 0 (overwriting what was there)
    t = G.torch()
    G.say("bwd_x N=0")
    cb = t.zeros(256, dtype=t.float32, device="cuda")
    idx = t.zeros((0, 48), dtype=t.uint8, device="cuda")
    dy = t.zeros((3, 0), dtype=t.float32, device="cuda")
    dx = t.full((3, 48), float("nan"), dtype=t.float32, device="cuda")
    hx.hxq_linear_bwd_x(hx.HXQ_FMT_U8, cb, idx, None, None, None, dy, dx, 48)
    assert bool((dx == 0).all())


def test_bwd_x_no_tokens_is_a_no_op():
    t = G.torch()
    G.say("bwd_x M=0")
    lay = gen.random_layer(95, 40, 64, "u8", nnz=3)
    d = G.dev_layer(lay)
    dy = t.zeros((0, 40), dtype=t.float32, device="cuda")
    dx = t.zeros((0, 64), dtype=t.float32, device="cuda")
    hx.hxq_linear_bwd_x(hx.HXQ_FMT_U8, d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], dy, dx, 64)
    t.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_x_adjoint_of_forward_on_device(fmt):
    # <dy, y - b> = <dx, x> with both products from the library (fp32 path),
    # at a decode shape of the MLP block
    t = G.torch()
    N, K, M = 11008, 2048, 2
    G.say("bwd_x %s adjoint" % fmt)
    lay = gen.random_layer(96, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    rng = np.random.Generator(np.random.PCG64(97))
    x = t.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda()
    dy = t.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda()
    y = G.run(lay, d, x, bias=False)
    dx = _run(lay, d, dy)
    lhs = float((dy.double() * y.double()).sum())
    rhs = float((dx.double() * x.double()).sum())
    scale = float((dy.abs().double() @ y.abs().double().t()).diagonal().sum()) + 1.0
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("share", [1.0, 0.5, 0.0, None])
def test_bwd_x_workspace_sizes(fmt, share):
    # the full workspace, part of it (fewer splits), one split's worth less
    # than two (no split) and none: the same sums within the fp32 tolerance;
    # the workspace starts out holding garbage
    t = G.torch()
    N, K, M = 11008, 2048, 3
    G.say("bwd_x %s workspace share %s" % (fmt, share))
    lay = gen.random_layer(98, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(99, M, N, "f32")
    need = hx.hxq_linear_bwd_x_workspace(_fmt(lay), hx.HXQ_F32, M, N, K, len(lay.rows))
    assert need >= 2 * M * K * 4  # this shape splits its rows
    nbytes = 0 if share is None else max(4, int(need * share) // 4 * 4)
    ws = t.full((nbytes // 4,), float("nan"), dtype=t.float32, device="cuda")
    dx = _run(lay, d, G.dev_x(dy_np, "f32"), workspace=ws)
    Y, B = _oracle(lay, dy_np, "f32")
    G.check(dx, Y, B, G.TOL_FP32, "bwd_x %s workspace %s" % (fmt, share))


MFMA_CASES = [
    # (N, K, M)
    (2048, 2048, 64),
    (11008, 2048, 128),
    (2048, 11008, 96),
    (256, 512, 16),
    (64, 128, 200),
    (32, 16384, 20),
]


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("N,K,M", MFMA_CASES)
def test_bwd_x_mfma_matches_oracle(fmt, N, K, M):
    G.say("bwd_x mfma %s N=%d K=%d M=%d" % (fmt, N, K, M))
    lay = gen.random_layer(7000 + N + 3 * K + 7 * M, N, K, fmt, nnz=max(1, N * K // 1000), duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(8000 + N + K + M, M, N, "bf16")
    dx = _run(lay, d, G.dev_x(dy_np, "bf16"), variant=hx.HXQ_VARIANT_GEMM_BF16)
    G.torch().cuda.synchronize()
    Y, B = _oracle(lay, dy_np, "bf16")
    G.check(dx, Y, B, G.TOL_BF16, "bwd_x mfma %s N=%d K=%d M=%d" % (fmt, N, K, M))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_bwd_x_mfma_dense_sidecar(fmt):
    # bins of several hundred triplets (past the 64 a wave prefetches) with
    # repeated coordinates; and the same layer without its sidecar
    N, K, M = 64, 1024, 48
    G.say("bwd_x mfma %s dense sidecar" % fmt)
    lay = gen.random_layer(101, N, K, fmt, nnz=N * K // 8, duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(102, M, N, "bf16")
    for sidecar in (True, False):
        dx = _run(lay, d, G.dev_x(dy_np, "bf16"), sidecar=sidecar, variant=hx.HXQ_VARIANT_GEMM_BF16)
        Y, B = _oracle(lay, dy_np, "bf16", sidecar=sidecar)
        G.check(dx, Y, B, G.TOL_BF16, "bwd_x mfma %s dense sidecar=%s" % (fmt, sidecar))


def test_bwd_x_mfma_needs_its_workspace():
    # forced onto the matrix cores with too little workspace: refused, nothing launched
    t = G.torch()
    N, K, M = 2048, 2048, 64
    lay = gen.random_layer(103, N, K, "u8", nnz=N * K // 1000)
    d = G.dev_layer(lay)
    dy = G.dev_x(_dy(104, M, N, "bf16"), "bf16")
    dx = t.zeros((M, K), dtype=t.float32, device="cuda")
    with pytest.raises(hx.HxqError):
        hx.hxq_linear_bwd_x(hx.HXQ_FMT_U8, d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], dy, dx,
                            K, variant=hx.HXQ_VARIANT_GEMM_BF16, workspace=t.zeros(4, dtype=t.uint8, device="cuda"))


G5_CASES = [
    # (N, K, M) on the 256 x 256 tile kernel (u8): row splits, token tails,
    # K with a half-empty last column tile, one and three stages, the
    # narrowest and widest K
    (2048, 2048, 256),
    (11008, 2048, 300),
    (2048, 11008, 200),
    (32, 384, 17),
    (96, 1152, 520),
    (4096, 128, 64),
    (64, 16384, 130),
]


@pytest.mark.parametrize("N,K,M", G5_CASES)
def test_bwd_x_g5_matches_oracle(N, K, M):
    G.say("bwd_x g5 N=%d K=%d M=%d" % (N, K, M))
    lay = gen.random_layer(9000 + N + 3 * K + 7 * M, N, K, "u8", nnz=max(1, N * K // 1000), duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(9500 + N + K + M, M, N, "bf16")
    dx = _run(lay, d, G.dev_x(dy_np, "bf16"), variant=hx.HXQ_VARIANT_GEMM_BF16_T256)
    G.torch().cuda.synchronize()
    Y, B = _oracle(lay, dy_np, "bf16")
    G.check(dx, Y, B, G.TOL_BF16, "bwd_x g5 N=%d K=%d M=%d" % (N, K, M))


def test_bwd_x_g5_dense_sidecar_and_repeats():
    # bins of several hundred patch words (past the 64 a wave reads at once)
    # with repeated coordinates, rows in every stage; the same layer without
    # its sidecar; and, without it, the same bits on a second call
    t = G.torch()
    N, K, M = 96, 1024, 256
    G.say("bwd_x g5 dense sidecar")
    lay = gen.random_layer(111, N, K, "u8", nnz=N * K // 8, duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(112, M, N, "bf16")
    dyd = G.dev_x(dy_np, "bf16")
    for sidecar in (True, False):
        dx = _run(lay, d, dyd, sidecar=sidecar, variant=hx.HXQ_VARIANT_GEMM_BF16_T256)
        Y, B = _oracle(lay, dy_np, "bf16", sidecar=sidecar)
        G.check(dx, Y, B, G.TOL_BF16, "bwd_x g5 dense sidecar=%s" % sidecar)
    again = _run(lay, d, dyd, sidecar=False, variant=hx.HXQ_VARIANT_GEMM_BF16_T256)
    assert t.equal(dx, again)


def test_bwd_x_g5_rejects_pk12():
    t = G.torch()
    N, K, M = 256, 512, 256
    lay = gen.random_layer(113, N, K, "pk12", nnz=100)
    d = G.dev_layer(lay)
    dy = G.dev_x(_dy(114, M, N, "bf16"), "bf16")
    dx = t.zeros((M, K), dtype=t.float32, device="cuda")
    with pytest.raises(hx.HxqError):
        hx.hxq_linear_bwd_x(hx.HXQ_FMT_PK12, d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], dy,
                            dx, K, variant=hx.HXQ_VARIANT_GEMM_BF16_T256)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_layer_autograd_input_gradient(fmt, xdt):
    # HelixLinear under autograd: y = layer(x), y.backward(dy) leaves dy W in
    # x.grad (computed by the library), in x's dtype
    t = G.torch()
    N, K, M = 1000, 1024, 5
    G.say("layer autograd %s x=%s" % (fmt, xdt))
    lay = gen.random_layer(105, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    m = hx.HelixLinear.from_layer(lay, device="cuda")
    rng = np.random.Generator(np.random.PCG64(106))
    x_np = rng.standard_normal((M, K)).astype(np.float32)
    x = G.dev_x(x_np if xdt == "f32" else gen.to_bf16_bits(x_np), xdt).requires_grad_(True)
    y = m(x)
    assert y.requires_grad and y.dtype == t.float32
    dy_np = _dy(107, M, N, "f32")
    y.backward(t.from_numpy(dy_np).cuda())
    t.cuda.synchronize()
    assert x.grad is not None and x.grad.dtype == x.dtype
    Y, B = _oracle(lay, dy_np, "f32")
    tol = G.TOL_FP32 if xdt == "f32" else G.TOL_BF16  # bf16 x: the gradient is rounded to bf16
    G.check(x.grad.float(), Y, B, tol, "layer autograd %s %s" % (fmt, xdt))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_x_vector_kernel_long_runs(fmt, dtype):
    # many tiles, so few row splits: each workgroup's run (4096 rows) is longer
    # than the rows of dy it stages at once (256 at 8 tokens), so dy is staged
    # again mid-run and the sidecar terms read dy from global memory; bf16 dy
    # forced onto the vector kernel
    N, K, M = 8192, 4096, 64
    G.say("bwd_x vector long runs %s %s" % (fmt, dtype))
    lay = gen.random_layer(108, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    dy_np = _dy(109, M, N, dtype)
    dx = _run(lay, d, G.dev_x(dy_np, dtype), variant=hx.HXQ_VARIANT_GEMV_VALU)
    Y, B = _oracle(lay, dy_np, dtype)
    G.check(dx, Y, B, G.TOL_FP32, "bwd_x vector long runs %s %s" % (fmt, dtype))


def test_bwd_x_split_sum_repeats():
    # row-split shapes at one token, called in turn several times on one
    # stream: within tolerance of the oracle every time, and without a
    # sidecar (whose terms within a tile are added in no fixed order) the
    # same bits every time (the row splits are summed in a fixed order)
    t = G.torch()
    shapes = [(2048, 2048), (11008, 2048), (2048, 11008), (257, 520)]
    runs = []
    for i, (N, K) in enumerate(shapes):
        lay = gen.random_layer(700 + i, N, K, "u8", nnz=N * K // 1000, duplicates=True)
        dy_np = _dy(800 + i, 1, N, "f32")
        Y, B = _oracle(lay, dy_np, "f32")
        Y0, B0 = _oracle(lay, dy_np, "f32", sidecar=False)
        runs.append((lay, G.dev_layer(lay), G.dev_x(dy_np, "f32"), Y, B, Y0, B0))
    first = []
    for rep in range(3):
        for i, (lay, d, dyd, Y, B, Y0, B0) in enumerate(runs):
            G.say("bwd_x split sum repeat %d shape %d" % (rep, i))
            G.check(_run(lay, d, dyd), Y, B, G.TOL_FP32, "bwd_x split sum shape %d repeat %d" % (i, rep))
            dx0 = _run(lay, d, dyd, sidecar=False).cpu().numpy()
            G.check(t.from_numpy(dx0), Y0, B0, G.TOL_FP32, "bwd_x split sum, no sidecar, shape %d" % i)
            if rep == 0:
                first.append(dx0)
            else:
                assert np.array_equal(dx0, first[i]), "repeat %d of shape %d differs" % (rep, i)
