"""GPU parity of the decode kernel and of hxq_linear_fwd_grouped (several
layers sharing x in one call) against the CPU oracle, through the C ABI."""

import numpy as np
import pytest

import gpu_util as G
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


def _x(seed, M, K, x_dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    xf = rng.standard_normal((M, K)).astype(np.float32)
    return gen.to_bf16_bits(xf) if x_dtype == "bf16" else xf


def _group(fmt, Ns, K, seed, nnz_den=1000):
    lays = [gen.random_layer(seed * 31 + i, N, K, fmt, nnz=max(1, N * K // nnz_den), duplicates=True)
            for i, N in enumerate(Ns)]
    return lays, [G.dev_layer(l) for l in lays]


def _grouped(fmt, lays, ds, xd, bias=True):
    t = G.torch()
    M = xd.shape[0]
    ys = [t.full((M, l.N), float("nan"), dtype=t.float32, device="cuda") for l in lays]
    desc = [dict(codebook=d["codebook"], indices=d["indices"], sc_rows=d["rows"], sc_cols=d["cols"],
                 sc_deltas=d["deltas"], bias=d["bias"] if bias else None, y=y)
            for d, y in zip(ds, ys)]
    hx.hxq_linear_fwd_grouped(hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12, desc, xd)
    return ys


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8, 13, 16])
def test_grouped_matches_oracle_and_single_calls(fmt, x_dtype, M):
    G.say("grouped %s %s M=%d" % (fmt, x_dtype, M))
    K = 2048
    lays, ds = _group(fmt, [1000, 96, 2500], K, seed=M)
    x_np = _x(M, M, K, x_dtype)
    xd = G.dev_x(x_np, x_dtype)
    ys = _grouped(fmt, lays, ds, xd)
    for lay, d, y in zip(lays, ds, ys):
        Y, B = G.oracle_fwd(lay, x_np, x_dtype)
        G.check(y, Y, B, G.TOL_FP32, "grouped %s N=%d" % (fmt, lay.N))
        # the same kernel and per-row arithmetic as the single-layer call
        # (more than four tokens go through it four at a time)
        y1 = G.run(lay, d, xd)
        assert G.torch().equal(y, y1), "grouped and single-layer results differ bitwise"


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("M", [20, 48, 64])
def test_grouped_token_groups_match_single_calls(fmt, M):
    # fp32 x past 16 tokens: the matrix-core GEMV with 32 / 64 staged tokens,
    # one launch for the group, the single-layer kernel's arithmetic
    G.say("grouped token groups %s M=%d" % (fmt, M))
    K = 2048
    lays, ds = _group(fmt, [1000, 96, 2500], K, seed=M + 100)
    x_np = _x(M + 1, M, K, "f32")
    xd = G.dev_x(x_np, "f32")
    ys = _grouped(fmt, lays, ds, xd)
    for lay, d, y in zip(lays, ds, ys):
        Y, B = G.oracle_fwd(lay, x_np, "f32")
        G.check(y, Y, B, G.TOL_FP32, "grouped %s N=%d" % (fmt, lay.N))
        assert G.torch().equal(y, G.run(lay, d, xd)), "grouped and single-layer results differ bitwise"


@pytest.mark.parametrize("fmt,M,K", [("u8", 17, 2048), ("u8", 130, 2048), ("u8", 300, 1024), ("u8", 130, 96),
                                      ("pk12", 17, 2048), ("pk12", 300, 1024), ("pk12", 130, 96),
                                      ("u8", 2000, 256), ("pk12", 2000, 256)])
def test_grouped_prefill_gemm(fmt, M, K):
    # bf16 x past the decode sizes: one matrix-core launch over all layers
    # (K % 32 == 0), else one call per layer (at 17 tokens these layers are
    # too narrow for the GEMM and take the fp32 matrix-core GEMV); all equal
    # single-layer calls bitwise.  At 2000 tokens the grouped launch takes
    # 256-output tiles while the 1000-output layer alone takes 128-output
    # ones: the tile width does not change any output's summation order.
    G.say("grouped gemm %s M=%d K=%d" % (fmt, M, K))
    lays, ds = _group(fmt, [1000, 96, 2500], K, seed=M + K)
    x_np = _x(M + 1, M, K, "bf16")
    xd = G.dev_x(x_np, "bf16")
    ys = _grouped(fmt, lays, ds, xd)
    for lay, d, y in zip(lays, ds, ys):
        Y, B = G.oracle_fwd(lay, x_np, "bf16")
        tol = G.TOL_BF16 if K % 32 == 0 or fmt == "u8" else G.TOL_FP32
        G.check(y, Y, B, tol, "grouped gemm %s N=%d" % (fmt, lay.N))
        assert G.torch().equal(y, G.run(lay, d, xd)), "grouped and single-layer results differ bitwise"


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("Ns,M", [([4096, 8192], 32), ([1000, 8000], 20), ([2048, 3968], 64)])
def test_grouped_bf16_narrow_and_wide_layers(fmt, Ns, M):
    # bf16 x at 17-64 tokens: the GEMM for layers with at least 32 output
    # tiles of 128 x 128, the fp32 matrix-core GEMV for narrower ones; a
    # group of both kinds runs its layers one by one.  Each layer equals its
    # single-layer call bitwise and the oracle within its path's tolerance.
    G.say("grouped bf16 %s Ns=%s M=%d" % (fmt, Ns, M))
    K = 2048
    lays, ds = _group(fmt, Ns, K, seed=M + sum(Ns))
    x_np = _x(M + 7, M, K, "bf16")
    xd = G.dev_x(x_np, "bf16")
    ys = _grouped(fmt, lays, ds, xd)
    for lay, d, y in zip(lays, ds, ys):
        Y, B = G.oracle_fwd(lay, x_np, "bf16")
        G.check(y, Y, B, G.TOL_BF16, "grouped bf16 %s N=%d" % (fmt, lay.N))
        assert G.torch().equal(y, G.run(lay, d, xd)), "grouped and single-layer results differ bitwise"
    if all(l.N <= 3968 for l in lays):
        for lay, y in zip(lays, ys):
            Y, B = G.oracle_fwd(lay, x_np, "bf16")
            G.check(y, Y, B, G.TOL_FP32, "grouped bf16 GEMV %s N=%d" % (fmt, lay.N))


@pytest.mark.parametrize("fmt,K", [("u8", 11008), ("pk12", 11008), ("u8", 16), ("u8", 4096 + 16)])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_decode_k_range(fmt, K, M):
    # K from one chunk to 11008 (several slices with a ragged last one); at
    # M = 4 and K = 11008 x does not fit LDS and the call takes another kernel
    G.say("decode %s K=%d M=%d" % (fmt, K, M))
    lay = gen.random_layer(K + M, 300, K, fmt, nnz=300 * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(K, M, K, "f32")
    y = G.run(lay, d, G.dev_x(x_np, "f32"))
    Y, B = G.oracle_fwd(lay, x_np, "f32")
    G.check(y, Y, B, G.TOL_FP32, "decode %s K=%d" % (fmt, K))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_decode_dense_sidecar(fmt):
    # more than one staging pass of sidecar triplets per workgroup
    lay = gen.random_layer(77, 24, 4096, fmt, nnz=24 * 4096 // 6, duplicates=True)
    d = G.dev_layer(lay)
    for M in (1, 2, 4):
        x_np = _x(M, M, 4096, "f32")
        y = G.run(lay, d, G.dev_x(x_np, "f32"))
        Y, B = G.oracle_fwd(lay, x_np, "f32")
        G.check(y, Y, B, G.TOL_FP32, "dense sidecar %s M=%d" % (fmt, M))


def test_decode_many_rows_per_block():
    # more rows than one workgroup's threads: the launcher adds workgroups
    lay = gen.random_layer(5, 300000, 16, "u8", nnz=5000, duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(5, 1, 16, "f32")
    y = G.run(lay, d, G.dev_x(x_np, "f32"))
    Y, B = G.oracle_fwd(lay, x_np, "f32")
    G.check(y, Y, B, G.TOL_FP32, "300000 rows")


def test_grouped_tiny_and_empty_layers():
    t = G.torch()
    K = 1024
    lays, ds = _group("u8", [1, 3000, 2], K, seed=9)
    x_np = _x(9, 1, K, "f32")
    xd = G.dev_x(x_np, "f32")
    ys = _grouped("u8", lays, ds, xd, bias=False)
    for lay, y in zip(lays, ys):
        Y, B = G.oracle_fwd(lay, x_np, "f32", bias=False)
        G.check(y, Y, B, G.TOL_FP32, "tiny layers N=%d" % lay.N)
    # a layer with N == 0 is skipped
    e = dict(codebook=ds[0]["codebook"], indices=t.empty((0, K), dtype=t.uint8, device="cuda"),
             y=t.empty((1, 0), device="cuda"))
    y1 = t.full((1, lays[1].N), float("nan"), device="cuda")
    hx.hxq_linear_fwd_grouped(hx.HXQ_FMT_U8, [e, dict(codebook=ds[1]["codebook"], indices=ds[1]["indices"],
                                                       sc_rows=ds[1]["rows"], sc_cols=ds[1]["cols"],
                                                       sc_deltas=ds[1]["deltas"], bias=ds[1]["bias"],
                                                       y=y1)], xd)
    Y, B = G.oracle_fwd(lays[1], x_np, "f32")
    G.check(y1, Y, B, G.TOL_FP32, "with an empty layer")


def test_grouped_is_deterministic():
    lays, ds = _group("u8", [2048, 256, 256], 2048, seed=3)
    xd = G.dev_x(_x(3, 1, 2048, "f32"), "f32")
    a = _grouped("u8", lays, ds, xd)
    for _ in range(3):
        b = _grouped("u8", lays, ds, xd)
        for ya, yb in zip(a, b):
            assert G.torch().equal(ya, yb)


@pytest.mark.parametrize("nbytes", [16, 1024 * 1024 + 48, 23 * 1000 * 1000 // 16 * 16])
@pytest.mark.parametrize("words", [8, 256, 1024, 4096 * 8])
@pytest.mark.parametrize("fn", ["hxq_stream_read", "hxq_stream_read_nt"])
def test_stream_read_digest(nbytes, words, fn):
    # the measurement helper reads every byte once whatever its grid (a word
    # per wave, words / 8 workgroups): XOR of the digests is the XOR of all
    # 32-bit words
    t = G.torch()
    rng = np.random.Generator(np.random.PCG64(nbytes))
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = t.from_numpy(host.view(np.int32)).cuda()
    sink = t.zeros(words, dtype=t.int32, device="cuda")
    st = getattr(hx.lib(), fn)(src.data_ptr(), nbytes, sink.data_ptr(), words,
                               t.cuda.current_stream().cuda_stream)
    assert st == 0
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [5, 8])
@pytest.mark.parametrize("Ns,K,nnz_den", [((20000,), 2048, 1000), ((11008, 11008), 1280, 1000),
                                          ((16392, 40), 2048, 100)])
def test_large_layers_m5_to_8(x_dtype, M, Ns, K, nnz_den):
    # 5-8 tokens on layers of gate|up size (tens of 4-row fragments per
    # workgroup, groups of two): a ragged last fragment, a K that gives the
    # waves different chunk counts, a tiny layer beside a large one, and a
    # sidecar dense enough for several epilogue passes
    G.say("large layers %s M=%d Ns=%s K=%d" % (x_dtype, M, Ns, K))
    lays, ds = _group("u8", list(Ns), K, seed=M * 7 + K, nnz_den=nnz_den)
    x_np = _x(M + K, M, K, x_dtype)
    xd = G.dev_x(x_np, x_dtype)
    ys = _grouped("u8", lays, ds, xd)
    for lay, y in zip(lays, ys):
        Y, B = G.oracle_fwd(lay, x_np, x_dtype)
        G.check(y, Y, B, G.TOL_FP32, "large layer N=%d" % lay.N)
    if len(lays) == 1:
        assert G.torch().equal(ys[0], G.run(lays[0], ds[0], xd)), "grouped and single-layer results differ bitwise"


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_grouped_streaming_launch(M):
    # a launch of more index bytes than the L2 caches hold (gate|up of the
    # Qwen set: 2 x 11008 x 2048 u8, 45 MB) takes the instances with
    # non-temporal index loads; each layer alone (22.5 MB) takes the ordinary
    # ones: the same arithmetic, so equal bit for bit, and equal to the oracle
    G.say("grouped streaming launch M=%d" % M)
    K = 2048
    lays, ds = _group("u8", [11008, 11008], K, seed=40 + M)
    x_np = _x(M + 77, M, K, "f32")
    xd = G.dev_x(x_np, "f32")
    ys = _grouped("u8", lays, ds, xd)
    for lay, d, y in zip(lays, ds, ys):
        Y, B = G.oracle_fwd(lay, x_np, "f32")
        G.check(y, Y, B, G.TOL_FP32, "streaming launch N=%d M=%d" % (lay.N, M))
        assert G.torch().equal(y, G.run(lay, d, xd)), "grouped and single-layer results differ bitwise"
