"""GPU parity of the matrix-core GEMV (5 <= M <= 64 tokens in one launch,
more in launches of 64; u8 and pk12, K % 64 == 0) against the CPU oracle,
through the C ABI."""

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


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [5, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(300, 2048), (2048, 576), (11008, 2048), (2048, 11008), (33, 64)])
def test_gemv_mfma_matches_oracle(x_dtype, M, N, K):
    # 16-row fragments with a ragged last one, slices with a ragged last one
    # (576 = 512 + 64), one to four fragments per workgroup
    G.say("gemv mfma %s M=%d N=%d K=%d" % (x_dtype, M, N, K))
    lay = gen.random_layer(N + K + M, N, K, "u8", nnz=max(1, N * K // 1000), duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(M + K, M, K, x_dtype)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype))
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma")


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [5, 9, 16])
@pytest.mark.parametrize("N,K", [(300, 2048), (8512, 2048), (2048, 4096 + 64)])
def test_gemv_mfma_pk12_matches_oracle(x_dtype, M, N, K):
    # 2D pairs: 12-bit indices three bytes per pair of pairs, the 4096-pair table
    G.say("gemv mfma pk12 %s M=%d N=%d K=%d" % (x_dtype, M, N, K))
    lay = gen.random_layer(N + K + M + 1, N, K, "pk12", nnz=max(1, N * K // 2000), duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(M + K + 1, M, K, x_dtype)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype))
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma pk12")


def test_gemv_mfma_dense_sidecar():
    # several epilogue passes of sidecar terms per workgroup, repeated coordinates
    lay = gen.random_layer(91, 40, 1024, "u8", nnz=40 * 1024 // 8, duplicates=True)
    d = G.dev_layer(lay)
    for M, xdt in ((6, "f32"), (16, "bf16")):
        x_np = _x(M, M, 1024, xdt)
        y = G.run(lay, d, G.dev_x(x_np, xdt))
        Y, B = G.oracle_fwd(lay, x_np, xdt)
        G.check(y, Y, B, G.TOL_FP32, "gemv mfma dense sidecar M=%d" % M)


def test_gemv_mfma_no_bias_no_sidecar_and_determinism():
    t = G.torch()
    lay = gen.random_layer(92, 1000, 2048, "u8", nnz=2000)
    d = G.dev_layer(lay)
    x_np = _x(3, 12, 2048, "f32")
    xd = G.dev_x(x_np, "f32")
    y = G.run(lay, d, xd, bias=False, sidecar=False)
    Y, B = G.oracle_fwd(lay, x_np, "f32", bias=False, sidecar=False)
    G.check(y, Y, B, G.TOL_FP32, "no bias, no sidecar")
    a = G.run(lay, d, xd)
    for _ in range(3):
        assert t.equal(a, G.run(lay, d, xd))


def test_gemv_mfma_constant_index_bit_exact():
    # idx == j, C[j] = 0.375, integer x: every product and partial sum is exact
    N, K, M = 300, 2048, 11
    lay = gen.random_layer(93, N, K, "u8")
    lay.codebook[17] = 0.375
    lay.indices[:] = 17
    lay.bias = (np.arange(N) % 7 - 3).astype(np.float32) / 4
    rng = np.random.Generator(np.random.PCG64(4))
    x_np = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    y = G.run(lay, G.dev_layer(lay), G.dev_x(x_np, "f32"), sidecar=False).cpu().numpy()
    want = (np.float32(0.375) * x_np.sum(1, dtype=np.float64)[:, None] + lay.bias[None, :]).astype(np.float32)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("M", [17, 24, 32, 33, 40, 64])
@pytest.mark.parametrize("N,K", [(300, 2048), (2048, 4096 + 64), (8512, 2048)])
def test_gemv_mfma_token_groups(fmt, M, N, K):
    # two and four 16-token groups per launch (teams of four and two waves,
    # 256- and 128-deep slices), ragged last group, fp32 x
    G.say("gemv mfma groups %s M=%d N=%d K=%d" % (fmt, M, N, K))
    den = 1000 if fmt == "u8" else 2000
    lay = gen.random_layer(N + K + 3 * M, N, K, fmt, nnz=max(1, N * K // den), duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(2 * M + K, M, K, "f32")
    y = G.run(lay, d, G.dev_x(x_np, "f32"))
    Y, B = G.oracle_fwd(lay, x_np, "f32")
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma %s M=%d" % (fmt, M))


@pytest.mark.parametrize("fmt,x_dtype", [("u8", "f32"), ("pk12", "f32"), ("pk12", "bf16")])
@pytest.mark.parametrize("M", [65, 130, 200])
def test_gemv_mfma_chunks_past_64(fmt, x_dtype, M):
    # launches of 64 tokens on offset x and y rows, ragged last launch
    G.say("gemv mfma chunks %s %s M=%d" % (fmt, x_dtype, M))
    N, K = 700, 1024
    lay = gen.random_layer(M + 7, N, K, fmt, nnz=N * K // 500, duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(M + 8, M, K, x_dtype)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype), variant=hx.HXQ_VARIANT_GEMV_MFMA)
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma chunks %s M=%d" % (fmt, M))


def test_gemv_mfma_dense_sidecar_token_groups():
    # several epilogue passes (128 and 64 triplets each) with 32 and 64 staged tokens
    lay = gen.random_layer(94, 40, 1024, "u8", nnz=40 * 1024 // 8, duplicates=True)
    d = G.dev_layer(lay)
    for M in (20, 64):
        x_np = _x(M, M, 1024, "f32")
        y = G.run(lay, d, G.dev_x(x_np, "f32"))
        Y, B = G.oracle_fwd(lay, x_np, "f32")
        G.check(y, Y, B, G.TOL_FP32, "gemv mfma dense sidecar M=%d" % M)


def test_gemv_mfma_token_groups_constant_index_bit_exact():
    N, K = 300, 4096
    lay = gen.random_layer(95, N, K, "u8")
    lay.codebook[5] = 0.375
    lay.indices[:] = 5
    lay.bias = (np.arange(N) % 5 - 2).astype(np.float32) / 8
    rng = np.random.Generator(np.random.PCG64(6))
    for M in (29, 64, 97):
        x_np = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
        y = G.run(lay, G.dev_layer(lay), G.dev_x(x_np, "f32"), sidecar=False).cpu().numpy()
        want = (np.float32(0.375) * x_np.sum(1, dtype=np.float64)[:, None] + lay.bias[None, :]).astype(np.float32)
        assert np.array_equal(y, want), M


@pytest.mark.parametrize("fmt,x_dtype", [("u8", "f32"), ("u8", "bf16"), ("pk12", "f32")])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 70])
def test_gemv_mfma_forced(fmt, x_dtype, M):
    # the kernel forced where the automatic choice takes another one (up to
    # four tokens, and bf16 x past 16 tokens for u8)
    G.say("gemv mfma forced %s %s M=%d" % (fmt, x_dtype, M))
    N, K = 1000, 2048
    lay = gen.random_layer(M + 50, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(M + 51, M, K, x_dtype)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype), variant=hx.HXQ_VARIANT_GEMV_MFMA)
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma forced %s M=%d" % (fmt, M))
