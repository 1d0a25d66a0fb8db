"""GPU parity of the 4x4-block matrix-core GEMV (2 to 8 tokens, u8 and pk12,
K % 256 == 0) against the CPU oracle, through the C ABI."""

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


def _case(fmt, x_dtype, M, N, K, seed, nnz_den=1000):
    lay = gen.random_layer(seed, N, K, fmt, nnz=max(1, N * K // nnz_den), duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(seed + 1, M, K, x_dtype)
    y = G.run(lay, d, G.dev_x(x_np, x_dtype))
    Y, B = G.oracle_fwd(lay, x_np, x_dtype)
    G.check(y, Y, B, G.TOL_FP32, "gemv mfma4 %s %s M=%d N=%d K=%d" % (fmt, x_dtype, M, N, K))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(97, 2048), (2048, 11008), (11008, 2048), (1000, 768), (5, 256)])
def test_gemv_mfma4_matches_oracle(fmt, x_dtype, M, N, K):
    # ragged last fragment, one to 43 chunks (waves without chunks at K < 2048),
    # one to six fragment groups per workgroup
    G.say("gemv mfma4 %s %s M=%d N=%d K=%d" % (fmt, x_dtype, M, N, K))
    _case(fmt, x_dtype, M, N, K, seed=N + K + M + (7 if fmt == "pk12" else 0))


@pytest.mark.parametrize("N", [24576, 24580])
@pytest.mark.parametrize("M", [3, 8])
def test_gemv_mfma4_fragment_limit(N, M):
    # 24 fragments per workgroup on 256 CUs fit; four rows more take the 16x16
    # kernel (8 tokens) or the decode kernel (3)
    G.say("gemv mfma4 limit N=%d M=%d" % (N, M))
    _case("u8", "f32", M, N, 256, seed=N + M)


def test_gemv_mfma4_dense_sidecar():
    # 1024 triplets per workgroup: two epilogue passes, repeated coordinates
    G.say("gemv mfma4 dense sidecar")
    for M, xdt in ((5, "f32"), (8, "bf16")):
        _case("u8", xdt, M, 40, 1024, seed=300 + M, nnz_den=4)


def test_gemv_mfma4_constant_index_bit_exact():
    N, K, M = 300, 2048, 7
    lay = gen.random_layer(96, N, K, "u8")
    lay.codebook[9] = 0.375
    lay.indices[:] = 9
    lay.bias = (np.arange(N) % 7 - 3).astype(np.float32) / 4
    rng = np.random.Generator(np.random.PCG64(8))
    x_np = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    y = G.run(lay, G.dev_layer(lay), G.dev_x(x_np, "f32"), sidecar=False).cpu().numpy()
    want = (np.float32(0.375) * x_np.sum(1, dtype=np.float64)[:, None] + lay.bias[None, :]).astype(np.float32)
    assert np.array_equal(y, want)


def test_gemv_mfma4_determinism_and_prefix():
    # bitwise repeatable; the first five token rows of an 8-token call match a
    # 5-token call within tolerance (same kernel, token groups of four)
    t = G.torch()
    lay = gen.random_layer(97, 3000, 2048, "pk12", nnz=3000)
    d = G.dev_layer(lay)
    x_np = _x(11, 8, 2048, "f32")
    xd = G.dev_x(x_np, "f32")
    a = G.run(lay, d, xd)
    for _ in range(3):
        assert t.equal(a, G.run(lay, d, xd))
    y5 = G.run(lay, d, xd[:5].contiguous())
    Y, B = G.oracle_fwd(lay, x_np[:5], "f32")
    G.check(y5, Y, B, G.TOL_FP32, "prefix")
    G.check(a[:5], Y, B, G.TOL_FP32, "prefix of 8")
