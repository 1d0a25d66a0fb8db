"""The allocation-free input gradient (hxq_linear_bwd_x_noalloc) through the
C ABI against the workspace entry point (hxq_linear_bwd_x) and the CPU oracle:
two calls in a row on one GPU, the second with a smaller input (the library's
scratch keeps the first call's contents), both formats, fp32 and bf16 dy."""

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


def _dy(seed, M, N, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    f = rng.standard_normal((M, N)).astype(np.float32)
    return (gen.to_bf16_bits(f), "bf16") if dtype == "bf16" else (f, "f32")


def _case(fmt, N, K, M, dtype, seed):
    lay = gen.random_layer(seed, N, K, fmt, nnz=N * K // 1000 + 3, duplicates=True)
    d = G.dev_layer(lay)
    dy_np, dt = _dy(seed + 1, M, N, dtype)
    dyd = G.dev_x(dy_np, dt)
    t = G.torch()
    dx_na = t.full((M, K), float("nan"), dtype=t.float32, device="cuda")
    dx_ws = t.full((M, K), float("nan"), dtype=t.float32, device="cuda")
    f = hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12
    G.say("noalloc bwd_x %s N=%d K=%d M=%d dy=%s" % (fmt, N, K, M, dtype))
    hx.hxq_linear_bwd_x_noalloc(f, d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], dyd, dx_na, K)
    hx.hxq_linear_bwd_x(f, d["codebook"], d["indices"], d["rows"], d["cols"], d["deltas"], dyd, dx_ws, K)
    t.cuda.synchronize()
    if fmt == "u8":
        DX, BX = oracle.hxq_linear_bwd_x_u8(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, dy_np, dt)
    else:
        DX, BX = oracle.hxq_linear_bwd_x_pk12(lay.codebook, lay.indices, lay.rows, lay.cols, lay.deltas, dy_np, dt,
                                              N, K)
    tol = G.TOL_BF16 if (dtype == "bf16" and M >= 16) else G.TOL_FP32
    G.check(dx_na, DX, BX, tol, "noalloc %s %s" % (fmt, dtype))
    G.check(dx_ws, DX, BX, tol, "workspace %s %s" % (fmt, dtype))
    # the same kernels and splits: the two entry points agree within the tolerance of each other
    a = dx_na.cpu().numpy().astype(np.float64)
    b = dx_ws.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - b) <= 2 * tol * BX)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_two_calls_second_smaller(fmt, dtype):
    # first call: splits and (bf16) sidecar bins fill a large part of the scratch
    _case(fmt, 2048, 2048, 64, dtype, seed=11)
    # second call, smaller, after the first left its partial sums behind
    _case(fmt, 1000, 256, 16, dtype, seed=12)


def test_noalloc_one_token():
    _case("u8", 11008, 2048, 1, "f32", seed=13)
    _case("u8", 2048, 11008, 1, "f32", seed=14)


def test_noalloc_256_tile_kernel():
    # from 128 tokens (u8, bf16 dy) the 256 x 256 tile kernel: row splits and
    # sidecar bins in the scratch, then a smaller call of the same kernel
    _case("u8", 2048, 2048, 256, "bf16", seed=15)
    _case("u8", 512, 1024, 128, "bf16", seed=16)
