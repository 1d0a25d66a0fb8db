"""The dense-weight helper behind the buffered comparison design (gather the
bf16 weight into a buffer, then a library matmul): its weight is bit-exact
against the oracle's dequantised weight with the sidecar added in fp32 and
rounded once, and the buffered product matches the oracle within the bf16
tolerance.  Through the C ABI."""

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


def _expected_bits(lay):
    """bf16 bits of C[idx] + the sidecar run at each position, the run's
    deltas added in fp32 in stored order, rounded once to nearest even."""
    if lay.fmt == "u8":
        W = oracle.dequant_u8(lay.codebook, oracle.unpack_u8(lay.indices)).astype(np.float32)
    else:
        W = oracle.dequant_pk12(lay.codebook, oracle.unpack_pk12(lay.indices, lay.N, lay.K), lay.K).astype(np.float32)
    rows, cols, dl = np.asarray(lay.rows), np.asarray(lay.cols), np.asarray(lay.deltas, dtype=np.float32)
    e = 0
    while e < len(rows):
        r, c = int(rows[e]), int(cols[e])
        v = np.float32(W[r, c])
        while e < len(rows) and rows[e] == r and cols[e] == c:
            v = np.float32(v + dl[e])
            e += 1
        W[r, c] = v
    return (oracle.bf16_round_f32(W).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
@pytest.mark.parametrize("N,K,den", [(300, 1024, 200), (2048, 2048, 1000), (5, 16, 4), (97, 4096 + 16, 50)])
def test_dequant_bit_exact(fmt, N, K, den):
    G.say("dequant %s N=%d K=%d" % (fmt, N, K))
    t = G.torch()
    lay = gen.random_layer(N + K + den, N, K, fmt, nnz=max(1, N * K // den), duplicates=True)
    d = G.dev_layer(lay)
    w = t.full((N, K), -1, dtype=t.int16, device="cuda")
    hx.hxq_dequant_bf16(hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12, d["codebook"], d["indices"],
                        d["rows"], d["cols"], d["deltas"], w)
    got = w.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _expected_bits(lay))


@pytest.mark.parametrize("fmt", ["u8", "pk12"])
def test_buffered_product_matches_oracle(fmt):
    # the comparison design end to end: bf16 weight, then a library matmul
    # (fp32 accumulation here), then the bias
    t = G.torch()
    N, K, M = 700, 2048, 130
    lay = gen.random_layer(77, N, K, fmt, nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    w = t.empty((N, K), dtype=t.bfloat16, device="cuda")
    hx.hxq_dequant_bf16(hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12, d["codebook"], d["indices"],
                        d["rows"], d["cols"], d["deltas"], w)
    rng = np.random.Generator(np.random.PCG64(78))
    x_np = gen.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    xd = G.dev_x(x_np, "bf16")
    y = (xd.float() @ w.float().t().contiguous()) + d["bias"]
    Y, B = G.oracle_fwd(lay, x_np, "bf16")
    G.check(y, Y, B, G.TOL_BF16, "buffered %s" % fmt)
