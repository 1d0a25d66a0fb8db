"""The forward with a workspace (hxq_linear_fwd_ws): layers whose 256 x 256
output tiles are too few to fill the GPU split their sum over k into runs,
each run's partial sums in the workspace, added into y in run order.  Checked
element by element against the oracle within the bf16 tolerance: the
Qwen2.5-3B down projection at 512 and 2048 tokens (sampled token rows at
2048), both formats, a ragged last output tile, sidecars on the patch path,
on the walk path (more triplets than a tile's patch area: its terms added by
the first run only) and mixed, K far past the patch bins of one launch (each
run takes its own stages' patches), repeat determinism; and that calls which
do not split, or get too little workspace, give exactly the plain forward.
"""

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


def _fmtc(fmt):
    return hx.HXQ_FMT_U8 if fmt == "u8" else hx.HXQ_FMT_PK12


def _x(seed, M, K):
    rng = np.random.Generator(np.random.PCG64(seed))
    return gen.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))


def _run_ws(lay, d, xd, workspace=None, sidecar=True):
    t = G.torch()
    M = xd.shape[0]
    y = t.full((M, lay.N), float("nan"), dtype=t.float32, device="cuda")
    r, c, dl = (d["rows"], d["cols"], d["deltas"]) if sidecar else (None, None, None)
    hx.hxq_linear_fwd_ws(_fmtc(lay.fmt), d["codebook"], d["indices"], r, c, dl, xd, d["bias"], y, lay.K,
                         workspace=workspace)
    return y


def _need(lay, M):
    return hx.lib().hxq_linear_fwd_workspace(_fmtc(lay.fmt), hx.HXQ_BF16, M, lay.N, lay.K)


CASES = [
    # (fmt, N, K, M, nnz): split launches
    ("u8", 2048, 11008, 512, 2048 * 11008 // 1000),
    ("pk12", 2048, 11008, 512, 2048 * 11008 // 2000),
    ("u8", 300, 4096, 200, 300 * 4096 // 1000),     # ragged last output tile, two runs
    ("u8", 64, 4096, 150, 8192),                    # walk path (past the patch area)
    ("u8", 300, 4096, 200, 12000),                  # patch path in some tiles, walk in others
    ("u8", 96, 33024, 130, 3000),                   # K past one launch's patch bins
    ("pk12", 96, 33024, 130, 3000),
]


@pytest.mark.parametrize("fmt,N,K,M,nnz", CASES)
def test_fwd_ws_split_matches_oracle(fmt, N, K, M, nnz):
    G.say("fwd_ws %s N=%d K=%d M=%d nnz=%d" % (fmt, N, K, M, nnz))
    lay = gen.random_layer(N + K + M, N, K, fmt, nnz=nnz, duplicates=True)
    assert _need(lay, M) > 0, "this shape is meant to split"
    d = G.dev_layer(lay)
    x_np = _x(M + 1, M, K)
    y = _run_ws(lay, d, G.dev_x(x_np, "bf16"))
    Y, B = G.oracle_fwd(lay, x_np, "bf16")
    G.check(y, Y, B, G.TOL_BF16, "fwd_ws %s N=%d K=%d M=%d" % (fmt, N, K, M))


def test_fwd_ws_down_2048_tokens_sampled():
    # the prefill step's down launch: four runs of 86 stages; one token row
    # in every 128-token block and 64 more compared, all outputs
    N, K, M = 2048, 11008, 2048
    lay = gen.random_layer(31, N, K, "u8", nnz=N * K // 1000, duplicates=True)
    d = G.dev_layer(lay)
    x_np = _x(32, M, K)
    y = _run_ws(lay, d, G.dev_x(x_np, "bf16"))
    rows = G.tile_rows(M)
    Y, B = G.oracle_fwd(lay, x_np, "bf16", m_rows=rows)
    G.check(y, Y, B, G.TOL_BF16, "fwd_ws down M=2048", m_rows=rows)


def test_fwd_ws_repeats_bitwise():
    t = G.torch()
    lay = gen.random_layer(33, 2048, 11008, "u8", nnz=2048 * 11008 // 1000, duplicates=True)
    d = G.dev_layer(lay)
    xd = G.dev_x(_x(34, 512, 11008), "bf16")
    a = _run_ws(lay, d, xd)
    b = _run_ws(lay, d, xd)
    assert t.equal(a, b)


@pytest.mark.parametrize("fmt,N,K,M", [("u8", 2048, 2048, 2048), ("u8", 700, 1024, 8), ("pk12", 11008, 2048, 2048),
                                       ("u8", 2048, 11008, 17)])
def test_fwd_ws_without_split_is_the_plain_forward(fmt, N, K, M):
    # shapes that do not split: bitwise the plain forward
    t = G.torch()
    lay = gen.random_layer(35 + N, N, K, fmt, nnz=N * K // 1000)
    assert _need(lay, M) == 0
    d = G.dev_layer(lay)
    xd = G.dev_x(_x(36, M, K), "bf16")
    assert t.equal(_run_ws(lay, d, xd), G.run(lay, d, xd))


def test_fwd_ws_too_little_workspace_is_the_plain_forward():
    t = G.torch()
    lay = gen.random_layer(37, 2048, 11008, "u8", nnz=2048 * 11008 // 1000)
    d = G.dev_layer(lay)
    xd = G.dev_x(_x(38, 512, 11008), "bf16")
    small = t.empty(int(_need(lay, 512)) - 256, dtype=t.uint8, device="cuda")
    assert t.equal(_run_ws(lay, d, xd, workspace=small), G.run(lay, d, xd))
