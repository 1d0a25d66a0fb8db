"""Parity at the five workload configurations, full sizes, through the entry
points the bench times (automatic kernel choice).

  0  single 256 x 256 u8 layer, M = 1, fp32 x
  1  Qwen2.5-3B-shaped u8 layer set, M = 1 and 8, fp32 x
  2  Mamba2-1.3B-shaped u8 projections, M = 1, 16, 64, fp32 and bf16 x
  3  pk12 gate/down shapes, M = 1 and 16, fp32 x
  4  prefill: the config-1 layers at M = 512 and 2048, and gate/up/down at
     M = 25600, bf16 x; checked on 64 random token rows plus one in every
     128-token block and the last of every 256-token block (all N outputs)
"""

import numpy as np
import pytest

import gpu_util as G
import vq_compressed_linear_amd as hx
from hxq_synth import gen

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("needs a GPU")
    hx.lib()
    yield
    t.cuda.synchronize()


def _layer(cfg, i):
    spec = gen.CONFIGS[cfg]
    name, N, K = spec["layers"][i]
    return gen.synth_layer(spec["wcfg"], i, N, K, spec["fmt"], spec["den"], name)


def _run_cfg(cfg, i, Ms, xdt, m_rows_for=None):
    lay = _layer(cfg, i)
    d = G.dev_layer(lay)
    x_full = gen.synth_x(cfg, i, max(Ms), lay.K)
    ratios = {}
    for M in Ms:
        x_np = x_full[:M]
        if xdt == "bf16":
            x_np = gen.to_bf16_bits(x_np)
        G.say("cfg %d layer %s M=%d x=%s" % (cfg, lay.name, M, xdt))
        y = G.run(lay, d, G.dev_x(x_np, xdt))
        rows = m_rows_for(M) if m_rows_for else None
        Y, B = G.oracle_fwd(lay, x_np, xdt, m_rows=rows)
        tol = G.TOL_BF16 if (xdt == "bf16" and M > 16) else G.TOL_FP32
        ratios[M] = G.check(y, Y, B, tol, "cfg%d %s M=%d" % (cfg, lay.name, M), m_rows=rows)
    return ratios


def test_config0():
    r = _run_cfg(0, 0, [1], "f32")
    G.say("config 0 max err/B", r)


@pytest.mark.parametrize("i", range(7))
def test_config1(i):
    G.say("config 1 max err/B", _run_cfg(1, i, [1, 8], "f32"))


@pytest.mark.parametrize("i", range(2))
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_config2(i, xdt):
    G.say("config 2 max err/B", _run_cfg(2, i, [1, 16, 64], xdt))


@pytest.mark.parametrize("i", range(2))
def test_config3(i):
    G.say("config 3 max err/B", _run_cfg(3, i, [1, 16], "f32"))


@pytest.mark.parametrize("i", range(7))
def test_config4(i):
    G.say("config 4 max err/B", _run_cfg(4, i, [512, 2048], "bf16", G.tile_rows))


@pytest.mark.parametrize("i", [4, 5, 6])
def test_config4_50x512(i):
    """gate, up, down at M = 25600 (50 chunks of 512 tokens): every 128-token
    block of the output has a compared row."""
    G.say("config 4 M=25600 max err/B", _run_cfg(4, i, [25600], "bf16", G.tile_rows))
