"""The seeded generator: determinism and the codec choices it states."""

import numpy as np

from hxq_synth import gen


def _nearest_lower(values, cb):
    d = np.abs(values.astype(np.float64)[:, None] - cb.astype(np.float64)[None, :])
    return np.argmin(d, axis=1)  # argmin returns the first (lowest) index on ties


def test_config0_structure():
    lay = gen.config_layers(0)[0]
    assert (lay.N, lay.K, lay.fmt) == (256, 256, "u8")
    assert lay.codebook.dtype == np.float32 and lay.codebook.shape == (256,)
    assert lay.indices.dtype == np.uint8 and lay.indices.shape == (256, 256)
    assert lay.nnz == 65
    pos = lay.rows.astype(np.int64) * lay.K + lay.cols
    assert np.all(np.diff(pos) > 0), "sidecar sorted by (row, col), unique"
    w = gen.draw_weights(0, 0, 256, 256)
    near = _nearest_lower(w.reshape(-1), lay.codebook)
    assert np.array_equal(near, lay.indices.reshape(-1).astype(np.int64))
    r = np.abs(w.astype(np.float64) - lay.codebook[lay.indices].astype(np.float64)).reshape(-1)
    chosen = np.zeros(r.size, bool)
    chosen[pos] = True
    assert r[chosen].min() >= r[~chosen].max()
    assert np.array_equal(lay.deltas, (w.reshape(-1)[pos].astype(np.float64)
                                       - lay.codebook[lay.indices.reshape(-1)[pos]]).astype(np.float32))


def test_kmeans1d_is_a_lloyd_fixed_point_nearly():
    rng = np.random.Generator(np.random.PCG64(3))
    w = (0.02 * rng.standard_normal(50000)).astype(np.float32)
    cb, idx = gen.kmeans1d(w, 256, 10)
    assert np.array_equal(idx, _nearest_lower(w, cb))
    # quantile initialisation keeps the entries ordered
    assert np.all(np.diff(cb.astype(np.float64)) >= 0)


def test_kmeans2d_final_assignment_is_nearest():
    rng = np.random.Generator(np.random.PCG64(4))
    p = (0.02 * rng.standard_normal((3000, 2))).astype(np.float32)
    cb, lab = gen.kmeans2d(p, np.random.Generator(np.random.PCG64(5)), 4096, 3)
    assert cb.shape == (4096, 2) and cb.dtype == np.float32
    d = ((p.astype(np.float64)[:, None, :] - cb.astype(np.float64)[None, :, :]) ** 2).sum(-1)
    best = d.min(axis=1)
    assert np.array_equal(d[np.arange(p.shape[0]), lab], best)


def test_generator_is_deterministic():
    a = gen.random_layer(3, 40, 64, "pk12", nnz=30, duplicates=True)
    b = gen.random_layer(3, 40, 64, "pk12", nnz=30, duplicates=True)
    assert a.sha256() == b.sha256()
    gen._MEM.clear()
    import os
    os.environ["HXQ_SYNTH_CACHE"] = ""
    try:
        x = gen.synth_layer(7, 1, 64, 96, "u8", 1000)
        gen._MEM.clear()
        y = gen.synth_layer(7, 1, 64, 96, "u8", 1000)
    finally:
        del os.environ["HXQ_SYNTH_CACHE"]
    assert x.sha256() == y.sha256()
    assert np.array_equal(gen.synth_x(1, 2, 8, 100)[:3], gen.synth_x(1, 2, 3, 100))


def test_small_pk12_layer():
    lay = gen.synth_layer(9, 0, 24, 40, "pk12", 2000)
    assert lay.indices.shape == (24, 30)
    assert lay.nnz == 24 * 40 // 2000


def test_generator_outputs_match_stored_sha256(monkeypatch):
    """The seeded generator reproduces, byte for byte, the outputs whose
    SHA-256 tests/golden/make_synth_sha256.py stored (u8 and pk12 layers,
    activations, a random parity layer)."""
    import importlib.util
    import os

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    monkeypatch.setenv("HXQ_SYNTH_CACHE", "")
    monkeypatch.setattr(gen, "_MEM", {})
    spec = importlib.util.spec_from_file_location("make_synth_sha256", os.path.join(here, "make_synth_sha256.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want = {}
    with open(os.path.join(here, "synth_sha256.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                label, field, h = line.split()
                want[(label, field)] = h
    got = {(label, field): h for label, field, h in mod.digests()}
    assert got == want
