"""Seeded generator for HelixLinear layers and activations.

Every array is drawn from
``np.random.Generator(PCG64(SeedSequence([20260403, cfg, layer, stream])))``
with ``stream`` 0 = weights, 1 = outlier positions, 2 = bias, 3 = activations,
4 = 2D k-means initialisation.

Codec steps follow the HXQ whitepaper (Fellows, Echo Labs, 2026), "Method":
per-tensor k-means (k = 256 scalar, k = 4096 over pairs), nearest-entry index
assignment, sidecar (row, col, delta) triplets for the weights with the largest
reconstruction error, and 12-bit packing of index pairs into 3 bytes.  Where the
pages leave a detail open (initialisation, iteration count, the threshold, the
byte order) this module takes one fixed choice:

* 1D k-means: quantile initialisation ``c_j = sorted(W)[floor((j + 1/2) NK / 256)]``,
  10 Lloyd iterations, nearest entry by the exact 1D midpoint rule with ties to
  the lower entry index, cluster means in fp64 rounded to fp32, an empty
  cluster keeps its entry, final indices re-assigned against the final codebook.
* 2D k-means: 4096 distinct pair positions drawn without replacement as the
  initial entries, 10 Lloyd iterations with exact Euclidean nearest-entry
  assignment (KD-tree, fp64 distances), same mean/empty rules, final
  re-assignment.  Pairs are (W[n, 2j], W[n, 2j+1]) along the input dimension.
* Sidecar: the floor(f N K) positions with the largest |W - C[idx]| (ties to the
  lower row-major position), delta = fp32(W - C[idx]), stored sorted by
  (row, col), rows and cols int32.
* 12-bit packing, per row: index pair (a, b) -> v = a | b << 12 -> bytes
  (v & 0xFF, (v >> 8) & 0xFF, v >> 16); a row of K weights has K/2 indices and
  3 * ceil(K/4) bytes, an odd trailing index is paired with a zero pad.

Weights W = fp32(0.02 N(0,1)) with floor(0.001 N K) distinct positions scaled
by 10; bias = fp32(0.01 N(0,1)); x = fp32(N(0,1)).
"""

from __future__ import annotations

import hashlib
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

SEED_ROOT = 20260403
STREAM_W, STREAM_OUTLIER, STREAM_BIAS, STREAM_X, STREAM_INIT2D = 0, 1, 2, 3, 4
GEN_VERSION = 1

QWEN_LAYERS = [
    ("q", 2048, 2048),
    ("k", 256, 2048),
    ("v", 256, 2048),
    ("o", 2048, 2048),
    ("gate", 11008, 2048),
    ("up", 11008, 2048),
    ("down", 2048, 11008),
]
MAMBA_LAYERS = [("in_proj", 8512, 2048), ("out_proj", 2048, 4096)]
PK12_LAYERS = [("gate", 11008, 2048), ("down", 2048, 11008)]

# Each config: index format, layer list (name, N out, K in), token counts,
# activation dtypes, sidecar fraction denominator (count = N K // den) and the
# config whose seeds the weights come from.
CONFIGS: Dict[int, dict] = {
    0: dict(workload="single HelixLinear 256x256, 1D VQ u8", fmt="u8",
            layers=[("single", 256, 256)], ms=(1,), xdtypes=("f32",),
            den=1000, wcfg=0),
    1: dict(workload="Qwen2.5-3B-shaped layer set, decode, 1D VQ u8", fmt="u8",
            layers=QWEN_LAYERS, ms=(1, 8), xdtypes=("f32",), den=1000, wcfg=1),
    2: dict(workload="Mamba2-1.3B-shaped projections, small batch, 1D VQ u8",
            fmt="u8", layers=MAMBA_LAYERS, ms=(1, 16, 64),
            xdtypes=("f32", "bf16"), den=1000, wcfg=2),
    3: dict(workload="2D VQ pk12, gate/down shapes", fmt="pk12",
            layers=PK12_LAYERS, ms=(1, 16), xdtypes=("f32",), den=2000,
            wcfg=3),
    4: dict(workload="Qwen2.5-3B-shaped layer set, prefill, 1D VQ u8", fmt="u8",
            layers=QWEN_LAYERS, ms=(512, 2048), xdtypes=("bf16",), den=1000,
            wcfg=1, big_m=25600, big_layers=("gate", "up", "down")),
}


def rng_for(cfg: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg, layer, stream])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Layer:
    """One compressed linear layer as the forward pass consumes it.

    ``codebook``: u8 -> float32 [256]; pk12 -> float32 [4096, 2].
    ``indices``:  u8 -> uint8 [N, K]; pk12 -> uint8 [N, 3*ceil(K/4)] packed.
    ``rows``/``cols``: int32 [nnz], sorted by (row, col); ``deltas`` float32.
    ``bias``: float32 [N].
    """

    name: str
    cfg: int
    layer_id: int
    N: int
    K: int
    fmt: str
    codebook: np.ndarray
    indices: np.ndarray
    rows: np.ndarray
    cols: np.ndarray
    deltas: np.ndarray
    bias: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.rows.size)

    def compressed_bytes(self) -> int:
        return int(self.codebook.nbytes + self.indices.nbytes + self.rows.nbytes
                   + self.cols.nbytes + self.deltas.nbytes)

    def sha256(self) -> Dict[str, str]:
        out = {}
        for k in ("codebook", "indices", "rows", "cols", "deltas", "bias"):
            out[k] = hashlib.sha256(np.ascontiguousarray(getattr(self, k)).tobytes()).hexdigest()
        return out


# ----------------------------------------------------------------- weights

def draw_weights(cfg: int, layer: int, N: int, K: int, outlier_den: int = 1000) -> np.ndarray:
    w = (0.02 * rng_for(cfg, layer, STREAM_W).standard_normal((N, K))).astype(np.float32)
    n_out = (N * K) // outlier_den
    if n_out:
        pos = rng_for(cfg, layer, STREAM_OUTLIER).choice(N * K, size=n_out, replace=False)
        flat = w.reshape(-1)
        flat[pos] = flat[pos] * np.float32(10.0)
    return w


def draw_bias(cfg: int, layer: int, N: int) -> np.ndarray:
    return (0.01 * rng_for(cfg, layer, STREAM_BIAS).standard_normal(N)).astype(np.float32)


def synth_x(cfg: int, layer: int, M: int, K: int) -> np.ndarray:
    """fp32 activations [M, K]; smaller token counts use row prefixes."""
    return rng_for(cfg, layer, STREAM_X).standard_normal((M, K)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ------------------------------------------------------------- 1D k-means

def _assign_ranges_sorted(s: np.ndarray, c: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """For sorted data ``s`` (fp64) return [lo, hi) of the points nearest to each
    entry of ``c``; ties go to the lower entry index."""
    k = c.size
    cv64 = c.astype(np.float64)
    perm = np.lexsort((np.arange(k), cv64))
    cv = cv64[perm]
    keep = np.ones(k, dtype=bool)
    keep[1:] = cv[1:] != cv[:-1]          # equal values: only the lowest index can win
    wid = perm[keep]
    wv = cv[keep]
    lo = np.zeros(k, dtype=np.int64)
    hi = np.zeros(k, dtype=np.int64)
    if wid.size == 1:
        lo[wid[0]], hi[wid[0]] = 0, s.size
        return lo, hi
    mid = (wv[:-1] + wv[1:]) * 0.5
    left_is_lower = wid[:-1] < wid[1:]
    cut = np.where(left_is_lower,
                   np.searchsorted(s, mid, side="right"),
                   np.searchsorted(s, mid, side="left"))
    edges = np.concatenate(([0], cut, [s.size]))
    lo[wid] = edges[:-1]
    hi[wid] = edges[1:]
    return lo, hi


def kmeans1d(w: np.ndarray, k: int = 256, iters: int = 10) -> Tuple[np.ndarray, np.ndarray]:
    """Scalar k-means over the values of ``w``; returns (codebook fp32 [k], indices [w.size])."""
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = flat.size
    s = np.sort(flat).astype(np.float64)
    csum = np.concatenate(([0.0], np.cumsum(s)))
    c = s[((2 * np.arange(k) + 1) * n) // (2 * k)].astype(np.float32)
    for _ in range(iters):
        lo, hi = _assign_ranges_sorted(s, c)
        cnt = hi - lo
        nz = cnt > 0
        c = c.copy()
        c[nz] = ((csum[hi[nz]] - csum[lo[nz]]) / cnt[nz]).astype(np.float32)
    return c, _assign_values(flat, c)


def _assign_values(flat: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Nearest entry of ``c`` for every value (ties to the lower entry index)."""
    k = c.size
    cv64 = c.astype(np.float64)
    perm = np.lexsort((np.arange(k), cv64))
    cv = cv64[perm]
    keep = np.ones(k, dtype=bool)
    keep[1:] = cv[1:] != cv[:-1]
    wid = perm[keep]
    wv = cv[keep]
    if wid.size == 1:
        return np.full(flat.size, wid[0], dtype=np.int64)
    mid = (wv[:-1] + wv[1:]) * 0.5
    # "w <= mid goes left" when the left entry has the lower index, else "w < mid";
    # the strict form is the non-strict one against the next fp64 value down.
    mid = np.where(wid[:-1] < wid[1:], mid, np.nextafter(mid, -np.inf))
    return wid[np.searchsorted(mid, flat.astype(np.float64), side="left")]


# ------------------------------------------------------------- 2D k-means

def _nearest2d(p: np.ndarray, c: np.ndarray) -> np.ndarray:
    from scipy.spatial import cKDTree

    tree = cKDTree(c.astype(np.float64))
    _, lab = tree.query(p, k=1, workers=_threads())
    return lab.astype(np.int64)


def kmeans2d(p: np.ndarray, rng: np.random.Generator, k: int = 4096,
             iters: int = 10) -> Tuple[np.ndarray, np.ndarray]:
    """k-means over 2-vectors ``p`` [P, 2] fp32; returns (codebook fp32 [k, 2], labels [P])."""
    P = p.shape[0]
    p64 = p.astype(np.float64)
    take = min(k, P)
    init = rng.choice(P, size=take, replace=False)
    c = np.empty((k, 2), dtype=np.float32)
    c[:take] = p[init]
    if take < k:  # fewer pairs than entries: the spare entries are random pairs
        c[take:] = (0.02 * rng.standard_normal((k - take, 2))).astype(np.float32)
    for _ in range(iters):
        lab = _nearest2d(p64, c)
        cnt = np.bincount(lab, minlength=k)
        s0 = np.bincount(lab, weights=p64[:, 0], minlength=k)
        s1 = np.bincount(lab, weights=p64[:, 1], minlength=k)
        nz = cnt > 0
        c = c.copy()
        c[nz, 0] = (s0[nz] / cnt[nz]).astype(np.float32)
        c[nz, 1] = (s1[nz] / cnt[nz]).astype(np.float32)
    return c, _nearest2d(p64, c)


# ---------------------------------------------------------------- packing

def pack12_rows(idx2: np.ndarray) -> np.ndarray:
    """Pack 12-bit indices [N, P] into bytes [N, 3*ceil(P/2)], pairs along each row."""
    idx2 = np.asarray(idx2)
    if idx2.ndim != 2:
        raise ValueError("idx2 must be 2-D")
    if idx2.size and (idx2.min() < 0 or idx2.max() > 0xFFF):
        raise ValueError("12-bit indices must lie in [0, 4096)")
    N, P = idx2.shape
    T = (P + 1) // 2
    padded = np.zeros((N, 2 * T), dtype=np.uint32)
    padded[:, :P] = idx2
    v = padded[:, 0::2] | (padded[:, 1::2] << 12)
    out = np.empty((N, T, 3), dtype=np.uint8)
    out[:, :, 0] = v & 0xFF
    out[:, :, 1] = (v >> 8) & 0xFF
    out[:, :, 2] = v >> 16
    return out.reshape(N, 3 * T)


# ---------------------------------------------------------------- sidecar

def select_sidecar(w: np.ndarray, wq: np.ndarray, count: int):
    """Largest |w - wq| positions (ties to lower row-major position), sorted by (row, col)."""
    N, K = w.shape
    if count <= 0:
        z = np.zeros(0, dtype=np.int32)
        return z, z.copy(), np.zeros(0, dtype=np.float32)
    r = w.astype(np.float64).reshape(-1) - wq.astype(np.float64).reshape(-1)
    a = np.abs(r)
    kth = a.size - count
    t = np.partition(a, kth)[kth]
    gt = np.flatnonzero(a > t)
    eq = np.flatnonzero(a == t)[: count - gt.size]
    pos = np.sort(np.concatenate((gt, eq)))
    rows = (pos // K).astype(np.int32)
    cols = (pos % K).astype(np.int32)
    return rows, cols, r[pos].astype(np.float32)


# ------------------------------------------------------------------ layers

def _cache_dir() -> Optional[str]:
    d = os.environ.get("HXQ_SYNTH_CACHE", os.path.join("/tmp", "hxq_synth_cache"))
    return d or None


_MEM: Dict[tuple, Layer] = {}


def synth_layer(cfg: int, layer: int, N: int, K: int, fmt: str = "u8",
                den: int = 1000, name: str = "") -> Layer:
    """Compress a freshly drawn N x K weight with the codec described above."""
    if fmt not in ("u8", "pk12"):
        raise ValueError(fmt)
    if fmt == "pk12" and K % 2:
        raise ValueError("pk12 needs an even K")
    key = (GEN_VERSION, cfg, layer, N, K, fmt, den)
    if key in _MEM:
        return _MEM[key]
    fields = ("codebook", "indices", "rows", "cols", "deltas", "bias")
    cdir = _cache_dir()
    path = None
    if cdir:
        path = os.path.join(cdir, "v%d_c%d_l%d_%dx%d_%s_%d.npz" % key)
        if os.path.exists(path):
            try:
                with np.load(path, allow_pickle=False) as z:
                    arrs = {f: z[f] for f in fields}
                lay = Layer(name, cfg, layer, N, K, fmt, **arrs)
                _MEM[key] = lay
                return lay
            except Exception:
                pass
    w = draw_weights(cfg, layer, N, K)
    bias = draw_bias(cfg, layer, N)
    if fmt == "u8":
        cb, idx = kmeans1d(w, 256, 10)
        idx = idx.reshape(N, K)
        wq = cb[idx]
        indices = idx.astype(np.uint8)
    else:
        pairs = w.reshape(N * K // 2, 2)
        cb, lab = kmeans2d(pairs, rng_for(cfg, layer, STREAM_INIT2D), 4096, 10)
        idx2 = lab.reshape(N, K // 2)
        wq = cb[idx2].reshape(N, K)
        indices = pack12_rows(idx2)
    rows, cols, deltas = select_sidecar(w, wq, (N * K) // den)
    lay = Layer(name, cfg, layer, N, K, fmt, cb.astype(np.float32), indices,
                rows, cols, deltas, bias)
    _MEM[key] = lay
    if path:
        try:
            os.makedirs(cdir, exist_ok=True)
            tmp = path + ".%d.tmp.npz" % os.getpid()
            np.savez(tmp, **{f: getattr(lay, f) for f in fields})
            os.replace(tmp, path)
        except OSError:
            pass
    return lay


def config_layers(cfg: int) -> List[Layer]:
    spec = CONFIGS[cfg]
    return [synth_layer(spec["wcfg"], i, N, K, spec["fmt"], spec["den"], name)
            for i, (name, N, K) in enumerate(spec["layers"])]


def random_layer(seed: int, N: int, K: int, fmt: str = "u8", nnz: int = 0,
                 duplicates: bool = False) -> Layer:
    """A layer with a random codebook, uniformly random indices over every
    codebook entry and ``nnz`` random sidecar triplets (sorted; optionally with
    repeated coordinates).  Used for parity cases that must touch every entry."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 99, seed])))
    if fmt == "u8":
        cb = (0.02 * rng.standard_normal(256)).astype(np.float32)
        indices = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    else:
        if K % 2:
            raise ValueError("pk12 needs an even K")
        cb = (0.02 * rng.standard_normal((4096, 2))).astype(np.float32)
        indices = pack12_rows(rng.integers(0, 4096, size=(N, K // 2)))
    if nnz and N * K:
        if duplicates:
            pos = rng.integers(0, N * K, size=nnz)
        else:
            pos = rng.choice(N * K, size=min(nnz, N * K), replace=False)
        pos = np.sort(pos)
        rows = (pos // K).astype(np.int32)
        cols = (pos % K).astype(np.int32)
        deltas = (0.2 * rng.standard_normal(pos.size)).astype(np.float32)
    else:
        rows = np.zeros(0, np.int32)
        cols = np.zeros(0, np.int32)
        deltas = np.zeros(0, np.float32)
    bias = (0.01 * rng.standard_normal(N)).astype(np.float32)
    return Layer("random", -1, seed, N, K, fmt, cb, indices, rows, cols, deltas, bias)
