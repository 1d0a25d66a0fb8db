"""Plain fp64 CPU oracle of the HelixLinear forward pass and of its product
with the transposed weight (the gradient with respect to the input).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module; the GPU
library and its Python binding never do, and this module imports neither.

What it computes.  The model cards ("Zamba2-1.2B-HXQ", "Mamba2-1.3B-HXQ",
"Qwen2.5-3B-Instruct-HXQ", section "What is HelixCode?") describe a layer
stored as a float32 codebook, an index matrix and optional sidecar corrections,
whose module computes ``codebook[indices] @ x`` for any ``nn.Linear``.  The HXQ
whitepaper (Fellows, Echo Labs, 2026), "Method", adds the sidecar as sparse
(row, col, delta) corrections of the weights with the largest reconstruction
error and the 2D variant whose 4096-entry codebook holds pairs of adjacent
weights with 12-bit indices packed two per 3 bytes; its inference paragraph
describes the forward as gather + sidecar + matmul.  The exact result is
therefore a dense product with the dequantised weight, and the oracle is that
definition written out:

    W = C[idx] (+ sidecar deltas, duplicates summed)     (N x K, fp64)
    Y = X @ W^T + bias                                   (M x N, fp64)
    B = |X| @ |W|^T                                      (tolerance scale)

The model cards ("Good to Know") keep the compressed weights frozen while
LoRA adapters train through each HelixLinear (via HelixLinearSTE).  Training
through a frozen layer needs the gradient of its output with respect to its
input, which for y = x W^T + b is the product with the untransposed weight:

    dX = dY @ W                                          (M x K, fp64)
    B  = |dY| @ |W|                                      (tolerance scale)

Readings of points the pages leave open (each also listed in the design notes):
  * orientation: W has nn.Linear's layout [out N, in K]; y = x W^T + b;
  * the sidecar is additive, W = C[idx] + delta, duplicate coordinates sum;
  * 2D pairs run along K: weights (2j, 2j+1) of a row share index j and take
    components 0 and 1 of the codebook pair;
  * 12-bit layout: triplet t of a row holds indices (a, b) = (2t, 2t+1) as the
    little-endian 24-bit word v = a | b << 12; a row has 3*ceil(K/4) bytes;
  * bf16 activations are given as bit patterns and upcast exactly;
  * the input gradient uses the same dequantised W, sidecar included (the
    weights are frozen, so no gradient flows to codebook, indices or deltas).

Pins (tests marked "not gpu"): brute-force fsum products on tiny non-square
inputs with repeated sidecar coordinates, the constant-index closed form, the
empty-sidecar difference, exhaustive 12-bit round trip and printed golden
bytes, one-hot column reconstruction, the u8/pk12 cross-format special case,
and bf16 rounding against the library cast.  The input gradient is pinned by
its own brute force, a hand-computed example, the constant-index closed form,
one-hot rows, and the adjoint identity sum(dY * (Y - b)) = sum(dX * X) that
ties it to the pinned forward.  The tolerance scales (error_bound,
error_bound_bwd and the bound of hxq_sidecar_add) are pinned by their own
fsum brute force on square and non-square shapes and by a hand-worked example
with exact values.  No function here is unpinned.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "unpack_u8",
    "unpack_pk12",
    "bf16_bits_to_f64",
    "bf16_round_f32",
    "activations_f64",
    "dequant_u8",
    "dequant_pk12",
    "apply_sidecar",
    "linear_forward",
    "error_bound",
    "hxq_linear_fwd_u8",
    "hxq_linear_fwd_pk12",
    "hxq_sidecar_add",
    "linear_backward_x",
    "error_bound_bwd",
    "hxq_linear_bwd_x_u8",
    "hxq_linear_bwd_x_pk12",
    "max_err_ratio",
]


# --------------------------------------------------------------- unpacking

def unpack_u8(indices: np.ndarray) -> np.ndarray:
    """One uint8 index per weight (model cards, "What is HelixCode?": uint8
    index matrix into a 256-entry codebook)."""
    return np.asarray(indices, dtype=np.uint8).astype(np.int64)


def unpack_pk12(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """12-bit indices from 3-byte groups (HXQ whitepaper, "Method", 12-bit
    index packing).  Returns [N, K/2] indices; index j of a row covers weights
    2j and 2j+1.  Byte layout: v = b0 | b1 << 8 | b2 << 16, first index
    v & 0xFFF, second v >> 12."""
    if K % 2:
        raise ValueError("pk12 rows hold pairs: K must be even")
    T = (K + 3) // 4
    p = np.asarray(packed, dtype=np.uint8).reshape(N, T, 3).astype(np.int64)
    v = p[:, :, 0] | (p[:, :, 1] << 8) | (p[:, :, 2] << 16)
    idx = np.empty((N, 2 * T), dtype=np.int64)
    idx[:, 0::2] = v & 0xFFF
    idx[:, 1::2] = v >> 12
    return idx[:, : K // 2]


# -------------------------------------------------------------- activations

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """A bf16 value is the upper half of an IEEE fp32 pattern; the upcast is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round_f32(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, ties to even (IEEE 754
    roundTiesToEven on the 16 dropped bits); returned as fp32.  NaN stays NaN."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    high = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((high & 1) == 1))
    r = ((high + up.astype(np.uint64)) << 16) & 0xFFFFFFFF
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(np.asarray(v, dtype=np.float32))
    return np.where(nan, np.float32(np.nan), out).astype(np.float32)


def activations_f64(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """x as fp64: fp32 values, or bf16 bit patterns (uint16)."""
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError(x_dtype)


# ------------------------------------------------------------------ dequant

def dequant_u8(codebook: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """W[n, k] = C[idx[n, k]] in fp64 (model cards, "What is HelixCode?")."""
    c = np.asarray(codebook, dtype=np.float32).astype(np.float64)
    if c.shape != (256,):
        raise ValueError("u8 codebook must hold 256 float32 entries")
    return c[idx]


def dequant_pk12(codebook2: np.ndarray, idx2: np.ndarray, K: int) -> np.ndarray:
    """W[n, 2j + s] = C2[idx2[n, j], s] in fp64 (HXQ whitepaper, "2D vector
    quantization": k = 4096 entries in R^2 over pairs of adjacent weights)."""
    c = np.asarray(codebook2, dtype=np.float32).astype(np.float64)
    if c.shape != (4096, 2):
        raise ValueError("pk12 codebook must hold 4096 float32 pairs")
    N = idx2.shape[0]
    return c[idx2].reshape(N, K)


def apply_sidecar(W: np.ndarray, rows, cols, deltas) -> np.ndarray:
    """W + S where S holds the (row, col, delta) triplets (HXQ whitepaper,
    "Method", sidecar outlier correction).  Repeated coordinates add up."""
    out = np.array(W, dtype=np.float64, copy=True)
    r = np.asarray(rows, dtype=np.int64)
    c = np.asarray(cols, dtype=np.int64)
    d = np.asarray(deltas, dtype=np.float32).astype(np.float64)
    if r.size:
        np.add.at(out, (r, c), d)
    return out


# ------------------------------------------------------------------ forward

def linear_forward(W: np.ndarray, X: np.ndarray, bias=None) -> np.ndarray:
    """Y = X @ W^T + bias, fp64 (nn.Linear semantics)."""
    Y = X @ W.T
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return Y


def error_bound(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """B = |X| @ |W|^T, the elementwise scale of the tolerance."""
    return np.abs(X) @ np.abs(W).T


def _rows(X: np.ndarray, m_rows):
    return X if m_rows is None else X[np.asarray(m_rows, dtype=np.int64)]


def hxq_linear_fwd_u8(codebook, indices, rows, cols, deltas, x, x_dtype, bias,
                      m_rows=None, want_bound=True):
    """Oracle of the u8 forward.  Returns (Y, B) for all rows of x, or for the
    rows listed in ``m_rows``."""
    W = apply_sidecar(dequant_u8(codebook, unpack_u8(indices)), rows, cols, deltas)
    X = _rows(activations_f64(x, x_dtype), m_rows)
    Y = linear_forward(W, X, bias)
    return Y, (error_bound(W, X) if want_bound else None)


def hxq_linear_fwd_pk12(codebook2, packed, rows, cols, deltas, x, x_dtype, bias,
                        N, K, m_rows=None, want_bound=True):
    """Oracle of the pk12 forward (2D VQ, 12-bit packed indices)."""
    W = dequant_pk12(codebook2, unpack_pk12(packed, N, K), K)
    W = apply_sidecar(W, rows, cols, deltas)
    X = _rows(activations_f64(x, x_dtype), m_rows)
    Y = linear_forward(W, X, bias)
    return Y, (error_bound(W, X) if want_bound else None)


def hxq_sidecar_add(rows, cols, deltas, x, x_dtype, N):
    """The sparse term alone: Z[m, r] = sum over triplets of delta * x[m, c]
    (the sidecar acting on the activations, W never formed).  Returns (Z, B)
    with B[m, r] = sum over the triplets of row r of |delta| * |x[m, c]|: the
    absolute values of the terms the sum adds, the scale of its rounding error
    (at least |X| @ |S|^T, where repeated coordinates would cancel first)."""
    X = activations_f64(x, x_dtype)
    M = X.shape[0]
    r = np.asarray(rows, dtype=np.int64)
    c = np.asarray(cols, dtype=np.int64)
    d = np.asarray(deltas, dtype=np.float32).astype(np.float64)
    Z = np.zeros((M, N), dtype=np.float64)
    B = np.zeros((M, N), dtype=np.float64)
    for i in range(r.size):
        Z[:, r[i]] += d[i] * X[:, c[i]]
        B[:, r[i]] += abs(d[i]) * np.abs(X[:, c[i]])
    return Z, B


# ------------------------------------------------ product with W (input gradient)

def linear_backward_x(W: np.ndarray, DY: np.ndarray) -> np.ndarray:
    """dX = dY @ W, fp64: the gradient of y = x W^T + b with respect to x, for
    a frozen W (model cards, "Good to Know": LoRA on frozen HelixLinear)."""
    return DY @ W


def error_bound_bwd(W: np.ndarray, DY: np.ndarray) -> np.ndarray:
    """B = |dY| @ |W|, the elementwise scale of the tolerance."""
    return np.abs(DY) @ np.abs(W)


def hxq_linear_bwd_x_u8(codebook, indices, rows, cols, deltas, dy, dy_dtype,
                        m_rows=None, want_bound=True):
    """Oracle of the u8 input gradient.  dy is [M, N] (fp32, or bf16 bit
    patterns); returns (dX, B) for all rows of dy or the rows in ``m_rows``."""
    W = apply_sidecar(dequant_u8(codebook, unpack_u8(indices)), rows, cols, deltas)
    DY = _rows(activations_f64(dy, dy_dtype), m_rows)
    return linear_backward_x(W, DY), (error_bound_bwd(W, DY) if want_bound else None)


def hxq_linear_bwd_x_pk12(codebook2, packed, rows, cols, deltas, dy, dy_dtype,
                          N, K, m_rows=None, want_bound=True):
    """Oracle of the pk12 input gradient (2D VQ, 12-bit packed indices)."""
    W = dequant_pk12(codebook2, unpack_pk12(packed, N, K), K)
    W = apply_sidecar(W, rows, cols, deltas)
    DY = _rows(activations_f64(dy, dy_dtype), m_rows)
    return linear_backward_x(W, DY), (error_bound_bwd(W, DY) if want_bound else None)


def max_err_ratio(y, Y, B) -> float:
    """max |y - Y| / B over the elements (0/0 counts as 0)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - Y)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(err == 0, 0.0, err / B)
    return float(np.max(ratio)) if ratio.size else 0.0
