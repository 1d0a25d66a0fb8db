"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments on the host before anything is launched."""

import ctypes

import pytest

from vq_compressed_linear_amd import _binding as B


@pytest.fixture(scope="module")
def L():
    try:
        return B.lib()
    except RuntimeError as e:  # pragma: no cover - build() runs before the suite
        pytest.fail(str(e))


def test_exports_every_declared_symbol(L):
    names = B.header_symbols()
    assert "hxq_linear_fwd_u8" in names and "hxq_linear_fwd_pk12" in names
    assert "hxq_sidecar_add" in names
    for n in names:
        assert hasattr(L, n), n
        assert n in B.SIGNATURES, "binding lacks a signature for %s" % n


def test_status_strings(L):
    for st in range(-6, 1):
        assert L.hxq_status_str(st)
    assert L.hxq_version() >= 100


FAKE = 0x100000  # a non-null, 16-byte aligned address that is never dereferenced


def fwd(L, fn="hxq_linear_fwd_u8_ex", codebook=FAKE, indices=FAKE, rows=FAKE, cols=FAKE,
        deltas=FAKE, nnz=0, x=FAKE, x_dtype=0, bias=FAKE, y=FAKE, M=1, N=1, K=16, variant=0):
    return getattr(L, fn)(codebook, indices, rows, cols, deltas, nnz, x, x_dtype, bias, y,
                          M, N, K, None, variant)


# Each case must fail validation, so no kernel is ever queued.
BAD = [
    (dict(x_dtype=2), B.HXQ_ERR_DTYPE),
    (dict(x_dtype=-1), B.HXQ_ERR_DTYPE),
    (dict(M=-1), B.HXQ_ERR_SHAPE),
    (dict(N=-5), B.HXQ_ERR_SHAPE),
    (dict(K=-16), B.HXQ_ERR_SHAPE),
    (dict(nnz=-1), B.HXQ_ERR_SHAPE),
    (dict(M=2 ** 31), B.HXQ_ERR_SHAPE),
    (dict(y=None), B.HXQ_ERR_NULL),
    (dict(x=None), B.HXQ_ERR_NULL),
    (dict(indices=None), B.HXQ_ERR_NULL),
    (dict(codebook=None), B.HXQ_ERR_NULL),
    (dict(nnz=3, rows=None), B.HXQ_ERR_NULL),
    (dict(nnz=3, deltas=None), B.HXQ_ERR_NULL),
    (dict(x=FAKE + 2), B.HXQ_ERR_ALIGN),
    (dict(x=FAKE + 1, x_dtype=1), B.HXQ_ERR_ALIGN),
    (dict(y=FAKE + 2), B.HXQ_ERR_ALIGN),
    (dict(bias=FAKE + 1), B.HXQ_ERR_ALIGN),
    (dict(nnz=1, cols=FAKE + 2), B.HXQ_ERR_ALIGN),
    (dict(variant=9), B.HXQ_ERR_UNSUPPORTED),
    (dict(variant=-1), B.HXQ_ERR_UNSUPPORTED),
    # the fp32 matrix-core GEMV needs K % 64 == 0 (checked on the host)
    (dict(variant=B.HXQ_VARIANT_GEMV_MFMA, K=16), B.HXQ_ERR_UNSUPPORTED),
    (dict(variant=B.HXQ_VARIANT_GEMV_MFMA, K=96, M=100), B.HXQ_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,want", BAD)
def test_u8_rejects(L, kw, want):
    assert fwd(L, **kw) == want


@pytest.mark.parametrize("kw,want", BAD)
def test_pk12_rejects(L, kw, want):
    assert fwd(L, fn="hxq_linear_fwd_pk12_ex", **kw) == want


def test_pk12_odd_k(L):
    assert fwd(L, fn="hxq_linear_fwd_pk12_ex", K=7) == B.HXQ_ERR_SHAPE


def test_empty_is_a_no_op(L):
    # M == 0 or N == 0 returns before any launch, NULL pointers allowed
    assert fwd(L, M=0, x=None, y=None, codebook=None, indices=None) == B.HXQ_OK
    assert fwd(L, N=0, x=None, y=None, codebook=None, indices=None) == B.HXQ_OK
    assert fwd(L, fn="hxq_linear_fwd_pk12_ex", M=0, y=None) == B.HXQ_OK
    assert L.hxq_sidecar_add(None, None, None, 0, None, 0, None, 4, 4, 4, None) == B.HXQ_OK


def test_sidecar_add_rejects(L):
    f = L.hxq_sidecar_add
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 3, FAKE, 1, 1, 1, None) == B.HXQ_ERR_DTYPE
    assert f(FAKE, FAKE, FAKE, -1, FAKE, 0, FAKE, 1, 1, 1, None) == B.HXQ_ERR_SHAPE
    assert f(None, FAKE, FAKE, 1, FAKE, 0, FAKE, 1, 1, 1, None) == B.HXQ_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 0, None, 1, 1, 1, None) == B.HXQ_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 1, FAKE + 2, 0, FAKE, 1, 1, 1, None) == B.HXQ_ERR_ALIGN


def test_variant_selection(L):
    sel = L.hxq_select_variant
    # bf16 x with M > 16 goes to the matrix-core GEMM (K % 32 == 0), everything else to a GEMV
    assert sel(0, B.HXQ_BF16, 2048, 11008, 2048) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(0, B.HXQ_BF16, 16, 11008, 2048) != B.HXQ_VARIANT_GEMM_BF16
    assert sel(0, B.HXQ_F32, 64, 8512, 2048) != B.HXQ_VARIANT_GEMM_BF16
    # from 17 to 64 tokens only layers with at least 32 output tiles of 128 x 128 (N > 3968)
    assert sel(0, B.HXQ_BF16, 64, 8512, 2048) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(0, B.HXQ_BF16, 17, 3969, 2048) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(0, B.HXQ_BF16, 64, 3968, 4096) == B.HXQ_VARIANT_GEMV_VALU
    assert sel(0, B.HXQ_BF16, 17, 2048, 4096) == B.HXQ_VARIANT_GEMV_VALU
    assert sel(1, B.HXQ_BF16, 64, 2048, 4096) == B.HXQ_VARIANT_GEMV_VALU
    assert sel(0, B.HXQ_BF16, 65, 2048, 4096) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(1, B.HXQ_BF16, 2048, 11008, 2048) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(1, B.HXQ_BF16, 2048, 11008, 96) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(1, B.HXQ_BF16, 2048, 11008, 80) != B.HXQ_VARIANT_GEMM_BF16
    assert sel(0, B.HXQ_BF16, 2048, 11008, 96) == B.HXQ_VARIANT_GEMM_BF16
    assert sel(1, B.HXQ_F32, 2048, 11008, 2048) != B.HXQ_VARIANT_GEMM_BF16
    # shapes the fast kernels do not take go to the generic kernel
    assert sel(0, B.HXQ_F32, 1, 100, 100) == B.HXQ_VARIANT_GENERIC
    assert sel(1, B.HXQ_F32, 1, 100, 6) == B.HXQ_VARIANT_GENERIC
    assert sel(0, B.HXQ_F32, 1, 100, 0) == B.HXQ_VARIANT_GENERIC
    assert sel(1, B.HXQ_F32, 1, 100, 7) == B.HXQ_ERR_SHAPE
    assert sel(0, 5, 1, 1, 16) == B.HXQ_ERR_DTYPE


def test_ctypes_signatures_match_header():
    # the binding's argument counts follow the header's parameter lists
    import re
    with open(B.HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    for name, (_, args) in B.SIGNATURES.items():
        m = re.search(r"\b%s\s*\(([^)]*)\)" % name, text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), name
    assert ctypes.sizeof(ctypes.c_int64) == 8


def _layers(n, **kw):
    arr = (B.HxqLayer * n)()
    for i in range(n):
        d = dict(codebook=FAKE, indices=FAKE, sc_rows=FAKE, sc_cols=FAKE, sc_deltas=FAKE, nnz=0,
                 bias=FAKE, y=FAKE, N=8)
        d.update(kw if i == n - 1 else {})
        arr[i] = B.HxqLayer(**d)
    return arr


def test_grouped_struct_layout():
    # struct hxq_layer: eight 8-byte fields and N, no padding
    assert ctypes.sizeof(B.HxqLayer) == 9 * 8
    assert B.HxqLayer.N.offset == 64 and B.HxqLayer.nnz.offset == 40


@pytest.mark.parametrize("kw,want", [
    (dict(y=None), B.HXQ_ERR_NULL),
    (dict(indices=None), B.HXQ_ERR_NULL),
    (dict(nnz=2, sc_cols=None), B.HXQ_ERR_NULL),
    (dict(N=-1), B.HXQ_ERR_SHAPE),
    (dict(nnz=-1), B.HXQ_ERR_SHAPE),
    (dict(y=FAKE + 2), B.HXQ_ERR_ALIGN),
    (dict(bias=FAKE + 1), B.HXQ_ERR_ALIGN),
])
def test_grouped_rejects(L, kw, want):
    # the last of three layers is bad: nothing may be launched for the others
    f = L.hxq_linear_fwd_grouped
    assert f(B.HXQ_FMT_U8, _layers(3, **kw), 3, FAKE, B.HXQ_F32, 1, 16, None) == want
    assert f(B.HXQ_FMT_PK12, _layers(3, **kw), 3, FAKE, B.HXQ_F32, 1, 16, None) == want


def test_grouped_rejects_call_arguments(L):
    f = L.hxq_linear_fwd_grouped
    good = _layers(2)
    assert f(2, good, 2, FAKE, B.HXQ_F32, 1, 16, None) == B.HXQ_ERR_SHAPE
    assert f(B.HXQ_FMT_U8, good, 0, FAKE, B.HXQ_F32, 1, 16, None) == B.HXQ_ERR_SHAPE
    assert f(B.HXQ_FMT_U8, _layers(9), 9, FAKE, B.HXQ_F32, 1, 16, None) == B.HXQ_ERR_SHAPE
    assert f(B.HXQ_FMT_U8, None, 1, FAKE, B.HXQ_F32, 1, 16, None) == B.HXQ_ERR_NULL
    assert f(B.HXQ_FMT_U8, good, 2, FAKE, 7, 1, 16, None) == B.HXQ_ERR_DTYPE
    assert f(B.HXQ_FMT_U8, good, 2, FAKE + 2, B.HXQ_F32, 1, 16, None) == B.HXQ_ERR_ALIGN
    assert f(B.HXQ_FMT_PK12, good, 2, FAKE, B.HXQ_F32, 1, 15, None) == B.HXQ_ERR_SHAPE
    assert f(B.HXQ_FMT_U8, good, 2, FAKE, B.HXQ_F32, -1, 16, None) == B.HXQ_ERR_SHAPE
    # M == 0 and all-empty layers launch nothing
    assert f(B.HXQ_FMT_U8, good, 2, FAKE, B.HXQ_F32, 0, 16, None) == B.HXQ_OK
    assert f(B.HXQ_FMT_U8, _layers(2, N=0), 1, FAKE, B.HXQ_F32, 0, 16, None) == B.HXQ_OK


@pytest.mark.parametrize("fn", ["hxq_stream_read", "hxq_stream_read_nt"])
def test_stream_read_rejects(L, fn):
    f = getattr(L, fn)
    assert f(FAKE, 15, FAKE, 8, None) == B.HXQ_ERR_SHAPE
    assert f(FAKE, -16, FAKE, 8, None) == B.HXQ_ERR_SHAPE
    assert f(FAKE, 16, FAKE, 0, None) == B.HXQ_ERR_SHAPE
    assert f(FAKE, 16, FAKE, 7, None) == B.HXQ_ERR_SHAPE  # a word per wave of at least one workgroup
    assert f(None, 16, FAKE, 8, None) == B.HXQ_ERR_NULL
    assert f(FAKE, 16, None, 8, None) == B.HXQ_ERR_NULL
    assert f(FAKE + 4, 16, FAKE, 8, None) == B.HXQ_ERR_ALIGN
    assert f(FAKE, 16, FAKE + 2, 8, None) == B.HXQ_ERR_ALIGN
    assert f(None, 0, None, 8, None) == B.HXQ_OK


def test_dequant_rejects(L):
    f = L.hxq_dequant_bf16
    U8, PK = B.HXQ_FMT_U8, B.HXQ_FMT_PK12

    def call(fmt=U8, cb=FAKE, idx=FAKE, r=FAKE, c=FAKE, d=FAKE, nnz=0, w=FAKE, N=4, K=32):
        return f(fmt, cb, idx, r, c, d, nnz, w, N, K, None)

    assert call(fmt=7) == B.HXQ_ERR_SHAPE
    assert call(N=-1) == B.HXQ_ERR_SHAPE
    assert call(K=-16) == B.HXQ_ERR_SHAPE
    assert call(nnz=-1) == B.HXQ_ERR_SHAPE
    assert call(fmt=PK, K=33) == B.HXQ_ERR_SHAPE
    assert call(w=None) == B.HXQ_ERR_NULL
    assert call(idx=None) == B.HXQ_ERR_NULL
    assert call(nnz=2, r=None) == B.HXQ_ERR_NULL
    assert call(idx=FAKE + 4) == B.HXQ_ERR_ALIGN
    assert call(fmt=PK, idx=FAKE + 2) == B.HXQ_ERR_ALIGN
    assert call(fmt=PK, cb=FAKE + 4) == B.HXQ_ERR_ALIGN
    assert call(w=FAKE + 8) == B.HXQ_ERR_ALIGN
    assert call(K=24) == B.HXQ_ERR_UNSUPPORTED
    # empty weights launch nothing
    assert call(N=0, cb=None, idx=None, w=None) == B.HXQ_OK
    assert call(K=0, cb=None, idx=None, w=None) == B.HXQ_OK


def test_bwd_x_rejects(L):
    f = L.hxq_linear_bwd_x_ex
    U8, PK = B.HXQ_FMT_U8, B.HXQ_FMT_PK12

    def call(fmt=U8, cb=FAKE, idx=FAKE, r=FAKE, c=FAKE, d=FAKE, nnz=0, dy=FAKE, dt=0, dx=FAKE,
             M=2, N=4, K=32, ws=None, wsb=0, variant=0):
        return f(fmt, cb, idx, r, c, d, nnz, dy, dt, dx, M, N, K, ws, wsb, None, variant)

    assert call(fmt=5) == B.HXQ_ERR_SHAPE
    assert call(dt=3) == B.HXQ_ERR_DTYPE
    assert call(M=-1) == B.HXQ_ERR_SHAPE
    assert call(N=-1) == B.HXQ_ERR_SHAPE
    assert call(K=-2) == B.HXQ_ERR_SHAPE
    assert call(nnz=-1) == B.HXQ_ERR_SHAPE
    assert call(K=2 ** 31) == B.HXQ_ERR_SHAPE
    assert call(fmt=PK, K=31) == B.HXQ_ERR_SHAPE
    assert call(variant=B.HXQ_VARIANT_GENERIC) == B.HXQ_ERR_UNSUPPORTED
    assert call(variant=99) == B.HXQ_ERR_UNSUPPORTED
    assert call(dx=None) == B.HXQ_ERR_NULL
    assert call(dy=None) == B.HXQ_ERR_NULL
    assert call(idx=None) == B.HXQ_ERR_NULL
    assert call(cb=None) == B.HXQ_ERR_NULL
    assert call(nnz=3, c=None) == B.HXQ_ERR_NULL
    assert call(dx=FAKE + 2) == B.HXQ_ERR_ALIGN
    assert call(dy=FAKE + 2) == B.HXQ_ERR_ALIGN
    assert call(dy=FAKE + 1, dt=1) == B.HXQ_ERR_ALIGN
    assert call(cb=FAKE + 2) == B.HXQ_ERR_ALIGN
    assert call(nnz=1, d=FAKE + 1) == B.HXQ_ERR_ALIGN
    assert call(ws=FAKE + 2, wsb=64) == B.HXQ_ERR_ALIGN
    assert call(wsb=-1) == B.HXQ_ERR_SHAPE
    # nothing to compute: no launch, no pointer needed
    assert call(M=0, cb=None, idx=None, dy=None, dx=None) == B.HXQ_OK
    assert call(K=0, cb=None, idx=None, dy=None, dx=None) == B.HXQ_OK


def test_bwd_x_workspace_query(L):
    q = L.hxq_linear_bwd_x_workspace
    F32, BF = B.HXQ_F32, B.HXQ_BF16
    assert q(9, F32, 1, 8, 8, 0) == B.HXQ_ERR_SHAPE
    assert q(B.HXQ_FMT_U8, 5, 1, 8, 8, 0) == B.HXQ_ERR_DTYPE
    assert q(B.HXQ_FMT_PK12, F32, 1, 8, 7, 0) == B.HXQ_ERR_SHAPE
    assert q(B.HXQ_FMT_U8, F32, -1, 8, 8, 0) == B.HXQ_ERR_SHAPE
    assert q(B.HXQ_FMT_U8, F32, 1, 8, 8, -1) == B.HXQ_ERR_SHAPE
    assert q(B.HXQ_FMT_U8, F32, 0, 8, 8, 0) == 0
    # the vector path's workspace holds whole [M][K] fp32 partial sums
    for M, N, K in ((1, 11008, 2048), (3, 2048, 11008), (64, 4096, 4096)):
        n = q(B.HXQ_FMT_U8, F32, M, N, K, 0)
        assert n >= 0 and n % (M * K * 4) == 0
    # the matrix-core path also keeps the sidecar bins there
    assert q(B.HXQ_FMT_U8, BF, 256, 2048, 2048, 4096) > q(B.HXQ_FMT_U8, BF, 256, 2048, 2048, 0)


def test_noalloc_bwd_rejects_oversize_before_any_hip_call(L):
    # a call whose workspace would exceed the library's scratch returns
    # HXQ_ERR_SCRATCH after validating its arguments and before touching a
    # device (this container has none); bad arguments still come first
    M, N, K = 512, 65536, 16384
    need = L.hxq_linear_bwd_x_workspace(B.HXQ_FMT_U8, B.HXQ_BF16, M, N, K, N * K // 1000)
    assert need > B.HXQ_SCRATCH_BYTES
    st = L.hxq_linear_bwd_x_noalloc(B.HXQ_FMT_U8, FAKE, FAKE, FAKE, FAKE, FAKE, N * K // 1000, FAKE, B.HXQ_BF16,
                                    FAKE, M, N, K, None)
    assert st == B.HXQ_ERR_SCRATCH
    assert b"scratch" in L.hxq_status_str(B.HXQ_ERR_SCRATCH)
    st = L.hxq_linear_bwd_x_noalloc(B.HXQ_FMT_U8, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 7, FAKE, M, N, K, None)
    assert st == B.HXQ_ERR_DTYPE
    st = L.hxq_linear_bwd_x_noalloc(B.HXQ_FMT_U8, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, B.HXQ_F32, None, M, N, K,
                                    None)
    assert st == B.HXQ_ERR_NULL
    # M == 0 does nothing
    assert L.hxq_linear_bwd_x_noalloc(B.HXQ_FMT_U8, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, B.HXQ_F32, FAKE, 0, N, K,
                                      None) == B.HXQ_OK


def _bwd_layers(specs):
    """hxq_bwd_layer array of (N, nnz) with stand-in pointers (never dereferenced)."""
    arr = (B.HxqBwdLayer * len(specs))()
    for i, (N, nnz) in enumerate(specs):
        arr[i] = B.HxqBwdLayer(FAKE, FAKE, FAKE, FAKE, FAKE, nnz, FAKE, N)
    return arr


def test_bwd_x_grouped_workspace_query(L):
    q = L.hxq_linear_bwd_x_grouped_workspace
    F32, BF, U8 = B.HXQ_F32, B.HXQ_BF16, B.HXQ_FMT_U8
    two = _bwd_layers([(2048, 10), (256, 3)])
    assert q(9, F32, two, 2, 1, 2048) == B.HXQ_ERR_SHAPE
    assert q(U8, 5, two, 2, 1, 2048) == B.HXQ_ERR_DTYPE
    assert q(U8, F32, two, 0, 1, 2048) == B.HXQ_ERR_SHAPE
    assert q(U8, F32, two, B.HXQ_MAX_GROUP + 1, 1, 2048) == B.HXQ_ERR_SHAPE
    assert q(U8, F32, None, 2, 1, 2048) == B.HXQ_ERR_NULL
    assert q(B.HXQ_FMT_PK12, F32, two, 2, 1, 2047) == B.HXQ_ERR_SHAPE
    assert q(U8, F32, _bwd_layers([(-1, 0), (8, 0)]), 2, 1, 64) == B.HXQ_ERR_SHAPE
    assert q(U8, F32, two, 2, 0, 2048) == 0
    assert q(U8, F32, _bwd_layers([(0, 0), (0, 0)]), 2, 4, 64) == 0
    # one layer with rows: what the single-layer call asks for
    for M, dt in ((1, F32), (256, BF)):
        assert q(U8, dt, _bwd_layers([(0, 0), (2048, 40)]), 2, M, 2048) == \
            L.hxq_linear_bwd_x_workspace(U8, dt, M, 2048, 2048, 40)
    # vector path: one partial sum of [M][K] fp32 per run of rows, at least one per layer
    for M in (1, 3, 8):
        n = q(U8, F32, _bwd_layers([(2048, 10), (256, 3), (256, 3)]), 3, M, 2048)
        assert n >= 3 * M * 2048 * 4 and n % (M * 2048 * 4) == 0
    # matrix-core path: the sidecar bins come on top of the partial sums
    assert q(U8, BF, _bwd_layers([(2048, 4096), (256, 400)]), 2, 256, 2048) > \
        q(U8, BF, _bwd_layers([(2048, 0), (256, 0)]), 2, 256, 2048)


def test_bwd_x_grouped_rejects_before_any_hip_call(L):
    g = L.hxq_linear_bwd_x_grouped
    F32, U8 = B.HXQ_F32, B.HXQ_FMT_U8
    two = _bwd_layers([(300, 5), (200, 5)])
    M, K = 2, 1024
    assert g(9, two, 2, F32, FAKE, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_SHAPE
    assert g(U8, two, 0, F32, FAKE, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_SHAPE
    assert g(U8, None, 2, F32, FAKE, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_NULL
    assert g(U8, two, 2, 7, FAKE, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_DTYPE
    assert g(U8, two, 2, F32, None, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_NULL
    assert g(U8, two, 2, F32, FAKE, M, K, FAKE + 8, 1 << 20, None) == B.HXQ_ERR_ALIGN
    assert g(U8, _bwd_layers([(300, 5), (-2, 0)]), 2, F32, FAKE, M, K, FAKE, 1 << 20, None) == B.HXQ_ERR_SHAPE
    # too little workspace for two layers: refused, nothing launched
    need = L.hxq_linear_bwd_x_grouped_workspace(U8, F32, two, 2, M, K)
    assert need > 0
    assert g(U8, two, 2, F32, FAKE, M, K, FAKE, need - 256, None) == B.HXQ_ERR_UNSUPPORTED
    assert g(U8, two, 2, F32, FAKE, M, K, None, 0, None) == B.HXQ_ERR_UNSUPPORTED
    # nothing to compute
    assert g(U8, two, 2, F32, FAKE, 0, K, None, 0, None) == B.HXQ_OK


def test_fwd_workspace_query(L):
    q = L.hxq_linear_fwd_workspace
    U8, PK, BF, F32 = B.HXQ_FMT_U8, B.HXQ_FMT_PK12, B.HXQ_BF16, B.HXQ_F32
    assert q(9, BF, 1, 8, 8) == B.HXQ_ERR_SHAPE
    assert q(U8, 5, 1, 8, 8) == B.HXQ_ERR_DTYPE
    assert q(U8, BF, -1, 8, 8) == B.HXQ_ERR_SHAPE
    assert q(PK, BF, 8, 8, 7) == B.HXQ_ERR_SHAPE
    assert q(U8, BF, 0, 8, 8) == 0
    # the down projection at 512 and 2048 tokens splits its k (whole [M][N] fp32 partial sums)
    for M in (512, 2048):
        n = q(U8, BF, M, 2048, 11008)
        assert n >= 2 * M * 2048 * 4 and n % (M * 2048 * 4) == 0
    # no split: fp32 x, enough output tiles, short K, or too few tokens for the GEMM
    assert q(U8, F32, 2048, 2048, 11008) == 0
    assert q(U8, BF, 2048, 11008, 2048) == 0
    assert q(U8, BF, 2048, 2048, 2048) == 0
    assert q(U8, BF, 17, 2048, 11008) == 0


def test_fwd_ws_rejects_before_any_hip_call(L):
    f = L.hxq_linear_fwd_ws
    U8, BF = B.HXQ_FMT_U8, B.HXQ_BF16
    args = lambda **k: (k.get("fmt", U8), FAKE, FAKE, None, None, None, 0, FAKE, BF, None, FAKE, 4, 64, 64,
                        k.get("ws", None), k.get("wsb", 0), None)
    assert f(*args(fmt=7)) == B.HXQ_ERR_SHAPE
    assert f(*args(wsb=-1)) == B.HXQ_ERR_SHAPE
    assert f(*args(ws=FAKE + 4, wsb=64)) == B.HXQ_ERR_ALIGN
    assert f(U8, FAKE, FAKE, None, None, None, 0, FAKE, 9, None, FAKE, 4, 64, 64, None, 0, None) == B.HXQ_ERR_DTYPE
    assert f(U8, FAKE, FAKE, None, None, None, 0, FAKE, BF, None, None, 4, 64, 64, None, 0, None) == B.HXQ_ERR_NULL
    assert f(U8, FAKE, FAKE, None, None, None, 0, FAKE, BF, None, FAKE, 0, 64, 64, None, 0, None) == B.HXQ_OK


def test_bwd_x_grouped_total_rows_limit(L):
    # the layers' rows are split as one range: their total must fit int32
    big = _bwd_layers([(2**31 - 2**17, 0), (2**17, 0)])
    assert L.hxq_linear_bwd_x_grouped_workspace(B.HXQ_FMT_U8, B.HXQ_F32, big, 2, 1, 64) == B.HXQ_ERR_SHAPE
    assert L.hxq_linear_bwd_x_grouped(B.HXQ_FMT_U8, big, 2, B.HXQ_F32, FAKE, 1, 64, FAKE, 1 << 20,
                                      None) == B.HXQ_ERR_SHAPE
