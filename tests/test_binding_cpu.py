"""The Python binding refuses host tensors before the library is touched.

The kernels read raw device pointers; a CPU tensor's pointer handed to them
would fault the GPU.  Every entry point of the binding must raise ValueError
for a tensor that is not on a GPU, without calling into libhxq (checked by
replacing the loader with one that fails the test)."""

import pytest
import torch

import vq_compressed_linear_amd as hx
from vq_compressed_linear_amd import _binding as B


@pytest.fixture
def no_lib(monkeypatch):
    def fail():
        raise AssertionError("the library was reached")

    monkeypatch.setattr(B, "lib", fail)


def _layer(N=8, K=16, pk12=False):
    cb = torch.zeros(8192 if pk12 else 256, dtype=torch.float32)
    idx = torch.zeros((N, 3 * ((K + 3) // 4) if pk12 else K), dtype=torch.uint8)
    rows = torch.zeros(2, dtype=torch.int32)
    cols = torch.zeros(2, dtype=torch.int32)
    dl = torch.zeros(2, dtype=torch.float32)
    return cb, idx, rows, cols, dl


def test_forward_u8_rejects_host_tensors(no_lib):
    cb, idx, r, c, d = _layer()
    x = torch.zeros((2, 16), dtype=torch.float32)
    y = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_linear_fwd_u8(cb, idx, r, c, d, x, None, y)


def test_forward_pk12_rejects_host_tensors(no_lib):
    cb, idx, r, c, d = _layer(pk12=True)
    x = torch.zeros((2, 16), dtype=torch.float32)
    y = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_linear_fwd_pk12(cb, idx, r, c, d, x, None, y)


def test_sidecar_add_rejects_host_tensors(no_lib):
    _, _, r, c, d = _layer()
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_sidecar_add(r, c, d, torch.zeros((2, 16)), torch.zeros((2, 8)))


def test_bwd_rejects_host_tensors(no_lib):
    cb, idx, r, c, d = _layer()
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_linear_bwd_x(hx.HXQ_FMT_U8, cb, idx, r, c, d, torch.zeros((2, 8)), torch.zeros((2, 16)), 16)


def test_dequant_rejects_host_tensors(no_lib):
    cb, idx, r, c, d = _layer()
    w = torch.zeros((8, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_dequant_bf16(hx.HXQ_FMT_U8, cb, idx, r, c, d, w)


def test_grouped_rejects_host_tensors(no_lib):
    cb, idx, r, c, d = _layer()
    x = torch.zeros((2, 16), dtype=torch.float32)
    lay = dict(codebook=cb, indices=idx, sc_rows=r, sc_cols=c, sc_deltas=d, bias=None,
               y=torch.zeros((2, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        B.hxq_linear_fwd_grouped(hx.HXQ_FMT_U8, [lay], x)


def test_layer_rejects_host_activations(no_lib):
    from hxq_synth import gen

    lay = gen.config_layers(0)[0]
    m = hx.HelixLinear.from_layer(lay, device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        m(torch.zeros((1, lay.K), dtype=torch.float32))


def test_library_built_from_these_sources():
    if not __import__("os").path.exists(B.LIB_PATH):
        pytest.skip("libhxq.so not built")
    B._lib = None
    handle = B.lib()
    assert handle.hxq_source_digest().decode() == B.source_digest()


def test_stale_library_is_refused(monkeypatch):
    if not __import__("os").path.exists(B.LIB_PATH):
        pytest.skip("libhxq.so not built")
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "source_digest", lambda: "0" * 32)
    with pytest.raises(RuntimeError, match="other sources"):
        B.lib()
