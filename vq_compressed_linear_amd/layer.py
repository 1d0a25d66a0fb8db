"""HelixLinear: a compressed nn.Linear whose forward runs in libhxq.

The layer keeps the compressed form resident on the GPU (codebook, indices or
packed 12-bit indices, sidecar triplets, bias) and calls the library for every
forward; the dense weight is never built (model cards, "What is HelixCode?").
The weights are frozen (model cards, "Good to Know": LoRA adapters train
through the layer): when x requires a gradient, the backward pass computes
dx = dy W with the library's input-gradient kernels and nothing else.
"""

from __future__ import annotations

from . import _binding as B


class HelixLinear:
    """Device-resident compressed layer of shape [out_features N, in_features K].

    ``fmt`` is "u8" (codebook [256]) or "pk12" (codebook [4096, 2], packed
    indices [N, 3*ceil(K/4)]).  Sidecar arrays are int32 rows/cols and float32
    deltas sorted by (row, col).
    """

    def __init__(self, fmt, codebook, indices, sc_rows, sc_cols, sc_deltas, bias, in_features,
                 device="cuda"):
        import torch

        if fmt not in ("u8", "pk12"):
            raise ValueError(fmt)
        self.fmt = fmt

        def dev(a, dtype):
            if a is None:
                return None
            t = torch.as_tensor(a)
            return t.to(device=device, dtype=dtype).contiguous()

        self.codebook = dev(codebook, torch.float32)
        self.indices = dev(indices, torch.uint8)
        self.sc_rows = dev(sc_rows, torch.int32)
        self.sc_cols = dev(sc_cols, torch.int32)
        self.sc_deltas = dev(sc_deltas, torch.float32)
        self.bias = dev(bias, torch.float32)
        self.out_features = int(self.indices.shape[0])
        self.in_features = int(in_features)

    @classmethod
    def from_layer(cls, layer, device="cuda") -> "HelixLinear":
        """From an object with codebook/indices/rows/cols/deltas/bias/K/fmt attributes."""
        return cls(layer.fmt, layer.codebook, layer.indices, layer.rows, layer.cols, layer.deltas,
                   layer.bias, layer.K, device=device)

    def forward(self, x, out=None, stream=None, variant: int = B.HXQ_VARIANT_AUTO):
        import torch

        if x.requires_grad and torch.is_grad_enabled() and out is None:
            return _helix_fn().apply(x, self)
        return self._forward(x, out, stream, variant)

    def _forward(self, x, out=None, stream=None, variant: int = B.HXQ_VARIANT_AUTO):
        import torch

        if x.shape[-1] != self.in_features:
            raise ValueError("x has %d features, layer expects %d" % (x.shape[-1], self.in_features))
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        y = out if out is not None else torch.empty((x2.shape[0], self.out_features),
                                                    dtype=torch.float32, device=x.device)
        if variant == B.HXQ_VARIANT_AUTO and x2.dtype == torch.bfloat16:
            # bf16 activations: the entry point with a workspace (from torch's
            # caching allocator), which splits the sum over k of layers with
            # too few output tiles to fill the GPU
            fmt = B.HXQ_FMT_U8 if self.fmt == "u8" else B.HXQ_FMT_PK12
            B.hxq_linear_fwd_ws(fmt, self.codebook, self.indices, self.sc_rows, self.sc_cols, self.sc_deltas, x2,
                                self.bias, y, self.in_features, stream=stream)
        else:
            fn = B.hxq_linear_fwd_u8 if self.fmt == "u8" else B.hxq_linear_fwd_pk12
            fn(self.codebook, self.indices, self.sc_rows, self.sc_cols, self.sc_deltas, x2,
               self.bias, y, stream=stream, variant=variant)
        return y.reshape(*lead, self.out_features)

    __call__ = forward

    def backward_input(self, dy, out=None, stream=None, variant: int = B.HXQ_VARIANT_AUTO):
        """dx = dy W (the gradient of the forward's output with respect to x) for
        dy [..., out_features] float32 or bfloat16; dx is float32 [..., in_features]."""
        import torch

        if dy.shape[-1] != self.out_features:
            raise ValueError("dy has %d features, layer has %d outputs" % (dy.shape[-1], self.out_features))
        lead = dy.shape[:-1]
        dy2 = dy.reshape(-1, self.out_features).contiguous()
        dx = out if out is not None else torch.empty((dy2.shape[0], self.in_features), dtype=torch.float32,
                                                     device=dy.device)
        fmt = B.HXQ_FMT_U8 if self.fmt == "u8" else B.HXQ_FMT_PK12
        B.hxq_linear_bwd_x(fmt, self.codebook, self.indices, self.sc_rows, self.sc_cols, self.sc_deltas, dy2, dx,
                           self.in_features, stream=stream, variant=variant)
        return dx.reshape(*lead, self.in_features)

    def compressed_bytes(self) -> int:
        n = 0
        for t in (self.codebook, self.indices, self.sc_rows, self.sc_cols, self.sc_deltas):
            if t is not None:
                n += t.numel() * t.element_size()
        return n

    def extra_repr(self) -> str:  # pragma: no cover - cosmetic
        return "fmt=%s, in=%d, out=%d, nnz=%d" % (
            self.fmt, self.in_features, self.out_features,
            0 if self.sc_rows is None else self.sc_rows.numel())


_FN = None


def _helix_fn():
    """torch.autograd.Function over the library: forward y = x W^T + b, backward
    dx = dy W (no gradient for the frozen compressed weights)."""
    global _FN
    if _FN is None:
        import torch

        class HelixFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x, layer):
                ctx.layer = layer
                ctx.x_dtype = x.dtype
                return layer._forward(x.detach())

            @staticmethod
            def backward(ctx, dy):
                dx = ctx.layer.backward_input(dy.contiguous())
                return dx.to(ctx.x_dtype), None

        _FN = HelixFn
    return _FN
