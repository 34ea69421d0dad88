"""A sparse MoE FFN layer object on one GPU: weights quantised once, workspace kept.

Weights are converted statically ("Hosting Qwen on Blackwell", section "Quantization")
by the library's quantisation kernels, to e4m3 codes with 128x128 block scales or, with
``fmt="mxfp8"``, to MXFP8 (1x32 blocks, E8M0 scales), with ``fmt="mxfp4"`` to MXFP4 (e2m1
codes packed two per byte, 1x32 blocks); ``forward`` runs the whole layer through
``moe_forward`` / ``moe_forward_mx`` / ``moe_forward_mxfp4``.
"""
from __future__ import annotations

from typing import Callable, Optional

import torch

from . import _lib


class MoELayer:
    def __init__(self, router_w: torch.Tensor, router_b: Optional[torch.Tensor], top_k: int,
                 w13: torch.Tensor, w13_scales: torch.Tensor, b13: Optional[torch.Tensor],
                 w2: torch.Tensor, w2_scales: torch.Tensor, b2: Optional[torch.Tensor]):
        self.router_w, self.router_b, self.top_k = router_w, router_b, top_k
        self.w13, self.w13_scales, self.b13 = w13, w13_scales, b13
        self.w2, self.w2_scales, self.b2 = w2, w2_scales, b2
        self.E, self.H = router_w.shape
        self.I = w13.shape[1] * 8 if w13.dim() == 5 else w2.shape[2]   # MXFP4 tiles: 2I/16 rows
        self._ws = {}

    @classmethod
    def from_expert_weights(cls, router_w, router_b, top_k: int, b13, b2,
                            w13_of: Callable[[int], torch.Tensor],
                            w2_of: Callable[[int], torch.Tensor], device="cuda",
                            fmt: str = "block") -> "MoELayer":
        """Quantise expert by expert: ``w13_of(e)`` -> [2I, H] fp32, ``w2_of(e)`` -> [H, I] fp32
        (on any device; moved to ``device`` one expert at a time).  ``fmt``: "block"
        (128x128 block scales), "mxfp8" or "mxfp4" (MXFP4 weights, MXFP8 activations)."""
        E, H = router_w.shape
        first = w2_of(0)
        I = first.shape[1]
        kb = _lib.kb
        if fmt == "mxfp4":
            (c13, t13), (c2, t2) = _lib.mxfp4_shapes(2 * I, H), _lib.mxfp4_shapes(H, I)
            w13 = torch.empty((E,) + c13, dtype=torch.uint8, device=device)
            w2 = torch.empty((E,) + c2, dtype=torch.uint8, device=device)
            s13 = torch.empty((E,) + t13, dtype=torch.uint8, device=device)
            s2 = torch.empty((E,) + t2, dtype=torch.uint8, device=device)
            quant = _lib.quantize_weights_mxfp4
        elif fmt == "mxfp8":
            w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
            w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
            s13 = torch.empty((E,) + _lib.mx_scale_shape(2 * I, H), dtype=torch.uint8, device=device)
            s2 = torch.empty((E,) + _lib.mx_scale_shape(H, I), dtype=torch.uint8, device=device)
            quant = _lib.quantize_weights_mx
        elif fmt == "block":
            w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
            w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
            s13 = torch.empty((E, kb(2 * I), kb(H)), dtype=torch.float32, device=device)
            s2 = torch.empty((E, kb(H), kb(I)), dtype=torch.float32, device=device)
            quant = _lib.quantize_weights
        else:
            raise ValueError(f"unknown weight format {fmt}")
        for e in range(E):
            a = w13_of(e).to(device=device, dtype=torch.float32).contiguous()
            quant(a, w13[e:e + 1], s13[e:e + 1])
            b = (first if e == 0 else w2_of(e)).to(device=device, dtype=torch.float32).contiguous()
            quant(b, w2[e:e + 1], s2[e:e + 1])
        return cls(router_w.to(device), None if router_b is None else router_b.to(device), top_k,
                   w13, s13, None if b13 is None else b13.to(device), w2, s2,
                   None if b2 is None else b2.to(device))

    def workspace(self, T: int) -> torch.Tensor:
        ws = self._ws.get(T)
        if ws is None:
            ws = _lib.new_workspace(T, self.H, self.E, self.top_k, self.I, self.w13.device)
            self._ws[T] = ws
        return ws

    def forward(self, x: torch.Tensor, out: torch.Tensor = None, routing: dict = None,
                fused: bool = False) -> torch.Tensor:
        """The layer on x [T, H] bf16; ``fused``: the decode-sized layer in one persistent
        kernel (moe_forward_fused) instead of the multi-kernel path."""
        fn = _lib.forward_fused if fused else _lib.forward
        return fn(x, self.router_w, self.router_b, self.w13, self.w13_scales, self.b13,
                  self.w2, self.w2_scales, self.b2, self.top_k, out=out, routing=routing,
                  workspace=self.workspace(x.shape[0]))

    __call__ = forward
