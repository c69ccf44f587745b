"""Drop-in replacement for a bf16 nn.Linear: weights quantized once per
output channel, activations per token on every call, fused int8 GEMM with
the dequant + bias epilogue."""
from __future__ import annotations

import torch

from . import ops


class W8A8Linear(torch.nn.Module):
    def __init__(self, wq: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None):
        super().__init__()
        self.register_buffer("wq", wq)
        self.register_buffer("w_scale", w_scale)
        self.register_buffer("bias", bias)
        self.out_features, self.in_features = wq.shape

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear) -> "W8A8Linear":
        w = lin.weight.detach().to(torch.bfloat16).contiguous()
        wq, ws = ops.quantize_weight(w)
        b = None if lin.bias is None else lin.bias.detach().to(torch.bfloat16).contiguous()
        return cls(wq, ws, b)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if x2.dtype != torch.bfloat16:
            raise TypeError("W8A8Linear expects bf16 activations")
        x2 = x2.contiguous()
        xq, xs = ops.quantize_act(x2)
        y = ops.linear(xq, xs, self.wq, self.w_scale, self.bias)
        return y.reshape(*lead, self.out_features)
