"""Quantisation-aware training with NVFP4 fake-quant (QAD page, sec. 3.2 and 4.1).

The forward pass runs the tensor through the fake-quantiser (quantise to E2M1 with an E4M3
scale per 16 values and an fp32 tensor scale, then dequantise); the backward pass hands the
incoming gradient straight back (straight-through estimator), clamped to [-clip, clip]
(clip = inf: no clamp). Activation scales follow a moving average of the per-batch tensor
scale. Every step runs in the HIP library; this module only wires it into autograd.
"""
from __future__ import annotations

import torch

from . import nvfp4


class FakeQuantSTE(torch.autograd.Function):
    """y = fakequant(x; S, block bytes); dx = clamp(dy, -clip, clip)."""

    @staticmethod
    def forward(ctx, x, S, scales=None, clip=float("inf")):
        ctx.clip = float(clip)
        return nvfp4.fakequant(x.contiguous(), S, scales)

    @staticmethod
    def backward(ctx, gy):
        return nvfp4.ste_backward(gy.contiguous(), ctx.clip), None, None, None


def fake_quant_ste(x: torch.Tensor, S: torch.Tensor, scales: torch.Tensor | None = None,
                   clip: float = float("inf")) -> torch.Tensor:
    return FakeQuantSTE.apply(x, S, scales, clip)


class NVFP4FakeQuant(torch.nn.Module):
    """Fake-quant layer for activations or weights.

    In training mode the tensor scale of each batch (amax / 2688) is folded into the running
    scale S <- m * S + (1 - m) * S_batch (the first batch sets S); in eval mode the running
    scale is used as is. `selector` picks the block bytes: "max" (amax / 6, the format's
    default, computed inside the fake-quant pass) or "mse" (search over all E4M3 candidates).
    """

    def __init__(self, momentum: float = 0.9, clip: float = float("inf"),
                 selector: str = "max"):
        super().__init__()
        if not 0.0 <= momentum <= 1.0:
            raise ValueError("momentum must lie in [0, 1]")
        if selector not in ("max", "mse"):
            raise ValueError("selector must be 'max' or 'mse'")
        self.momentum, self.clip, self.selector = momentum, clip, selector
        self.register_buffer("scale", torch.ones(1, dtype=torch.float32))
        self.register_buffer("initialised", torch.zeros((), dtype=torch.bool))
        self._started = None  # host copy of `initialised`, read once

    def _load_from_state_dict(self, *args, **kwargs):
        super()._load_from_state_dict(*args, **kwargs)
        self._started = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dim() != 2:
            raise ValueError("expected a 2-D tensor [rows, cols]")
        if self.scale.device != x.device:
            raise ValueError("module buffers and input are on different devices")
        if self.training:
            with torch.no_grad():
                s_batch = nvfp4.global_scale(x.detach().contiguous())
                if self._started is None:
                    self._started = bool(self.initialised)
                # momentum 0 on the first batch: S = fmaf(0, S, 1 * S_batch) = S_batch exactly
                nvfp4.scale_ema(self.scale, s_batch, self.momentum if self._started else 0.0)
                if not self._started:
                    self.initialised.fill_(True)
                    self._started = True
        scales = None
        if self.selector == "mse":
            with torch.no_grad():
                scales = nvfp4.scale_search_mse(x.detach().contiguous(), self.scale)
        return fake_quant_ste(x, self.scale, scales, self.clip)
