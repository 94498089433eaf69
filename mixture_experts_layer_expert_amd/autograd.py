"""torch.autograd wrapper of the layer: every step runs in the library's HIP
kernels through the C ABI (binding.py); this module only orders the calls
and hands tensors between them.

Forward:  logits = x W_r (moe_router_fwd) -> top-K routing and sort by expert
          (moe_route_sort) -> y = the routed SwiGLU experts combined with the
          router weights (moe_fwd).
Backward (routing held fixed): moe_bwd gives dX through the experts, the
          expert weight gradients and dL/d(router weights); moe_router_bwd
          turns the latter into dW_r and adds the router path's share of dX.

Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design"
(Forward pass / Backward pass); the router step is the input side of the
same layer.
"""
from __future__ import annotations

import torch

from . import binding as B

ROUTE_KEYS = ("topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted")


class MoEFunction(torch.autograd.Function):
    """y = MoE(x; W_r, W_gate, W_up, W_down) with top-K routing.

    x bf16 [T, D]; w_r fp32 [D, E]; w_gate, w_up bf16 [E, I, D]; w_down bf16
    [E, D, I].  Gradients come back in each input's dtype (the weight
    gradients are accumulated in fp32 by the kernels)."""

    @staticmethod
    def forward(ctx, x, w_r, w_gate, w_up, w_down, K: int, score: int):
        x = x.contiguous()
        logits = B.moe_router_fwd(x, w_r)
        route = B.moe_route_sort(logits, K, score)
        y = B.moe_fwd(x, w_gate, w_up, w_down, route, K, score)
        ctx.save_for_backward(x, w_r, w_gate, w_up, w_down, *(route[k] for k in ROUTE_KEYS))
        ctx.K, ctx.score = K, score
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_r, w_gate, w_up, w_down, *rt = ctx.saved_tensors
        route = dict(zip(ROUTE_KEYS, rt))
        g = B.moe_bwd(x, w_gate, w_up, w_down, route, dy.contiguous().to(torch.bfloat16),
                      ctx.K, ctx.score)
        dw_r = B.moe_router_bwd(x, w_r, route, g["d_topk_w"], g["dx"], ctx.K, ctx.score)
        return (g["dx"], dw_r.to(w_r.dtype), g["dw_gate"].to(w_gate.dtype),
                g["dw_up"].to(w_up.dtype), g["dw_down"].to(w_down.dtype), None, None)


def moe(x, w_r, w_gate, w_up, w_down, K: int, score: int = B.MOE_SCORE_SOFTMAX_TOPK):
    """Functional form of MoEFunction."""
    return MoEFunction.apply(x, w_r, w_gate, w_up, w_down, int(K), int(score))


class MoELayer(torch.nn.Module):
    """The routed SwiGLU MoE layer with its router as module parameters
    (router projection fp32 [D, E]; expert weights bf16 in the linear-layer
    layout [out, in])."""

    def __init__(self, D: int, I: int, E: int, K: int, score: int = B.MOE_SCORE_SOFTMAX_TOPK,
                 device=None, generator=None):
        super().__init__()
        self.K, self.score = int(K), int(score)

        def init(shape, fan_in, dtype):
            t = torch.randn(shape, generator=generator, device="cpu") / fan_in ** 0.5
            return torch.nn.Parameter(t.to(device=device, dtype=dtype))

        self.w_r = init((D, E), D, torch.float32)
        self.w_gate = init((E, I, D), D, torch.bfloat16)
        self.w_up = init((E, I, D), D, torch.bfloat16)
        self.w_down = init((E, D, I), I, torch.bfloat16)

    def forward(self, x):
        return moe(x, self.w_r, self.w_gate, self.w_up, self.w_down, self.K, self.score)
