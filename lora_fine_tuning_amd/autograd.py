"""PyTorch autograd glue over the C ABI: the LoRA linear layer as a
torch.autograd.Function and a module holding a frozen weight and one adapter.

The forward saves what the library's backward consumes (X, S and the mask
bits; W, A and B by reference), so the layer drops in where a PEFT-style LoRA
layer sits (juhe.plus blog on LoRAFusion, section 6: the fused kernels plug
into existing LoRA stacks as replacements).  Every step runs in the library;
this file only reshapes tensors and keeps the dropout counter.
"""
from __future__ import annotations

import torch

from . import _lib


class LoraLinearFunction(torch.autograd.Function):
    """Y = X W + alpha * (dropout(X) A) B for X (..., k) bf16; W k x n is frozen
    (no gradient); A k x r and B r x n receive gradients."""

    @staticmethod
    def forward(ctx, X, W, A, B, alpha: float, p: float, seed: int, offset: int):
        lead = X.shape[:-1]
        X2 = X.reshape(-1, X.shape[-1]).contiguous()
        Y, S, keep = _lib.lora_linear_fwd(X2, W, A, B, alpha, p, seed, offset)
        ctx.save_for_backward(X2, W, A, B, S, keep if keep is not None else torch.empty(0, device=X.device))
        ctx.alpha, ctx.p, ctx.lead, ctx.has_keep = alpha, p, lead, keep is not None
        return Y.reshape(*lead, W.shape[1])

    @staticmethod
    def backward(ctx, dY):
        X2, W, A, B, S, keep = ctx.saved_tensors
        dY2 = dY.reshape(-1, dY.shape[-1]).contiguous()
        want_dX = ctx.needs_input_grad[0]
        dX, dA, dB = _lib.lora_linear_bwd(dY2, X2, W, A, B, S, keep if ctx.has_keep else None,
                                          ctx.alpha, ctx.p, want_dX=want_dX)
        dX = dX.reshape(*ctx.lead, W.shape[0]) if want_dX else None
        return dX, None, dA, dB, None, None, None, None


def lora_linear(X, W, A, B, alpha: float, p: float = 0.0, seed: int = 0, offset: int = 0):
    return LoraLinearFunction.apply(X, W, A, B, alpha, p, seed, offset)


class MultiLoraLinearFunction(torch.autograd.Function):
    """Mixed-adapter batch: rows [seg_off[s], seg_off[s+1]) of X (m x k) use
    adapter seg_adapter[s]; the adapters come as A0, B0, A1, B1, ... and each
    gets its gradients summed over its rows (papers.chlience.com notes, section
    5 "FusedMultiLoRA")."""

    @staticmethod
    def forward(ctx, X, W, seg_off, seg_adapter, alphas, ps, seed: int, offset: int, *AB):
        As, Bs = AB[0::2], AB[1::2]
        r_max = max(a.shape[1] for a in As)
        table = _lib.adapter_table(As, Bs, alphas, ps)
        Y, S, keep = _lib.multi_lora_linear_fwd(X, W, table, len(As), seg_off, seg_adapter, r_max, seed, offset)
        ctx.save_for_backward(X, W, seg_off, seg_adapter, S, keep, *AB)
        ctx.alphas, ctx.ps, ctx.r_max = list(alphas), list(ps), r_max
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, W, seg_off, seg_adapter, S, keep, *AB = ctx.saved_tensors
        As, Bs = AB[0::2], AB[1::2]
        dAs = [torch.empty_like(a) for a in As]
        dBs = [torch.empty_like(b) for b in Bs]
        table = _lib.adapter_table(As, Bs, ctx.alphas, ctx.ps, dAs, dBs)
        dX = _lib.multi_lora_linear_bwd(dY.contiguous(), X, W, table, len(As), seg_off, seg_adapter, S, keep,
                                        ctx.r_max, want_dX=ctx.needs_input_grad[0])
        grads = []
        for da, db in zip(dAs, dBs):
            grads += [da, db]
        return (dX, None, None, None, None, None, None, None, *grads)


def multi_lora_linear(X, W, seg_off, seg_adapter, As, Bs, alphas, ps, seed: int = 0, offset: int = 0):
    AB = [t for pair in zip(As, Bs) for t in pair]
    return MultiLoraLinearFunction.apply(X, W, seg_off, seg_adapter, list(alphas), list(ps), seed, offset, *AB)


class LoraLinear(torch.nn.Module):
    """A frozen k x n weight with one LoRA adapter (A k x r, B r x n; B starts
    at zero).  Dropout draws from the library's counter-based generator under
    this module's own seed; each training call advances the counter past the
    elements it used, so successive calls get fresh masks and a rerun from the
    same state reproduces them.  In eval mode dropout is off."""

    def __init__(self, weight: torch.Tensor, r: int, alpha: float, p: float = 0.0, seed: int = 0):
        super().__init__()
        k, n = weight.shape
        self.register_buffer("weight", weight.detach().to(torch.bfloat16).contiguous())
        gen = torch.Generator(device="cpu").manual_seed(seed)
        a = torch.randn(k, r, generator=gen) / k ** 0.5
        self.A = torch.nn.Parameter(a.to(device=weight.device, dtype=torch.bfloat16))
        self.B = torch.nn.Parameter(torch.zeros(r, n, device=weight.device, dtype=torch.bfloat16))
        self.alpha, self.p, self.seed = float(alpha), float(p), int(seed)
        self.offset = 0  # next unused dropout counter (a multiple of 8)

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        p = self.p if self.training else 0.0
        offset = self.offset
        if p > 0.0:
            used = X.numel() // X.shape[-1] * X.shape[-1]
            self.offset += (used + 7) // 8 * 8
        return LoraLinearFunction.apply(X, self.weight, self.A, self.B, self.alpha, p, self.seed, offset)
