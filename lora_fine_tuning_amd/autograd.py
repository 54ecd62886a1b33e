"""PyTorch autograd glue over the C ABI: the LoRA linear layer as a
torch.autograd.Function and a module holding a frozen weight and one adapter.

The forward saves what the library's backward consumes (X, S and the mask
bits; W, A and B by reference), so the layer drops in where a PEFT-style LoRA
layer sits (juhe.plus blog on LoRAFusion, section 6: the fused kernels plug
into existing LoRA stacks as replacements).  Every step runs in the library;
this file only reshapes tensors and keeps the dropout counter.
"""
from __future__ import annotations

from collections import OrderedDict

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


class _AdapterSet:
    """The device adapter table of one set of adapter tensors, built once and
    reused by every call with the same tensors, scales and dropout ratios.

    The backward writes all gradients of the set into one flat bf16 buffer per
    call; the table's dA / dB pointer slots are set to that buffer's pieces
    by one device-side add (constant piece offsets plus the buffer's base
    address, a kernel argument), so no call after the first copies from host
    memory or waits for the device, and the calls can be captured in a graph.
    Calls that share a set must run in stream order (one stream)."""

    def __init__(self, As, Bs, alphas, ps):
        self.table = _lib.adapter_table(As, Bs, alphas, ps)
        self.k, self.n, ranks = self.table._lora_meta
        self.num = len(As)
        self.r_max = max(ranks)
        self.shapes = [(tuple(a.shape), tuple(b.shape)) for a, b in zip(As, Bs)]
        offs, pos = [], 0
        for sa, sb in self.shapes:
            na, nb = sa[0] * sa[1], sb[0] * sb[1]
            offs.append((pos, pos + (na + 7) // 8 * 8))  # pieces start on 16-byte boundaries
            pos += (na + 7) // 8 * 8 + (nb + 7) // 8 * 8
        self.total = pos
        self.elem_off = offs
        self.byte_off = torch.tensor([[2 * a, 2 * b] for a, b in offs], dtype=torch.int64,
                                     device=self.table.device)

    def gradient_buffers(self):
        flat = torch.empty(max(self.total, 1), dtype=torch.bfloat16, device=self.table.device)
        slots = self.table.view(torch.int64).view(self.num, 6)[:, 2:4]  # dA, dB of each record
        torch.add(self.byte_off, flat.data_ptr(), out=slots)
        dAs, dBs = [], []
        for (oa, ob), (sa, sb) in zip(self.elem_off, self.shapes):
            dAs.append(flat[oa:oa + sa[0] * sa[1]].view(sa))
            dBs.append(flat[ob:ob + sb[0] * sb[1]].view(sb))
        return dAs, dBs


_SETS: "OrderedDict[tuple, _AdapterSet]" = OrderedDict()
_SETS_MAX = 256


def _adapter_set(As, Bs, alphas, ps) -> _AdapterSet:
    # layout is part of the key: a tensor that would fail the checks never hits the cache
    key = (As[0].device,) + tuple((a.data_ptr(), tuple(a.shape), a.dtype, a.is_contiguous(), a.device,
                                   b.data_ptr(), tuple(b.shape), b.dtype, b.is_contiguous(), b.device,
                                   float(al), float(p)) for a, b, al, p in zip(As, Bs, alphas, ps))
    st = _SETS.get(key)
    if st is None:
        st = _SETS[key] = _AdapterSet(As, Bs, alphas, ps)
        while len(_SETS) > _SETS_MAX:
            _SETS.popitem(last=False)
    else:
        _SETS.move_to_end(key)
    return st


class MultiLoraLinearFunction(torch.autograd.Function):
    """Mixed-adapter batch: rows [seg_off[s], seg_off[s+1]) of X (m x k) use
    adapter seg_adapter[s]; the adapters come as A0, B0, A1, B1, ... and each
    gets its gradients summed over its rows (papers.chlience.com notes, section
    5 "FusedMultiLoRA")."""

    @staticmethod
    def forward(ctx, X, W, seg_off, seg_adapter, alphas, ps, seed: int, offset: int, *AB):
        As, Bs = AB[0::2], AB[1::2]
        st = _adapter_set(As, Bs, alphas, ps)
        Y, S, keep = _lib.multi_lora_linear_fwd(X, W, st.table, st.num, seg_off, seg_adapter, st.r_max, seed,
                                                offset)
        ctx.save_for_backward(X, W, seg_off, seg_adapter, S, keep)
        ctx.adapter_set = st
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, W, seg_off, seg_adapter, S, keep = ctx.saved_tensors
        st = ctx.adapter_set
        dAs, dBs = st.gradient_buffers()
        dX = _lib.multi_lora_linear_bwd(dY.contiguous(), X, W, st.table, st.num, seg_off, seg_adapter, S, keep,
                                        st.r_max, want_dX=ctx.needs_input_grad[0])
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
