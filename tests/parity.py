"""Shared helpers of the GPU parity tests: the tolerance rule, running the HIP
path through the C ABI, and running the oracle on the same inputs.

Tolerance (the spec bar, read for tensors whose entries exceed O(1)):
for every output T,  ||T - T_ref||_F / ||T_ref||_F <= 5e-3  and, element by
element, |T - T_ref| <= 3e-2 * max(1, rms(T_ref)) + 2^-8 * |T_ref|.  The last
term is half a bf16 ulp of the reference value: the output format cannot get
closer than that, and in a large tensor with heavy-tailed rows (a mixed batch
where one adapter has alpha = 4) elements of 16 and more occur, whose rounding
alone is 0.0625.  The dropout mask must match bit for bit.  S is an fp32
output and is held to 1e-4 (relative Frobenius).
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import lora_fine_tuning_amd as lf
import oracle

REL_FRO = 5e-3
ABS_MAX = 3e-2
HALF_ULP_BF16 = 2.0 ** -8


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check_close(name: str, got, ref, rel: float = REL_FRO, absf: float = ABS_MAX) -> dict:
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return {}
    nref = float(np.linalg.norm(ref))
    err = got - ref
    if nref == 0.0:
        assert not np.any(got), f"{name}: expected exact zeros"
        return {"fro": 0.0, "max": 0.0}
    fro = float(np.linalg.norm(err)) / nref
    rms = nref / np.sqrt(ref.size)
    aerr = np.abs(err)
    mx = float(aerr.max())
    bound = absf * max(1.0, rms) + HALF_ULP_BF16 * np.abs(ref)
    worst = int(np.argmax(aerr - bound))
    stats = {"fro": fro, "max": mx, "rms": rms}
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert fro <= rel, f"{name}: relative Frobenius error {fro:.3e} > {rel:.1e} ({stats})"
    assert np.all(aerr <= bound), (
        f"{name}: abs error {aerr.flat[worst]:.3e} at ref {ref.flat[worst]:.4g} > "
        f"{absf}*max(1,{rms:.3g}) + 2^-8*|ref| (flat index {worst})")
    return stats


def bits_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def assert_bits_equal(name: str, got: torch.Tensor, ref: np.ndarray) -> None:
    g = bits_u32(got)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    diff = np.count_nonzero(g != ref)
    assert diff == 0, f"{name}: {diff} of {g.size} mask words differ"


# ----------------------------------------------------------------------------
# HIP path
# ----------------------------------------------------------------------------
def gpu_single(X, W, A, B, dY, alpha, p, seed=0, offset=0, stream=None):
    dev = "cuda"
    Xd, Wd, Ad, Bd, dYd = (t.to(dev) for t in (X, W, A, B, dY))
    Y, S, keep = lf.lora_linear_fwd(Xd, Wd, Ad, Bd, alpha, p, seed, offset, stream=stream)
    dX, dA, dB = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, keep, alpha, p, stream=stream)
    torch.cuda.synchronize()
    return {"Y": Y.cpu(), "S": S.cpu(), "keep": None if keep is None else keep.cpu(),
            "dX": dX.cpu(), "dA": dA.cpu(), "dB": dB.cpu()}


def offset_view(t: torch.Tensor) -> torch.Tensor:
    """The same values on the GPU, one element (2 bytes) past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t.to("cuda"))
    return v


def gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed=0, offset=0, r_max=None, unaligned=()):
    """The mixed-adapter forward and backward on the GPU.  Adapters listed in
    `unaligned` get A, B, dA and dB one element past a 16-byte boundary."""
    dev = "cuda"
    Xd, Wd, dYd = X.to(dev), W.to(dev), dY.to(dev)
    place = lambda a, t: offset_view(t) if a in unaligned else t.to(dev)
    Ad = [place(a, t) for a, t in enumerate(As)]
    Bd = [place(a, t) for a, t in enumerate(Bs)]
    # garbage: outputs must be overwritten
    dAd = [place(a, torch.full(t.shape, 7.0, dtype=t.dtype)) for a, t in enumerate(As)]
    dBd = [place(a, torch.full(t.shape, 7.0, dtype=t.dtype)) for a, t in enumerate(Bs)]
    r_max = r_max or max(a.shape[1] for a in As)
    table = lf.adapter_table(Ad, Bd, alphas, ps, dAd, dBd)
    so = torch.as_tensor(np.asarray(seg_off, dtype=np.int64)).to(dev)
    sa = torch.as_tensor(np.asarray(seg_ad, dtype=np.int32)).to(dev)
    Y, S, keep = lf.multi_lora_linear_fwd(Xd, Wd, table, len(As), so, sa, r_max, seed, offset)
    dX = lf.multi_lora_linear_bwd(dYd, Xd, Wd, table, len(As), so, sa, S, keep, r_max)
    torch.cuda.synchronize()
    return {"Y": Y.cpu(), "S": S.cpu(), "keep": keep.cpu(), "dX": dX.cpu(),
            "dA": [a.cpu() for a in dAd], "dB": [b.cpu() for b in dBd]}


# ----------------------------------------------------------------------------
# Oracle on the same inputs
# ----------------------------------------------------------------------------
def oracle_single(X, W, A, B, dY, alpha, p, seed=0, offset=0):
    Xn, Wn, An, Bn, dYn = (f64(t) for t in (X, W, A, B, dY))
    p32 = np.float32(p)
    fw = oracle.lora_fwd(Xn, Wn, An, Bn, alpha, p32, seed, offset)
    bw = oracle.lora_bwd(dYn, Xn, Wn, An, Bn, alpha, p32, seed, offset)
    return {"Y": fw["Y"], "S": fw["S"], "bits": oracle.pack_bits(fw["keep"]), "dX": bw["dX"],
            "dA": bw["dA"], "dB": bw["dB"]}


def oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed=0, offset=0, r_max=None):
    r_max = r_max or max(a.shape[1] for a in As)
    ads = [{"A": f64(a), "B": f64(b), "alpha": al, "p": np.float32(p)}
           for a, b, al, p in zip(As, Bs, alphas, ps)]
    Xn, Wn, dYn = f64(X), f64(W), f64(dY)
    fw = oracle.multi_lora_fwd(Xn, Wn, ads, seg_off, seg_ad, r_max, seed, offset)
    bw = oracle.multi_lora_bwd(dYn, Xn, Wn, ads, seg_off, seg_ad, r_max, seed, offset)
    return {"Y": fw["Y"], "S": fw["S"], "bits": oracle.pack_bits(fw["keep"]), "dX": bw["dX"],
            "dA": bw["dA"], "dB": bw["dB"]}


def compare_single(g, o, p) -> dict:
    out = {}
    if p != 0.0:
        assert_bits_equal("keep_bits", g["keep"], o["bits"])
    out["S"] = check_close("S", g["S"], o["S"], rel=1e-4)
    for name in ("Y", "dX", "dA", "dB"):
        out[name] = check_close(name, g[name], o[name])
    return out


def bf16_randn(shape, std, gen):
    t = torch.empty(shape, dtype=torch.float32)
    t.normal_(0.0, 1.0, generator=gen)
    return (t * std).to(torch.bfloat16)
