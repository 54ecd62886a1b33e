"""Seeded synthetic inputs for the LoRA linear layer workloads.

This module only draws random tensors and segment tables; it holds none of the
layer's arithmetic, and both the oracle-side tests and the HIP-side tests and
benchmark take their inputs from here.

Recipe (stand-in for the pages' LLaMA-3.1 projection shapes and summarisation
datasets, which are not available here):

* values come from a torch CPU generator seeded ``1000 + config_id`` (plus 100
  per shape variant), drawn as float32 in the fixed order X, W, then A_a and
  B_a for each adapter, then dY; each is scaled by its standard deviation and
  rounded to bf16 (round-to-nearest-even);
* X ~ N(0, 1), W ~ N(0, 1/k), A ~ N(0, 1/k), B ~ N(0, 0.02) (the second
  argument read as a variance), dY ~ N(0, 1);
* segment tables come from ``numpy.random.Generator(PCG64(2000 + config_id))``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


@dataclass
class AdapterSpec:
    r: int
    alpha: float
    p: float


@dataclass
class Workload:
    name: str
    config_id: int
    variant: int
    m: int
    k: int
    n: int
    adapters: List[AdapterSpec]
    seg_off: Optional[np.ndarray] = None  # int64 [S+1]; None = single adapter
    seg_adapter: Optional[np.ndarray] = None  # int32 [S]
    seed: int = 0
    offset: int = 0
    notes: str = ""

    @property
    def multi(self) -> bool:
        return self.seg_off is not None

    @property
    def r_max(self) -> int:
        return max(a.r for a in self.adapters)


def lognormal_packed_segments(rng: np.random.Generator, total: int, median: float, sigma: float,
                              lo: int, hi: int, num_adapters: int):
    """Sample lengths ~ lognormal(ln median, sigma) clipped to [lo, hi] until
    their sum reaches `total`; the last sample is cut so the sum is exact.
    Each sample draws its adapter uniformly.  Segments stay in draw order."""
    lengths, adapters = [], []
    acc = 0
    while acc < total:
        L = int(round(float(np.exp(rng.normal(math.log(median), sigma)))))
        L = max(lo, min(hi, L))
        L = min(L, total - acc)
        lengths.append(L)
        adapters.append(int(rng.integers(0, num_adapters)))
        acc += L
    seg_off = np.zeros(len(lengths) + 1, dtype=np.int64)
    seg_off[1:] = np.cumsum(lengths)
    return seg_off, np.asarray(adapters, dtype=np.int32)


def dirichlet_segments(rng: np.random.Generator, total: int, parts: int):
    """Split `total` rows into `parts` segments with Dirichlet(1,...,1)
    proportions and largest-remainder rounding (zero lengths allowed)."""
    w = rng.dirichlet(np.ones(parts))
    raw = w * total
    base = np.floor(raw).astype(np.int64)
    rem = total - int(base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:rem]] += 1
    seg_off = np.zeros(parts + 1, dtype=np.int64)
    seg_off[1:] = np.cumsum(base)
    return seg_off, np.arange(parts, dtype=np.int32)


def workload(config_id: int, variant: int = 0, *, m: Optional[int] = None,
             r: Optional[int] = None) -> Workload:
    """The five workloads, made concrete.

    0: m 512, k = n 1024, r 16, alpha 2, p 0.1.
    1: m 8192, k 4096 -> n 4096 (variant 0) or n 14336 (variant 1), r 16.
    2: 4 adapters (r 16; alpha 1,2,2,4; p 0, .05, .1, .1), k = n 8192, 16384
       tokens packed from lognormal lengths (median 900, sigma 0.75, clipped
       128..4096), adapter uniform per sample.
    3: k = n 4096, r in {8..128}, m in {2048, 8192, 32768}, p 0.1 (sweep; the
       variant indexes r, `m` chooses the token count).
    4: k 28672 -> n 8192, m 8192, 8 adapters r {8,16,16,32,32,64,64,128} in 8
       Dirichlet(1) segments, alpha 2, p 0.1.
    """
    if config_id == 0:
        return Workload("small m512 k1024 n1024 r16", 0, 0, m or 512, 1024, 1024,
                        [AdapterSpec(r or 16, 2.0, 0.1)])
    if config_id == 1:
        n = 4096 if variant == 0 else 14336
        return Workload(f"llama8b-proj m8192 k4096 n{n} r16", 1, variant, m or 8192, 4096, n,
                        [AdapterSpec(r or 16, 2.0, 0.1)])
    if config_id == 2:
        rng = np.random.Generator(np.random.PCG64(2000 + config_id))
        total = m or 16384
        seg_off, seg_ad = lognormal_packed_segments(rng, total, 900.0, 0.75, 128, 4096, 4)
        ads = [AdapterSpec(16, 1.0, 0.0), AdapterSpec(16, 2.0, 0.05),
               AdapterSpec(16, 2.0, 0.1), AdapterSpec(16, 4.0, 0.1)]
        return Workload(f"multi4 packed m{total} k8192 n8192 r16", 2, 0, total, 8192, 8192, ads,
                        seg_off, seg_ad)
    if config_id == 3:
        ranks = [8, 16, 32, 64, 128]
        rr = r or ranks[variant]
        mm = m or 8192
        return Workload(f"sweep m{mm} k4096 n4096 r{rr}", 3, variant, mm, 4096, 4096,
                        [AdapterSpec(rr, 2.0, 0.1)])
    if config_id == 4:
        rng = np.random.Generator(np.random.PCG64(2000 + config_id))
        total = m or 8192
        seg_off, seg_ad = dirichlet_segments(rng, total, 8)
        ads = [AdapterSpec(rk, 2.0, 0.1) for rk in (8, 16, 16, 32, 32, 64, 64, 128)]
        return Workload(f"multi8 down-proj m{total} k28672 n8192 r8..128", 4, 0, total, 28672, 8192, ads,
                        seg_off, seg_ad)
    raise ValueError(f"unknown config {config_id}")


# the seven LoRA projections of one LLaMA-8B-shaped decoder layer: name, k, n
DECODER_PROJECTIONS = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
                       ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]


def decoder_projection(index: int, m: int = 8192, r: int = 16) -> Workload:
    """Projection `index` of DECODER_PROJECTIONS as a single-adapter workload
    (alpha 2, p 0.1), drawn with variant 10 + index of config 1's seeds."""
    nm, kk, nn = DECODER_PROJECTIONS[index]
    return Workload(f"{nm} m{m} k{kk} n{nn} r{r}", 1, 10 + index, m, kk, nn, [AdapterSpec(r, 2.0, 0.1)])


def wide_mixed_workload(m: int = 8192) -> Workload:
    """Four adapters r {8, 200, 13, 128} (alpha 2, 1, 0.5, 2; p 0.1, 0.1, 0.2,
    0) over k = n 4096 in 6 Dirichlet(1) segments that use the adapters in the
    order 0 1 2 3 1 2: a batch whose widest adapter exceeds 128 ranks next to
    one whose rank is not a multiple of 8."""
    rng = np.random.Generator(np.random.PCG64(2105))
    seg_off, _ = dirichlet_segments(rng, m, 6)
    ads = [AdapterSpec(8, 2.0, 0.1), AdapterSpec(200, 1.0, 0.1), AdapterSpec(13, 0.5, 0.2),
           AdapterSpec(128, 2.0, 0.0)]
    return Workload(f"mixed wide m{m} k4096 n4096 r8,200,13,128", 3, 50, m, 4096, 4096, ads, seg_off,
                    np.array([0, 1, 2, 3, 1, 2], dtype=np.int32))


def _bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def make_tensors(w: Workload, device: str = "cpu", *, with_dy: bool = True,
                 seed_override: Optional[int] = None) -> dict:
    """Draw X, W, A_a, B_a, dY for workload `w` (bf16, on `device`).

    The draw always happens on the CPU generator (so the values do not depend on
    the device) and the tensors are then moved."""
    seed = seed_override if seed_override is not None else 1000 + w.config_id + 100 * w.variant
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)

    def normal(shape, var):
        t = torch.empty(shape, dtype=torch.float32)
        t.normal_(0.0, 1.0, generator=g)
        return _bf16(t * math.sqrt(var))

    X = normal((w.m, w.k), 1.0)
    W = normal((w.k, w.n), 1.0 / w.k)
    As, Bs = [], []
    for ad in w.adapters:
        As.append(normal((w.k, ad.r), 1.0 / w.k))
        Bs.append(normal((ad.r, w.n), 0.02))
    dY = normal((w.m, w.n), 1.0) if with_dy else None
    out = {"X": X, "W": W, "A": As, "B": Bs, "dY": dY}
    if device != "cpu":
        for key in ("X", "W", "dY"):
            if out[key] is not None:
                out[key] = out[key].to(device)
        out["A"] = [a.to(device) for a in As]
        out["B"] = [b.to(device) for b in Bs]
    return out


def make_tensors_device(w: Workload, device: str, seed: int = 0) -> dict:
    """Same distributions drawn directly on the device (fast, for timing only;
    values differ from `make_tensors`)."""
    g = torch.Generator(device=device)
    g.manual_seed(1000 + w.config_id + 100 * w.variant + seed)

    def normal(shape, var):
        t = torch.empty(shape, dtype=torch.float32, device=device)
        t.normal_(0.0, 1.0, generator=g)
        return _bf16(t * math.sqrt(var))

    X = normal((w.m, w.k), 1.0)
    W = normal((w.k, w.n), 1.0 / w.k)
    As = [normal((w.k, ad.r), 1.0 / w.k) for ad in w.adapters]
    Bs = [normal((ad.r, w.n), 0.02) for ad in w.adapters]
    dY = normal((w.m, w.n), 1.0)
    return {"X": X, "W": W, "A": As, "B": Bs, "dY": dY}
