"""GPU parity on seeded random shapes: the fixed cases elsewhere pick each code
path on purpose; these draw m, k, n, ranks, dropout, alpha, segment layouts and
adapter alignment at random (seeded per case, so a failure names a
reproducible case) over the ranges the C ABI accepts at sizes the oracle
finishes in seconds.  Ranks are drawn from the three kernel regimes (1..32 in
one rank block, 33..128 in one pass, 129..256 in rank tiles); segment cuts may
coincide (empty segments) and adapters may be unused or placed off 16-byte
boundaries.  A wide tier draws k and n from 1024..4096 (half of them exactly
2048 or 4096), where the dA pass and, with mixed adapters, the dS/dB pass take
their XCD-aware work orders (a multiple of 8 column tiles of 256).  Same bar as
the other parity tests: the dropout mask bit for bit, every floating-point
output within the tolerance rule of `parity.py`."""
import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as lf
from parity import (assert_bits_equal, bf16_randn, check_close, compare_single, gpu_multi,
                    gpu_single, log, oracle_multi, oracle_single)

pytestmark = pytest.mark.gpu

N_SINGLE = 32
N_MULTI = 24
N_WIDE = 12


def _rank(rng) -> int:
    u = rng.random()
    if u < 0.45:
        return int(rng.integers(1, 33))
    if u < 0.85:
        return int(rng.integers(33, 129))
    return int(rng.integers(129, 257))


def _dims(rng, mmax, wide=False):
    m = int(rng.integers(1, mmax + 1))
    if wide:
        k = int(rng.choice([2048, 4096])) if rng.random() < 0.5 else 8 * int(rng.integers(128, 513))
        n = int(rng.choice([2048, 4096])) if rng.random() < 0.5 else 8 * int(rng.integers(128, 513))
        return m, k, n
    k = 8 * int(rng.integers(1, 129))
    n = 8 * int(rng.integers(1, 129))
    return m, k, n


def single_params(case, wide=False):
    rng = np.random.default_rng((9100 if wide else 5100) + case)
    m, k, n = _dims(rng, 600 if wide else 1500, wide)
    r = _rank(rng)
    alpha = float(rng.choice([0.5, 1.0, 2.0, 4.0]))
    p = float(rng.choice([0.0, 0.05, 0.1, 0.3, 0.7]))
    seed = int(rng.integers(0, 2 ** 31))
    offset = 8 * int(rng.integers(0, 4096))
    return m, k, n, r, alpha, p, seed, offset


def multi_params(case, wide=False):
    rng = np.random.default_rng((9200 if wide else 6100) + case)
    na = int(rng.integers(1, 6))
    ranks = [_rank(rng) for _ in range(na)]
    m, k, n = _dims(rng, 600 if wide else 1500, wide)
    nseg = int(rng.integers(1, 13))
    cuts = sorted(int(c) for c in rng.integers(0, m + 1, size=nseg - 1))
    seg_off = [0] + cuts + [m]
    seg_ad = [int(rng.integers(0, na)) for _ in range(nseg)]
    alphas = [float(rng.choice([0.5, 1.0, 2.0, 4.0])) for _ in range(na)]
    ps = [float(rng.choice([0.0, 0.1, 0.3])) for _ in range(na)]
    unaligned = tuple(a for a in range(na) if rng.random() < 0.25)
    seed = int(rng.integers(0, 2 ** 31))
    offset = 8 * int(rng.integers(0, 4096))
    return m, k, n, ranks, alphas, ps, seg_off, seg_ad, unaligned, seed, offset


def _tensors(m, k, n, ranks, seed):
    g = torch.Generator().manual_seed(seed)
    X = bf16_randn((m, k), 1.0, g)
    W = bf16_randn((k, n), (1.0 / k) ** 0.5, g)
    As = [bf16_randn((k, r), (1.0 / k) ** 0.5, g) for r in ranks]
    Bs = [bf16_randn((r, n), 0.02 ** 0.5, g) for r in ranks]
    dY = bf16_randn((m, n), 1.0, g)
    return X, W, As, Bs, dY


SINGLE_IDS = [(c, False) for c in range(N_SINGLE)] + [(c, True) for c in range(N_WIDE)]
MULTI_IDS = [(c, False) for c in range(N_MULTI)] + [(c, True) for c in range(N_WIDE)]


@pytest.mark.parametrize("case,wide", SINGLE_IDS, ids=[f"{'wide' if w else 'small'}{c}" for c, w in SINGLE_IDS])
def test_random_single(case, wide):
    m, k, n, r, alpha, p, seed, offset = single_params(case, wide)
    log(f"random single {'wide ' if wide else ''}{case}: m={m} k={k} n={n} r={r} alpha={alpha} p={p} "
        f"seed={seed} offset={offset}")
    X, W, As, Bs, dY = _tensors(m, k, n, [r], (7500 if wide else 7000) + case)
    g = gpu_single(X, W, As[0], Bs[0], dY, alpha, p, seed, offset)
    o = oracle_single(X, W, As[0], Bs[0], dY, alpha, p, seed, offset)
    log(f"  {compare_single(g, o, p)}")


@pytest.mark.parametrize("case,wide", MULTI_IDS, ids=[f"{'wide' if w else 'small'}{c}" for c, w in MULTI_IDS])
def test_random_multi(case, wide):
    m, k, n, ranks, alphas, ps, seg_off, seg_ad, unaligned, seed, offset = multi_params(case, wide)
    log(f"random multi {'wide ' if wide else ''}{case}: m={m} k={k} n={n} ranks={ranks} segs={seg_off} "
        f"adapters={seg_ad} unaligned={unaligned} seed={seed} offset={offset}")
    lf.multi_lora_check_segments(seg_off, seg_ad, m, ranks, max(ranks))
    X, W, As, Bs, dY = _tensors(m, k, n, ranks, (8500 if wide else 8000) + case)
    g = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset, unaligned=unaligned)
    o = oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset)
    assert_bits_equal("keep_bits", g["keep"], o["bits"])
    check_close("S", g["S"], o["S"], rel=1e-4)
    check_close("Y", g["Y"], o["Y"])
    check_close("dX", g["dX"], o["dX"])
    for a in range(len(ranks)):
        check_close(f"dA[{a}]", g["dA"][a], o["dA"][a])
        check_close(f"dB[{a}]", g["dB"][a], o["dB"][a])
