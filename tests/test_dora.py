"""DoRA norm of the adapted weight: norm[j] = || W[:, j] + alpha (A B)[:, j] ||_2.

Oracle pins (CPU): the oracle's dense double-precision definition against
* numpy.linalg.norm of the dense W + alpha A B (a library routine on the
  definition);
* B = 0: the column norms of W; W = 0 with orthonormal A: |alpha| ||B[:, j]||;
* the page's factored identity (base + 2 alpha cross + alpha^2 Gram term with
  U = W^T A and G = A^T A), computed separately in numpy.

GPU parity (through the C ABI): element by element against the oracle,
|got - ref| <= 1e-4 ref + 1e-6.  The library sums fp32 squares of exact bf16
products added in fp32; over k = 8192 terms the accumulated rounding is a few
1e-6 relative, well inside the bound.  Cases span ragged row and column tiles
(k, n not multiples of 32 or 256), ranks that are not multiples of 8 (the
element-wise A reads), every rank-step count (r up to 32, 64, 128, 256), a
single row, and the page's 8192 x 8192 shapes on sampled columns.
"""
import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as lf
import oracle
from parity import bf16_randn, log

REL = 1e-4
ABS = 1e-6


def rand_case(k, n, r, seed):
    g = torch.Generator().manual_seed(seed)
    W = bf16_randn((k, n), (1.0 / k) ** 0.5, g)
    A = bf16_randn((k, r), (1.0 / k) ** 0.5, g)
    B = bf16_randn((r, n), 0.02 ** 0.5, g)
    return W, A, B


def f64(t):
    return t.to(torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float64)


# ---- oracle pins ---------------------------------------------------------------

@pytest.mark.parametrize("k,n,r,alpha", [(64, 40, 8, 2.0), (37, 24, 5, -0.7), (128, 16, 32, 4.0)])
def test_oracle_matches_dense_numpy(k, n, r, alpha):
    W, A, B = rand_case(k, n, r, seed=k + n + r)
    ref = np.linalg.norm(f64(W) + alpha * f64(A) @ f64(B), axis=0)
    got = oracle.dora_norm(f64(W), f64(A), f64(B), alpha)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)


def test_oracle_special_cases():
    W, A, B = rand_case(48, 24, 6, seed=3)
    got = oracle.dora_norm(f64(W), f64(A), np.zeros(f64(B).shape), 3.0)
    np.testing.assert_allclose(got, np.linalg.norm(f64(W), axis=0), rtol=1e-14)
    q, _ = np.linalg.qr(np.random.default_rng(0).standard_normal((48, 6)))
    got = oracle.dora_norm(np.zeros((48, 24)), q, f64(B), -2.5)
    np.testing.assert_allclose(got, 2.5 * np.linalg.norm(f64(B), axis=0), rtol=1e-12)
    # sampled columns are those of the full result
    full = oracle.dora_norm(f64(W), f64(A), f64(B), 1.5)
    np.testing.assert_array_equal(oracle.dora_norm(f64(W), f64(A), f64(B), 1.5, cols=[5, 0, 23]),
                                  full[[5, 0, 23]])


def test_oracle_matches_factored_identity():
    # ||w + a A b||^2 = ||w||^2 + 2a <w, A b> + a^2 b^T (A^T A) b, per column
    W, A, B = rand_case(96, 32, 12, seed=5)
    w, a, b, alpha = f64(W), f64(A), f64(B), 0.8
    U = w.T @ a                      # n x r
    G = a.T @ a                      # r x r
    sq = (w * w).sum(0) + 2 * alpha * (b.T * U).sum(1) + alpha ** 2 * ((b.T @ G) * b.T).sum(1)
    np.testing.assert_allclose(oracle.dora_norm(w, a, b, alpha), np.sqrt(sq), rtol=1e-12)


# ---- library (host) ----------------------------------------------------------------

def test_workspace_size():
    assert lf.lora_dora_norm_workspace_size(8192, 8192, 16) > 0
    assert lf.lora_dora_norm_workspace_size(0, 8192, 16) == 0


# ---- GPU parity ----------------------------------------------------------------------

def check_norm(got, ref, name):
    got = got.to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"{name}: column {worst}: {got[worst]!r} vs {ref[worst]!r}"
    return float((err / np.maximum(np.abs(ref), 1e-30)).max())


DORA_CASES = [
    # k, n, r, alpha
    (264, 264, 16, 2.0),      # ragged sub-block and column tile
    (1000, 520, 36, -1.5),    # rank not a multiple of 8: element-wise A reads
    (4096, 4096, 16, 2.0),
    (777, 1032, 64, 0.5),
    (512, 264, 100, 3.0),     # three rank steps of 32 in a four-step build
    (300, 512, 256, 1.0),
    (1, 8, 3, 2.0),           # a single row, one 8-column group
    (4104, 256, 8, 2.0),      # several row splits, the last one ragged
    # above rank 128 (eight waves, one half of each sub-block per wave)
    (520, 776, 129, 2.0),     # the first such rank: element-wise A reads
    (1000, 1032, 203, -0.7),  # ragged sub-block and column tile, element-wise A reads
    (8200, 264, 160, 1.5),    # 33 row splits, the last one 8 rows
    (5, 264, 256, 1.0),       # one sub-block of 5 rows (both halves partly empty)
    (40, 8, 250, -2.0),       # one 8-column group, element-wise A reads
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(DORA_CASES)))
def test_dora_parity(case):
    k, n, r, alpha = DORA_CASES[case]
    log(f"dora case {case}: k={k} n={n} r={r} alpha={alpha}")
    W, A, B = rand_case(k, n, r, seed=500 + case)
    got = lf.lora_dora_norm(W.cuda(), A.cuda(), B.cuda(), alpha)
    torch.cuda.synchronize()
    ref = oracle.dora_norm(f64(W), f64(A), f64(B), alpha)
    rel = check_norm(got, ref, f"norm k={k} n={n} r={r}")
    log(f"  max rel err {rel:.2e}")


@pytest.mark.gpu
def test_dora_large_alpha_dominated():
    # the low-rank term dominates (B large): no cancellation issue in the direct form
    k, n, r = 512, 256, 16
    W, A, B = rand_case(k, n, r, seed=9)
    B = (B.float() * 50).bfloat16()
    got = lf.lora_dora_norm(W.cuda(), A.cuda(), B.cuda(), -3.0)
    check_norm(got, oracle.dora_norm(f64(W), f64(A), f64(B), -3.0), "alpha-dominated")


@pytest.mark.gpu
@pytest.mark.parametrize("r", [32, 200])
def test_dora_deterministic(r):
    W, A, B = rand_case(2048, 1024, r, seed=11)
    W, A, B = W.cuda(), A.cuda(), B.cuda()
    a = lf.lora_dora_norm(W, A, B, 2.0)
    b = lf.lora_dora_norm(W, A, B, 2.0)
    assert torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("r", [16, 256])
def test_dora_full_size_sampled(r):
    # the page's shape: 8192 x 8192; 48 sampled columns (first, last, random)
    k = n = 8192
    log(f"dora full size r={r}")
    g = torch.Generator(device="cuda").manual_seed(21 + r)
    W = (torch.randn(k, n, device="cuda", generator=g) / k ** 0.5).bfloat16()
    A = (torch.randn(k, r, device="cuda", generator=g) / k ** 0.5).bfloat16()
    B = (torch.randn(r, n, device="cuda", generator=g) * 0.02 ** 0.5).bfloat16()
    got = lf.lora_dora_norm(W, A, B, 2.0)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([[0, 255, 256, n - 1], np.random.default_rng(r).integers(0, n, 44)]))
    ref = oracle.dora_norm(f64(W.cpu()), f64(A.cpu()), f64(B.cpu()), 2.0, cols=cols)
    check_norm(got.cpu()[torch.as_tensor(cols)], ref, f"full size r={r}")
