"""Pins for the CPU oracle: each check ties it to something other than itself.

* the Philox4x32-10 block function against PyTorch's own header-only
  implementation of the same published generator (compiled here with g++);
* the mask's bit layout against numpy.packbits; its drop rate against the
  binomial law; p = 0 keeps everything; independence of neighbouring bits;
  the counter layout through the row-offset shift;
* the forward against numpy matmul chains in the cases that reduce to one
  (B = 0, A = 0, alpha = 0: Y = XW; p = 0: Y = XW + alpha (XA) B);
* the inverted-dropout scale through E_mask[S] = XA (average over seeds);
* the backward against central finite differences (exact up to rounding,
  since L = <Y, dY> is affine in every single scalar of X, A and B once the
  mask is fixed) and against the Euler identities of a degree-1 map;
* the multi-adapter oracle against single-adapter runs per segment;
* everything against brute-force pure-Python loops on a tiny case.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from synth import workload, make_tensors

TORCH_INCLUDE = None
try:
    import torch  # noqa: F401
    TORCH_INCLUDE = os.path.join(os.path.dirname(torch.__file__), "include")
except Exception:  # pragma: no cover
    pass


def rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Philox4x32-10 against PyTorch's implementation of the same generator
# ---------------------------------------------------------------------------
_ATEN_SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned long long seed, block;
  while (std::scanf("%llu %llu", &seed, &block) == 2) {
    at::Philox4_32 eng(seed, 0, block);   // key = seed, counter = (block, 0)
    unsigned a = eng(), b = eng(), c = eng(), d = eng();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def aten_philox():
    hdr = os.path.join(TORCH_INCLUDE or "", "ATen", "core", "PhiloxRNGEngine.h")
    if not TORCH_INCLUDE or not os.path.exists(hdr) or shutil.which("g++") is None:
        pytest.skip("PyTorch Philox header or g++ not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(_ATEN_SRC)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", TORCH_INCLUDE, src, "-o", exe], check=True)

    def run(pairs):
        inp = "".join(f"{s} {b}\n" for s, b in pairs)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]

    yield run
    shutil.rmtree(d, ignore_errors=True)


PHILOX_CASES = [(0, 0), (0, 1), (1, 0), (12345, 67890), (2**32 - 1, 2**32 - 1),
                (2**64 - 1, 2**64 - 1), (0x243F6A8885A308D3, 0x13198A2E03707344),
                (7, 2**40 + 3), (2**63, 5)]


def test_philox_block_matches_pytorch(aten_philox):
    ref = aten_philox(PHILOX_CASES)
    for (seed, block), want in zip(PHILOX_CASES, ref):
        got = oracle.philox4x32_10([block & 0xFFFFFFFF, block >> 32, 0, 0],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        assert tuple(int(v) for v in got) == want, (seed, block)


def test_u16_lane_layout_matches_pytorch(aten_philox):
    # uniform of element counter c = 16-bit half (c & 7) of block c >> 3,
    # lowest half of the lowest word first
    pairs = [(99, 0), (99, 1), (2**40 + 9, 12345678901)]
    ref = aten_philox(pairs)
    for (seed, block), words in zip(pairs, ref):
        for q in range(8):
            w = words[q >> 1]
            want = (w >> 16) if (q & 1) else (w & 0xFFFF)
            assert oracle.u16(seed, block * 8 + q) == want


# ---------------------------------------------------------------------------
# Mask
# ---------------------------------------------------------------------------
def test_threshold_closed_forms():
    assert oracle.threshold(0.0) == 0
    assert oracle.threshold(0.5) == 32768
    # float32(0.1) = 0.100000001490116..., 0.1*65536 + 0.5 = 6554.10...
    assert oracle.threshold(np.float32(0.1)) == 6554
    assert oracle.threshold(np.float32(0.05)) == 3277
    assert oracle.threshold(np.float32(0.25)) == 16384
    # float32(0.9999) = 0x1.fff2e4p-1 = 0.99989998340606689...; * 65536 + 0.5 = 65529.945...
    assert oracle.threshold(np.float32(0.9999)) == 65529
    # float32(0.95) = 0x1.e66666p-1 = 0.94999998807907104...; * 65536 + 0.5 = 62259.699...
    assert oracle.threshold(np.float32(0.95)) == 62259
    # float32(0.3) = 0x1.333334p-2 = 0.30000001192092896...; * 65536 + 0.5 = 19661.300...
    assert oracle.threshold(np.float32(0.3)) == 19661


def test_pack_bits_layout_matches_numpy_packbits():
    rng = np.random.default_rng(1)
    for k in (8, 32, 40, 96, 1000):
        keep = (rng.random((5, k)) < 0.7).astype(np.uint8)
        bits = oracle.pack_bits(keep)
        words = (k + 31) // 32
        padded = np.zeros((5, words * 32), dtype=np.uint8)
        padded[:, :k] = keep
        ref = np.packbits(padded, axis=1, bitorder="little").view("<u4")
        np.testing.assert_array_equal(bits, ref)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.05])
def test_mask_drop_rate_binomial(p):
    m, k = 256, 1024
    keep = oracle.keep_mask(0, 0, np.arange(m), k, p)
    q = oracle.threshold(p) / 65536.0
    N = m * k
    drops = N - int(keep.sum())
    sigma = np.sqrt(N * q * (1 - q))
    assert abs(drops - N * q) < 5 * sigma


def test_mask_threshold_boundary():
    # keep iff u16 >= T: an element whose uniform equals T is kept, and raising
    # T by one drops it (p = u/65536 gives T = u exactly)
    seed, k = 4, 64
    for c in (0, 5, 77, 1000):
        u = oracle.u16(seed, c)
        i, j = divmod(c, k)
        at = oracle.keep_mask(seed, 0, [i], k, np.float32(u / 65536.0))
        above = oracle.keep_mask(seed, 0, [i], k, np.float32((u + 1) / 65536.0))
        assert oracle.threshold(np.float32(u / 65536.0)) == u
        assert at[0, j] == 1 and above[0, j] == 0
    # p just below 1 gives T = 65536: everything dropped
    assert not oracle.keep_mask(1, 0, [0, 1], 64, np.float32(0.99999994)).any()


def test_mask_p0_keeps_everything():
    keep = oracle.keep_mask(123, 8 * 77, np.arange(64), 256, 0.0)
    assert keep.all()


def test_mask_u16_uniform_histogram():
    vals = np.array([oracle.u16(5, c) for c in range(64 * 1024)], dtype=np.int64)
    hist = np.bincount(vals >> 12, minlength=16)
    exp = vals.size / 16
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 50  # 15 dof; P(chi2 > 50) ~ 1e-5


def _pair_chi2(a, b, q):
    # 2x2 pattern counts of (a, b) against independence with keep prob 1-q
    pk = 1.0 - q
    exp = np.array([(1 - pk) ** 2, (1 - pk) * pk, pk * (1 - pk), pk * pk]) * a.size
    obs = np.array([((a == x) & (b == y)).sum() for x in (0, 1) for y in (0, 1)])
    return ((obs - exp) ** 2 / exp).sum()


def test_mask_neighbours_independent():
    p = 0.5
    keep = oracle.keep_mask(77, 0, np.arange(128), 512, p).astype(np.int64)
    q = oracle.threshold(p) / 65536.0
    assert _pair_chi2(keep[:, :-1], keep[:, 1:], q) < 25  # along a row
    assert _pair_chi2(keep[:-1, :], keep[1:, :], q) < 25  # down a column
    # neighbouring 128-bit blocks (elements 8 apart) must not be correlated either
    assert _pair_chi2(keep[:, :-8], keep[:, 8:], q) < 25


def test_mask_row_offset_shift():
    # counter c = offset + i*k + j: shifting offset by i0*k shifts rows by i0
    k, m, i0 = 96, 40, 13
    full = oracle.keep_mask(9, 64, np.arange(m), k, 0.3)
    shifted = oracle.keep_mask(9, 64 + i0 * k, np.arange(m - i0), k, 0.3)
    np.testing.assert_array_equal(full[i0:], shifted)
    # and a global-row request equals the same rows of a full request
    rows = np.array([3, 17, 39])
    np.testing.assert_array_equal(oracle.keep_mask(9, 64, rows, k, 0.3), full[rows])


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------
def _case(rng, m=24, k=40, n=32, r=5):
    return (rand((m, k), rng), rand((k, n), rng, 0.2), rand((k, r), rng, 0.2),
            rand((r, n), rng, 0.2), rand((m, n), rng))


def test_forward_reduces_to_xw():
    rng = np.random.default_rng(2)
    X, W, A, B, _ = _case(rng)
    ref = X @ W
    out = oracle.lora_fwd(X, W, A, np.zeros_like(B), 2.0, 0.3, 4, 0)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12)
    out = oracle.lora_fwd(X, W, np.zeros_like(A), B, 2.0, 0.3, 4, 0)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12)
    out = oracle.lora_fwd(X, W, A, B, 0.0, 0.3, 4, 0)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12)


def test_forward_p0_equals_unfused_chain():
    rng = np.random.default_rng(3)
    X, W, A, B, _ = _case(rng)
    out = oracle.lora_fwd(X, W, A, B, 1.7, 0.0, 11, 0)
    np.testing.assert_allclose(out["S"], X @ A, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["Y"], X @ W + 1.7 * ((X @ A) @ B), rtol=1e-12, atol=1e-12)


def test_forward_uses_mask_for_adapter_only():
    # with a mask, S = (s*keep*X) A and the base path stays X W
    rng = np.random.default_rng(4)
    X, W, A, B, _ = _case(rng)
    p = np.float32(0.25)
    out = oracle.lora_fwd(X, W, A, B, 1.5, p, 21, 0)
    keep = out["keep"].astype(np.float64)
    s = 1.0 / (1.0 - float(p))
    Xh = s * keep * X
    np.testing.assert_allclose(out["S"], Xh @ A, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["Y"], X @ W + 1.5 * (Xh @ A) @ B, rtol=1e-12, atol=1e-12)
    assert 0 < keep.mean() < 1


def test_inverted_dropout_expectation():
    # E_mask[S] = X A pins the scale s = 1/(1-p)
    rng = np.random.default_rng(5)
    m, k, r = 6, 64, 3
    X, A = rand((m, k), rng), rand((k, r), rng)
    p = 0.5
    trials = 600
    acc = np.zeros((m, r))
    for seed in range(trials):
        keep = oracle.keep_mask(seed, 0, np.arange(m), k, p)
        acc += oracle.lora_s(X, keep, A, p)
    mean = acc / trials
    q = 1 - oracle.threshold(p) / 65536.0  # keep probability
    s = 1 / (1 - p)
    var = s * s * q * (1 - q) * ((X ** 2) @ (A ** 2))
    z = (mean - X @ A) / np.sqrt(var / trials)
    assert np.abs(z).max() < 5.0


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def _loss(X, W, A, B, dY, alpha, p, keep):
    S = oracle.lora_s(X, keep, A, p)
    return float((oracle.lora_y(X, W, S, B, alpha) * dY).sum())


def test_backward_finite_differences():
    rng = np.random.default_rng(6)
    m, k, n, r = 5, 12, 7, 3
    X, W, A, B, dY = (rand((m, k), rng), rand((k, n), rng), rand((k, r), rng),
                      rand((r, n), rng), rand((m, n), rng))
    alpha, p, seed = 1.3, np.float32(0.3), 8
    g = oracle.lora_bwd(dY, X, W, A, B, alpha, p, seed, 0)
    keep = g["keep"]
    assert 0 < keep.mean() < 1
    h = 1e-3
    for name, T, grad in (("X", X, g["dX"]), ("A", A, g["dA"]), ("B", B, g["dB"])):
        fd = np.zeros_like(T)
        for idx in np.ndindex(*T.shape):
            args = {"X": X, "A": A, "B": B}
            Tp, Tm = T.copy(), T.copy()
            Tp[idx] += h
            Tm[idx] -= h
            args[name] = Tp
            lp = _loss(args["X"], W, args["A"], args["B"], dY, alpha, p, keep)
            args[name] = Tm
            lm = _loss(args["X"], W, args["A"], args["B"], dY, alpha, p, keep)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-9, err_msg=name)


def test_backward_euler_identities():
    rng = np.random.default_rng(7)
    m, k, n, r = 33, 48, 40, 6
    X, W, A, B, dY = (rand((m, k), rng), rand((k, n), rng, 0.2), rand((k, r), rng, 0.2),
                      rand((r, n), rng, 0.2), rand((m, n), rng))
    alpha, p, seed = 2.0, np.float32(0.1), 3
    f = oracle.lora_fwd(X, W, A, B, alpha, p, seed, 16)
    g = oracle.lora_bwd(dY, X, W, A, B, alpha, p, seed, 16)
    L = (f["Y"] * dY).sum()
    Llora = ((f["Y"] - X @ W) * dY).sum()
    assert np.isclose((g["dX"] * X).sum(), L, rtol=1e-10)
    assert np.isclose((g["dA"] * A).sum(), Llora, rtol=1e-10)
    assert np.isclose((g["dB"] * B).sum(), Llora, rtol=1e-10)


# ---------------------------------------------------------------------------
# Multi-adapter
# ---------------------------------------------------------------------------
def test_multi_equals_single_per_segment():
    rng = np.random.default_rng(8)
    m, k, n = 50, 24, 16
    X, W, dY = rand((m, k), rng), rand((k, n), rng, 0.3), rand((m, n), rng)
    ranks = [2, 5, 3]
    adapters = [{"A": rand((k, rr), rng, 0.3), "B": rand((rr, n), rng, 0.3),
                 "alpha": a, "p": np.float32(p)}
                for rr, a, p in zip(ranks, (1.0, 2.0, 0.5), (0.0, 0.2, 0.4))]
    seg_off = np.array([0, 7, 7, 20, 33, 50])
    seg_ad = np.array([1, 0, 2, 1, 0])
    seed, offset = 5, 24
    f = oracle.multi_lora_fwd(X, W, adapters, seg_off, seg_ad, 5, seed, offset)
    g = oracle.multi_lora_bwd(dY, X, W, adapters, seg_off, seg_ad, 5, seed, offset)
    dA = [np.zeros_like(a["A"]) for a in adapters]
    dB = [np.zeros_like(a["B"]) for a in adapters]
    for s in range(len(seg_ad)):
        lo, hi = seg_off[s], seg_off[s + 1]
        if hi == lo:
            continue
        a = adapters[seg_ad[s]]
        # a standalone call on the segment's rows with the offset moved by lo*k
        fs = oracle.lora_fwd(X[lo:hi], W, a["A"], a["B"], a["alpha"], a["p"], seed, offset + lo * k)
        gs = oracle.lora_bwd(dY[lo:hi], X[lo:hi], W, a["A"], a["B"], a["alpha"], a["p"], seed,
                             offset + lo * k)
        np.testing.assert_allclose(f["Y"][lo:hi], fs["Y"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g["dX"][lo:hi], gs["dX"], rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(f["keep"][lo:hi], fs["keep"])
        dA[seg_ad[s]] += gs["dA"]
        dB[seg_ad[s]] += gs["dB"]
    for a in range(3):
        np.testing.assert_allclose(g["dA"][a], dA[a], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dB"][a], dB[a], rtol=1e-12, atol=1e-12)


def test_multi_unused_adapter_gets_zero_gradients():
    rng = np.random.default_rng(9)
    m, k, n = 12, 16, 8
    X, W, dY = rand((m, k), rng), rand((k, n), rng), rand((m, n), rng)
    adapters = [{"A": rand((k, 2), rng), "B": rand((2, n), rng), "alpha": 1.0, "p": 0.1}
                for _ in range(3)]
    g = oracle.multi_lora_bwd(dY, X, W, adapters, np.array([0, 12]), np.array([2]), 2, 0, 0)
    assert not g["dA"][0].any() and not g["dB"][1].any()
    assert g["dA"][2].any()


# ---------------------------------------------------------------------------
# Sampled evaluation (used for the full-size GPU checks) = the full oracle
# restricted to the samples, exactly
# ---------------------------------------------------------------------------
def test_sampled_equals_full_single():
    rng = np.random.default_rng(11)
    m, k, n, r = 40, 24, 32, 3
    X, W, A, B, dY = (rand((m, k), rng), rand((k, n), rng, 0.3), rand((k, r), rng, 0.3),
                      rand((r, n), rng, 0.3), rand((m, n), rng))
    out_rows, a_rows, b_cols = [0, 7, 39], [1, 23], [0, 5, 31]
    f = oracle.lora_fwd(X, W, A, B, 2.0, np.float32(0.3), 9, 16)
    g = oracle.lora_bwd(dY, X, W, A, B, 2.0, np.float32(0.3), 9, 16)
    s = oracle.lora_sampled(X, W, A, B, dY, 2.0, np.float32(0.3), 9, 16, out_rows, a_rows, b_cols)
    np.testing.assert_array_equal(s["keep"], f["keep"])
    np.testing.assert_array_equal(s["S"], f["S"])
    np.testing.assert_array_equal(s["dS"], g["dS"])
    np.testing.assert_array_equal(s["Y"], f["Y"][out_rows])
    np.testing.assert_array_equal(s["dX"], g["dX"][out_rows])
    np.testing.assert_array_equal(s["dA"], g["dA"][a_rows])
    np.testing.assert_array_equal(s["dB"], g["dB"][:, b_cols])


def test_sampled_equals_full_multi():
    rng = np.random.default_rng(12)
    m, k, n = 50, 24, 16
    X, W, dY = rand((m, k), rng), rand((k, n), rng, 0.3), rand((m, n), rng)
    adapters = [{"A": rand((k, rr), rng, 0.3), "B": rand((rr, n), rng, 0.3),
                 "alpha": a, "p": np.float32(p)}
                for rr, a, p in zip((2, 5, 3), (1.0, 2.0, 0.5), (0.0, 0.2, 0.4))]
    seg_off, seg_ad = np.array([0, 7, 7, 20, 33, 50]), np.array([1, 0, 2, 1, 0])
    out_rows, a_rows, b_cols = [0, 6, 7, 19, 20, 49], [0, 11, 23], [3, 15]
    f = oracle.multi_lora_fwd(X, W, adapters, seg_off, seg_ad, 5, 5, 24)
    g = oracle.multi_lora_bwd(dY, X, W, adapters, seg_off, seg_ad, 5, 5, 24)
    s = oracle.multi_lora_sampled(X, W, adapters, dY, seg_off, seg_ad, 5, 5, 24, out_rows,
                                  a_rows, b_cols)
    np.testing.assert_array_equal(s["keep"], f["keep"])
    np.testing.assert_array_equal(s["S"], f["S"])
    np.testing.assert_array_equal(s["Y"], f["Y"][out_rows])
    np.testing.assert_array_equal(s["dX"], g["dX"][out_rows])
    for a in range(3):
        np.testing.assert_array_equal(s["dA"][a], g["dA"][a][a_rows])
        np.testing.assert_array_equal(s["dB"][a], g["dB"][a][:, b_cols])


# ---------------------------------------------------------------------------
# Brute force: pure-Python loops on a tiny case
# ---------------------------------------------------------------------------
def test_against_python_loops():
    rng = np.random.default_rng(10)
    m, k, n, r = 3, 8, 4, 2
    X, W, A, B, dY = (rand((m, k), rng), rand((k, n), rng), rand((k, r), rng),
                      rand((r, n), rng), rand((m, n), rng))
    alpha, p, seed, offset = 0.7, np.float32(0.4), 31, 8
    T = oracle.threshold(p)
    s = 1.0 / (1.0 - float(p))
    keep = [[1 if oracle.u16(seed, offset + i * k + j) >= T else 0 for j in range(k)]
            for i in range(m)]
    S = [[sum(s * keep[i][j] * X[i, j] * A[j, c] for j in range(k)) for c in range(r)]
         for i in range(m)]
    Y = [[sum(X[i, t] * W[t, j] for t in range(k)) + alpha * sum(S[i][c] * B[c, j]
          for c in range(r)) for j in range(n)] for i in range(m)]
    dS = [[alpha * sum(dY[i, j] * B[c, j] for j in range(n)) for c in range(r)] for i in range(m)]
    dB = [[alpha * sum(S[i][c] * dY[i, j] for i in range(m)) for j in range(n)] for c in range(r)]
    dA = [[sum(s * keep[i][t] * X[i, t] * dS[i][c] for i in range(m)) for c in range(r)]
          for t in range(k)]
    dX = [[sum(dY[i, j] * W[t, j] for j in range(n)) +
           s * keep[i][t] * sum(dS[i][c] * A[t, c] for c in range(r)) for t in range(k)]
          for i in range(m)]
    f = oracle.lora_fwd(X, W, A, B, alpha, p, seed, offset)
    g = oracle.lora_bwd(dY, X, W, A, B, alpha, p, seed, offset)
    np.testing.assert_array_equal(f["keep"], np.array(keep))
    for got, want in ((f["S"], S), (f["Y"], Y), (g["dS"], dS), (g["dB"], dB), (g["dA"], dA),
                      (g["dX"], dX)):
        np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The synthetic workloads are well-formed
# ---------------------------------------------------------------------------
def test_workload_segments_cover_rows():
    for cid in (2, 4):
        w = workload(cid)
        assert w.seg_off[0] == 0 and w.seg_off[-1] == w.m
        assert np.all(np.diff(w.seg_off) >= 0)
        assert w.seg_adapter.min() >= 0 and w.seg_adapter.max() < len(w.adapters)
    w2 = workload(2)
    lens = np.diff(w2.seg_off)
    assert lens[:-1].min() >= 128 and lens.max() <= 4096


def test_workload_tensors_small_config():
    w = workload(0)
    t = make_tensors(w)
    assert t["X"].shape == (512, 1024) and t["W"].shape == (1024, 1024)
    assert abs(float(t["X"].float().std()) - 1.0) < 0.02
    assert abs(float(t["B"][0].float().var()) - 0.02) < 0.003
