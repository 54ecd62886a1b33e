"""GPU parity of the HIP path against the oracle, element by element, at sizes
the oracle finishes in seconds (several tiles plus ragged tails), and the edge
cases: m = 0, ragged m/k/n, ranks 1..256, p = 0, mixed-adapter tiles, empty
and tile-straddling segments, unused adapters, determinism, a non-default
stream, 0xFF-filled workspaces, and the frozen GEMMs against the oracle."""
import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as lf
import oracle
from parity import (assert_bits_equal, bf16_randn, check_close, compare_single, gpu_multi,
                    gpu_single, log, offset_view, oracle_multi, oracle_single)
from synth import make_tensors, workload

pytestmark = pytest.mark.gpu


def small_case(m, k, n, r, seed=1):
    g = torch.Generator().manual_seed(seed)
    X = bf16_randn((m, k), 1.0, g)
    W = bf16_randn((k, n), (1.0 / k) ** 0.5, g)
    A = bf16_randn((k, r), (1.0 / k) ** 0.5, g)
    B = bf16_randn((r, n), 0.02 ** 0.5, g)
    dY = bf16_randn((m, n), 1.0, g)
    return X, W, A, B, dY


@pytest.mark.parametrize("m,k,n,seed,offset,p", [
    (37, 1000, 8, 0, 0, 0.1),
    (64, 64, 8, 2 ** 40 + 3, 8 * 12345, 0.5),
    (5, 8, 8, 7, 2 ** 33, 0.3),
    (300, 4096, 8, 0, 0, 0.1),
    (3, 48, 8, 1, 0, 0.0),
])
def test_mask_bit_exact(m, k, n, seed, offset, p):
    log(f"mask m={m} k={k} seed={seed} offset={offset} p={p}")
    bits = lf.lora_dropout_mask(seed, offset, m, k, p)
    torch.cuda.synchronize()
    ref = oracle.pack_bits(oracle.keep_mask(seed, offset, np.arange(m), k, np.float32(p)))
    assert_bits_equal("mask", bits, ref)


SINGLE_CASES = [
    # m, k, n, r, alpha, p
    (512, 1024, 1024, 16, 2.0, 0.1),   # the small workload
    (300, 200, 136, 5, 2.0, 0.1),      # ragged everywhere
    (257, 264, 520, 17, 1.5, 0.3),     # one row past a tile, rank past a block
    (64, 128, 128, 1, 4.0, 0.0),       # rank 1, no dropout
    (1000, 512, 384, 33, 0.5, 0.1),
    (130, 1024, 256, 128, 2.0, 0.2),
    (96, 256, 264, 256, 2.0, 0.1),     # largest rank
    (8, 8, 8, 3, 1.0, 0.25),           # tiny
    (300, 264, 136, 8, 2.0, 0.1),      # all-loads-first epilogue, ragged m and n
    (257, 512, 520, 24, 1.5, 0.3),     # same epilogue, rank 24
    (1000, 1024, 776, 32, 2.0, 0.0),   # same epilogue, rank 32, no dropout
    (700, 512, 520, 64, 2.0, 0.1),     # two rank tiles of 32
    (333, 264, 264, 36, 1.0, 0.2),     # rank tiles, second one ragged (rank not a multiple of 8)
    (520, 1024, 264, 96, 0.5, 0.1),    # three rank tiles
    (300, 264, 136, 80, 1.0, 0.1),     # ranks past 64 with a ragged last column tile of dX
    (200, 136, 8, 4, 0.0, 0.5),        # alpha 0 (the LoRA term and its gradients vanish), n = 8
    (128, 256, 264, 16, 2.0, 0.95),    # heavy dropout: scale 20
    (300, 2048, 264, 64, 2.0, 0.1),    # 8 column tiles of k: the dA pass's XCD-aware work order
    (520, 4096, 136, 16, 1.0, 0.2),    # 16 column tiles of k, rank 16
]


@pytest.mark.parametrize("m,k,n,r,alpha,p", SINGLE_CASES)
def test_single_parity(m, k, n, r, alpha, p):
    log(f"single m={m} k={k} n={n} r={r} alpha={alpha} p={p}")
    X, W, A, B, dY = small_case(m, k, n, r, seed=m + r)
    seed, offset = 1234 + m, 8 * (m % 7)
    g = gpu_single(X, W, A, B, dY, alpha, p, seed, offset)
    o = oracle_single(X, W, A, B, dY, alpha, p, seed, offset)
    stats = compare_single(g, o, p)
    log(f"  {stats}")


@pytest.mark.parametrize("m,k,n,r", [(300, 264, 264, 16), (333, 264, 264, 64), (257, 512, 136, 24)])
def test_single_unaligned_adapter(m, k, n, r):
    # A, B, dA and dB only need 2-byte alignment: the 16-byte paths must step aside
    log(f"unaligned adapter m={m} k={k} n={n} r={r}")
    X, W, A, B, dY = small_case(m, k, n, r, seed=3 * m + r)
    Ad, Bd = offset_view(A), offset_view(B)
    assert Ad.data_ptr() % 16 == 2 and Bd.data_ptr() % 16 == 2
    dA, dB = offset_view(torch.zeros_like(A)), offset_view(torch.zeros_like(B))
    Xd, Wd, dYd = X.cuda(), W.cuda(), dY.cuda()
    Y, S, keep = lf.lora_linear_fwd(Xd, Wd, Ad, Bd, 2.0, 0.1, 5, 0)
    dX, _, _ = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, keep, 2.0, 0.1, dA=dA, dB=dB)
    torch.cuda.synchronize()
    g = {"Y": Y.cpu(), "S": S.cpu(), "keep": keep.cpu(), "dX": dX.cpu(), "dA": dA.cpu(), "dB": dB.cpu()}
    o = oracle_single(X, W, A, B, dY, 2.0, 0.1, 5, 0)
    log(f"  {compare_single(g, o, 0.1)}")


def test_bwd_without_input_gradient():
    # dX = NULL skips the dX GEMM; dA and dB are those of the full call, bit for bit
    m, k, n, r = 520, 264, 264, 24
    X, W, A, B, dY = small_case(m, k, n, r, seed=77)
    Xd, Wd, Ad, Bd, dYd = (t.cuda() for t in (X, W, A, B, dY))
    Y, S, keep = lf.lora_linear_fwd(Xd, Wd, Ad, Bd, 2.0, 0.1, 3, 0)
    _, dA, dB = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, keep, 2.0, 0.1)
    dX0, dA0, dB0 = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, keep, 2.0, 0.1, want_dX=False)
    torch.cuda.synchronize()
    assert dX0 is None and torch.equal(dA, dA0) and torch.equal(dB, dB0)
    # the same through autograd: an input without requires_grad gets no gradient
    Ag, Bg = Ad.clone().requires_grad_(), Bd.clone().requires_grad_()
    lf.lora_linear(Xd, Wd, Ag, Bg, 2.0, 0.1, 3, 0).backward(dYd)
    torch.cuda.synchronize()
    assert Xd.grad is None and torch.equal(Ag.grad, dA) and torch.equal(Bg.grad, dB)


CONCAT_CASES = [
    # m, k, n, r, alpha
    (512, 1024, 1024, 16, 2.0),   # the small workload's shape
    (300, 200, 136, 8, 1.5),      # ragged everywhere; K ends inside a 64-deep stage
    (257, 264, 520, 16, 0.5),     # one row past a tile
    (1000, 4096, 264, 8, 2.0),    # 64 K stages
    (8, 8, 8, 16, 1.0),           # tiny
    (600, 520, 776, 16, 0.0),     # alpha 0: Y is the frozen product, S still X A
]


@pytest.mark.parametrize("m,k,n,r,alpha", CONCAT_CASES)
def test_concat_forward_p0(m, k, n, r, alpha):
    # the forward with [W | A] as one operand at p = 0: Y and S against the
    # oracle, S feeding the backward, and the split forward agreeing
    log(f"concatenated forward m={m} k={k} n={n} r={r} alpha={alpha}")
    X, W, A, B, dY = small_case(m, k, n, r, seed=7 * m + r)
    Xd, Wd, Ad, Bd, dYd = (t.cuda() for t in (X, W, A, B, dY))
    Y, S = lf.lora_linear_fwd_concat(Xd, Wd, Ad, Bd, alpha)
    Y2, S2, _ = lf.lora_linear_fwd(Xd, Wd, Ad, Bd, alpha, 0.0)
    dX, dA, dB = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, None, alpha, 0.0)
    torch.cuda.synchronize()
    o = oracle_single(X, W, A, B, dY, alpha, 0.0)
    stats = {"S": check_close("S", S.cpu(), o["S"], rel=1e-4),
             "Y": check_close("Y", Y.cpu(), o["Y"]),
             "dX": check_close("dX", dX.cpu(), o["dX"]),
             "dA": check_close("dA", dA.cpu(), o["dA"]),
             "dB": check_close("dB", dB.cpu(), o["dB"]),
             "S vs split": check_close("S vs split", S.cpu(), S2.cpu().double().numpy(), rel=1e-5),
             "Y vs split": check_close("Y vs split", Y.cpu(), Y2.cpu().double().numpy())}
    log(f"  {stats}")


def test_concat_forward_deterministic_and_unsupported():
    X, W, A, B, _ = small_case(520, 512, 264, 16, seed=13)
    Xd, Wd, Ad, Bd = (t.cuda() for t in (X, W, A, B))
    a = lf.lora_linear_fwd_concat(Xd, Wd, Ad, Bd, 2.0)
    b = lf.lora_linear_fwd_concat(Xd, Wd, Ad, Bd, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # other ranks are refused before any launch (the general forward covers them)
    A24 = torch.zeros((512, 24), dtype=torch.bfloat16, device="cuda")
    B24 = torch.zeros((24, 264), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lf.LoraError):
        lf.lora_linear_fwd_concat(Xd, Wd, A24, B24, 2.0)


@pytest.mark.parametrize("m,k,n,r", [(300, 264, 264, 33), (333, 264, 264, 36), (300, 264, 136, 80),
                                     (520, 1024, 264, 96), (96, 256, 264, 256), (257, 264, 520, 17)])
def test_single_garbage_workspace(m, k, n, r):
    # workspaces filled with 0xFF bytes (NaN as bf16 or fp32): every value the
    # kernels read from them must have been written by the same call
    log(f"0xFF workspaces m={m} k={k} n={n} r={r}")
    X, W, A, B, dY = small_case(m, k, n, r, seed=5 * m + r)
    Xd, Wd, Ad, Bd, dYd = (t.cuda() for t in (X, W, A, B, dY))
    wsf = torch.full((max(lf.lora_linear_fwd_workspace_size(m, k, n, r), 1),), 0xFF, dtype=torch.uint8,
                     device="cuda")
    wsb = torch.full((lf.lora_linear_bwd_workspace_size(m, k, n, r),), 0xFF, dtype=torch.uint8, device="cuda")
    Y, S, keep = lf.lora_linear_fwd(Xd, Wd, Ad, Bd, 2.0, 0.1, 6, 0, workspace=wsf)
    dX, dA, dB = lf.lora_linear_bwd(dYd, Xd, Wd, Ad, Bd, S, keep, 2.0, 0.1, workspace=wsb)
    torch.cuda.synchronize()
    g = {"Y": Y.cpu(), "S": S.cpu(), "keep": keep.cpu(), "dX": dX.cpu(), "dA": dA.cpu(), "dB": dB.cpu()}
    log(f"  {compare_single(g, oracle_single(X, W, A, B, dY, 2.0, 0.1, 6, 0), 0.1)}")


def test_single_config0_workload():
    w = workload(0)
    t = make_tensors(w)
    ad = w.adapters[0]
    log("config 0 workload")
    g = gpu_single(t["X"], t["W"], t["A"][0], t["B"][0], t["dY"], ad.alpha, ad.p, w.seed, w.offset)
    o = oracle_single(t["X"], t["W"], t["A"][0], t["B"][0], t["dY"], ad.alpha, ad.p, w.seed, w.offset)
    log(f"  {compare_single(g, o, ad.p)}")


def test_single_deterministic():
    X, W, A, B, dY = small_case(700, 512, 520, 16, seed=3)
    a = gpu_single(X, W, A, B, dY, 2.0, 0.1, 5, 0)
    b = gpu_single(X, W, A, B, dY, 2.0, 0.1, 5, 0)
    for name in ("Y", "S", "keep", "dX", "dA", "dB"):
        assert torch.equal(a[name], b[name]), name


def test_single_m0_zero_gradients():
    k, n, r = 64, 64, 8
    X = torch.empty((0, k), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, n), dtype=torch.bfloat16, device="cuda")
    W = torch.randn((k, n), device="cuda").to(torch.bfloat16)
    A = torch.randn((k, r), device="cuda").to(torch.bfloat16)
    B = torch.randn((r, n), device="cuda").to(torch.bfloat16)
    Y, S, keep = lf.lora_linear_fwd(X, W, A, B, 2.0, 0.1)
    dA = torch.full((k, r), 3.0, dtype=torch.bfloat16, device="cuda")
    dB = torch.full((r, n), 3.0, dtype=torch.bfloat16, device="cuda")
    dX, dA, dB = lf.lora_linear_bwd(dY, X, W, A, B, S, keep, 2.0, 0.1, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, n) and dX.shape == (0, k)
    assert not dA.float().abs().sum().item() and not dB.float().abs().sum().item()


def test_single_row_block_with_offset():
    # rows [r0, r1) called alone with offset + r0*k reproduce the full call
    m, k, n, r = 600, 256, 264, 16
    X, W, A, B, dY = small_case(m, k, n, r, seed=11)
    full = gpu_single(X, W, A, B, dY, 2.0, 0.1, 9, 64)
    r0, r1 = 200, 457
    part = gpu_single(X[r0:r1], W, A, B, dY[r0:r1], 2.0, 0.1, 9, 64 + r0 * k)
    assert torch.equal(part["keep"], full["keep"][r0:r1])
    check_close("Y rows", part["Y"], full["Y"][r0:r1], rel=1e-6, absf=1e-6)
    check_close("dX rows", part["dX"], full["dX"][r0:r1], rel=1e-6, absf=1e-6)


def test_single_nondefault_stream():
    X, W, A, B, dY = small_case(300, 256, 256, 8, seed=5)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = gpu_single(X, W, A, B, dY, 2.0, 0.1, 1, 0, stream=s)
    o = oracle_single(X, W, A, B, dY, 2.0, 0.1, 1, 0)
    compare_single(g, o, 0.1)


# ----------------------------------------------------------------------------
# Mixed-adapter batches
# ----------------------------------------------------------------------------
def multi_case(m, k, n, ranks, seed):
    g = torch.Generator().manual_seed(seed)
    X = bf16_randn((m, k), 1.0, g)
    W = bf16_randn((k, n), (1.0 / k) ** 0.5, g)
    As = [bf16_randn((k, r), (1.0 / k) ** 0.5, g) for r in ranks]
    Bs = [bf16_randn((r, n), 0.02 ** 0.5, g) for r in ranks]
    dY = bf16_randn((m, n), 1.0, g)
    return X, W, As, Bs, dY


MULTI_CASES = [
    # m, k, n, ranks, alphas, ps, seg_off, seg_adapter
    (700, 256, 264, [16, 3, 40], [2.0, 1.0, 0.5], [0.1, 0.0, 0.25],
     [0, 10, 10, 300, 301, 520, 700], [0, 1, 2, 0, 1, 2]),      # empty + straddling segments
    (512, 512, 512, [16, 16, 16, 16], [1.0, 2.0, 2.0, 4.0], [0.0, 0.05, 0.1, 0.1],
     [0, 512], [2]),                                          # one segment; others unused
    (1100, 384, 136, [8, 64, 128], [2.0, 2.0, 2.0], [0.1, 0.1, 0.1],
     [0, 1, 65, 129, 700, 1100], [2, 0, 1, 0, 2]),             # 1-row segment, ranks up to 128
    (333, 136, 520, [5, 17], [3.0, 0.7], [0.3, 0.1],
     [0, 100, 200, 333], [1, 1, 0]),                           # same adapter twice in a row
    (600, 256, 264, [64, 16, 24], [2.0, 1.0, 0.5], [0.1, 0.2, 0.0],
     [0, 520, 600], [0, 2]),                                   # whole 128-row waves inside a rank-64 segment
    (600, 264, 136, [128, 120], [1.0, 2.0], [0.1, 0.2],
     [0, 300, 600], [0, 1]),                                   # a 16-row band meeting ranks 128 and 120 (8 chunks)
    (520, 136, 264, [128, 64, 8], [2.0, 0.5, 4.0], [0.1, 0.0, 0.3],
     [0, 200, 390, 520], [1, 0, 2]),                           # bands meeting ranks 64 | 128 and 128 | 8
    (700, 2048, 136, [16, 64, 128], [2.0, 1.0, 0.5], [0.1, 0.0, 0.2],
     [0, 200, 450, 700], [2, 0, 1]),                           # 8 column tiles of k: XCD-aware dA order
    (1210, 264, 136, [8, 40, 128], [2.0, 1.0, 0.5], [0.1, 0.2, 0.1],
     [0] + [11 * i + (i % 3) for i in range(1, 110)] + [1210], [i % 3 for i in range(110)]),
                                                               # 110 segments (past one wave of the router)
]


@pytest.mark.parametrize("case", range(len(MULTI_CASES)))
def test_multi_parity(case):
    m, k, n, ranks, alphas, ps, seg_off, seg_ad = MULTI_CASES[case]
    log(f"multi case {case}: m={m} k={k} n={n} ranks={ranks} segs={seg_off}")
    lf.multi_lora_check_segments(seg_off, seg_ad, m, ranks, max(ranks))
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=100 + case)
    seed, offset = 77 + case, 8 * case
    g = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset)
    o = oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset)
    assert_bits_equal("keep_bits", g["keep"], o["bits"])
    check_close("S", g["S"], o["S"], rel=1e-4)
    check_close("Y", g["Y"], o["Y"])
    check_close("dX", g["dX"], o["dX"])
    for a in range(len(ranks)):
        check_close(f"dA[{a}]", g["dA"][a], o["dA"][a])
        check_close(f"dB[{a}]", g["dB"][a], o["dB"][a])


MIXED_WIDE_CASES = [
    # m, k, n, ranks, alphas, ps, seg_off, seg_adapter, adapters placed off 16-byte boundaries
    (600, 264, 264, [200, 13, 64], [2.0, 1.0, 0.5], [0.1, 0.2, 0.0],
     [0, 150, 151, 400, 600], [1, 0, 2, 1], (1,)),            # rank 200 beside an unaligned rank-13 adapter
    (520, 264, 136, [129, 256, 8], [1.0, 2.0, 4.0], [0.1, 0.1, 0.3],
     [0, 100, 300, 520], [2, 1, 0], (2,)),                     # ranks 129 and 256, unaligned rank 8
    (700, 520, 264, [16, 24, 64], [2.0, 0.5, 1.0], [0.1, 0.0, 0.2],
     [0, 250, 500, 700], [0, 1, 2], (1,)),                     # ranks <= 64, unaligned rank 24
    (640, 264, 264, [128, 40, 96], [1.0, 2.0, 0.5], [0.1, 0.1, 0.1],
     [0, 64, 320, 640], [0, 1, 2], (0, 2)),                    # ranks <= 128, unaligned 128 and 96
]


@pytest.mark.parametrize("case", range(len(MIXED_WIDE_CASES)))
def test_multi_wide_rank_and_unaligned_adapters(case):
    m, k, n, ranks, alphas, ps, seg_off, seg_ad, unaligned = MIXED_WIDE_CASES[case]
    log(f"mixed wide/unaligned case {case}: m={m} k={k} n={n} ranks={ranks} segs={seg_off} "
        f"unaligned={unaligned}")
    lf.multi_lora_check_segments(seg_off, seg_ad, m, ranks, max(ranks))
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=300 + case)
    seed, offset = 91 + case, 16 * case
    g = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset, unaligned=unaligned)
    o = oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, seed, offset)
    assert_bits_equal("keep_bits", g["keep"], o["bits"])
    check_close("S", g["S"], o["S"], rel=1e-4)
    check_close("Y", g["Y"], o["Y"])
    check_close("dX", g["dX"], o["dX"])
    for a in range(len(ranks)):
        check_close(f"dA[{a}]", g["dA"][a], o["dA"][a])
        check_close(f"dB[{a}]", g["dB"][a], o["dB"][a])


def test_multi_parity_packed_microbatch():
    # the host packer's output end to end: samples of four adapters packed into
    # microbatches of at most 640 tokens; the segment table (rows grouped by
    # adapter) of the one with the most adapters, then the most rows, drives
    # the mixed-adapter forward and backward
    rng = np.random.Generator(np.random.PCG64(41))
    lengths = [int(v) for v in np.clip(np.rint(rng.lognormal(np.log(90.0), 0.75, 40)), 16, 400)]
    adapters = [int(v) for v in rng.integers(0, 4, len(lengths))]
    mb, count = lf.lora_pack_greedy(lengths, 640)
    tables = [lf.lora_microbatch_segments(lengths, adapters, mb, 4, q) for q in range(count)]
    _, seg_off, seg_ad = max(tables, key=lambda t: (len(t[2]), t[1][-1]))
    m, k, n = seg_off[-1], 256, 264
    ranks, alphas, ps = [16, 8, 32, 24], [2.0, 1.0, 0.5, 4.0], [0.1, 0.0, 0.2, 0.05]
    log(f"packed microbatch: m={m} segs={seg_off} adapters={seg_ad}")
    lf.multi_lora_check_segments(seg_off, seg_ad, m, ranks, max(ranks))
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=141)
    g = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, 9, 0)
    o = oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, 9, 0)
    assert_bits_equal("keep_bits", g["keep"], o["bits"])
    check_close("S", g["S"], o["S"], rel=1e-4)
    check_close("Y", g["Y"], o["Y"])
    check_close("dX", g["dX"], o["dX"])
    for a in range(len(ranks)):
        check_close(f"dA[{a}]", g["dA"][a], o["dA"][a])
        check_close(f"dB[{a}]", g["dB"][a], o["dB"][a])


@pytest.mark.parametrize("k,r", [(512, 16), (2048, 16), (512, 32), (2048, 64), (4096, 128), (512, 200)])
def test_multi_single_segment_equals_single_bitwise(k, r):
    # k = 2048 and 4096 give 8 and 16 column tiles of 256: the dA pass then
    # takes its XCD-aware work order (k = 512: grid order).  The mask, S and
    # every gradient match bit for bit.  Y does too, except for ranks 33..128,
    # where the single-adapter forward accumulates alpha S B as extra K stages
    # of the GEMM and the mixed form adds it after the K loop: one rounding
    # apart (at most one bf16 step).
    m, n = 640, 264
    log(f"single vs one-segment mixed, bitwise: m={m} k={k} n={n} r={r}")
    X, W, As, Bs, dY = multi_case(m, k, n, [r], seed=7)
    s = gpu_single(X, W, As[0], Bs[0], dY, 2.0, 0.1, 3, 16)
    mu = gpu_multi(X, W, As, Bs, [2.0], [0.1], [0, m], [0], dY, 3, 16)
    assert torch.equal(s["keep"], mu["keep"])
    if 32 < r <= 128:
        a, b = s["Y"].float(), mu["Y"].float()
        assert torch.all((a - b).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), b.abs()) + 2.0 ** -16), "Y beyond one bf16 step"
    else:
        assert torch.equal(s["Y"], mu["Y"])
    assert torch.equal(s["S"], mu["S"])
    assert torch.equal(s["dX"], mu["dX"])
    assert torch.equal(s["dA"], mu["dA"][0])
    assert torch.equal(s["dB"], mu["dB"][0])


def test_multi_garbage_workspace():
    m, k, n, ranks, alphas, ps, seg_off, seg_ad = MULTI_CASES[2]
    log("mixed adapters, 0xFF workspaces")
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=102)
    dev = "cuda"
    Xd, Wd, dYd = X.to(dev), W.to(dev), dY.to(dev)
    Ad, Bd = [a.to(dev) for a in As], [b.to(dev) for b in Bs]
    dAd = [torch.full_like(a, 7.0) for a in Ad]
    dBd = [torch.full_like(b, 7.0) for b in Bd]
    r_max, na, ns = max(ranks), len(ranks), len(seg_ad)
    table = lf.adapter_table(Ad, Bd, alphas, ps, dAd, dBd)
    so = torch.as_tensor(np.asarray(seg_off, dtype=np.int64)).to(dev)
    sa = torch.as_tensor(np.asarray(seg_ad, dtype=np.int32)).to(dev)
    wsf = torch.full((lf.multi_lora_fwd_workspace_size(m, k, n, r_max, na, ns),), 0xFF, dtype=torch.uint8,
                     device=dev)
    wsb = torch.full((lf.multi_lora_bwd_workspace_size(m, k, n, r_max, na, ns),), 0xFF, dtype=torch.uint8,
                     device=dev)
    Y, S, keep = lf.multi_lora_linear_fwd(Xd, Wd, table, na, so, sa, r_max, 5, 0, workspace=wsf)
    dX = lf.multi_lora_linear_bwd(dYd, Xd, Wd, table, na, so, sa, S, keep, r_max, workspace=wsb)
    torch.cuda.synchronize()
    o = oracle_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, 5, 0)
    assert_bits_equal("keep_bits", keep.cpu(), o["bits"])
    check_close("S", S.cpu(), o["S"], rel=1e-4)
    check_close("Y", Y.cpu(), o["Y"])
    check_close("dX", dX.cpu(), o["dX"])
    for a in range(na):
        check_close(f"dA[{a}]", dAd[a].cpu(), o["dA"][a])
        check_close(f"dB[{a}]", dBd[a].cpu(), o["dB"][a])


def test_multi_bwd_without_input_gradient():
    # dX = NULL skips the dX GEMM of the mixed form too; dA and dB are those of
    # the full call bit for bit, directly and through the autograd wrapper
    m, k, n, ranks = 600, 256, 264, [16, 64, 8]
    alphas, ps = [2.0, 1.0, 0.5], [0.1, 0.2, 0.0]
    seg_off, seg_ad = [0, 100, 430, 600], [2, 0, 1]
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=91)
    dev = "cuda"
    Xd, Wd, dYd = X.to(dev), W.to(dev), dY.to(dev)
    Ad, Bd = [a.to(dev) for a in As], [b.to(dev) for b in Bs]
    so = torch.as_tensor(np.asarray(seg_off, dtype=np.int64)).to(dev)
    sa = torch.as_tensor(np.asarray(seg_ad, dtype=np.int32)).to(dev)
    full = ([torch.empty_like(a) for a in Ad], [torch.empty_like(b) for b in Bd])
    part = ([torch.empty_like(a) for a in Ad], [torch.empty_like(b) for b in Bd])
    t_full = lf.adapter_table(Ad, Bd, alphas, ps, *full)
    t_part = lf.adapter_table(Ad, Bd, alphas, ps, *part)
    Y, S, keep = lf.multi_lora_linear_fwd(Xd, Wd, t_full, 3, so, sa, 64, 4, 0)
    dX = lf.multi_lora_linear_bwd(dYd, Xd, Wd, t_full, 3, so, sa, S, keep, 64)
    dX0 = lf.multi_lora_linear_bwd(dYd, Xd, Wd, t_part, 3, so, sa, S, keep, 64, want_dX=False)
    torch.cuda.synchronize()
    assert dX is not None and dX0 is None
    for i in range(3):
        assert torch.equal(full[0][i], part[0][i]) and torch.equal(full[1][i], part[1][i]), i
    Ag = [a.clone().requires_grad_() for a in Ad]
    Bg = [b.clone().requires_grad_() for b in Bd]
    Y2 = lf.multi_lora_linear(Xd, Wd, so, sa, Ag, Bg, alphas, ps, 4, 0)
    assert torch.equal(Y2.detach(), Y)
    Y2.backward(dYd)
    torch.cuda.synchronize()
    assert Xd.grad is None
    for i in range(3):
        assert torch.equal(Ag[i].grad, full[0][i]) and torch.equal(Bg[i].grad, full[1][i]), i


def test_multi_deterministic():
    m, k, n, ranks, alphas, ps, seg_off, seg_ad = MULTI_CASES[0]
    X, W, As, Bs, dY = multi_case(m, k, n, ranks, seed=100)
    a = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, 1, 0)
    b = gpu_multi(X, W, As, Bs, alphas, ps, seg_off, seg_ad, dY, 1, 0)
    for name in ("Y", "S", "keep", "dX"):
        assert torch.equal(a[name], b[name]), name
    for i in range(len(ranks)):
        assert torch.equal(a["dA"][i], b["dA"][i]) and torch.equal(a["dB"][i], b["dB"][i])


# ----------------------------------------------------------------------------
# Frozen GEMMs against the oracle's products (its forward with B = 0 is X W;
# its input gradient with dS = 0 is dY W^T)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("m,k,n", [(512, 1024, 1024), (300, 200, 136), (1000, 264, 520)])
def test_frozen_gemms(m, k, n):
    g = torch.Generator().manual_seed(m)
    X = bf16_randn((m, k), 1.0, g)
    W = bf16_randn((k, n), (1.0 / k) ** 0.5, g)
    dY = bf16_randn((m, n), 1.0, g)
    Y = lf.lora_frozen_fwd(X.cuda(), W.cuda())
    dX = lf.lora_frozen_bwd(dY.cuda(), W.cuda())
    torch.cuda.synchronize()
    Xn, Wn, dYn = (np.ascontiguousarray(t.to(torch.float64).numpy()) for t in (X, W, dY))
    r = 1
    Y_ref = oracle.lora_y(Xn, Wn, np.zeros((m, r)), np.zeros((r, n)), 1.0)
    dX_ref = oracle.lora_dx(dYn, Wn, np.zeros((m, r)), np.zeros((k, r)), np.ones((m, k), dtype=np.uint8),
                            np.float32(0.0))
    check_close("XW", Y.cpu(), Y_ref)
    check_close("dY W^T", dX.cpu(), dX_ref)
