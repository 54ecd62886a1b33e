"""GPU parity at the full workload sizes, through the C ABI with the library's
own workspace sizing, as the benchmark launches it.

Against the oracle:
* the dropout mask, every word, bit for bit;
* S, every element;
* Y and dX on sampled rows: the first and last rows, rows on both sides of
  256-row tile edges and of every segment boundary, and seeded random rows;
* dA on sampled input features and dB on sampled output columns (all ranks),
  each summed over every row of the batch.

Over every element:
* Y and dX against a plain PyTorch fp32 product on the GPU, with the mask
  taken from the oracle;
* the Euler identity <dX, X> = <Y, dY> of the layer (Y is linear in X once the
  mask is fixed), within the spread that bf16 rounding of Y and dX allows.
"""
import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as lf
import oracle
from parity import assert_bits_equal, check_close, f64, log, offset_view
from synth import decoder_projection, make_tensors_device, wide_mixed_workload, workload

pytestmark = pytest.mark.gpu

N_RANDOM_ROWS = 24
N_FEATURES = 96


def sample_rows(m, seg_off=None, seed=0):
    rows = {0, m - 1}
    for edge in (256, 512, m // 2 // 256 * 256):
        if 0 < edge < m:
            rows.update((edge - 1, edge))
    if seg_off is not None:
        for lo, hi in zip(seg_off[:-1], seg_off[1:]):
            if hi > lo:
                rows.update((int(lo), int(hi) - 1))
    rng = np.random.default_rng(seed)
    rows.update(int(v) for v in rng.integers(0, m, N_RANDOM_ROWS))
    return np.array(sorted(rows), dtype=np.int64)


def sample_features(size, seed):
    cols = {0, size - 1, min(255, size - 1), min(256, size - 1)}
    rng = np.random.default_rng(seed)
    cols.update(int(v) for v in rng.integers(0, size, N_FEATURES))
    return np.array(sorted(cols), dtype=np.int64)


def euler_check(X, Y, dY, dX):
    """<dX, X> = <Y, dY>.  bf16 rounding of each element of Y and dX has a
    relative spread of about 2^-8/sqrt(3); the bound is about 8 such standard
    deviations of each side's sum."""
    Xd, Yd, dYd, dXd = (t.to(torch.float64) for t in (X, Y, dY, dX))
    lhs = float((dXd * Xd).sum())
    rhs = float((Yd * dYd).sum())
    scale = float(((Yd * dYd) ** 2).sum().sqrt() + ((dXd * Xd) ** 2).sum().sqrt())
    log(f"  euler <dX,X>={lhs:.6g} <Y,dY>={rhs:.6g} scale={scale:.4g}")
    assert abs(lhs - rhs) <= 0.02 * scale, (lhs, rhs, scale)


def torch_reference_rows(X, W, dY, items, k):
    """Y and dX of every row in fp32 torch ops on the GPU.  `items` are
    (lo, hi, A, B, alpha, p, keep) with keep the oracle's uint8 mask rows."""
    X32, W32, dY32 = X.float(), W.float(), dY.float()
    Yr = X32 @ W32
    dXr = dY32 @ W32.t().contiguous()
    for lo, hi, A, B, alpha, p, keep in items:
        s = 1.0 / (1.0 - float(np.float32(p)))
        km = torch.from_numpy(keep).to(X.device, torch.float32)
        A32, B32 = A.float(), B.float()
        Sr = (s * km * X32[lo:hi]) @ A32
        Yr[lo:hi] += alpha * (Sr @ B32)
        dS = alpha * (dY32[lo:hi] @ B32.t().contiguous())
        dXr[lo:hi] += s * km * (dS @ A32.t().contiguous())
    return Yr, dXr


def run_single(w, variant_seed=0):
    ad = w.adapters[0]
    log(f"full-size single: {w.name} alpha={ad.alpha} p={ad.p}")
    t = make_tensors_device(w, "cuda", seed=variant_seed)
    X, W, A, B, dY = t["X"], t["W"], t["A"][0], t["B"][0], t["dY"]
    Y, S, keep = lf.lora_linear_fwd(X, W, A, B, ad.alpha, ad.p, w.seed, w.offset)
    dX, dA, dB = lf.lora_linear_bwd(dY, X, W, A, B, S, keep, ad.alpha, ad.p)
    torch.cuda.synchronize()
    log("  GPU path done; oracle on samples")

    rows = sample_rows(w.m, seed=w.m + ad.r)
    a_rows = sample_features(w.k, seed=1)
    b_cols = sample_features(w.n, seed=2)
    o = oracle.lora_sampled(f64(X), f64(W), f64(A), f64(B), f64(dY), ad.alpha, np.float32(ad.p),
                            w.seed, w.offset, rows, a_rows, b_cols)
    assert_bits_equal("keep_bits", keep, oracle.pack_bits(o["keep"]))
    stats = {"S": check_close("S", S, o["S"], rel=1e-4),
             "Y rows": check_close("Y rows", Y[torch.from_numpy(rows).cuda()], o["Y"]),
             "dX rows": check_close("dX rows", dX[torch.from_numpy(rows).cuda()], o["dX"]),
             "dA features": check_close("dA features", dA[torch.from_numpy(a_rows).cuda()], o["dA"]),
             "dB columns": check_close("dB columns", dB[:, torch.from_numpy(b_cols).cuda()], o["dB"])}
    log(f"  oracle: {stats}")

    Yr, dXr = torch_reference_rows(X, W, dY, [(0, w.m, A, B, ad.alpha, ad.p, o["keep"])], w.k)
    log(f"  torch fp32, all rows: Y {check_close('Y', Y, Yr)} dX {check_close('dX', dX, dXr)}")
    del Yr, dXr
    euler_check(X, Y, dY, dX)


@pytest.mark.parametrize("variant", [0, 1], ids=["n4096", "n14336"])
def test_full_llama8b_projection(variant):
    run_single(workload(1, variant))


@pytest.mark.parametrize("m", [2048, 8192, 32768])
@pytest.mark.parametrize("r", [8, 16, 32, 64, 128])
def test_full_rank_token_sweep(m, r):
    run_single(workload(3, m=m, r=r))


@pytest.mark.parametrize("index", [1, 6], ids=["k_proj_4096x1024", "down_proj_14336x4096"])
def test_full_decoder_projection(index):
    # the decoder layer's shapes that the two projection workloads above do
    # not cover (q and o are k = n 4096; gate and up are 4096 -> 14336; v is k's)
    run_single(decoder_projection(index))


def run_multi(w, unaligned=()):
    log(f"full-size multi: {w.name} ranks={[a.r for a in w.adapters]} "
        f"segments={w.seg_off.tolist()} adapters={w.seg_adapter.tolist()} unaligned={list(unaligned)}")
    t = make_tensors_device(w, "cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    # adapters listed in `unaligned` sit one element past a 16-byte boundary
    place = lambda a, v: offset_view(v) if a in unaligned else v
    As = [place(a, v) for a, v in enumerate(t["A"])]
    Bs = [place(a, v) for a, v in enumerate(t["B"])]
    alphas = [a.alpha for a in w.adapters]
    ps = [a.p for a in w.adapters]
    r_max = w.r_max
    lf.multi_lora_check_segments(w.seg_off, w.seg_adapter, w.m, [a.r for a in w.adapters], r_max)
    dAs = [place(a, torch.full_like(v, 7.0)) for a, v in enumerate(As)]  # outputs must be overwritten
    dBs = [place(a, torch.full_like(v, 7.0)) for a, v in enumerate(Bs)]
    table = lf.adapter_table(As, Bs, alphas, ps, dAs, dBs)
    so = torch.as_tensor(w.seg_off).cuda()
    sa = torch.as_tensor(w.seg_adapter).cuda()
    Y, S, keep = lf.multi_lora_linear_fwd(X, W, table, len(As), so, sa, r_max, w.seed, w.offset)
    dX = lf.multi_lora_linear_bwd(dY, X, W, table, len(As), so, sa, S, keep, r_max)
    torch.cuda.synchronize()
    log("  GPU path done; oracle on samples")

    rows = sample_rows(w.m, w.seg_off, seed=w.m)
    a_rows = sample_features(w.k, seed=3)
    b_cols = sample_features(w.n, seed=4)
    ads = [{"A": f64(a), "B": f64(b), "alpha": al, "p": np.float32(p)}
           for a, b, al, p in zip(As, Bs, alphas, ps)]
    o = oracle.multi_lora_sampled(f64(X), f64(W), ads, f64(dY), w.seg_off, w.seg_adapter, r_max,
                                  w.seed, w.offset, rows, a_rows, b_cols)
    assert_bits_equal("keep_bits", keep, oracle.pack_bits(o["keep"]))
    ri = torch.from_numpy(rows).cuda()
    log(f"  S {check_close('S', S, o['S'], rel=1e-4)}")
    log(f"  Y rows {check_close('Y rows', Y[ri], o['Y'])}")
    log(f"  dX rows {check_close('dX rows', dX[ri], o['dX'])}")
    used = set(int(a) for lo, hi, a in oracle.segments_rows(w.seg_off, w.seg_adapter))
    for a in range(len(As)):
        gA = dAs[a][torch.from_numpy(a_rows).cuda()]
        gB = dBs[a][:, torch.from_numpy(b_cols).cuda()]
        if a not in used:
            assert not dAs[a].float().abs().sum().item() and not dBs[a].float().abs().sum().item()
            continue
        log(f"  adapter {a}: dA {check_close(f'dA[{a}]', gA, o['dA'][a])} "
            f"dB {check_close(f'dB[{a}]', gB, o['dB'][a])}")

    items = [(lo, hi, As[a], Bs[a], alphas[a], ps[a], o["keep"][lo:hi])
             for lo, hi, a in oracle.segments_rows(w.seg_off, w.seg_adapter)]
    Yr, dXr = torch_reference_rows(X, W, dY, items, w.k)
    log(f"  torch fp32, all rows: Y {check_close('Y', Y, Yr)} dX {check_close('dX', dX, dXr)}")
    del Yr, dXr
    euler_check(X, Y, dY, dX)


def test_full_mixed_four_adapters():
    run_multi(workload(2))


def test_full_70b_down_proj_eight_adapters():
    run_multi(workload(4))


def test_full_wide_rank_and_unaligned_adapters():
    # ranks 8, 200, 13, 128: the widest is past 128, rank 13 is not a multiple
    # of 8 and its A and B sit off 16-byte boundaries
    run_multi(wide_mixed_workload(), unaligned=(2,))


@pytest.mark.parametrize("variant", [0, 1], ids=["n4096", "n14336"])
def test_full_concat_forward_p0(variant):
    # the forward with [W | A] as one operand at p = 0 on the projection shapes
    w = workload(1, variant)
    ad = w.adapters[0]
    log(f"full-size concatenated forward: {w.name} alpha={ad.alpha} p=0")
    t = make_tensors_device(w, "cuda")
    X, W, A, B, dY = t["X"], t["W"], t["A"][0], t["B"][0], t["dY"]
    Y, S = lf.lora_linear_fwd_concat(X, W, A, B, ad.alpha)
    torch.cuda.synchronize()
    rows = sample_rows(w.m, seed=w.m + ad.r)
    a_rows = sample_features(w.k, seed=1)
    b_cols = sample_features(w.n, seed=2)
    o = oracle.lora_sampled(f64(X), f64(W), f64(A), f64(B), f64(dY), ad.alpha, np.float32(0.0),
                            w.seed, w.offset, rows, a_rows, b_cols)
    log(f"  S {check_close('S', S, o['S'], rel=1e-4)}")
    log(f"  Y rows {check_close('Y rows', Y[torch.from_numpy(rows).cuda()], o['Y'])}")
    ones = np.ones((w.m, w.k), dtype=np.uint8)
    Yr, _ = torch_reference_rows(X, W, dY, [(0, w.m, A, B, ad.alpha, 0.0, ones)], w.k)
    log(f"  torch fp32, all rows: Y {check_close('Y', Y, Yr)}")
