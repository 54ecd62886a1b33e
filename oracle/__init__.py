"""CPU oracle for the LoRA linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library under
``lora_fine_tuning_amd/``) never imports it and shares no code with it.

The arithmetic lives in ``lora_oracle.c`` (plain double-precision C, see the
header comment there for the definitions and where the pages state them).  This
module only builds that file, marshals numpy arrays into it, and composes its
functions in the order the definition gives:

* forward  (juhe.plus blog on LoRAFusion, section 2, Y = XW + alpha*S*B;
  papers.chlience.com notes, section 3, S = X^ A with X^ = dropout(X)):
  mask -> S -> Y.
* backward (chain rule; W is frozen, juhe.plus blog section 2):
  dS, dB from dY; dA from X^ and dS; dX from dY, W, dS, A and the mask.
* multi-adapter (papers.chlience.com notes, section 5 "FusedMultiLoRA": each
  tile carries an adapter id, rank, scaling factor and dropout ratio):
  the single-adapter steps applied per segment with that segment's adapter;
  mask counters use the global row index; dA/dB of an adapter sum over all its
  segments, and adapters without rows get zero gradients.

All inputs are float64 arrays holding exact bf16 values; outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblora_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile lora_oracle.c into liblora_oracle.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    U64 = ctypes.c_uint64
    F32 = ctypes.c_float
    F64 = ctypes.c_double
    U32 = ctypes.c_uint32
    sig = {
        "oracle_philox4x32_10": (None, [P, P, P]),
        "oracle_u16": (U32, [U64, U64]),
        "oracle_threshold": (U32, [F32]),
        "oracle_keep": (None, [U64, U64, P, I64, I64, U32, P]),
        "oracle_pack_bits": (None, [P, I64, I64, P]),
        "oracle_lora_s": (None, [P, P, P, I64, I64, I64, F32, P]),
        "oracle_lora_y": (None, [P, P, P, P, I64, I64, I64, I64, F64, P]),
        "oracle_lora_ds": (None, [P, P, I64, I64, I64, F64, P]),
        "oracle_lora_dx": (None, [P, P, P, P, P, I64, I64, I64, I64, F32, P]),
        "oracle_lora_db_acc": (None, [P, P, I64, I64, I64, F64, P]),
        "oracle_lora_da_acc": (None, [P, P, P, I64, I64, I64, F32, P]),
        "oracle_num_threads": (ctypes.c_int, []),
        "oracle_dora_norm": (None, [P, P, P, I64, I64, I64, F64, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------------------
# Dropout mask
# ----------------------------------------------------------------------------
def philox4x32_10(counter: Sequence[int], key: Sequence[int]) -> np.ndarray:
    """Raw Philox4x32-10 block for a 4-word counter and 2-word key."""
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def u16(seed: int, counter: int) -> int:
    return int(_load().oracle_u16(seed, counter))


def threshold(p: float) -> int:
    return int(_load().oracle_threshold(p))


def keep_mask(seed: int, offset: int, rows, k: int, p: float) -> np.ndarray:
    """0/1 uint8 mask for the given global row indices (len(rows) x k)."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    keep = np.zeros((rows.size, k), dtype=np.uint8)
    if rows.size and k:
        _load().oracle_keep(seed, offset, _p(rows), rows.size, k, threshold(p), _p(keep))
    return keep


def pack_bits(keep: np.ndarray) -> np.ndarray:
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    m, k = keep.shape
    words = (k + 31) // 32
    bits = np.zeros((m, words), dtype=np.uint32)
    if m and k:
        _load().oracle_pack_bits(_p(keep), m, k, _p(bits))
    return bits


# ----------------------------------------------------------------------------
# Single adapter, on an arbitrary set of rows
# ----------------------------------------------------------------------------
def lora_s(X, keep, A, p) -> np.ndarray:
    X, A = _f64(X), _f64(A)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    nrows, k = X.shape
    r = A.shape[1]
    S = np.zeros((nrows, r))
    if nrows:
        _load().oracle_lora_s(_p(X), _p(keep), _p(A), nrows, k, r, p, _p(S))
    return S


def lora_y(X, W, S, B, alpha) -> np.ndarray:
    X, W, S, B = _f64(X), _f64(W), _f64(S), _f64(B)
    nrows, k = X.shape
    n = W.shape[1]
    r = B.shape[0]
    Y = np.zeros((nrows, n))
    if nrows:
        _load().oracle_lora_y(_p(X), _p(W), _p(S), _p(B), nrows, k, n, r, alpha, _p(Y))
    return Y


def lora_ds(dY, B, alpha) -> np.ndarray:
    dY, B = _f64(dY), _f64(B)
    nrows, n = dY.shape
    r = B.shape[0]
    dS = np.zeros((nrows, r))
    if nrows:
        _load().oracle_lora_ds(_p(dY), _p(B), nrows, n, r, alpha, _p(dS))
    return dS


def lora_dx(dY, W, dS, A, keep, p) -> np.ndarray:
    dY, W, dS, A = _f64(dY), _f64(W), _f64(dS), _f64(A)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    nrows, n = dY.shape
    k = W.shape[0]
    r = A.shape[1]
    dX = np.zeros((nrows, k))
    if nrows:
        _load().oracle_lora_dx(_p(dY), _p(W), _p(dS), _p(A), _p(keep), nrows, k, n, r, p, _p(dX))
    return dX


def dora_norm(W, A, B, alpha, cols=None) -> np.ndarray:
    """|| W[:, j] + alpha (A B)[:, j] ||_2 for j in cols (all columns by default);
    the page on the factored DoRA norm, "core method" (the norm of W + sBA per
    output feature), written densely."""
    W, A, B = _f64(W), _f64(A), _f64(B)
    k, n = W.shape
    r = A.shape[1]
    cols = np.arange(n, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    out = np.zeros(len(cols), dtype=np.float64)
    if len(cols):
        _load().oracle_dora_norm(_p(W), _p(A), _p(B), k, n, r, float(alpha), _p(cols), len(cols), _p(out))
    return out


def lora_db_acc(S, dY, alpha, dB: np.ndarray) -> None:
    S, dY = _f64(S), _f64(dY)
    nrows, n = dY.shape
    r = S.shape[1]
    assert dB.dtype == np.float64 and dB.flags.c_contiguous and dB.shape == (r, n)
    if nrows:
        _load().oracle_lora_db_acc(_p(S), _p(dY), nrows, n, r, alpha, _p(dB))


def lora_da_acc(X, keep, dS, p, dA: np.ndarray) -> None:
    X, dS = _f64(X), _f64(dS)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    nrows, k = X.shape
    r = dS.shape[1]
    assert dA.dtype == np.float64 and dA.flags.c_contiguous and dA.shape == (k, r)
    if nrows:
        _load().oracle_lora_da_acc(_p(X), _p(keep), _p(dS), nrows, k, r, p, _p(dA))


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
def lora_fwd(X, W, A, B, alpha, p, seed, offset, rows=None):
    """Forward for one adapter.  ``rows`` (global indices of the rows of X
    given) defaults to 0..m-1.  Returns dict(Y, S, keep)."""
    X = _f64(X)
    if rows is None:
        rows = np.arange(X.shape[0], dtype=np.int64)
    keep = keep_mask(seed, offset, rows, X.shape[1], p)
    S = lora_s(X, keep, A, p)
    Y = lora_y(X, W, S, B, alpha)
    return {"Y": Y, "S": S, "keep": keep}


def lora_bwd(dY, X, W, A, B, alpha, p, seed, offset, rows=None):
    """Backward for one adapter (recomputes the forward's mask and S).
    Returns dict(dX, dA, dB, dS, S, keep)."""
    X = _f64(X)
    if rows is None:
        rows = np.arange(X.shape[0], dtype=np.int64)
    keep = keep_mask(seed, offset, rows, X.shape[1], p)
    S = lora_s(X, keep, A, p)
    dS = lora_ds(dY, B, alpha)
    r = np.asarray(A).shape[1]
    dB = np.zeros((r, np.asarray(W).shape[1]))
    lora_db_acc(S, dY, alpha, dB)
    dA = np.zeros((X.shape[1], r))
    lora_da_acc(X, keep, dS, p, dA)
    dX = lora_dx(dY, W, dS, A, keep, p)
    return {"dX": dX, "dA": dA, "dB": dB, "dS": dS, "S": S, "keep": keep}


def segments_rows(seg_off, seg_adapter):
    """Yield (lo, hi, adapter) for every non-empty segment, in order."""
    for s in range(len(seg_adapter)):
        lo, hi = int(seg_off[s]), int(seg_off[s + 1])
        if hi > lo:
            yield lo, hi, int(seg_adapter[s])


def multi_lora_fwd(X, W, adapters, seg_off, seg_adapter, r_max, seed, offset):
    """adapters: list of dicts with A, B, alpha, p.  Returns dict(Y, S, keep)
    with S m x r_max (zero beyond each row's rank)."""
    X, W = _f64(X), _f64(W)
    m, k = X.shape
    n = W.shape[1]
    Y = np.zeros((m, n))
    S = np.zeros((m, r_max))
    keep = np.ones((m, k), dtype=np.uint8)
    for lo, hi, a in segments_rows(seg_off, seg_adapter):
        ad = adapters[a]
        out = lora_fwd(X[lo:hi], W, ad["A"], ad["B"], ad["alpha"], ad["p"], seed, offset,
                       rows=np.arange(lo, hi, dtype=np.int64))
        Y[lo:hi] = out["Y"]
        S[lo:hi, : out["S"].shape[1]] = out["S"]
        keep[lo:hi] = out["keep"]
    return {"Y": Y, "S": S, "keep": keep}


def multi_lora_bwd(dY, X, W, adapters, seg_off, seg_adapter, r_max, seed, offset):
    """Returns dict(dX, dA: list, dB: list, dS m x r_max)."""
    X, W, dY = _f64(X), _f64(W), _f64(dY)
    m, k = X.shape
    n = W.shape[1]
    dX = np.zeros((m, k))
    dS = np.zeros((m, r_max))
    dA = [np.zeros((k, np.asarray(ad["A"]).shape[1])) for ad in adapters]
    dB = [np.zeros((np.asarray(ad["B"]).shape[0], n)) for ad in adapters]
    for lo, hi, a in segments_rows(seg_off, seg_adapter):
        ad = adapters[a]
        out = lora_bwd(dY[lo:hi], X[lo:hi], W, ad["A"], ad["B"], ad["alpha"], ad["p"], seed,
                       offset, rows=np.arange(lo, hi, dtype=np.int64))
        dX[lo:hi] = out["dX"]
        dS[lo:hi, : out["dS"].shape[1]] = out["dS"]
        dA[a] += out["dA"]
        dB[a] += out["dB"]
    return {"dX": dX, "dA": dA, "dB": dB, "dS": dS}


# ----------------------------------------------------------------------------
# Sampled evaluation for large shapes
# ----------------------------------------------------------------------------
def lora_sampled(X, W, A, B, dY, alpha, p, seed, offset, out_rows, a_rows, b_cols, rows=None):
    """Forward and backward of one adapter where the m*k*n-sized results are
    evaluated only at samples: Y and dX on local rows ``out_rows``, dA on rows
    ``a_rows`` (input features), dB on columns ``b_cols``.  The mask, S and dS
    are computed in full.  Every sampled entry is what ``lora_fwd`` /
    ``lora_bwd`` give at that position: the same functions run on a subset of
    rows (Y, dX) or columns (dA, dB), each entry's sum in the same order."""
    X, dY = _f64(X), _f64(dY)
    m, k = X.shape
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    out_rows = np.asarray(out_rows, dtype=np.int64)
    a_rows = np.asarray(a_rows, dtype=np.int64)
    b_cols = np.asarray(b_cols, dtype=np.int64)
    r = np.asarray(A).shape[1]
    keep = keep_mask(seed, offset, rows, k, p)
    S = lora_s(X, keep, A, p)
    dS = lora_ds(dY, B, alpha)
    Y = lora_y(X[out_rows], W, S[out_rows], B, alpha)
    dX = lora_dx(dY[out_rows], W, dS[out_rows], A, np.ascontiguousarray(keep[out_rows]), p)
    dB = np.zeros((r, b_cols.size))
    lora_db_acc(S, np.ascontiguousarray(dY[:, b_cols]), alpha, dB)
    dA = np.zeros((a_rows.size, r))
    lora_da_acc(np.ascontiguousarray(X[:, a_rows]), np.ascontiguousarray(keep[:, a_rows]), dS, p, dA)
    return {"Y": Y, "dX": dX, "dA": dA, "dB": dB, "S": S, "dS": dS, "keep": keep}


def multi_lora_sampled(X, W, adapters, dY, seg_off, seg_adapter, r_max, seed, offset, out_rows,
                       a_rows, b_cols):
    """Mixed-adapter counterpart of ``lora_sampled``: ``out_rows`` are sorted
    global row indices; Y and dX come back in that order, dA / dB per adapter
    on the sampled features / columns (summed over the adapter's segments, in
    segment order, as in ``multi_lora_bwd``), S (m x r_max) and the mask in
    full."""
    X, dY = _f64(X), _f64(dY)
    m, k = X.shape
    n = np.asarray(W).shape[1]
    out_rows = np.asarray(out_rows, dtype=np.int64)
    a_rows = np.asarray(a_rows, dtype=np.int64)
    b_cols = np.asarray(b_cols, dtype=np.int64)
    Y = np.zeros((out_rows.size, n))
    dX = np.zeros((out_rows.size, k))
    S = np.zeros((m, r_max))
    keep = np.ones((m, k), dtype=np.uint8)
    dA = [np.zeros((a_rows.size, np.asarray(ad["A"]).shape[1])) for ad in adapters]
    dB = [np.zeros((np.asarray(ad["B"]).shape[0], b_cols.size)) for ad in adapters]
    for lo, hi, a in segments_rows(seg_off, seg_adapter):
        ad = adapters[a]
        sel = np.nonzero((out_rows >= lo) & (out_rows < hi))[0]
        out = lora_sampled(X[lo:hi], W, ad["A"], ad["B"], dY[lo:hi], ad["alpha"], ad["p"], seed,
                           offset, out_rows[sel] - lo, a_rows, b_cols,
                           rows=np.arange(lo, hi, dtype=np.int64))
        Y[sel] = out["Y"]
        dX[sel] = out["dX"]
        S[lo:hi, : out["S"].shape[1]] = out["S"]
        keep[lo:hi] = out["keep"]
        dA[a] += out["dA"]
        dB[a] += out["dB"]
    return {"Y": Y, "dX": dX, "dA": dA, "dB": dB, "S": S, "keep": keep}
