"""ctypes binding of liblora_fused.so.

Argument marshalling only: every function here has the name of a C-ABI entry
point in include/lora_fused.h, takes torch device tensors, checks their dtype
and contiguity, and passes raw pointers plus the current HIP stream.  PyTorch
supplies device memory and streams; every step of the layer runs in the
library's HIP kernels.  There is no fallback: if the library is missing or was
built for something else, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblora_fused.so")

LORA_OK = 0
STATUS_NAMES = {0: "LORA_OK", -1: "LORA_ERR_INVALID_ARG", -2: "LORA_ERR_UNSUPPORTED",
                -3: "LORA_ERR_WORKSPACE", -4: "LORA_ERR_HIP"}

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = [
    "lora_linear_fwd_workspace_size", "lora_linear_fwd", "lora_linear_bwd_workspace_size",
    "lora_linear_bwd", "multi_lora_fwd_workspace_size", "multi_lora_linear_fwd",
    "multi_lora_bwd_workspace_size", "multi_lora_linear_bwd", "multi_lora_check_segments",
    "lora_dropout_mask", "lora_frozen_fwd", "lora_frozen_bwd", "lora_profiling_enable",
    "lora_profiling_reset", "lora_profiling_query", "lora_status_string",
    "lora_last_error_message", "lora_pack_greedy", "lora_microbatch_segments",
    "lora_check_bubble_lemma", "lora_dora_norm_workspace_size", "lora_dora_norm",
    "lora_linear_bwd_noalloc_max_scratch", "lora_linear_bwd_noalloc", "lora_linear_fwd_concat",
]


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class LoraAdapter(ctypes.Structure):
    """Mirror of lora_adapter (48 bytes)."""
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("dA", ctypes.c_void_p),
                ("dB", ctypes.c_void_p), ("r", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("p", ctypes.c_float), ("reserved", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with __graft_entry__.build() "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, I32, I64, U64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_float, ctypes.c_size_t)
    sigs = {
        "lora_linear_fwd_workspace_size": (SZ, [I64, I64, I64, I32]),
        "lora_linear_bwd_workspace_size": (SZ, [I64, I64, I64, I32]),
        "multi_lora_fwd_workspace_size": (SZ, [I64, I64, I64, I32, I32, I32]),
        "multi_lora_bwd_workspace_size": (SZ, [I64, I64, I64, I32, I32, I32]),
        "lora_linear_fwd": (I32, [P, P, P, P, I64, I64, I64, I32, F32, F32, U64, U64, P, P, P, P,
                                  SZ, P]),
        "lora_linear_bwd": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I32, F32, F32, P, P, P, P,
                                  SZ, P]),
        "lora_linear_fwd_concat": (I32, [P, P, P, P, I64, I64, I64, I32, F32, P, P, P]),
        "lora_linear_bwd_noalloc_max_scratch": (SZ, []),
        "lora_linear_bwd_noalloc": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I32, F32, F32, P, P, P, P]),
        "multi_lora_linear_fwd": (I32, [P, P, P, I32, P, P, I32, I64, I64, I64, I32, U64, U64, P,
                                        P, P, P, SZ, P]),
        "multi_lora_linear_bwd": (I32, [P, P, P, P, I32, P, P, I32, P, P, I64, I64, I64, I32, P,
                                        P, SZ, P]),
        "multi_lora_check_segments": (I32, [P, P, I32, I64, P, I32, I32]),
        "lora_pack_greedy": (I32, [P, I32, I64, P, P]),
        "lora_dora_norm_workspace_size": (SZ, [I64, I64, I32]),
        "lora_dora_norm": (I32, [P, P, P, I64, I64, I32, F32, P, P, SZ, P]),
        "lora_microbatch_segments": (I32, [P, P, P, I32, I32, I32, P, P, P, P, P]),
        "lora_check_bubble_lemma": (I32, [P, P, P, I32, I32, I32, P]),
        "lora_dropout_mask": (I32, [U64, U64, I64, I64, F32, P, P]),
        "lora_frozen_fwd": (I32, [P, P, I64, I64, I64, P, P]),
        "lora_frozen_bwd": (I32, [P, P, I64, I64, I64, P, P]),
        "lora_profiling_enable": (I32, [I32, I32]),
        "lora_profiling_reset": (I32, []),
        "lora_profiling_query": (I32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_double)]),
        "lora_status_string": (ctypes.c_char_p, [I32]),
        "lora_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != LORA_OK:
        msg = load().lora_last_error_message().decode(errors="replace")
        raise LoraError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def lora_linear_fwd_workspace_size(m, k, n, r) -> int:
    return int(load().lora_linear_fwd_workspace_size(m, k, n, r))


def lora_linear_bwd_workspace_size(m, k, n, r) -> int:
    return int(load().lora_linear_bwd_workspace_size(m, k, n, r))


def multi_lora_fwd_workspace_size(m, k, n, r_max, num_adapters, num_segments) -> int:
    return int(load().multi_lora_fwd_workspace_size(m, k, n, r_max, num_adapters, num_segments))


def multi_lora_bwd_workspace_size(m, k, n, r_max, num_adapters, num_segments) -> int:
    return int(load().multi_lora_bwd_workspace_size(m, k, n, r_max, num_adapters, num_segments))


def lora_linear_fwd(X, W, A, B, alpha: float, p: float, seed: int = 0, offset: int = 0, *,
                    Y=None, S=None, keep_bits=None, workspace=None, stream=None):
    """Returns (Y, S, keep_bits); outputs are allocated when not given."""
    for t, nm in ((X, "X"), (W, "W"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm)
    m, k = X.shape
    n = W.shape[1]
    r = A.shape[1]
    dev = X.device
    if Y is None:
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    if S is None:
        S = torch.empty((m, r), dtype=torch.float32, device=dev)
    if keep_bits is None and p != 0.0:
        keep_bits = torch.empty((m, (k + 31) // 32), dtype=torch.int32, device=dev)
    ws = _workspace(lora_linear_fwd_workspace_size(m, k, n, r), dev, workspace)
    _check(load().lora_linear_fwd(_ptr(X), _ptr(W), _ptr(A), _ptr(B), m, k, n, r, alpha, p, seed,
                                  offset, _ptr(Y), _ptr(S), _ptr(keep_bits), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return Y, S, keep_bits


def lora_linear_fwd_concat(X, W, A, B, alpha: float, *, Y=None, S=None, stream=None):
    """The forward at p = 0 with [W | A] as one operand.  Returns (Y, S);
    outputs are allocated when not given.  r must be 8 or 16."""
    for t, nm in ((X, "X"), (W, "W"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm)
    m, k = X.shape
    n = W.shape[1]
    r = A.shape[1]
    dev = X.device
    if Y is None:
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    if S is None:
        S = torch.empty((m, r), dtype=torch.float32, device=dev)
    _check(load().lora_linear_fwd_concat(_ptr(X), _ptr(W), _ptr(A), _ptr(B), m, k, n, r, alpha, _ptr(Y),
                                         _ptr(S), _stream(stream)))
    return Y, S


def lora_linear_bwd(dY, X, W, A, B, S, keep_bits, alpha: float, p: float, *, dX=None, dA=None,
                    dB=None, workspace=None, stream=None, want_dX: bool = True):
    """Returns (dX, dA, dB); dX is None (and its GEMM skipped) when want_dX is False."""
    for t, nm in ((dY, "dY"), (X, "X"), (W, "W"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm)
    _need(S, torch.float32, "S")
    m, k = X.shape
    n = W.shape[1]
    r = A.shape[1]
    dev = X.device
    if want_dX and dX is None:
        dX = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    if not want_dX:
        dX = None
    dA = torch.empty((k, r), dtype=torch.bfloat16, device=dev) if dA is None else dA
    dB = torch.empty((r, n), dtype=torch.bfloat16, device=dev) if dB is None else dB
    ws = _workspace(lora_linear_bwd_workspace_size(m, k, n, r), dev, workspace)
    _check(load().lora_linear_bwd(_ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(S),
                                  _ptr(keep_bits), m, k, n, r, alpha, p, _ptr(dX), _ptr(dA),
                                  _ptr(dB), _ptr(ws), ws.numel(), _stream(stream)))
    return dX, dA, dB


def lora_linear_bwd_noalloc_max_scratch() -> int:
    return int(load().lora_linear_bwd_noalloc_max_scratch())


def lora_linear_bwd_noalloc(dY, X, W, A, B, S, keep_bits, alpha: float, p: float, dX, dA, dB, *,
                            stream=None):
    """lora_linear_bwd without a workspace (the library's static scratch);
    every output must be given, since the point is to allocate nothing."""
    for t, nm in ((dY, "dY"), (X, "X"), (W, "W"), (A, "A"), (B, "B"), (dA, "dA"), (dB, "dB")):
        _need(t, torch.bfloat16, nm)
    _need(S, torch.float32, "S")
    if dX is not None:
        _need(dX, torch.bfloat16, "dX")
    m, k = X.shape
    n = W.shape[1]
    r = A.shape[1]
    _check(load().lora_linear_bwd_noalloc(_ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(S),
                                          _ptr(keep_bits), m, k, n, r, alpha, p, _ptr(dX), _ptr(dA),
                                          _ptr(dB), _stream(stream)))
    return dX, dA, dB


def _check_adapters(As, Bs, alphas, ps, dAs=None, dBs=None, k=None, n=None):
    """Host checks of a mixed-adapter set that the library cannot make (its
    table lives on the device): bf16, contiguous device tensors; A_i k x r_i and
    B_i r_i x n with 1 <= r_i <= 256 and the same k and n for every adapter;
    finite alpha; 0 <= p < 1 (as the float32 the table stores); gradient
    buffers shaped like their parameters.  Returns (k, n, ranks)."""
    na = len(As)
    if na < 1 or len(Bs) != na or len(alphas) != na or len(ps) != na:
        raise ValueError("As, Bs, alphas and ps must have the same, non-zero length")
    for grads, nm in ((dAs, "dAs"), (dBs, "dBs")):
        if grads is not None and len(grads) != na:
            raise ValueError(f"{nm} must have one tensor per adapter")
    k = As[0].shape[0] if k is None else int(k)
    n = Bs[0].shape[1] if n is None else int(n)
    dev = As[0].device
    ranks = []
    for i in range(na):
        A, B = As[i], Bs[i]
        for t, nm in ((A, f"A[{i}]"), (B, f"B[{i}]")):
            if t.dtype != torch.bfloat16:
                raise TypeError(f"{nm} must be torch.bfloat16, got {t.dtype}")
            if not t.is_contiguous():
                raise ValueError(f"{nm} must be contiguous")
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError(f"adapter {i}: A and B must be 2-D")
        r = A.shape[1]
        if A.shape[0] != k or B.shape != (r, n):
            raise ValueError(f"adapter {i}: A {tuple(A.shape)} and B {tuple(B.shape)} do not fit "
                             f"k = {k}, n = {n} (A must be k x r, B r x n)")
        if not 1 <= r <= 256:
            raise ValueError(f"adapter {i}: rank {r} outside [1, 256]")
        with np.errstate(over="ignore"):
            a32, p32 = np.float32(alphas[i]), np.float32(ps[i])
        if not np.isfinite(a32):
            raise ValueError(f"adapter {i}: alpha {alphas[i]} is not finite")
        if not (p32 >= 0.0 and p32 < 1.0):
            raise ValueError(f"adapter {i}: dropout p = {ps[i]} must be in [0, 1)")
        for grads, ref, nm in ((dAs, A, "dA"), (dBs, B, "dB")):
            if grads is None:
                continue
            g = grads[i]
            if g.dtype != torch.bfloat16 or not g.is_contiguous() or g.shape != ref.shape:
                raise ValueError(f"adapter {i}: {nm} must be a contiguous bf16 {tuple(ref.shape)} tensor")
        ranks.append(r)
    # device last, so that host tests can reach every other check with CPU tensors
    for i in range(na):
        ts = [As[i], Bs[i]] + [g[i] for g in (dAs, dBs) if g is not None]
        if any(t.device.type != "cuda" or t.device != dev for t in ts):
            raise ValueError(f"adapter {i}: every tensor must be on one GPU ({dev})")
    return k, n, ranks


def _pack_table(As, Bs, alphas, ps, dA_ptrs, dB_ptrs) -> bytes:
    na = len(As)
    recs = (LoraAdapter * na)()
    for i in range(na):
        recs[i].A = As[i].data_ptr()
        recs[i].B = Bs[i].data_ptr()
        recs[i].dA = dA_ptrs[i]
        recs[i].dB = dB_ptrs[i]
        recs[i].r = As[i].shape[1]
        recs[i].alpha = float(alphas[i])
        recs[i].p = float(ps[i])
        recs[i].reserved = 0
    return bytes(recs)


def adapter_table(As: Sequence[torch.Tensor], Bs: Sequence[torch.Tensor], alphas, ps,
                  dAs: Optional[Sequence[torch.Tensor]] = None,
                  dBs: Optional[Sequence[torch.Tensor]] = None, device=None, *,
                  k: Optional[int] = None, n: Optional[int] = None) -> torch.Tensor:
    """Pack lora_adapter records into a device uint8 tensor (the table the
    multi-adapter calls read on the device), after the host checks of
    _check_adapters.  The table remembers k, n and the ranks, which the
    multi-adapter wrappers check against X, W and r_max."""
    k, n, ranks = _check_adapters(As, Bs, alphas, ps, dAs, dBs, k, n)
    raw = _pack_table(As, Bs, alphas, ps,
                      [d.data_ptr() for d in dAs] if dAs is not None else [0] * len(As),
                      [d.data_ptr() for d in dBs] if dBs is not None else [0] * len(As))
    host = torch.frombuffer(bytearray(raw), dtype=torch.uint8)
    table = host.to(device if device is not None else As[0].device)
    table._lora_meta = (k, n, tuple(ranks))
    return table


def _check_table(adapters: torch.Tensor, num_adapters: int, k: int, n: int, r_max: int) -> None:
    if adapters.dtype != torch.uint8 or adapters.device.type != "cuda" or not adapters.is_contiguous():
        raise ValueError("adapters must be a contiguous device uint8 table (see adapter_table)")
    if adapters.numel() < num_adapters * ctypes.sizeof(LoraAdapter):
        raise ValueError(f"adapter table holds fewer than {num_adapters} records")
    meta = getattr(adapters, "_lora_meta", None)
    if meta is not None:
        tk, tn, ranks = meta
        if (tk, tn) != (k, n):
            raise ValueError(f"adapter table was built for k = {tk}, n = {tn}; X and W give k = {k}, n = {n}")
        if len(ranks) != num_adapters:
            raise ValueError(f"adapter table has {len(ranks)} adapters, num_adapters = {num_adapters}")
        if max(ranks) > r_max:
            raise ValueError(f"r_max = {r_max} is below the largest adapter rank {max(ranks)}")


def multi_lora_linear_fwd(X, W, adapters: torch.Tensor, num_adapters: int, seg_off, seg_adapter,
                          r_max: int, seed: int = 0, offset: int = 0, *, Y=None, S=None,
                          keep_bits=None, workspace=None, stream=None):
    _need(X, torch.bfloat16, "X")
    _need(W, torch.bfloat16, "W")
    _need(seg_off, torch.int64, "seg_off")
    _need(seg_adapter, torch.int32, "seg_adapter")
    m, k = X.shape
    n = W.shape[1]
    _check_table(adapters, num_adapters, k, n, r_max)
    nseg = seg_adapter.numel()
    dev = X.device
    Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if Y is None else Y
    S = torch.empty((m, r_max), dtype=torch.float32, device=dev) if S is None else S
    if keep_bits is None:
        keep_bits = torch.empty((m, (k + 31) // 32), dtype=torch.int32, device=dev)
    ws = _workspace(multi_lora_fwd_workspace_size(m, k, n, r_max, num_adapters, nseg), dev,
                    workspace)
    _check(load().multi_lora_linear_fwd(_ptr(X), _ptr(W), _ptr(adapters), num_adapters,
                                        _ptr(seg_off), _ptr(seg_adapter), nseg, m, k, n, r_max,
                                        seed, offset, _ptr(Y), _ptr(S), _ptr(keep_bits), _ptr(ws),
                                        ws.numel(), _stream(stream)))
    return Y, S, keep_bits


def multi_lora_linear_bwd(dY, X, W, adapters: torch.Tensor, num_adapters: int, seg_off,
                          seg_adapter, S, keep_bits, r_max: int, *, dX=None, workspace=None,
                          stream=None, want_dX: bool = True):
    _need(dY, torch.bfloat16, "dY")
    _need(X, torch.bfloat16, "X")
    _need(W, torch.bfloat16, "W")
    _need(S, torch.float32, "S")
    m, k = X.shape
    n = W.shape[1]
    _check_table(adapters, num_adapters, k, n, r_max)
    nseg = seg_adapter.numel()
    dev = X.device
    if want_dX and dX is None:
        dX = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    if not want_dX:
        dX = None
    ws = _workspace(multi_lora_bwd_workspace_size(m, k, n, r_max, num_adapters, nseg), dev,
                    workspace)
    _check(load().multi_lora_linear_bwd(_ptr(dY), _ptr(X), _ptr(W), _ptr(adapters), num_adapters,
                                        _ptr(seg_off), _ptr(seg_adapter), nseg, _ptr(S),
                                        _ptr(keep_bits), m, k, n, r_max, _ptr(dX), _ptr(ws),
                                        ws.numel(), _stream(stream)))
    return dX


def multi_lora_check_segments(seg_off: Sequence[int], seg_adapter: Sequence[int], m: int,
                              ranks: Sequence[int], r_max: int) -> None:
    so = (ctypes.c_int64 * len(seg_off))(*[int(v) for v in seg_off])
    sa = (ctypes.c_int32 * len(seg_adapter))(*[int(v) for v in seg_adapter])
    rk = (ctypes.c_int32 * len(ranks))(*[int(v) for v in ranks])
    _check(load().multi_lora_check_segments(so, sa, len(seg_adapter), m, rk, len(ranks), r_max))


def lora_dora_norm_workspace_size(k: int, n: int, r: int) -> int:
    return int(load().lora_dora_norm_workspace_size(k, n, r))


def lora_dora_norm(W, A, B, alpha: float, *, norm=None, workspace=None, stream=None):
    """norm[j] = || W[:, j] + alpha (A B)[:, j] ||_2 (fp32, n values)."""
    _need(W, torch.bfloat16, "W")
    _need(A, torch.bfloat16, "A")
    _need(B, torch.bfloat16, "B")
    k, n = W.shape
    r = A.shape[1]
    norm = torch.empty(n, dtype=torch.float32, device=W.device) if norm is None else norm
    ws = _workspace(lora_dora_norm_workspace_size(k, n, r), W.device, workspace)
    _check(load().lora_dora_norm(_ptr(W), _ptr(A), _ptr(B), k, n, r, alpha, _ptr(norm), _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return norm


def _i32_array(values: Sequence[int]):
    return (ctypes.c_int32 * max(len(values), 1))(*[int(v) for v in values])


def lora_pack_greedy(lengths: Sequence[int], capacity: int) -> Tuple[List[int], int]:
    """(microbatch of each sample, number of microbatches); host only."""
    n = len(lengths)
    mb = (ctypes.c_int32 * max(n, 1))()
    nmb = ctypes.c_int32(0)
    _check(load().lora_pack_greedy(_i32_array(lengths), n, capacity, mb, ctypes.byref(nmb)))
    return list(mb[:n]), nmb.value


def lora_microbatch_segments(lengths: Sequence[int], adapter_of_sample: Sequence[int],
                             mb_of_sample: Sequence[int], num_adapters: int,
                             mb: int) -> Tuple[List[int], List[int], List[int]]:
    """(sample order, seg_off, seg_adapter) of microbatch `mb`; host only."""
    n = len(lengths)
    order = (ctypes.c_int32 * max(n, 1))()
    so = (ctypes.c_int64 * (num_adapters + 1))()
    sa = (ctypes.c_int32 * num_adapters)()
    nm, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().lora_microbatch_segments(_i32_array(lengths), _i32_array(adapter_of_sample),
                                           _i32_array(mb_of_sample), n, num_adapters, mb, order,
                                           ctypes.byref(nm), so, sa, ctypes.byref(ns)))
    return list(order[:nm.value]), list(so[:ns.value + 1]), list(sa[:ns.value])


def lora_check_bubble_lemma(mb_of_sample: Sequence[int], adapter_of_sample: Sequence[int],
                            batch_of_sample: Sequence[int], num_adapters: int, stages: int) -> int:
    """Number of (adapter, batch) pairs whose next batch starts too early; host only."""
    v = ctypes.c_int64(0)
    _check(load().lora_check_bubble_lemma(_i32_array(mb_of_sample), _i32_array(adapter_of_sample),
                                          _i32_array(batch_of_sample), len(mb_of_sample),
                                          num_adapters, stages, ctypes.byref(v)))
    return v.value


def lora_dropout_mask(seed: int, offset: int, m: int, k: int, p: float, keep_bits=None,
                      device="cuda", stream=None):
    if keep_bits is None:
        keep_bits = torch.empty((m, (k + 31) // 32), dtype=torch.int32, device=device)
    _check(load().lora_dropout_mask(seed, offset, m, k, p, _ptr(keep_bits), _stream(stream)))
    return keep_bits


def lora_frozen_fwd(X, W, *, Y=None, stream=None):
    m, k = X.shape
    n = W.shape[1]
    Y = torch.empty((m, n), dtype=torch.bfloat16, device=X.device) if Y is None else Y
    _check(load().lora_frozen_fwd(_ptr(X), _ptr(W), m, k, n, _ptr(Y), _stream(stream)))
    return Y


def lora_frozen_bwd(dY, W, *, dX=None, stream=None):
    m, n = dY.shape
    k = W.shape[0]
    dX = torch.empty((m, k), dtype=torch.bfloat16, device=dY.device) if dX is None else dX
    _check(load().lora_frozen_bwd(_ptr(dY), _ptr(W), m, k, n, _ptr(dX), _stream(stream)))
    return dX


def lora_profiling_enable(enable: bool = True, capacity: int = 4096) -> None:
    _check(load().lora_profiling_enable(1 if enable else 0, capacity))


def lora_profiling_reset() -> None:
    _check(load().lora_profiling_reset())


def lora_profiling_query(name_substring: str):
    """(launches, total_ms) of timed kernels whose name contains the string."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(load().lora_profiling_query(name_substring.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)
