"""Thin Python binding of libgdn (include/gdn.h): same names as the C entry points.

Only argument marshalling happens here: tensors become device pointers, lists
become host int32 arrays, and shapes, dtypes and devices are checked against
the call's dims so that no buffer the C library cannot size-check is ever
under-allocated.  Every step of the computation runs in the HIP kernels; if the
built library is missing this module raises instead of falling back to anything.
PyTorch only provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY: another build of the library to load instead (the host-only sanitizer
# build, whose launches are stubbed out, runs the validation tests under ASan/UBSan)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "libgdn.so")
_lib = None

GDN_OK = 0
ROUTE_RECURRENT = 0
ROUTE_CHUNKED = 1
MAX_K = 3
QK_L2NORM = 1  # gdn_dims.flags: q and k are raw; the kernels normalise them (q also by 1/sqrt(d_k))

_ERRORS = {-1: "GDN_E_NULL", -2: "GDN_E_UNSUPPORTED", -3: "GDN_E_RANGE", -4: "GDN_E_ALIAS",
           -5: "GDN_E_ALIGN", -6: "GDN_E_WORKSPACE", -7: "GDN_E_HIP"}


class GdnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__("%s returned %s (%d)" % (fn, _ERRORS.get(code, "?"), code))


class _Dims(ctypes.Structure):
    _fields_ = [("n_qk_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


@dataclass(frozen=True)
class Dims:
    n_qk_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    k_max: int = 3
    flags: int = 0  # 0 or QK_L2NORM

    def c(self) -> _Dims:
        return _Dims(self.n_qk_heads, self.n_v_heads, self.d_k, self.d_v, self.k_max, self.flags)


_VP = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "gdn_decode_step": [ctypes.POINTER(_Dims), ctypes.c_int32] + [_VP] * 8 + [ctypes.c_int32] + [_VP] * 4,
    "gdn_verify_window": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P] + [_VP] * 8 +
                         [ctypes.c_int32, _I32P, _VP, _VP, _VP],
    "gdn_commit_accepted": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _VP, _VP, _VP,
                            ctypes.c_int32, _I32P, _VP, _VP],
    "gdn_verify_tree": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _I32P] + [_VP] * 8 +
                       [ctypes.c_int32, _I32P, _VP, _VP, _VP],
    "gdn_verify_window_delta": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P] + [_VP] * 8 +
                               [ctypes.c_int32, _I32P, _VP, _VP, _VP],
    "gdn_verify_window_delta_fold": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P] + [_VP] * 8 +
                                    [ctypes.c_int32, _I32P, _VP, _VP, _I32P, _VP, _VP, _VP, _VP, _VP],
    "gdn_commit_delta": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _VP, _VP, _VP, _VP,
                         ctypes.c_int32, _I32P, _I32P, _VP, _VP],
    "gdn_verify_window_select": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P] + [_VP] * 8 +
                                [ctypes.c_int32, _VP, _I32P, _VP, _VP, _VP],
    "gdn_verify_window_select_commit": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _I32P, _I32P, _VP] +
                                       [_VP] * 8 + [ctypes.c_int32, _VP, _I32P, _VP, _VP, _VP],
    "gdn_commit_select": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _VP, _I32P, ctypes.c_int32, _VP, _VP,
                          _VP],
    "gdn_commit_replay": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P] + [_VP] * 8 +
                         [_VP, ctypes.c_int32, _I32P, _I32P, _VP, _VP],
    "gdn_chunked_workspace_bytes": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, ctypes.c_int32],
    "gdn_chunked_prefill_with_checkpoints": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P,
                                             ctypes.c_int32, _I32P] + [_VP] * 8 +
                                            [ctypes.c_int32, _I32P, _I32P, _VP, _VP, _VP,
                                             ctypes.c_size_t, _VP],
    "gdn_chunked_prefill_with_checkpoints_static": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P,
                                                    ctypes.c_int32, _I32P] + [_VP] * 8 +
                                                   [ctypes.c_int32, _I32P, _I32P, _VP, _VP, _VP],
    "gdn_plan_transaction": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _I32P],
    "gdn_run_transaction": [ctypes.POINTER(_Dims), ctypes.c_int32, _I32P, _I32P] + [_VP] * 8 +
                           [ctypes.c_int32, _I32P, _I32P, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "gdn_status_str": [ctypes.c_int],
    "gdn_version": [],
}
_RES = {"gdn_chunked_workspace_bytes": ctypes.c_size_t, "gdn_status_str": ctypes.c_char_p}


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: the library's HIP runtime dependency then resolves to the one
        # torch loaded, so both share one runtime (streams, device memory)
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError("libgdn.so is not built (%s); run "
                              "`python -m gateddeltanet_linear_attention_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = _RES.get(name, ctypes.c_int)
        _lib = l
    return _lib


# ------------------------------------------------------------------ marshalling

def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32).ravel())


def _ip(arr: np.ndarray):
    return arr.ctypes.data_as(_I32P)


def _dev(t, name: str, dtype, shape):
    """Pointer of a contiguous device tensor after checking dtype and shape."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return _VP(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return _VP(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, rc: int):
    if rc != GDN_OK:
        raise GdnError(fn, rc)


def _token_ptrs(dims: Dims, N: int, q, k, v, a, b, A_log, dt_bias, o):
    import torch
    Hq, Hv, d = dims.n_qk_heads, dims.n_v_heads, dims.d_k
    return [_dev(q, "q", torch.bfloat16, (N, Hq, d)), _dev(k, "k", torch.bfloat16, (N, Hq, d)),
            _dev(v, "v", torch.bfloat16, (N, Hv, dims.d_v)),
            _dev(a, "a", torch.float32, (N, Hv)), _dev(b, "b", torch.float32, (N, Hv)),
            _dev(A_log, "A_log", torch.float32, (Hv,)), _dev(dt_bias, "dt_bias", torch.float32, (Hv,))], \
        _dev(o, "o", torch.bfloat16, (N, Hv, dims.d_v))


def _pool(dims: Dims, state_pool):
    import torch
    n_slots = int(state_pool.shape[0]) if hasattr(state_pool, "shape") else 0
    return _dev(state_pool, "state_pool", torch.float32,
                (n_slots, dims.n_v_heads, dims.d_v, dims.d_k)), n_slots


def _ckpt(dims: Dims, ckpt, n_rows: int, optional: bool = False):
    import torch
    if ckpt is None and optional:
        return _VP(0)
    return _dev(ckpt, "ckpt", torch.float32,
                (n_rows, dims.k_max + 1, dims.n_v_heads, dims.d_v, dims.d_k))


def _token_in_ptrs(dims: Dims, N: int, q, k, v, a, b, A_log, dt_bias):
    import torch
    Hq, Hv, d = dims.n_qk_heads, dims.n_v_heads, dims.d_k
    return [_dev(q, "q", torch.bfloat16, (N, Hq, d)), _dev(k, "k", torch.bfloat16, (N, Hq, d)),
            _dev(v, "v", torch.bfloat16, (N, Hv, dims.d_v)),
            _dev(a, "a", torch.float32, (N, Hv)), _dev(b, "b", torch.float32, (N, Hv)),
            _dev(A_log, "A_log", torch.float32, (Hv,)), _dev(dt_bias, "dt_bias", torch.float32, (Hv,))]


# ------------------------------------------------------------------ entry points

def gdn_version() -> int:
    return lib().gdn_version()


def gdn_status_str(code: int) -> str:
    return lib().gdn_status_str(code).decode()


def _decode_args(dims: Dims, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, dst_slot, o, stream):
    src, dst = _i32(src_slot), _i32(dst_slot)
    n_rows = src.size
    if dst.size != n_rows:
        raise ValueError("src_slot and dst_slot lengths differ")
    toks, op = _token_ptrs(dims, n_rows, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, *toks, pp, n_slots, _ip(src), _ip(dst), op, _stream(stream))
    return args, (cd, src, dst, q, k, v, a, b, A_log, dt_bias, state_pool, o)


def gdn_decode_step(dims: Dims, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, dst_slot, o,
                    stream=None) -> None:
    """One token per row; new state of row r to slot dst_slot[r]."""
    args, _keep = _decode_args(dims, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, dst_slot, o, stream)
    _check("gdn_decode_step", lib().gdn_decode_step(*args))


def prepare_decode_step(dims: Dims, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, dst_slot, o,
                        stream=None) -> "PreparedCall":
    args, keep = _decode_args(dims, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, dst_slot, o, stream)
    return PreparedCall("gdn_decode_step", args, keep)


def gdn_verify_window(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                      ckpt, o, stream=None) -> None:
    """Each row's window from its committed slot; writes o and checkpoint slots 0..T_r-1
    (ckpt None: outputs only, for commit by replay)."""
    T, src = _i32(row_tokens), _i32(src_slot)
    n_rows = T.size
    if src.size != n_rows:
        raise ValueError("row_tokens and src_slot lengths differ")
    N = int(T.sum())
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows, optional=True)
    rc = lib().gdn_verify_window(ctypes.byref(dims.c()), n_rows, _ip(T), *toks, pp, n_slots, _ip(src),
                                 cp, op, _stream(stream))
    _check("gdn_verify_window", rc)


def gdn_verify_tree(dims: Dims, row_tokens, parents, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                    ckpt, o, stream=None) -> None:
    """Token-tree windows: token t of a row runs from its parent's state (parents per
    packed token, -1 = the committed state); checkpoint slot t = node t's state."""
    T, par, src = _i32(row_tokens), _i32(parents), _i32(src_slot)
    n_rows = T.size
    if src.size != n_rows:
        raise ValueError("row_tokens and src_slot lengths differ")
    N = int(T.sum())
    if par.size != N:
        raise ValueError("parents must hold one entry per packed token")
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows)
    rc = lib().gdn_verify_tree(ctypes.byref(dims.c()), n_rows, _ip(T), _ip(par), *toks, pp, n_slots,
                               _ip(src), cp, op, _stream(stream))
    _check("gdn_verify_tree", rc)


def gdn_commit_accepted(dims: Dims, row_tokens, ckpt, accepted, state_pool, dst_slot, status,
                        stream=None) -> None:
    """Copy checkpoint slot accepted[r] (device int32) of each row to slot dst_slot[r]."""
    import torch
    T, dst = _i32(row_tokens), _i32(dst_slot)
    n_rows = T.size
    if dst.size != n_rows:
        raise ValueError("row_tokens and dst_slot lengths differ")
    cp = _ckpt(dims, ckpt, n_rows)
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    pp, n_slots = _pool(dims, state_pool)
    rc = lib().gdn_commit_accepted(ctypes.byref(dims.c()), n_rows, _ip(T), cp, ap, pp, n_slots,
                                   _ip(dst), sp, _stream(stream))
    _check("gdn_commit_accepted", rc)


def delta_shape(dims: Dims, n_rows: int) -> tuple:
    """Shape of the fp32 delta-checkpoint buffer of gdn_verify_window_delta."""
    return (n_rows, dims.k_max + 1, dims.n_v_heads, dims.d_v + 4)


def _verify_delta_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot, delta, o,
                       stream):
    import torch
    T, src = _i32(row_tokens), _i32(src_slot)
    n_rows = T.size
    if src.size != n_rows:
        raise ValueError("row_tokens and src_slot lengths differ")
    toks, op = _token_ptrs(dims, int(T.sum()), q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    dp = _dev(delta, "delta", torch.float32, delta_shape(dims, n_rows))
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), *toks, pp, n_slots, _ip(src), dp, op, _stream(stream))
    return args, (cd, T, src, q, k, v, a, b, A_log, dt_bias, state_pool, delta, o)


def _commit_delta_args(dims, row_tokens, k, delta, accepted, state_pool, src_slot, dst_slot, status, stream):
    import torch
    T, src, dst = _i32(row_tokens), _i32(src_slot), _i32(dst_slot)
    n_rows = T.size
    if not (src.size == dst.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    kp = _dev(k, "k", torch.bfloat16, (int(T.sum()), dims.n_qk_heads, dims.d_k))
    dp = _dev(delta, "delta", torch.float32, delta_shape(dims, n_rows))
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    pp, n_slots = _pool(dims, state_pool)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), kp, dp, ap, pp, n_slots, _ip(src), _ip(dst), sp, _stream(stream))
    return args, (cd, T, src, dst, k, delta, accepted, state_pool, status)


def _verify_fold_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot, delta, o,
                      prev_row_tokens, prev_k, prev_delta, prev_accepted, status, stream):
    import torch
    T, sl, pT = _i32(row_tokens), _i32(slot), _i32(prev_row_tokens)
    n_rows = T.size
    if not (sl.size == pT.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    toks, op = _token_ptrs(dims, int(T.sum()), q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    dp = _dev(delta, "delta", torch.float32, delta_shape(dims, n_rows))
    pkp = _dev(prev_k, "prev_k", torch.bfloat16, (int(pT.sum()), dims.n_qk_heads, dims.d_k))
    pdp = _dev(prev_delta, "prev_delta", torch.float32, delta_shape(dims, n_rows))
    ap = _dev(prev_accepted, "prev_accepted", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), *toks, pp, n_slots, _ip(sl), dp, op, _ip(pT), pkp, pdp, ap, sp,
            _stream(stream))
    return args, (cd, T, sl, pT, q, k, v, a, b, A_log, dt_bias, state_pool, delta, o, prev_k, prev_delta,
                  prev_accepted, status)


def gdn_verify_window_delta_fold(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot,
                                 delta, o, prev_row_tokens, prev_k, prev_delta, prev_accepted, status,
                                 stream=None) -> None:
    """Commit each row's previous window (fold its delta checkpoints into slot[r]) and
    verify the new window from the result, storing its delta checkpoints: one launch."""
    args, _keep = _verify_fold_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot, delta,
                                    o, prev_row_tokens, prev_k, prev_delta, prev_accepted, status, stream)
    _check("gdn_verify_window_delta_fold", lib().gdn_verify_window_delta_fold(*args))


def prepare_verify_window_delta_fold(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot,
                                     delta, o, prev_row_tokens, prev_k, prev_delta, prev_accepted, status,
                                     stream=None) -> PreparedCall:
    args, keep = _verify_fold_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot, delta,
                                   o, prev_row_tokens, prev_k, prev_delta, prev_accepted, status, stream)
    return PreparedCall("gdn_verify_window_delta_fold", args, keep)


def gdn_verify_window_delta(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                            delta, o, stream=None) -> None:
    """Verify windows storing each step's rank-1 factors (delta checkpoints)."""
    args, _keep = _verify_delta_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                                     delta, o, stream)
    _check("gdn_verify_window_delta", lib().gdn_verify_window_delta(*args))


def gdn_commit_delta(dims: Dims, row_tokens, k, delta, accepted, state_pool, src_slot, dst_slot, status,
                     stream=None) -> None:
    """Fold tokens 0..accepted[r] of each row's delta checkpoints into slot src_slot[r]."""
    args, _keep = _commit_delta_args(dims, row_tokens, k, delta, accepted, state_pool, src_slot, dst_slot,
                                     status, stream)
    _check("gdn_commit_delta", lib().gdn_commit_delta(*args))


def prepare_verify_window_delta(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                                delta, o, stream=None) -> PreparedCall:
    args, keep = _verify_delta_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, src_slot,
                                    delta, o, stream)
    return PreparedCall("gdn_verify_window_delta", args, keep)


def prepare_commit_delta(dims: Dims, row_tokens, k, delta, accepted, state_pool, src_slot, dst_slot, status,
                         stream=None) -> PreparedCall:
    args, keep = _commit_delta_args(dims, row_tokens, k, delta, accepted, state_pool, src_slot, dst_slot,
                                    status, stream)
    return PreparedCall("gdn_commit_delta", args, keep)


def _verify_select_args(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table, bank, o,
                        status, stream):
    import torch
    T, bk = _i32(row_tokens), _i32(bank)
    n_rows = T.size
    if bk.size != n_rows:
        raise ValueError("per-row arrays differ in length")
    toks, op = _token_ptrs(dims, int(T.sum()), q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    tp = _dev(slot_table, "slot_table", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), *toks, pp, n_slots, tp, _ip(bk), op, sp, _stream(stream))
    return args, (cd, T, bk, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table, o, status)


def _verify_select_commit_args(dims: Dims, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a, b, A_log,
                               dt_bias, state_pool, slot_table, bank, o, status, stream):
    import torch
    T, PT, PB, bk = _i32(row_tokens), _i32(prev_row_tokens), _i32(prev_bank), _i32(bank)
    n_rows = T.size
    if not (PT.size == PB.size == bk.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    toks, op = _token_ptrs(dims, int(T.sum()), q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    tp = _dev(slot_table, "slot_table", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), _ip(PT), _ip(PB), ap, *toks, pp, n_slots, tp, _ip(bk), op, sp,
            _stream(stream))
    return args, (cd, T, PT, PB, bk, accepted, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table, o, status)


def _commit_select_args(dims: Dims, row_tokens, accepted, bank, state_pool, slot_table, status, stream):
    import torch
    T, bk = _i32(row_tokens), _i32(bank)
    n_rows = T.size
    if bk.size != n_rows:
        raise ValueError("per-row arrays differ in length")
    _, n_slots = _pool(dims, state_pool)
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    tp = _dev(slot_table, "slot_table", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), ap, _ip(bk), n_slots, tp, sp, _stream(stream))
    return args, (cd, T, bk, accepted, slot_table, status)


def gdn_verify_window_select(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table, bank,
                             o, status, stream=None) -> None:
    """Verify windows writing their checkpoints into the pool, row r into slots
    bank[r] * (k_max + 1) + j, from the source slot slot_table[r] (device int32)."""
    args, _keep = _verify_select_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table,
                                      bank, o, status, stream)
    _check("gdn_verify_window_select", lib().gdn_verify_window_select(*args))


def gdn_commit_select(dims: Dims, row_tokens, accepted, bank, state_pool, slot_table, status, stream=None) -> None:
    """slot_table[r] = bank[r] * (k_max + 1) + accepted[r] (device): select, not copy.
    state_pool is passed for its slot count only; nothing in it is read or written."""
    args, _keep = _commit_select_args(dims, row_tokens, accepted, bank, state_pool, slot_table, status, stream)
    _check("gdn_commit_select", lib().gdn_commit_select(*args))


def gdn_verify_window_select_commit(dims: Dims, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a, b,
                                    A_log, dt_bias, state_pool, slot_table, bank, o, status, stream=None) -> None:
    """gdn_commit_select of the previous window (prev_row_tokens, prev_bank, accepted on the
    device), then gdn_verify_window_select of this one, in one launch."""
    args, _keep = _verify_select_commit_args(dims, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a, b,
                                             A_log, dt_bias, state_pool, slot_table, bank, o, status, stream)
    _check("gdn_verify_window_select_commit", lib().gdn_verify_window_select_commit(*args))


def prepare_verify_window_select_commit(dims: Dims, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a,
                                        b, A_log, dt_bias, state_pool, slot_table, bank, o, status,
                                        stream=None) -> PreparedCall:
    args, keep = _verify_select_commit_args(dims, row_tokens, prev_row_tokens, prev_bank, accepted, q, k, v, a, b,
                                            A_log, dt_bias, state_pool, slot_table, bank, o, status, stream)
    return PreparedCall("gdn_verify_window_select_commit", args, keep)


def prepare_verify_window_select(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table,
                                 bank, o, status, stream=None) -> PreparedCall:
    args, keep = _verify_select_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool, slot_table,
                                     bank, o, status, stream)
    return PreparedCall("gdn_verify_window_select", args, keep)


def prepare_commit_select(dims: Dims, row_tokens, accepted, bank, state_pool, slot_table, status,
                          stream=None) -> PreparedCall:
    args, keep = _commit_select_args(dims, row_tokens, accepted, bank, state_pool, slot_table, status, stream)
    return PreparedCall("gdn_commit_select", args, keep)


def _replay_args(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, accepted, state_pool,
                 src_slot, dst_slot, status, stream):
    import torch
    T, src, dst = _i32(row_tokens), _i32(src_slot), _i32(dst_slot)
    n_rows = T.size
    if not (src.size == dst.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    toks = _token_in_ptrs(dims, int(T.sum()), q, k, v, a, b, A_log, dt_bias)
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    pp, n_slots = _pool(dims, state_pool)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), *toks, ap, pp, n_slots, _ip(src), _ip(dst), sp,
            _stream(stream))
    return args, (cd, T, src, dst, q, k, v, a, b, A_log, dt_bias, accepted, state_pool, status)


def gdn_commit_replay(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, accepted, state_pool,
                      src_slot, dst_slot, status, stream=None) -> None:
    """Re-run each row's first accepted[r] + 1 window tokens (device int32) from slot
    src_slot[r]; the resulting state goes to slot dst_slot[r]."""
    args, _keep = _replay_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, accepted, state_pool,
                               src_slot, dst_slot, status, stream)
    _check("gdn_commit_replay", lib().gdn_commit_replay(*args))


def gdn_chunked_workspace_bytes(dims: Dims, row_tokens, chunk: int = 64) -> int:
    T = _i32(row_tokens)
    return int(lib().gdn_chunked_workspace_bytes(ctypes.byref(dims.c()), T.size, _ip(T), chunk))


def gdn_chunked_prefill_with_checkpoints(dims: Dims, row_tokens, n_tail, q, k, v, a, b, A_log,
                                         dt_bias, state_pool, src_slot, dst_slot, ckpt, o,
                                         workspace, chunk: int = 64, stream=None) -> None:
    """Long rows in the chunked form; final state to dst_slot (-1: none), tail checkpoints."""
    import torch
    T, nt, src, dst = _i32(row_tokens), _i32(n_tail), _i32(src_slot), _i32(dst_slot)
    n_rows = T.size
    if not (nt.size == src.size == dst.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    N = int(T.sum())
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows)
    need = gdn_chunked_workspace_bytes(dims, T, chunk)
    if workspace is None:
        wp, wb = _VP(0), 0
    else:
        wp = _dev(workspace, "workspace", torch.uint8, (workspace.numel(),))
        wb = workspace.numel()
    if wb < need:
        raise GdnError("gdn_chunked_prefill_with_checkpoints", -6)
    rc = lib().gdn_chunked_prefill_with_checkpoints(
        ctypes.byref(dims.c()), n_rows, _ip(T), chunk, _ip(nt), *toks, pp, n_slots, _ip(src), _ip(dst),
        cp, op, wp, wb, _stream(stream))
    _check("gdn_chunked_prefill_with_checkpoints", rc)


STATIC_WS_BYTES = 128 << 20  # GDN_STATIC_WS_BYTES


def gdn_chunked_prefill_with_checkpoints_static(dims: Dims, row_tokens, n_tail, q, k, v, a, b, A_log,
                                                dt_bias, state_pool, src_slot, dst_slot, ckpt, o,
                                                chunk: int = 64, stream=None) -> None:
    """gdn_chunked_prefill_with_checkpoints on the library's own per-GPU workspace
    (STATIC_WS_BYTES): the call allocates no device memory.  Calls that overlap on one
    GPU share that workspace and must be ordered by the caller."""
    T, nt, src, dst = _i32(row_tokens), _i32(n_tail), _i32(src_slot), _i32(dst_slot)
    n_rows = T.size
    if not (nt.size == src.size == dst.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    N = int(T.sum())
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows)
    rc = lib().gdn_chunked_prefill_with_checkpoints_static(
        ctypes.byref(dims.c()), n_rows, _ip(T), chunk, _ip(nt), *toks, pp, n_slots, _ip(src), _ip(dst),
        cp, op, _stream(stream))
    _check("gdn_chunked_prefill_with_checkpoints_static", rc)


def gdn_plan_transaction(dims: Dims, row_tokens) -> np.ndarray:
    """Route per row: ROUTE_RECURRENT (0) or ROUTE_CHUNKED (1)."""
    T = _i32(row_tokens)
    route = np.zeros(T.size, np.int32)
    rc = lib().gdn_plan_transaction(ctypes.byref(dims.c()), T.size, _ip(T), _ip(route))
    _check("gdn_plan_transaction", rc)
    return route


def gdn_run_transaction(dims: Dims, row_tokens, n_ckpt, q, k, v, a, b, A_log, dt_bias, state_pool,
                        src_slot, dst_slot, ckpt, o, workspace=None, stream=None) -> None:
    """A mixed ragged transaction, planned per row and launched on both routes."""
    import torch
    T, nc, src, dst = _i32(row_tokens), _i32(n_ckpt), _i32(src_slot), _i32(dst_slot)
    n_rows = T.size
    if not (nc.size == src.size == dst.size == n_rows):
        raise ValueError("per-row arrays differ in length")
    N = int(T.sum())
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows)
    if workspace is None:
        wp, wb = _VP(0), 0
    else:
        wp = _dev(workspace, "workspace", torch.uint8, (workspace.numel(),))
        wb = workspace.numel()
    rc = lib().gdn_run_transaction(ctypes.byref(dims.c()), n_rows, _ip(T), _ip(nc), *toks, pp, n_slots,
                                   _ip(src), _ip(dst), cp, op, wp, wb, _stream(stream))
    _check("gdn_run_transaction", rc)


# ------------------------------------------------------------------ prepared calls

class PreparedCall:
    """One entry-point call with its arguments checked and marshalled once; calling it
    re-issues the same C call (same buffers, same stream).  For tight loops where the
    per-call Python checks would dominate the host time, and for capture into a HIP
    graph.  It holds a reference to every host array and device tensor its pointers
    refer to, so none of them can be freed (and its memory reused) while the call
    exists."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.name = name
        self._fn = getattr(lib(), name)
        self._args = args
        self._keep = keep  # host arrays and tensors the pointers refer to

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != GDN_OK:
            raise GdnError(self.name, rc)


def prepare_verify_window(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, state_pool,
                          src_slot, ckpt, o, stream=None) -> PreparedCall:
    T, src = _i32(row_tokens), _i32(src_slot)
    n_rows = T.size
    N = int(T.sum())
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows, optional=True)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), *toks, pp, n_slots, _ip(src), cp, op, _stream(stream))
    return PreparedCall("gdn_verify_window", args,
                        (cd, T, src, q, k, v, a, b, A_log, dt_bias, state_pool, ckpt, o))


def prepare_verify_tree(dims: Dims, row_tokens, parents, q, k, v, a, b, A_log, dt_bias, state_pool,
                        src_slot, ckpt, o, stream=None) -> PreparedCall:
    T, par, src = _i32(row_tokens), _i32(parents), _i32(src_slot)
    n_rows = T.size
    N = int(T.sum())
    if par.size != N:
        raise ValueError("parents must hold one entry per packed token")
    toks, op = _token_ptrs(dims, N, q, k, v, a, b, A_log, dt_bias, o)
    pp, n_slots = _pool(dims, state_pool)
    cp = _ckpt(dims, ckpt, n_rows)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), _ip(par), *toks, pp, n_slots, _ip(src), cp, op, _stream(stream))
    return PreparedCall("gdn_verify_tree", args,
                        (cd, T, par, src, q, k, v, a, b, A_log, dt_bias, state_pool, ckpt, o))


def prepare_commit_replay(dims: Dims, row_tokens, q, k, v, a, b, A_log, dt_bias, accepted, state_pool,
                          src_slot, dst_slot, status, stream=None) -> PreparedCall:
    args, keep = _replay_args(dims, row_tokens, q, k, v, a, b, A_log, dt_bias, accepted, state_pool,
                              src_slot, dst_slot, status, stream)
    return PreparedCall("gdn_commit_replay", args, keep)


def prepare_commit_accepted(dims: Dims, row_tokens, ckpt, accepted, state_pool, dst_slot, status,
                            stream=None) -> PreparedCall:
    import torch
    T, dst = _i32(row_tokens), _i32(dst_slot)
    n_rows = T.size
    cp = _ckpt(dims, ckpt, n_rows)
    ap = _dev(accepted, "accepted", torch.int32, (n_rows,))
    sp = _dev(status, "status", torch.int32, ((n_rows + 31) // 32,))
    pp, n_slots = _pool(dims, state_pool)
    cd = dims.c()
    args = (ctypes.byref(cd), n_rows, _ip(T), cp, ap, pp, n_slots, _ip(dst), sp, _stream(stream))
    return PreparedCall("gdn_commit_accepted", args, (cd, T, dst, ckpt, accepted, state_pool, status))
