"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE.

Only the test suite (``tests/``), ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The GPU library never does, and
the two share no code: the C source here (``gdn_oracle.c``) is compiled with gcc
on its own, and the only thing both sides consume is the seeded input arrays.

Every function takes and returns numpy fp64 arrays; bf16 / fp32 inputs are
widened exactly.  The arithmetic (gates, the state update, the chunkwise form)
lives in ``gdn_oracle.c``; the Python layer here only marshals arrays and
expresses the verify / commit / decode calls through it:

* verify window (a row's K+1 draft-verification tokens, run from the committed
  state, every intermediate state kept as a checkpoint) -- the checkpoints that
  let a rejected draft roll back, onnxruntime-genai pull request "Run chained
  MTP drafting in the batch Engine", section "Correctness fix";
* commit(a) -- the committed state becomes the state after a+1 window tokens
  (the previous bonus token plus a accepted drafts), same page, sections
  "Correctness fix" and "Rollback fix and corrected quality disposition";
* decode -- one token; the verify window is, by definition, repeated decode;
* verify tree -- a draft tree instead of a chain: each node runs from its
  parent's state (the pages run chains only and refuse tree shapes, "Occamy 1.0
  MTP", section "MTP1 runtime"; built as an extension, checked against brute force).
* l2norm_qk -- the input step of the rule when q and k arrive unnormalised: unit
  Euclidean norm per (token, head) vector, q also scaled by 1/sqrt(d_k) (the gated
  delta rule normalises queries and keys, Yang, Kautz & Hatamizadeh, ICLR 2025; the
  pages are silent on it).  Plain numpy, fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIBRARY: a prebuilt copy to load instead (the sanitizer build below);
# it is then never rebuilt here
_LIB = os.environ.get("GDN_ORACLE_LIBRARY") or os.path.join(_HERE, "libgdn_oracle.so")
_PREBUILT = bool(os.environ.get("GDN_ORACLE_LIBRARY"))
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no contraction, OpenMP over units).  out: another
    path to write; sanitize: with AddressSanitizer and UndefinedBehaviorSanitizer (any
    finding aborts), for a run with the ASan runtime preloaded."""
    lib = out or _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=all"] if sanitize else ["-O2"])
        subprocess.run(["gcc", *opt, "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _PREBUILT:
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.gdn_oracle_gates.argtypes = [ctypes.c_int, _D, _D, ctypes.c_double, ctypes.c_double, _D, _D]
        lib.gdn_oracle_gates.restype = None
        common = [ctypes.c_int] * 5 + [_I, _I, ctypes.c_int]
        tail = [_D] * 11 + [ctypes.c_int]
        lib.gdn_oracle_sequential.argtypes = common + tail
        lib.gdn_oracle_sequential.restype = ctypes.c_int
        lib.gdn_oracle_chunked.argtypes = common + [ctypes.c_int] + tail
        lib.gdn_oracle_chunked.restype = ctypes.c_int
        lib.gdn_oracle_threads_used.argtypes = []
        lib.gdn_oracle_threads_used.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def threads_used() -> int:
    return _load().gdn_oracle_threads_used()


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return None if x is None else x.ctypes.data_as(_D)


L2NORM_EPS = 1e-6  # under the square root: a zero vector maps to zero, not NaN


def l2norm_qk(q, k) -> tuple[np.ndarray, np.ndarray]:
    """(q_hat, k_hat) in fp64: k_hat = k / sqrt(sum_j k_j^2 + eps), and
    q_hat = q / sqrt(sum_j q_j^2 + eps) / sqrt(d_k), over the last axis."""
    q, k = _f64(q), _f64(k)
    d = q.shape[-1]
    k_hat = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + L2NORM_EPS)
    q_hat = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + L2NORM_EPS) / np.sqrt(d)
    return q_hat, k_hat


def gates(a, b, A_log: float, dt_bias: float) -> tuple[np.ndarray, np.ndarray]:
    """alpha = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b), for one head."""
    a, b = _f64(a).ravel(), _f64(b).ravel()
    assert a.shape == b.shape
    al, be = np.empty_like(a), np.empty_like(a)
    _load().gdn_oracle_gates(a.size, _p(a), _p(b), float(A_log), float(dt_bias), _p(al), _p(be))
    return al, be


def _out(buf, shape):
    """A caller-provided output array of the right shape, or a fresh one."""
    if buf is None:
        fresh = np.empty(shape)
        fresh.fill(0.0)  # first touch on one thread: page faults under OpenMP are slow
        return fresh
    if buf.shape != tuple(shape) or buf.dtype != np.float64 or not buf.flags.c_contiguous:
        raise ValueError("output buffer must be contiguous float64 of shape %s" % (tuple(shape),))
    return buf


def _run(fn_name, row_tokens, q, k, v, a, b, A_log, dt_bias, S0, n_tail, n_slot, chunk, n_threads,
         nan_fill=True, out=None):
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias = _f64(A_log).ravel(), _f64(dt_bias).ravel()
    N, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == N and a.shape == (N, Hv) and b.shape == (N, Hv)
    L = np.ascontiguousarray(np.asarray(row_tokens, dtype=np.int32).ravel())
    B = L.size
    assert int(L.sum()) == N, "row_tokens must add up to the packed token count"
    S0 = np.zeros((B, Hv, dv, dk)) if S0 is None else _f64(S0)
    assert S0.shape == (B, Hv, dv, dk)
    nt = np.zeros(B, np.int32) if n_tail is None else np.ascontiguousarray(np.asarray(n_tail, np.int32).ravel())
    if n_slot is None:
        n_slot = int(nt.max()) if B else 0
    out = out or {}
    S_final = _out(out.get("S_final"), (B, Hv, dv, dk))
    ckpt = None
    if n_slot > 0:
        ckpt = _out(out.get("ckpt"), (B, n_slot, Hv, dv, dk))
        if nan_fill:
            ckpt.fill(np.nan)  # also takes the page faults on one thread
    o = _out(out.get("o"), (N, Hv, dv))
    nthr = default_threads() if n_threads is None else int(n_threads)
    lib = _load()
    args = [B, Hqk, Hv, dk, dv, L.ctypes.data_as(_I), nt.ctypes.data_as(_I), n_slot]
    if chunk is not None:
        args.append(int(chunk))
    args += [_p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log), _p(dt_bias), _p(S0), _p(S_final),
             _p(ckpt), _p(o), nthr]
    rc = getattr(lib, fn_name)(*args)
    if rc != 0:
        raise ValueError("%s rejected its arguments" % fn_name)
    return S_final, ckpt, o


def run_sequential(row_tokens, q, k, v, a, b, A_log, dt_bias, S0=None, n_tail=None, n_slot=None,
                   n_threads=None, nan_fill=True, out=None):
    """Token-by-token recurrence over a packed ragged batch.

    Returns (S_final [B][H_v][d_v][d_k], ckpt [B][n_slot][H_v][d_v][d_k] or None,
    o [N][H_v][d_v]); checkpoint slot j of row r is the state after
    L_r - n_tail_r + j + 1 of its tokens; slots >= n_tail_r hold NaN (or are left
    uninitialised with nan_fill=False).  `out` may hold preallocated float64 arrays
    under the keys "S_final", "ckpt" and "o" (reused buffers avoid page faults).
    """
    return _run("gdn_oracle_sequential", row_tokens, q, k, v, a, b, A_log, dt_bias, S0, n_tail,
                n_slot, None, n_threads, nan_fill, out)


def run_chunked(row_tokens, q, k, v, a, b, A_log, dt_bias, S0=None, n_tail=None, n_slot=None,
                chunk=64, n_threads=None, nan_fill=True):
    """Same function as run_sequential, evaluated in the chunkwise UT form."""
    return _run("gdn_oracle_chunked", row_tokens, q, k, v, a, b, A_log, dt_bias, S0, n_tail,
                n_slot, chunk, n_threads, nan_fill)


def verify_window(row_tokens, q, k, v, a, b, A_log, dt_bias, S_committed, k_max=3, n_threads=None,
                  nan_fill=True, out=None):
    """Run each row's window (T_r = row_tokens[r] <= k_max+1 tokens) from its committed
    state, keeping checkpoint slot j = state after j+1 window tokens, j < T_r.

    Returns (ckpt [B][k_max+1][H_v][d_v][d_k], o)."""
    T = np.asarray(row_tokens, np.int32)
    assert np.all((T >= 1) & (T <= k_max + 1))
    _, ckpt, o = run_sequential(T, q, k, v, a, b, A_log, dt_bias, S_committed, n_tail=T,
                                n_slot=k_max + 1, n_threads=n_threads, nan_fill=nan_fill, out=out)
    return ckpt, o


def verify_tree(row_tokens, parents, q, k, v, a, b, A_log, dt_bias, S_committed, k_max=3):
    """Token-tree windows, by the plain definition: node t of row r is its root path
    (its ancestors in order, then t itself; parents[cu_r + t] = -1 means the
    committed state) run token by token from the committed state -- one sequential
    run per node.  A chain (parent t - 1) is the verify window.

    Returns (ckpt [B][k_max+1][H_v][d_v][d_k] with slot t = node t's state, NaN past
    T_r, o [N][H_v][d_v] with o_t = S_t q_t)."""
    T = np.asarray(row_tokens, np.int64)
    par = np.asarray(parents, np.int64).ravel()
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    S_committed = _f64(S_committed)
    B, Hv, dv, dk = S_committed.shape
    assert np.all((T >= 1) & (T <= k_max + 1)) and par.size == int(T.sum())
    cu = np.concatenate([[0], np.cumsum(T)])
    ckpt = np.full((B, k_max + 1, Hv, dv, dk), np.nan)
    o = np.zeros((int(T.sum()), Hv, dv))
    for r in range(B):
        if par[cu[r]] != -1:
            raise ValueError("row %d: the first window token must follow the committed state" % r)
        for t in range(int(T[r])):
            p = int(par[cu[r] + t])
            if not -1 <= p < t:
                raise ValueError("row %d token %d: parent %d is not an earlier node" % (r, t, p))
            path, x = [], t
            while x >= 0:
                path.append(x)
                x = int(par[cu[r] + x])
            idx = cu[r] + np.array(path[::-1])
            S_fin, _, o_path = run_sequential([len(idx)], q[idx], k[idx], v[idx], a[idx], b[idx], A_log,
                                              dt_bias, S_committed[r:r + 1])
            ckpt[r, t] = S_fin[0]
            o[cu[r] + t] = o_path[-1]
    return ckpt, o


def commit(ckpt, row_tokens, accepted) -> np.ndarray:
    """Committed state of each row after accepting a_r drafts: checkpoint slot a_r,
    the state after the previous bonus token and the a_r accepted drafts."""
    acc = np.asarray(accepted, np.int64)
    T = np.asarray(row_tokens, np.int64)
    if np.any(acc < 0) or np.any(acc >= T):
        raise ValueError("accepted count out of range for the window")
    return np.stack([ckpt[r, acc[r]] for r in range(len(acc))])


def decode_step(q, k, v, a, b, A_log, dt_bias, S, n_threads=None):
    """One token per row.  Returns (new state [B][H_v][d_v][d_k], o [B][H_v][d_v])."""
    B = np.asarray(S).shape[0]
    S_final, _, o = run_sequential(np.ones(B, np.int32), q, k, v, a, b, A_log, dt_bias, S,
                                   n_threads=n_threads)
    return S_final, o
