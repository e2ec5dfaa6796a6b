"""Helpers shared by the GPU parity tests: moving the seeded inputs to the device,
reading results back, and the tolerance checks.

Tolerances (both sides run the same inputs; the oracle in fp64):
  * state: relative L2 per (row, head) unit, ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-4
    (absolute when the reference is zero);
  * outputs (bf16): max |o_gpu - o_ref| <= 1e-2 over all elements, and the tighter
    per-element bound |o_gpu - o_ref| <= 2^-8 |o_ref| + 1e-5 (bf16 round-to-nearest
    alone contributes at most 2^-9 |o|; fp32 accumulation adds ~1e-7 at these
    magnitudes).
"""
from __future__ import annotations

import sys

import numpy as np

from gateddeltanet_linear_attention_amd import binding as gb
from gateddeltanet_linear_attention_amd import synth

STATE_TOL = 1e-4
O_ABS_TOL = 1e-2
O_REL_TOL = 2.0 ** -8
O_FLOOR = 1e-5


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dims_of(shape: synth.HeadShape, k_max: int = 3, raw_qk: bool = False) -> gb.Dims:
    """raw_qk: q and k are unnormalised and the library normalises them (GDN_QK_L2NORM)."""
    return gb.Dims(shape.n_qk_heads, shape.n_v_heads, shape.d, shape.d, k_max,
                   gb.QK_L2NORM if raw_qk else 0)


def ref_qk(tok: synth.Tokens, raw_qk: bool):
    """The q and k the oracle runs on: normalised by the oracle when the inputs are raw."""
    import oracle
    return oracle.l2norm_qk(tok.q, tok.k) if raw_qk else (tok.q, tok.k)


def dev_tokens(tok: synth.Tokens) -> dict:
    import torch
    return dict(
        q=torch.from_numpy(np.ascontiguousarray(tok.q)).to(torch.bfloat16).cuda(),
        k=torch.from_numpy(np.ascontiguousarray(tok.k)).to(torch.bfloat16).cuda(),
        v=torch.from_numpy(np.ascontiguousarray(tok.v)).to(torch.bfloat16).cuda(),
        a=torch.from_numpy(np.ascontiguousarray(tok.a)).cuda(),
        b=torch.from_numpy(np.ascontiguousarray(tok.b)).cuda(),
    )


def dev_params(A_log, dt_bias) -> dict:
    import torch
    return dict(A_log=torch.from_numpy(np.ascontiguousarray(A_log)).cuda(),
                dt_bias=torch.from_numpy(np.ascontiguousarray(dt_bias)).cuda())


def index_tokens(t: dict, idx) -> dict:
    """Gather packed tokens (device) at the given token indices (a new contiguous block)."""
    import torch
    ii = torch.as_tensor(np.asarray(idx, np.int64), device=t["q"].device)
    return {k: v.index_select(0, ii).contiguous() for k, v in t.items()}


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def state_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over units (all leading dims) of the relative Frobenius error."""
    g = gpu.reshape(-1, gpu.shape[-2] * gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(err.max()) if err.size else 0.0


def o_err(gpu: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """(max |delta o|, max of |delta o| / (2^-8 |o_ref| + 1e-5)) -- the second must be <= 1."""
    d = np.abs(gpu - ref)
    return float(d.max()) if d.size else 0.0, \
        float((d / (O_REL_TOL * np.abs(ref) + O_FLOOR)).max()) if d.size else 0.0


def assert_o(gpu: np.ndarray, ref: np.ndarray, what: str):
    mx, rel = o_err(gpu, ref)
    assert mx <= O_ABS_TOL, "%s: max |do| = %.3g > %.3g" % (what, mx, O_ABS_TOL)
    assert rel <= 1.0, "%s: per-element |do| bound exceeded by %.3gx" % (what, rel)
    return mx


def assert_state(gpu: np.ndarray, ref: np.ndarray, what: str):
    e = state_err(gpu, ref)
    assert e <= STATE_TOL, "%s: state rel-L2 %.3g > %.3g" % (what, e, STATE_TOL)
    return e


def bits(t):
    """int32 view of an fp32 device tensor (bitwise comparisons, NaN-safe)."""
    import torch
    return t.contiguous().view(torch.int32)


def _raw(t):
    import torch
    return t.contiguous().view({4: torch.int32, 2: torch.int16}[t.element_size()])


def assert_same_bits(a, b, what: str = "tensors"):
    """Bitwise equality of two device tensors of one shape and element size (fp32 states,
    bf16 outputs; NaN-safe).  On a mismatch the message gives how many elements differ,
    the index of the first one and both values with their bit patterns."""
    assert tuple(a.shape) == tuple(b.shape), "%s: shapes %s and %s" % (what, tuple(a.shape), tuple(b.shape))
    ra, rb = _raw(a), _raw(b)
    if bool((ra == rb).all()):
        return
    diff = (ra != rb).flatten()
    n = int(diff.sum())
    first = int(diff.nonzero()[0])
    idx = tuple(int(i) for i in np.unravel_index(first, tuple(a.shape)))
    fa, fb = a.contiguous().flatten()[first], b.contiguous().flatten()[first]
    mask = (1 << (8 * a.element_size())) - 1
    raise AssertionError("%s: %d of %d elements differ; first at %s: %r (0x%0*x) vs %r (0x%0*x)" % (
        what, n, a.numel(), idx, float(fa), 2 * a.element_size(), int(ra.flatten()[first]) & mask,
        float(fb), 2 * b.element_size(), int(rb.flatten()[first]) & mask))
