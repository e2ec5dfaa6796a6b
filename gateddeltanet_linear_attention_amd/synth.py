"""Seeded synthetic inputs for the gated-delta-rule decode / verify / prefill path.

This module only draws random numbers and rounds them to the storage types the
kernels take (bfloat16 for q/k/v, float32 for gate logits and head parameters).
It holds none of the method's arithmetic: gates, state updates and outputs are
computed by the GPU library and, independently, by the fp64 oracle.  Both sides
receive exactly the arrays produced here.

Distributions (one draw per element unless stated):
  * q, k ~ N(0, 1), each (token, qk-head) vector L2-normalised; q then scaled by
    1/sqrt(d_k); rounded to bfloat16 (ties to even).  With raw_qk the normalisation
    and the scale are left to the consumer (the library's fused input mode): q, k
    are the N(0, 1) draws themselves, rounded to bfloat16.
  * v ~ N(0, 1), rounded to bfloat16.
  * gate logits a, b ~ N(0, 1), float32, one per (token, v-head).
  * per v-head parameters: A_log ~ U(log 1, log 16), dt_bias ~ N(0, 0.1^2), float32.
  * accepted draft counts ~ Binomial(K_r, 0.85), the weighted accepted/evaluated
    draft rate reported for K=3 on the onnxruntime-genai pull request "Run chained
    MTP drafting in the batch Engine", section "Validation".
The shapes follow a hybrid GatedDeltaNet layer with 16 query/key heads and 32
value heads of width 128 (every q/k head shared by two adjacent v-heads).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ACCEPT_P = 0.85


@dataclass(frozen=True)
class HeadShape:
    n_qk_heads: int
    n_v_heads: int
    d: int  # d_k == d_v


TINY = HeadShape(1, 1, 16)
FULL = HeadShape(16, 32, 128)


def streams(seed: int, n: int) -> list[np.random.Generator]:
    """Independent generators spawned from one seed (parameters, tokens, lengths...)."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even); result stored as float32.

    Values are first taken to float32.  Inputs here are finite normal draws.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(f.shape)


def head_params(rng: np.random.Generator, shape: HeadShape) -> tuple[np.ndarray, np.ndarray]:
    """Per v-head A_log ~ U(log 1, log 16) and dt_bias ~ N(0, 0.1^2), float32."""
    A_log = rng.uniform(np.log(1.0), np.log(16.0), size=shape.n_v_heads).astype(np.float32)
    dt_bias = (0.1 * rng.standard_normal(shape.n_v_heads)).astype(np.float32)
    return A_log, dt_bias


@dataclass
class Tokens:
    """A packed block of n tokens: q, k [n][H_qk][d], v [n][H_v][d] (bf16 values held
    as float32), a, b [n][H_v] float32."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray

    @property
    def n(self) -> int:
        return self.q.shape[0]

    def slice(self, lo: int, hi: int) -> "Tokens":
        return Tokens(self.q[lo:hi], self.k[lo:hi], self.v[lo:hi], self.a[lo:hi], self.b[lo:hi])

    @staticmethod
    def concat(parts: list["Tokens"]) -> "Tokens":
        return Tokens(*(np.concatenate([getattr(p, f) for p in parts], axis=0)
                        for f in ("q", "k", "v", "a", "b")))


def _unit_rows(rng: np.random.Generator, n: int, h: int, d: int) -> np.ndarray:
    x = rng.standard_normal((n, h, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def tokens(rng: np.random.Generator, shape: HeadShape, n: int, gate_shift: float = 0.0,
           raw_qk: bool = False) -> Tokens:
    """n fresh tokens.  gate_shift is added to the decay logit a (a negative shift makes
    the decay slow, alpha close to 1: a stress case for long memory).  raw_qk: q and k
    are not normalised (same draws, same stream positions)."""
    d = shape.d
    if raw_qk:
        q = round_to_bf16(rng.standard_normal((n, shape.n_qk_heads, d)))
        k = round_to_bf16(rng.standard_normal((n, shape.n_qk_heads, d)))
    else:
        q = round_to_bf16(_unit_rows(rng, n, shape.n_qk_heads, d) / np.sqrt(d))
        k = round_to_bf16(_unit_rows(rng, n, shape.n_qk_heads, d))
    v = round_to_bf16(rng.standard_normal((n, shape.n_v_heads, d)))
    a = (rng.standard_normal((n, shape.n_v_heads)) + gate_shift).astype(np.float32)
    b = rng.standard_normal((n, shape.n_v_heads)).astype(np.float32)
    return Tokens(q, k, v, a, b)


def accepted_counts(rng: np.random.Generator, draft_lens: np.ndarray, p: float = ACCEPT_P) -> np.ndarray:
    """Accepted draft count per row, Binomial(K_r, p), int32."""
    return rng.binomial(np.asarray(draft_lens, dtype=np.int64), p).astype(np.int32)


# ---------------------------------------------------------------------------
# Config-shaped workloads.  Each stream is keyed by (seed, purpose, index), so a
# window's tokens can be drawn in any order and are the same for every consumer.

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=key))


_PARAMS, _WARM, _WIN, _ACC, _LENS, _DECODE = 1, 2, 3, 4, 5, 6


@dataclass
class VerifyWorkload:
    """Rows warmed by prior tokens, then repeated verify windows with per-row draft
    lengths K_r (T_r = K_r + 1 tokens per window) and accepted counts per window.

    The accepted count is how many drafts survive; the committed state after a
    window is the state after a_r + 1 of its tokens."""

    name: str
    seed: int
    shape: HeadShape
    A_log: np.ndarray
    dt_bias: np.ndarray
    warm_lens: np.ndarray      # [B] prior tokens per row
    draft_lens: np.ndarray     # [B] K_r
    n_windows: int
    accept: str = "binomial"   # "binomial" (p = 0.85) or "uniform" (0..K_r)
    gate_shift: float = 0.0
    raw_qk: bool = False       # q, k left unnormalised (fused input mode)

    @property
    def n_rows(self) -> int:
        return int(self.warm_lens.size)

    @property
    def window_lens(self) -> np.ndarray:
        return (self.draft_lens + 1).astype(np.int32)

    def warm_tokens(self) -> Tokens:
        """Packed prior tokens, row r owning warm_lens[r] consecutive tokens."""
        return tokens(_rng(self.seed, _WARM), self.shape, int(self.warm_lens.sum()), self.gate_shift,
                      self.raw_qk)

    def window_tokens(self, i: int) -> Tokens:
        return tokens(_rng(self.seed, _WIN, i), self.shape, int(self.window_lens.sum()), self.gate_shift,
                      self.raw_qk)

    def accepted(self, i: int) -> np.ndarray:
        g = _rng(self.seed, _ACC, i)
        if self.accept == "uniform":
            return g.integers(0, self.draft_lens + 1).astype(np.int32)
        return accepted_counts(g, self.draft_lens)


VERIFY_WORKLOADS = ("tiny", "batch1", "conc16")


def verify_workload(name: str, *, seed: int | None = None, all_k3: bool = False,
                    n_windows: int | None = None, raw_qk: bool = False) -> VerifyWorkload:
    """The verify-window workloads.

    "tiny":   one request, one head, d = 16; 8 prompt tokens decoded one by one, then
              one K=3 window with an accepted count uniform in 0..3.
    "batch1": one request, 16 q/k heads / 32 v-heads, d = 128; warmed by 512 tokens,
              then 256 K=3 windows, accepted ~ Binomial(3, 0.85), commit after each.
    "conc16": 16 requests, same heads; warm lengths ~ U{128..2048}; per-request K_r in
              {1, 2, 3} (each value present; all_k3 gives every row K=3); 512 windows,
              accepted ~ Binomial(K_r, 0.85), per-row rollback.
    """
    base = {"tiny": 1001, "batch1": 1002, "conc16": 1003}
    if name not in base:
        raise ValueError("unknown verify workload %r" % name)
    seed = base[name] if seed is None else seed
    if name == "tiny":
        shape, B, warm, K, nw, acc = TINY, 1, np.array([8]), np.array([3]), 1, "uniform"
    elif name == "batch1":
        shape, B, warm, K, nw, acc = FULL, 1, np.array([512]), np.array([3]), 256, "binomial"
    else:
        shape, B, nw, acc = FULL, 16, 512, "binomial"
        g = _rng(seed, _LENS)
        warm = g.integers(128, 2049, size=B)
        if all_k3:
            K = np.full(B, 3)
        else:
            K = np.concatenate([[1, 2, 3], g.integers(1, 4, size=B - 3)])
            g.shuffle(K)
    A_log, dt_bias = head_params(_rng(seed, _PARAMS), shape)
    return VerifyWorkload(name=name + ("_k3" if all_k3 else ""), seed=seed, shape=shape,
                          A_log=A_log, dt_bias=dt_bias, warm_lens=np.asarray(warm, np.int32),
                          draft_lens=np.asarray(K, np.int32),
                          n_windows=nw if n_windows is None else n_windows, accept=acc, raw_qk=raw_qk)


@dataclass
class PrefillWorkload:
    """One packed prefill: rows of lengths L_r from the zero state, with the states
    after the last n_tail_r positions requested as checkpoints."""

    seed: int
    shape: HeadShape
    A_log: np.ndarray
    dt_bias: np.ndarray
    lens: np.ndarray
    n_tail: np.ndarray
    chunk: int = 64
    gate_shift: float = 0.0
    raw_qk: bool = False

    def tokens(self) -> Tokens:
        return tokens(_rng(self.seed, _WARM), self.shape, int(self.lens.sum()), self.gate_shift, self.raw_qk)


def prefill_workload(*, seed: int = 1004, lens=(2048,), n_tail=None, shape: HeadShape = FULL,
                     gate_shift: float = 0.0, raw_qk: bool = False) -> PrefillWorkload:
    """Default: one request, 2048 new tokens, d = 128 heads, chunk 64, checkpoints at
    the last 4 positions (other lengths / tails for tests)."""
    lens = np.asarray(lens, np.int32)
    nt = np.minimum(lens, 4) if n_tail is None else np.asarray(n_tail, np.int32)
    A_log, dt_bias = head_params(_rng(seed, _PARAMS), shape)
    return PrefillWorkload(seed=seed, shape=shape, A_log=A_log, dt_bias=dt_bias, lens=lens,
                           n_tail=nt.astype(np.int32), gate_shift=gate_shift, raw_qk=raw_qk)


@dataclass
class MixedWorkload:
    """Mixed ragged transaction: 16 rows in one packed transaction -- 4 prefills of L ~ U{256..4096} from
    the zero state and 12 K=3 verify windows on rows warmed by U{128..2048} tokens --
    then commit, then 64 decode-only K=3 windows over all 16 rows."""

    seed: int
    shape: HeadShape
    A_log: np.ndarray
    dt_bias: np.ndarray
    is_prefill: np.ndarray     # [16] bool
    prefill_lens: np.ndarray   # [16] (0 for verify rows)
    warm_lens: np.ndarray      # [16] (0 for prefill rows)
    n_windows: int = 64
    raw_qk: bool = False

    @property
    def n_rows(self) -> int:
        return int(self.is_prefill.size)

    def warm_tokens(self) -> Tokens:
        return tokens(_rng(self.seed, _WARM), self.shape, int(self.warm_lens.sum()), raw_qk=self.raw_qk)

    def transaction_lens(self) -> np.ndarray:
        return np.where(self.is_prefill, self.prefill_lens, 4).astype(np.int32)

    def transaction_tokens(self) -> Tokens:
        return tokens(_rng(self.seed, _DECODE), self.shape, int(self.transaction_lens().sum()), raw_qk=self.raw_qk)

    def transaction_accepted(self) -> np.ndarray:
        """Accepted drafts of the verify rows (prefill rows: unused, 0)."""
        acc = accepted_counts(_rng(self.seed, _ACC, 10**6), np.full(self.n_rows, 3))
        return np.where(self.is_prefill, 0, acc).astype(np.int32)

    def window_tokens(self, i: int) -> Tokens:
        return tokens(_rng(self.seed, _WIN, i), self.shape, 4 * self.n_rows, raw_qk=self.raw_qk)

    def accepted(self, i: int) -> np.ndarray:
        return accepted_counts(_rng(self.seed, _ACC, i), np.full(self.n_rows, 3))


def mixed_workload(*, seed: int = 1005, n_windows: int = 64, raw_qk: bool = False) -> MixedWorkload:
    g = _rng(seed, _LENS)
    B = 16
    is_prefill = np.zeros(B, bool)
    is_prefill[g.choice(B, 4, replace=False)] = True
    prefill_lens = np.where(is_prefill, g.integers(256, 4097, size=B), 0).astype(np.int32)
    warm_lens = np.where(is_prefill, 0, g.integers(128, 2049, size=B)).astype(np.int32)
    A_log, dt_bias = head_params(_rng(seed, _PARAMS), FULL)
    return MixedWorkload(seed=seed, shape=FULL, A_log=A_log, dt_bias=dt_bias, is_prefill=is_prefill,
                         prefill_lens=prefill_lens, warm_lens=warm_lens, n_windows=n_windows, raw_qk=raw_qk)
