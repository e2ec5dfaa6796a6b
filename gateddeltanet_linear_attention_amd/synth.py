"""Seeded synthetic inputs for the gated-delta-rule decode / verify / prefill path.

This module only draws random numbers and rounds them to the storage types the
kernels take (bfloat16 for q/k/v, float32 for gate logits and head parameters).
It holds none of the method's arithmetic: gates, state updates and outputs are
computed by the GPU library and, independently, by the fp64 oracle.  Both sides
receive exactly the arrays produced here.

Distributions (one draw per element unless stated):
  * q, k ~ N(0, 1), each (token, qk-head) vector L2-normalised; q then scaled by
    1/sqrt(d_k); rounded to bfloat16 (ties to even).
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


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are exactly bfloat16-representable."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


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


def tokens(rng: np.random.Generator, shape: HeadShape, n: int, gate_shift: float = 0.0) -> Tokens:
    """n fresh tokens.  gate_shift is added to the decay logit a (a negative shift makes
    the decay slow, alpha close to 1: a stress case for long memory)."""
    d = shape.d
    q = round_to_bf16(_unit_rows(rng, n, shape.n_qk_heads, d) / np.sqrt(d))
    k = round_to_bf16(_unit_rows(rng, n, shape.n_qk_heads, d))
    v = round_to_bf16(rng.standard_normal((n, shape.n_v_heads, d)))
    a = (rng.standard_normal((n, shape.n_v_heads)) + gate_shift).astype(np.float32)
    b = rng.standard_normal((n, shape.n_v_heads)).astype(np.float32)
    return Tokens(q, k, v, a, b)


def accepted_counts(rng: np.random.Generator, draft_lens: np.ndarray, p: float = ACCEPT_P) -> np.ndarray:
    """Accepted draft count per row, Binomial(K_r, p), int32."""
    return rng.binomial(np.asarray(draft_lens, dtype=np.int64), p).astype(np.int32)
