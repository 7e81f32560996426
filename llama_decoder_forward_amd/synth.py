"""Seeded synthetic inputs shared by the HIP path's callers and the oracle.

This module holds no arithmetic of the decoder itself: it only draws the
integers and uniforms that stand in for prompts and for the sampler's random
numbers.  Every value comes from SplitMix64 (Steele, Lea & Flood, OOPSLA
2014): output n of the generator started at state s is mix(s + (n+1)*gamma).

* Row b of a token matrix uses the stream whose state is output b of the
  generator started at the seed; token t of that row is
  ``(out_t >> 32) * V >> 32`` (uniform over [0, V)).
* Sampler uniforms use the same per-row streams: ``(out_step >> 40) * 2^-24``,
  a float32 on the 24-bit grid in [0, 1).
* Prompt lengths (ragged batches) use the stream at index 2^40 of the seed:
  ``lo + ((out_b >> 32) * (hi - lo + 1) >> 32)``.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(state, n) -> np.ndarray:
    """Output(s) n of the SplitMix64 generator started at `state` (vectorised)."""
    with np.errstate(over="ignore"):
        s = np.asarray(state, dtype=np.uint64)
        k = np.asarray(n, dtype=np.uint64) + np.uint64(1)
        return _mix(s + k * _GAMMA)


def _row_states(seed: int, B: int) -> np.ndarray:
    return splitmix64(np.uint64(seed), np.arange(B, dtype=np.uint64))


def tokens(seed: int, B: int, T: int, vocab: int) -> np.ndarray:
    """int32[B][T] token ids uniform over [0, vocab)."""
    st = _row_states(seed, B)[:, None]
    h = splitmix64(st, np.arange(T, dtype=np.uint64)[None, :])
    with np.errstate(over="ignore"):
        v = ((h >> np.uint64(32)) * np.uint64(vocab)) >> np.uint64(32)
    return v.astype(np.int32)


def uniforms(seed: int, steps: int, B: int) -> np.ndarray:
    """float32[steps][B] on the 24-bit grid in [0, 1)."""
    st = _row_states(seed, B)[None, :]
    h = splitmix64(st, np.arange(steps, dtype=np.uint64)[:, None])
    return ((h >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def prompt_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """int32[B] lengths uniform over [lo, hi]."""
    st = splitmix64(np.uint64(seed), np.uint64(1 << 40))
    h = splitmix64(st, np.arange(B, dtype=np.uint64))
    with np.errstate(over="ignore"):
        v = ((h >> np.uint64(32)) * np.uint64(hi - lo + 1)) >> np.uint64(32)
    return (v.astype(np.int64) + lo).astype(np.int32)
