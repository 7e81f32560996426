"""Helpers for GPU tests: device buffers via torch (memory only), seeded
synthetic activations, and comparison against the oracle."""
import sys

import numpy as np


def say(*a):
    """Progress line flushed immediately (names the case before GPU work)."""
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """Copy a numpy array to a new device tensor (fp16 arrays go as float16)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a)).to("cuda")
    t.cuda.synchronize()
    return x


def host(x) -> np.ndarray:
    torch().cuda.synchronize()
    return x.detach().cpu().numpy()


def empty(shape, dtype):
    t = torch()
    return t.empty(shape, dtype={np.float16: t.float16, np.float32: t.float32,
                                 np.int32: t.int32}[dtype], device="cuda")


def randn_f16(rng, shape, scale=1.0) -> np.ndarray:
    """Seeded normal values rounded to fp16 (returned as float16)."""
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def f16_ulp(x: np.ndarray) -> np.ndarray:
    return np.spacing(np.abs(x).astype(np.float16)).astype(np.float32)


def within_one_f16_step(got, want) -> np.ndarray:
    """True where two fp16 values are at most one rounding step apart (the
    larger spacing of the two, so a step across a power of two counts)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    return np.abs(got - want) <= np.maximum(f16_ulp(got), f16_ulp(want)) * 1.0001 + 1e-7


def cosine(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sum(a * b, -1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1))
