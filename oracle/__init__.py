"""CPU oracle for the Llama-2 decoder forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does, and the
two share no code: this wrapper loads ``liboracle.so`` built from
``oracle/oracle.c`` with gcc and nothing else.

Every array crosses the boundary as a numpy array; activations are float32
arrays whose values are already rounded to the model's storage type.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16 = 0, 1


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no fast-math,
    no FMA contraction so every fp32 operation rounds on its own)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-mavx2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-std=gnu11", "-Wall", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


class Params(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("dim", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("vocab_size", C.c_int32), ("multiple_of", C.c_int32),
                ("ffn_dim_multiplier", C.c_float), ("norm_eps", C.c_float),
                ("rope_theta", C.c_float), ("max_batch_size", C.c_int32),
                ("max_seq_len", C.c_int32), ("dtype", C.c_int32)]


_lib = None


def lib():
    """The loaded oracle library.  ORACLE_LIB names another build of
    oracle.c to load instead (the planted-mistake tests use it)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            build()
            path = _LIB
        L = C.CDLL(path)
        P = C.POINTER
        vp = C.c_void_p
        sig = {
            "orc_f64_to_f16": (C.c_uint16, [C.c_double]),
            "orc_f32_to_f16": (C.c_uint16, [C.c_float]),
            "orc_f16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_splitmix64_at": (C.c_uint64, [C.c_uint64, C.c_uint64]),
            "orc_weight_value": (C.c_double, [C.c_uint64, C.c_int32, C.c_uint64]),
            "orc_gen_tensor": (None, [C.c_uint64, C.c_int32, C.c_uint64, C.c_uint64, C.c_int32, vp]),
            "orc_ffn_hidden": (C.c_int32, [C.c_int32, C.c_int32, C.c_float]),
            "orc_rope_table": (None, [C.c_int32, C.c_int32, C.c_float, vp, vp]),
            "orc_rmsnorm": (None, [vp, vp, C.c_int32, C.c_float, C.c_int32, C.c_int32, vp]),
            "orc_rope_apply": (None, [vp, C.c_int32, vp, vp, C.c_int32]),
            "orc_attention_row": (None, [vp, vp, vp, C.c_int32, C.c_int32, C.c_int64, C.c_int32,
                                         C.c_int32, vp]),
            "orc_silu": (C.c_float, [C.c_float]),
            "orc_model_create": (vp, [P(Params), C.c_uint64, C.c_int32]),
            "orc_model_destroy": (None, [vp]),
            "orc_model_forward": (C.c_int, [vp, vp, C.c_int32, C.c_int32, C.c_int32, vp]),
            "orc_model_weights": (C.c_int, [vp, C.c_int32, C.c_uint64, C.c_uint64, vp]),
            "orc_forward_stream": (C.c_int, [P(Params), C.c_uint64, C.c_int32, vp, C.c_int32,
                                             C.c_int32, C.c_int32, vp]),
            "orc_layer_apply": (C.c_int, [P(Params), C.c_uint64, C.c_int32, C.c_int32, vp, C.c_int32,
                                          C.c_int32]),
            "orc_model_forward_resid": (C.c_int, [vp, vp, C.c_int32, C.c_int32, C.c_int32, vp, vp]),
            "orc_forward_stream_resid": (C.c_int, [P(Params), C.c_uint64, C.c_int32, vp, C.c_int32,
                                                   C.c_int32, C.c_int32, vp, vp]),
            "orc_argmax": (C.c_int32, [vp, C.c_int32]),
            "orc_softmax_temp": (None, [vp, C.c_int32, C.c_float, vp]),
            "orc_top_p": (C.c_int32, [vp, C.c_int32, C.c_float, C.c_float, P(C.c_int32)]),
            "orc_num_threads": (C.c_int32, []),
            "orc_model_set_weights": (C.c_int, [vp, C.c_int32, vp]),
            "orc_linear": (None, [vp, C.c_int32, C.c_int32, C.c_int32, vp, C.c_int32, C.c_int32,
                                  C.c_int32, vp]),
            "orc_f64_to_f16_vec": (None, [vp, C.c_int64, vp]),
            "orc_f32_to_f16_vec": (None, [vp, C.c_int64, vp]),
            "orc_f16_to_f32_vec": (None, [vp, C.c_int64, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------
# Scalar helpers
# ----------------------------------------------------------------------------
def f64_to_f16_bits(v: float) -> int:
    return lib().orc_f64_to_f16(float(v))


def f32_to_f16_bits(v: float) -> int:
    return lib().orc_f32_to_f16(float(v))


def f16_bits_to_f32(h: int) -> float:
    return lib().orc_f16_to_f32(int(h))


def f32_to_f16_array(x) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_vec(_ptr(x), x.size, _ptr(out))
    return out


def f64_to_f16_array(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f64_to_f16_vec(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f32_array(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_vec(_ptr(h), h.size, _ptr(out))
    return out


def splitmix64_at(state: int, n: int) -> int:
    return lib().orc_splitmix64_at(state & (2**64 - 1), n)


def weight_value(seed: int, tensor_id: int, e: int) -> float:
    return lib().orc_weight_value(seed, tensor_id, e)


def gen_tensor(seed: int, tensor_id: int, first: int, count: int, dtype: int) -> np.ndarray:
    """Stored elements [first, first+count) of a seeded weight tensor:
    uint16 bit patterns for fp16 models, float32 for fp32 models."""
    out = np.empty(count, dtype=np.uint16 if dtype == F16 else np.float32)
    lib().orc_gen_tensor(seed, tensor_id, first, count, dtype, _ptr(out))
    return out


def ffn_hidden(dim: int, multiple_of: int, mult: float | None) -> int:
    return lib().orc_ffn_hidden(dim, multiple_of, float(mult) if mult else 0.0)


def rope_table(head_dim: int, n_pos: int, theta: float):
    c = np.empty((n_pos, head_dim // 2), np.float32)
    s = np.empty((n_pos, head_dim // 2), np.float32)
    lib().orc_rope_table(head_dim, n_pos, theta, _ptr(c), _ptr(s))
    return c, s


def rmsnorm(x, eps: float = 1e-5, dtype: int = F16, acc64: bool = False, w=None) -> np.ndarray:
    x = _f32(x)
    y = np.empty_like(x)
    wp = None if w is None else _f32(w)
    lib().orc_rmsnorm(_ptr(x), None if wp is None else _ptr(wp), x.size, eps, dtype, int(acc64),
                      _ptr(y))
    return y


def rope_apply(v, cos_row, sin_row, dtype: int = F32) -> np.ndarray:
    v = _f32(v).copy()
    lib().orc_rope_apply(_ptr(v), v.size, _ptr(_f32(cos_row)), _ptr(_f32(sin_row)), dtype)
    return v


def attention_row(q, K, V, dtype: int = F32, acc64: bool = False) -> np.ndarray:
    """One query against keys K[L][d] / values V[L][d] (all visible)."""
    q, K, V = _f32(q), _f32(K), _f32(V)
    L, d = K.shape
    out = np.empty(d, np.float32)
    lib().orc_attention_row(_ptr(q), _ptr(K), _ptr(V), L, d, d, dtype, int(acc64), _ptr(out))
    return out


def linear(W, X, out_dtype: int = F16, acc64: bool = False) -> np.ndarray:
    """Y[M][N] = round(W X) for weights W[N][K] given as uint16 binary16 bit
    patterns or float32, and float32 rows X[M][K]."""
    W = np.ascontiguousarray(W)
    wd = F16 if W.dtype == np.uint16 else F32
    if wd == F32:
        W = W.astype(np.float32)
    X = _f32(X)
    N, K = W.shape
    M = X.shape[0]
    Y = np.empty((M, N), np.float32)
    lib().orc_linear(_ptr(W), wd, N, K, _ptr(X), M, out_dtype, int(acc64), _ptr(Y))
    return Y


def silu(x: float) -> float:
    return lib().orc_silu(float(x))


def argmax(logits) -> int:
    lg = _f32(logits)
    return lib().orc_argmax(_ptr(lg), lg.size)


def softmax_temp(logits, temperature: float) -> np.ndarray:
    lg = _f32(logits)
    p = np.empty_like(lg)
    lib().orc_softmax_temp(_ptr(lg), lg.size, float(temperature), _ptr(p))
    return p


def top_p(probs, top_p_: float, u: float):
    """Returns (token, number of kept tokens)."""
    p = _f32(probs)
    k = C.c_int32(0)
    tok = lib().orc_top_p(_ptr(p), p.size, float(top_p_), float(u), C.byref(k))
    return tok, k.value


def sample(logits, temperature: float, top_p_: float, u: float) -> int:
    """Greedy when temperature <= 0, else temperature softmax then top-p."""
    if temperature <= 0:
        return argmax(logits)
    return top_p(softmax_temp(logits, temperature), top_p_, u)[0]


def num_threads() -> int:
    return lib().orc_num_threads()


# ----------------------------------------------------------------------------
# Models
# ----------------------------------------------------------------------------
@dataclass
class Cfg:
    n_layers: int
    dim: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int
    multiple_of: int
    ffn_dim_multiplier: float = 0.0
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    max_batch_size: int = 1
    max_seq_len: int = 32
    dtype: int = F16

    def params(self) -> Params:
        return Params(self.n_layers, self.dim, self.n_heads, self.n_kv_heads, self.vocab_size,
                      self.multiple_of, self.ffn_dim_multiplier, self.norm_eps, self.rope_theta,
                      self.max_batch_size, self.max_seq_len, self.dtype)


class Model:
    """Resident oracle model with its own static KV cache."""

    def __init__(self, cfg: Cfg, seed: int, acc64: bool = False):
        self.cfg = cfg
        self._p = cfg.params()
        self._h = lib().orc_model_create(C.byref(self._p), seed, int(acc64))
        if not self._h:
            raise MemoryError("oracle model allocation failed")

    def forward(self, tokens, start_pos: int, resid: bool = False):
        """tokens[B][T] at positions start_pos.. -> fp32 logits[B][V] of the
        last position of each row; the KV cache is updated.  With resid the
        residual stream at every layer boundary is returned too, shaped
        [n_layers + 1][B][T][dim] (entry 0 the embedding rows, entry l + 1
        the output of layer l): (logits, resid)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        B, T = t.shape
        out = np.empty((B, self.cfg.vocab_size), np.float32)
        r = np.empty((self.cfg.n_layers + 1, B, T, self.cfg.dim), np.float32) if resid else None
        rc = lib().orc_model_forward_resid(self._h, _ptr(t), B, T, start_pos, _ptr(out),
                                           None if r is None else _ptr(r))
        if rc != 0:
            raise ValueError("oracle forward rejected its arguments")
        return (out, r) if resid else out

    def weights(self, tensor_id: int, first: int, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.uint16 if self.cfg.dtype == F16 else np.float32)
        if lib().orc_model_weights(self._h, tensor_id, first, count, _ptr(out)) != 0:
            raise ValueError("bad tensor range")
        return out

    def set_weights(self, tensor_id: int, data: np.ndarray):
        data = np.ascontiguousarray(data, dtype=np.uint16 if self.cfg.dtype == F16 else np.float32)
        if lib().orc_model_set_weights(self._h, tensor_id, _ptr(data)) != 0:
            raise ValueError("bad tensor id")

    def close(self):
        if self._h:
            lib().orc_model_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def forward_stream(cfg: Cfg, seed: int, tokens, first_pos: int, acc64: bool = False,
                   resid: bool = False):
    """Layer-major forward of whole sequences tokens[B][N]; returns the fp32
    logits of positions first_pos..N-1, shaped [B][N-first_pos][V].  With
    resid also the residual stream at every layer boundary, shaped
    [n_layers + 1][B][N][dim]: (logits, resid)."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    B, N = t.shape
    out = np.empty((B, N - first_pos, cfg.vocab_size), np.float32)
    r = np.empty((cfg.n_layers + 1, B, N, cfg.dim), np.float32) if resid else None
    p = cfg.params()
    rc = lib().orc_forward_stream_resid(C.byref(p), seed, int(acc64), _ptr(t), B, N, first_pos,
                                        _ptr(out), None if r is None else _ptr(r))
    if rc != 0:
        raise ValueError("oracle stream forward rejected its arguments")
    return (out, r) if resid else out


def layer_apply(cfg: Cfg, seed: int, layer: int, x, acc64: bool = False) -> np.ndarray:
    """One TransformerBlock of the seeded model on residual rows x[B][N][dim]
    (positions 0..N-1 of each row, causal); returns the rows leaving it."""
    y = np.array(x, dtype=np.float32, order="C", copy=True)
    B, N, _ = y.shape
    p = cfg.params()
    if lib().orc_layer_apply(C.byref(p), seed, layer, int(acc64), _ptr(y), B, N) != 0:
        raise ValueError("oracle layer_apply rejected its arguments")
    return y
