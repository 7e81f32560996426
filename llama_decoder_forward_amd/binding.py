"""ctypes binding of libllm.so: the C ABI of include/llm.h under the same
names.  Argument marshalling only -- every step of the forward pass runs in
the library's HIP kernels.  Importing this module fails loudly when the
library has not been built."""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllm.so")

LLM_OK, LLM_EINVAL, LLM_ESTATE, LLM_ENOMEM, LLM_EDEVICE = 0, -1, -2, -3, -4
LLM_F32, LLM_F16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m llama_decoder_forward_amd.build` "
                      "(or __graft_entry__.build()); there is no fallback path")

# One HIP runtime per process: torch ships its own libamdhip64 /
# libhsa-runtime64 under the same sonames as ROCm's.  Importing torch first
# makes libllm.so bind to that copy; loading ROCm's copy first and torch's
# afterwards leaves two runtimes in the process and torch then sees no GPU.
try:
    import torch  # noqa: F401
except ImportError:  # torch is optional for the C ABI itself
    torch = None

_lib = C.CDLL(LIB_PATH)


class llm_params(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("dim", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("vocab_size", C.c_int32), ("multiple_of", C.c_int32),
                ("ffn_dim_multiplier", C.c_float), ("norm_eps", C.c_float),
                ("rope_theta", C.c_float), ("max_batch_size", C.c_int32),
                ("max_seq_len", C.c_int32), ("dtype", C.c_int32)]


class llm_paging(C.Structure):
    _fields_ = [("block_size", C.c_int32), ("num_blocks", C.c_int32),
                ("gpu_memory_utilization", C.c_float)]


_vp = C.c_void_p
_P = C.POINTER(llm_params)
_PG = C.POINTER(llm_paging)
EXPORTS = {
    "llm_ffn_hidden": (C.c_int64, [_P]),
    "llm_kv_cache_bytes": (C.c_int64, [_P]),
    "llm_weight_bytes": (C.c_int64, [_P]),
    "llm_check_params": (C.c_int, [_P]),
    "llm_create": (C.c_int, [_P, C.c_uint64, _vp, C.POINTER(_vp)]),
    "llm_create_dry": (C.c_int, [_P, C.POINTER(_vp)]),
    "llm_destroy": (None, [_vp]),
    "llm_last_error": (C.c_char_p, [_vp]),
    "llm_get_stream": (_vp, [_vp]),
    "llm_prefill": (C.c_int, [_vp, _vp, C.c_int32, C.c_int32]),
    "llm_prefill_d": (C.c_int, [_vp, _vp, C.c_int32, C.c_int32]),
    "llm_decode": (C.c_int, [_vp, C.c_int32]),
    "llm_sample": (C.c_int, [_vp, C.c_float, C.c_float, _vp, _vp]),
    "llm_sample_d": (C.c_int, [_vp, C.c_float, C.c_float, _vp, _vp]),
    "llm_set_tokens": (C.c_int, [_vp, C.c_int32, _vp, _vp]),
    "llm_set_tokens_d": (C.c_int, [_vp, C.c_int32, _vp, _vp]),
    "llm_prefill_at": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32, C.c_int32]),
    "llm_prefill_varlen": (C.c_int, [_vp, _vp, _vp, C.c_int32]),
    "llm_prefill_varlen_d": (C.c_int, [_vp, _vp, _vp, C.c_int32]),
    "llm_decode_rows": (C.c_int, [_vp]),
    "llm_set_tokens_rows": (C.c_int, [_vp, _vp, _vp]),
    "llm_prefill_at_d": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32, C.c_int32]),
    "llm_profile_decode": (C.c_int, [_vp, C.c_int32, C.c_int32, _vp]),
    "llm_profile_prefill": (C.c_int, [_vp, _vp, C.c_int32, C.c_int32, C.c_int32, _vp]),
    "llm_profile_projections": (C.c_int, [_vp, C.c_int32, _vp]),
    "llm_get_logits": (C.c_int, [_vp, _vp]),
    "llm_get_logits_d": (C.c_int, [_vp, _vp]),
    "llm_get_tokens": (C.c_int, [_vp, C.c_int32, _vp]),
    "llm_sample_probs": (C.c_int, [_vp, _vp, C.c_int32, C.c_float, _vp, _vp]),
    "llm_sync": (C.c_int, [_vp]),
    "llm_read_weights": (C.c_int, [_vp, C.c_int32, C.c_int64, C.c_int64, _vp]),
    "llm_op_rmsnorm": (C.c_int, [_vp, _vp, C.c_int32, _vp]),
    "llm_op_linear": (C.c_int, [_vp, C.c_int32, C.c_int32, _vp, C.c_int32, _vp]),
    "llm_op_kv_write": (C.c_int, [_vp, C.c_int32, _vp, _vp, C.c_int32, C.c_int32, C.c_int32]),
    "llm_op_attention": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32, C.c_int32, C.c_int32, _vp]),
    "llm_op_layer": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32, C.c_int32, C.c_int32]),
    "llm_sample_logits_static": (C.c_int, [_vp, C.c_int32, C.c_int32, C.c_float, C.c_float, _vp, _vp, _vp]),
    "llm_kv_block_bytes": (C.c_int64, [_P, C.c_int32]),
    "llm_create_paged": (C.c_int, [_P, _PG, C.c_uint64, _vp, C.POINTER(_vp)]),
    "llm_create_paged_dry": (C.c_int, [_P, _PG, C.POINTER(_vp)]),
    "llm_kv_num_blocks": (C.c_int32, [_vp]),
    "llm_kv_free_blocks": (C.c_int32, [_vp]),
    "llm_kv_table_width": (C.c_int32, [_vp]),
    "llm_kv_block_table": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32]),
    "llm_kv_set_block_table": (C.c_int, [_vp, C.c_int32, _vp, C.c_int32]),
}
for _name, (_res, _args) in EXPORTS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class LlmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


def make_params(n_layers, dim, n_heads, n_kv_heads, vocab_size, multiple_of, ffn_dim_multiplier=0.0,
                norm_eps=1e-5, rope_theta=10000.0, max_batch_size=1, max_seq_len=2048,
                dtype=LLM_F16) -> llm_params:
    return llm_params(n_layers, dim, n_heads, n_kv_heads, vocab_size, multiple_of,
                      float(ffn_dim_multiplier or 0.0), norm_eps, rope_theta, max_batch_size,
                      max_seq_len, dtype)


def llm_ffn_hidden(p: llm_params) -> int:
    return _lib.llm_ffn_hidden(C.byref(p))


def llm_kv_cache_bytes(p: llm_params) -> int:
    return _lib.llm_kv_cache_bytes(C.byref(p))


def llm_weight_bytes(p: llm_params) -> int:
    return _lib.llm_weight_bytes(C.byref(p))


def llm_check_params(p: llm_params) -> int:
    return _lib.llm_check_params(C.byref(p))


def llm_kv_block_bytes(p: llm_params, block_size: int) -> int:
    return _lib.llm_kv_block_bytes(C.byref(p), block_size)


class Handle:
    """An llm_t* with the library's calls as methods (same names, minus the
    prefix) and errors raised as LlmError."""

    def __init__(self, ptr, params: llm_params):
        self.ptr = ptr
        self.params = params
        self.B = 0

    def _ck(self, rc):
        if rc != LLM_OK:
            msg = _lib.llm_last_error(self.ptr)
            raise LlmError(rc, msg.decode() if msg else "error")
        return rc

    @property
    def V(self):
        return self.params.vocab_size

    def stream(self) -> int:
        return _lib.llm_get_stream(self.ptr) or 0

    def prefill(self, tokens):
        t, p = _arr(tokens, np.int32)
        B, T = t.shape
        self._ck(_lib.llm_prefill(self.ptr, p, B, T))
        self.B = B

    def prefill_d(self, tokens_ptr: int, B: int, T: int):
        self._ck(_lib.llm_prefill_d(self.ptr, C.c_void_p(tokens_ptr), B, T))
        self.B = B

    def prefill_at(self, start_pos: int, tokens):
        t, p = _arr(tokens, np.int32)
        B, T = t.shape
        self._ck(_lib.llm_prefill_at(self.ptr, start_pos, p, B, T))
        self.B = B

    def prefill_at_d(self, start_pos: int, tokens_ptr: int, B: int, T: int):
        self._ck(_lib.llm_prefill_at_d(self.ptr, start_pos, C.c_void_p(tokens_ptr), B, T))
        self.B = B

    def prefill_varlen(self, rows):
        """rows: a list of 1-D token arrays of different lengths."""
        lens = np.ascontiguousarray([len(r) for r in rows], dtype=np.int32)
        packed = np.ascontiguousarray(np.concatenate([np.asarray(r, np.int32) for r in rows]))
        self._ck(_lib.llm_prefill_varlen(self.ptr, packed.ctypes.data_as(C.c_void_p),
                                         lens.ctypes.data_as(C.c_void_p), len(rows)))
        self.B = len(rows)

    def prefill_varlen_d(self, tokens_ptr: int, lens):
        ln = np.ascontiguousarray(lens, dtype=np.int32)
        self._ck(_lib.llm_prefill_varlen_d(self.ptr, C.c_void_p(tokens_ptr), ln.ctypes.data_as(C.c_void_p),
                                           len(ln)))
        self.B = len(ln)

    def decode_rows(self):
        self._ck(_lib.llm_decode_rows(self.ptr))

    def set_tokens_rows(self, tokens, mask=None):
        t, p = _arr(tokens, np.int32)
        mp = None
        if mask is not None:
            m, mp = _arr(mask, np.uint8)
        self._ck(_lib.llm_set_tokens_rows(self.ptr, p, mp))

    def decode(self, prev_pos: int):
        self._ck(_lib.llm_decode(self.ptr, prev_pos))

    def sample(self, temperature: float, top_p: float = 1.0, uniforms=None, want_tokens=True):
        up = None
        if uniforms is not None:
            u, up = _arr(uniforms, np.float32)
        out = np.empty(self.B, np.int32) if want_tokens else None
        self._ck(_lib.llm_sample(self.ptr, temperature, top_p, up,
                                 out.ctypes.data_as(C.c_void_p) if want_tokens else None))
        return out

    def sample_d(self, temperature: float, top_p: float, uniforms_ptr: int, out_ptr: int = 0):
        self._ck(_lib.llm_sample_d(self.ptr, temperature, top_p, C.c_void_p(uniforms_ptr or None),
                                   C.c_void_p(out_ptr or None)))

    def set_tokens(self, pos: int, tokens, mask=None):
        t, tp = _arr(tokens, np.int32)
        mp = None
        if mask is not None:
            m, mp = _arr(np.asarray(mask).astype(np.uint8), np.uint8)
        self._ck(_lib.llm_set_tokens(self.ptr, pos, tp, mp))

    def set_tokens_d(self, pos: int, tokens_ptr: int, mask_ptr: int = 0):
        self._ck(_lib.llm_set_tokens_d(self.ptr, pos, C.c_void_p(tokens_ptr), C.c_void_p(mask_ptr or None)))

    PROFILE_CLASSES = ("embed", "rmsnorm", "qkv", "attention", "o", "w13", "w2", "head", "step")

    def profile_decode(self, prev_pos: int, reps: int) -> dict:
        out = np.zeros(len(self.PROFILE_CLASSES), np.float32)
        self._ck(_lib.llm_profile_decode(self.ptr, prev_pos, reps, out.ctypes.data_as(C.c_void_p)))
        return dict(zip(self.PROFILE_CLASSES, out.tolist()))

    def profile_prefill_d(self, tokens_ptr: int, B: int, T: int, reps: int) -> dict:
        out = np.zeros(len(self.PROFILE_CLASSES), np.float32)
        self._ck(_lib.llm_profile_prefill(self.ptr, C.c_void_p(tokens_ptr), B, T, reps,
                                          out.ctypes.data_as(C.c_void_p)))
        self.B = B
        return dict(zip(self.PROFILE_CLASSES, out.tolist()))

    PRODUCT_KINDS = ("qkv", "o", "w13", "w2", "head", "step_order")

    def profile_projections(self, reps: int) -> dict:
        """Mean microseconds per launch of each decode weight product and of
        all of them in forward order, replayed from captured graphs; the
        handle needs a new prefill afterwards."""
        out = np.zeros(6, np.float32)
        self._ck(_lib.llm_profile_projections(self.ptr, reps, out.ctypes.data_as(C.c_void_p)))
        return dict(zip(self.PRODUCT_KINDS, out.tolist()))

    def get_logits(self) -> np.ndarray:
        out = np.empty((self.B, self.V), np.float32)
        self._ck(_lib.llm_get_logits(self.ptr, out.ctypes.data_as(C.c_void_p)))
        return out

    def get_logits_d(self, out_ptr: int):
        self._ck(_lib.llm_get_logits_d(self.ptr, C.c_void_p(out_ptr)))

    def get_tokens(self, n_cols: int) -> np.ndarray:
        out = np.empty((self.B, n_cols), np.int32)
        self._ck(_lib.llm_get_tokens(self.ptr, n_cols, out.ctypes.data_as(C.c_void_p)))
        return out

    def sample_probs(self, probs, top_p: float, uniforms) -> np.ndarray:
        p, pp = _arr(probs, np.float32)
        u, up = _arr(uniforms, np.float32)
        B = p.shape[0]
        out = np.empty(B, np.int32)
        self._ck(_lib.llm_sample_probs(self.ptr, pp, B, top_p, up, out.ctypes.data_as(C.c_void_p)))
        return out

    def sync(self):
        self._ck(_lib.llm_sync(self.ptr))

    def read_weights(self, tensor_id: int, first: int, count: int) -> np.ndarray:
        dt = np.uint16 if self.params.dtype == LLM_F16 else np.float32
        out = np.empty(count, dt)
        self._ck(_lib.llm_read_weights(self.ptr, tensor_id, first, count, out.ctypes.data_as(C.c_void_p)))
        return out

    def op_rmsnorm(self, x_ptr: int, M: int, y_ptr: int):
        self._ck(_lib.llm_op_rmsnorm(self.ptr, C.c_void_p(x_ptr), M, C.c_void_p(y_ptr)))

    def op_linear(self, layer: int, mat: int, x_ptr: int, M: int, y_ptr: int):
        self._ck(_lib.llm_op_linear(self.ptr, layer, mat, C.c_void_p(x_ptr), M, C.c_void_p(y_ptr)))

    def op_kv_write(self, layer: int, k_ptr: int, v_ptr: int, B: int, T: int, pos0: int):
        self._ck(_lib.llm_op_kv_write(self.ptr, layer, C.c_void_p(k_ptr), C.c_void_p(v_ptr), B, T, pos0))

    def op_attention(self, layer: int, q_ptr: int, B: int, T: int, pos0: int, out_ptr: int):
        self._ck(_lib.llm_op_attention(self.ptr, layer, C.c_void_p(q_ptr), B, T, pos0, C.c_void_p(out_ptr)))

    def op_layer(self, layer: int, x_ptr: int, B: int, T: int, pos0: int):
        self._ck(_lib.llm_op_layer(self.ptr, layer, C.c_void_p(x_ptr), B, T, pos0))

    def kv_num_blocks(self) -> int:
        return _lib.llm_kv_num_blocks(self.ptr)

    def kv_free_blocks(self) -> int:
        return _lib.llm_kv_free_blocks(self.ptr)

    def kv_table_width(self) -> int:
        return _lib.llm_kv_table_width(self.ptr)

    def kv_block_table(self, row: int) -> np.ndarray:
        n = self.kv_table_width()
        out = np.empty(n, np.int32)
        self._ck(_lib.llm_kv_block_table(self.ptr, row, out.ctypes.data_as(C.c_void_p), n))
        return out

    def kv_set_block_table(self, row: int, blocks):
        b, bp = _arr(blocks, np.int32)
        self._ck(_lib.llm_kv_set_block_table(self.ptr, row, bp if b.size else None, b.size))

    def destroy(self):
        if self.ptr:
            _lib.llm_destroy(self.ptr)
            self.ptr = None

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.destroy()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def llm_sample_logits_static(logits_ptr: int, B: int, V: int, temperature: float, top_p: float,
                             uniforms_ptr: int, out_ptr: int, hip_stream: int | None = None) -> None:
    """Handle-free, allocation-free sampling on device buffers (asynchronous)."""
    rc = _lib.llm_sample_logits_static(C.c_void_p(logits_ptr), B, V, temperature, top_p,
                                       C.c_void_p(uniforms_ptr) if uniforms_ptr else None,
                                       C.c_void_p(out_ptr), C.c_void_p(hip_stream) if hip_stream else None)
    if rc != LLM_OK:
        msg = _lib.llm_last_error(None)
        raise LlmError(rc, msg.decode() if msg else "error")


def llm_create(params: llm_params, seed: int, hip_stream: int | None = None) -> Handle:
    out = C.c_void_p()
    rc = _lib.llm_create(C.byref(params), seed, C.c_void_p(hip_stream or None), C.byref(out))
    if rc != LLM_OK:
        raise LlmError(rc, "llm_create failed")
    return Handle(out, params)


def llm_create_dry(params: llm_params) -> Handle:
    out = C.c_void_p()
    rc = _lib.llm_create_dry(C.byref(params), C.byref(out))
    if rc != LLM_OK:
        raise LlmError(rc, "llm_create_dry failed")
    return Handle(out, params)


def make_paging(block_size: int, num_blocks: int = 0, gpu_memory_utilization: float = 0.9) -> llm_paging:
    return llm_paging(block_size, num_blocks, gpu_memory_utilization)


def llm_create_paged(params: llm_params, paging: llm_paging, seed: int, hip_stream: int | None = None) -> Handle:
    out = C.c_void_p()
    rc = _lib.llm_create_paged(C.byref(params), C.byref(paging), seed, C.c_void_p(hip_stream or None),
                               C.byref(out))
    if rc != LLM_OK:
        raise LlmError(rc, "llm_create_paged failed")
    return Handle(out, params)


def llm_create_paged_dry(params: llm_params, paging: llm_paging) -> Handle:
    out = C.c_void_p()
    rc = _lib.llm_create_paged_dry(C.byref(params), C.byref(paging), C.byref(out))
    if rc != LLM_OK:
        raise LlmError(rc, "llm_create_paged_dry failed")
    return Handle(out, params)


def params_for(workload, max_batch_size=None, max_seq_len=None) -> llm_params:
    """llm_params of a configs.Workload."""
    return make_params(**workload.model_kwargs(max_batch_size, max_seq_len))
