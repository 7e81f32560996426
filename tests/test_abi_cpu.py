"""Host-side checks of the C ABI that need no GPU: every symbol declared in
include/llm.h is exported, sizing arithmetic, parameter validation, and the
call protocol on a dry handle (no device memory, no kernels)."""
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT, golden
from llama_decoder_forward_amd import configs

b = pytest.importorskip("llama_decoder_forward_amd.binding")


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "llm.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"\b(llm_[a-z_]+)\s*\(", hdr))
    assert len(names) >= 20
    for n in names:
        assert hasattr(b._lib, n), n
    assert names == set(b.EXPORTS), names ^ set(b.EXPORTS)


def test_sizing_matches_printed_kv_cache():
    g = golden("printed_values.txt")
    w = configs.L70B_BS32
    p = b.params_for(w)
    total = b.llm_kv_cache_bytes(p)
    assert total == int(g["kv_bytes_total_70b_b32_s4096"])
    assert total // w.n_layers == int(g["kv_bytes_per_layer_70b_b32_s4096"])
    assert round(total / 1e9, 1) == float(g["kv_gb_decimal_70b_mp1"])


def test_sizing_ffn_and_weights():
    for w in configs.WORKLOADS.values():
        p = b.params_for(w)
        assert b.llm_ffn_hidden(p) == w.ffn_hidden()
        assert b.llm_weight_bytes(p) == w.weight_bytes()
    assert b.llm_ffn_hidden(b.params_for(configs.L7B_BS1)) == int(golden("printed_values.txt")["ffn_hidden_dim4096_mo256"])
    # 70B weights: about 138 GB of fp16 (layer matrices + head)
    assert 137e9 < b.llm_weight_bytes(b.params_for(configs.L70B_BS32)) < 138e9


@pytest.mark.parametrize("field,value", [("n_layers", 0), ("dim", 100), ("n_kv_heads", 3),
                                         ("vocab_size", 1), ("max_seq_len", 100), ("max_batch_size", 0),
                                         ("dtype", 7), ("norm_eps", 0.0), ("rope_theta", -1.0)])
def test_param_validation(field, value):
    p = b.params_for(configs.L7B_BS1)
    assert b.llm_check_params(p) == b.LLM_OK
    setattr(p, field, value)
    assert b.llm_check_params(p) == b.LLM_EINVAL
    with pytest.raises(b.LlmError) as e:
        b.llm_create_dry(p)
    assert e.value.code == b.LLM_EINVAL


def test_dry_handle_protocol():
    w = configs.TINY
    h = b.llm_create_dry(b.params_for(w, max_batch_size=2))
    S, V = w.max_seq_len, w.vocab_size
    tok = np.zeros((2, 8), np.int32)

    def code(fn, *a):
        try:
            fn(*a)
            return b.LLM_OK
        except b.LlmError as e:
            return e.code

    assert code(h.decode, 8) == b.LLM_ESTATE                  # decode before prefill
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_ESTATE
    assert code(h.prefill, np.zeros((3, 8), np.int32)) == b.LLM_EINVAL   # B > max_batch
    assert code(h.prefill, np.zeros((1, S + 1), np.int32)) == b.LLM_EINVAL
    assert code(h.prefill, np.full((1, 4), V, np.int32)) == b.LLM_EINVAL  # token out of range
    assert code(h.prefill, np.full((1, 4), -1, np.int32)) == b.LLM_EINVAL
    assert code(h.prefill, tok) == b.LLM_OK
    assert code(h.decode, 8) == b.LLM_ESTATE                  # column 8 not written yet
    assert code(h.decode, 0) == b.LLM_EINVAL
    assert code(h.decode, S) == b.LLM_EINVAL
    assert code(h.sample, 0.8, 0.0, np.zeros(2, np.float32), False) == b.LLM_EINVAL   # top_p
    assert code(h.sample, 0.8, 1.5, np.zeros(2, np.float32), False) == b.LLM_EINVAL
    assert code(h.sample, float("nan"), 0.9, np.zeros(2, np.float32), False) == b.LLM_EINVAL
    assert code(h.sample, 0.8, 0.9, None, False) == b.LLM_EINVAL         # uniforms needed
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK             # writes column 8
    assert code(h.decode, 8) == b.LLM_OK
    assert code(h.decode, 10) == b.LLM_ESTATE                 # skips KV position 9
    assert code(h.set_tokens, 9, np.array([1, 2]), np.array([1, 0])) == b.LLM_OK  # partial mask
    assert code(h.decode, 9) == b.LLM_ESTATE
    assert code(h.set_tokens, 9, np.array([1, V])) == b.LLM_EINVAL
    assert code(h.set_tokens, 9, np.array([1, 2])) == b.LLM_OK
    assert code(h.decode, 9) == b.LLM_OK
    assert code(h.decode, 5) == b.LLM_OK                      # re-running an earlier position
    for p in range(10, S):                                      # fill to the end of the cache
        assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK
        assert code(h.decode, p) == b.LLM_ESTATE if p > 6 else True
        break
    assert code(h.get_logits) == b.LLM_ESTATE                 # dry handles return no values
    h.destroy()


def test_dry_handle_prefill_at():
    """Prefill at an offset: needs the cache prefix of the same batch and may
    not skip positions or run past the cache."""
    w = configs.TINY
    h = b.llm_create_dry(b.params_for(w, max_batch_size=2))
    S = w.max_seq_len

    def code(fn, *a):
        try:
            fn(*a)
            return b.LLM_OK
        except b.LlmError as e:
            return e.code

    z = lambda B, T: np.zeros((B, T), np.int32)
    assert code(h.prefill_at, 4, z(1, 4)) == b.LLM_ESTATE      # no prefix yet
    assert code(h.prefill_at, -1, z(1, 4)) == b.LLM_EINVAL
    assert code(h.prefill_at, 0, z(2, 6)) == b.LLM_OK          # start 0: a plain prefill
    assert code(h.prefill_at, 7, z(2, 4)) == b.LLM_ESTATE      # skips position 6
    assert code(h.prefill_at, 6, z(1, 4)) == b.LLM_ESTATE      # batch differs from the prefix
    assert code(h.prefill_at, 6, z(2, S - 5)) == b.LLM_EINVAL  # runs past the cache
    assert code(h.prefill_at, 6, np.full((2, 4), w.vocab_size, np.int32)) == b.LLM_EINVAL
    assert code(h.prefill_at, 6, z(2, 4)) == b.LLM_OK          # positions 6..9
    assert code(h.decode, 10) == b.LLM_ESTATE                  # column 10 not written
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK   # writes column 10
    assert code(h.decode, 10) == b.LLM_OK
    assert code(h.prefill_at, 3, z(2, 2)) == b.LLM_OK          # rewrite an earlier stretch
    assert code(h.decode, 5) == b.LLM_OK
    assert code(h.prefill_at, S - 2, z(2, 2)) == b.LLM_ESTATE  # beyond last position + 1
    h.destroy()


def test_dry_handle_varlen_rows():
    """Varlen prefill puts the rows at their own positions: per-row decode and
    tokens work, the uniform-position calls are refused until a plain
    prefill."""
    w = configs.TINY
    h = b.llm_create_dry(b.params_for(w, max_batch_size=2))
    S = w.max_seq_len

    def code(fn, *a):
        try:
            fn(*a)
            return b.LLM_OK
        except b.LlmError as e:
            return e.code

    r = lambda n: np.zeros(n, np.int32)
    assert code(h.decode_rows) == b.LLM_ESTATE                       # no varlen prefill yet
    assert code(h.prefill_varlen, [r(3), r(0)]) == b.LLM_EINVAL       # empty row
    assert code(h.prefill_varlen, [r(3), r(S + 1)]) == b.LLM_EINVAL   # longer than the cache
    assert code(h.prefill_varlen, [r(1)] * 3) == b.LLM_EINVAL         # B > max_batch_size
    assert code(h.prefill_varlen, [r(3), np.full(2, w.vocab_size, np.int32)]) == b.LLM_EINVAL
    assert code(h.prefill_varlen, [r(3), r(8)]) == b.LLM_OK
    assert code(h.decode_rows) == b.LLM_ESTATE                        # next columns not written
    assert code(h.decode, 8) == b.LLM_ESTATE                          # uniform calls refused
    assert code(h.set_tokens, 8, np.array([1, 2])) == b.LLM_ESTATE
    assert code(h.prefill_at, 3, np.zeros((2, 2), np.int32)) == b.LLM_ESTATE
    assert code(h.set_tokens_rows, np.array([1, 2]), np.array([1, 0])) == b.LLM_OK
    assert code(h.decode_rows) == b.LLM_ESTATE                        # row 1 still unwritten
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK          # writes both next columns
    assert code(h.decode_rows) == b.LLM_OK                            # rows now at 3 and 8
    assert code(h.set_tokens_rows, np.array([1, w.vocab_size])) == b.LLM_EINVAL
    for _ in range(S - 9):                                            # row 1 reaches S - 1
        assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK
        assert code(h.decode_rows) == b.LLM_OK
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK          # row 1's token has no column
    assert code(h.decode_rows) == b.LLM_EINVAL
    assert code(h.prefill, np.zeros((2, 4), np.int32)) == b.LLM_OK     # back to uniform rows
    assert code(h.sample, 0.0, 1.0, None, False) == b.LLM_OK
    assert code(h.decode, 4) == b.LLM_OK
    assert code(h.decode_rows) == b.LLM_ESTATE
    h.destroy()


def test_dry_handle_last_slot():
    """With prompt 8 and 24 steps the last decode runs at position S-1 = 31
    and its sampled token has no column left (it is returned, not stored)."""
    w = configs.TINY
    h = b.llm_create_dry(b.params_for(w))
    h.prefill(np.zeros((1, w.prompt_len), np.int32))
    h.sample(0.0, 1.0, None, False)
    for p in range(w.prompt_len, w.prompt_len + w.decode_steps):
        h.decode(p)
        h.sample(0.0, 1.0, None, False)
    assert w.prompt_len + w.decode_steps == w.max_seq_len
    with pytest.raises(b.LlmError):
        h.decode(w.max_seq_len)
    h.destroy()


def _code(fn, *a):
    try:
        fn(*a)
        return b.LLM_OK
    except b.LlmError as e:
        return e.code


def test_paging_parameters():
    """Block size, pool size and budget checks; block bytes follow
    2 * layers * block * kv_heads * head_dim * element size."""
    w = configs.TINY
    p = b.params_for(w, max_batch_size=3, max_seq_len=256)
    hd = w.dim // w.n_heads
    assert b.llm_kv_block_bytes(p, 32) == 2 * w.n_layers * 32 * w.n_kv_heads * hd * 4
    for bs, n in [(16, 4), (48, 4), (131072, 4), (32, -1), (32, 3 * 8 + 1), (32, 0)]:
        with pytest.raises(b.LlmError) as e:
            b.llm_create_paged_dry(p, b.make_paging(bs, n))
        assert e.value.code == b.LLM_EINVAL, (bs, n)
    h = b.llm_create_paged_dry(p, b.make_paging(64, 3 * 4))   # the largest pool: every row at 256
    assert (h.kv_num_blocks(), h.kv_free_blocks(), h.kv_table_width()) == (12, 12, 4)
    h.destroy()
    s = b.llm_create_dry(p)
    assert (s.kv_num_blocks(), s.kv_table_width()) == (0, 0)
    assert _code(s.kv_set_block_table, 0, [0]) == b.LLM_EINVAL       # not a paged handle
    s.destroy()


def test_paged_block_bookkeeping():
    """Blocks are handed out lowest id first as passes reach new positions,
    kept by their row, returned by a prefill from position 0 (rows >= B) or
    an explicit table; an exhausted pool and uncovered cached positions are
    refused before anything changes."""
    w = configs.TINY
    p = b.params_for(w, max_batch_size=3, max_seq_len=256)
    h = b.llm_create_paged_dry(p, b.make_paging(32, 10))
    tab = lambda r: [int(x) for x in h.kv_block_table(r) if x >= 0]
    zeros = lambda B, T: np.zeros((B, T), np.int32)
    assert _code(h.prefill, zeros(3, 40)) == b.LLM_OK                 # 2 blocks per row
    assert [tab(r) for r in range(3)] == [[0, 1], [2, 3], [4, 5]]
    for pos in range(40, 64):
        assert _code(h.set_tokens, pos, np.ones(3, np.int32)) == b.LLM_OK
        assert _code(h.decode, pos) == b.LLM_OK
    assert h.kv_free_blocks() == 4
    assert _code(h.set_tokens, 64, np.ones(3, np.int32)) == b.LLM_OK
    assert _code(h.decode, 64) == b.LLM_OK                            # a third block each
    assert [tab(r) for r in range(3)] == [[0, 1, 6], [2, 3, 7], [4, 5, 8]]
    for pos in range(65, 96):
        assert _code(h.set_tokens, pos, np.ones(3, np.int32)) == b.LLM_OK
        assert _code(h.decode, pos) == b.LLM_OK
    assert _code(h.set_tokens, 96, np.ones(3, np.int32)) == b.LLM_OK
    assert _code(h.decode, 96) == b.LLM_ENOMEM                        # 3 needed, 1 free
    assert h.kv_free_blocks() == 1 and tab(0) == [0, 1, 6]             # nothing changed
    assert _code(h.decode, 95) == b.LLM_OK                            # recomputing a position is fine
    h.kv_set_block_table(2, [])                                       # release row 2
    assert h.kv_free_blocks() == 4
    assert _code(h.decode, 96) == b.LLM_ESTATE                        # row 2's cache is gone
    # validation of explicit tables
    assert _code(h.kv_set_block_table, 2, [9, 9]) == b.LLM_EINVAL     # twice
    assert _code(h.kv_set_block_table, 2, [10]) == b.LLM_EINVAL       # out of the pool
    assert _code(h.kv_set_block_table, 2, [0]) == b.LLM_EINVAL        # row 0 holds it
    assert _code(h.kv_set_block_table, 2, list(range(4, 9)) + [9] * 4) == b.LLM_EINVAL  # wider than the table
    assert _code(h.kv_set_block_table, 3, [9]) == b.LLM_EINVAL        # no such row
    h.kv_set_block_table(2, [9, 5])
    assert tab(2) == [9, 5] and h.kv_free_blocks() == 2
    h.kv_set_block_table(0, [6, 1, 0])                                # a row may reorder its own blocks
    assert tab(0) == [6, 1, 0]
    # a prefill from 0 of two rows releases row 2 and extends rows 0 and 1
    assert _code(h.prefill, zeros(2, 100)) == b.LLM_OK
    assert [tab(r) for r in range(3)] == [[6, 1, 0, 4], [2, 3, 7, 5], []]
    assert h.kv_free_blocks() == 2
    assert _code(h.prefill_at, 100, zeros(2, 100)) == b.LLM_ENOMEM    # 3 more each, 2 free
    assert _code(h.prefill_at, 100, zeros(2, 28)) == b.LLM_OK         # stays in block 3
    # varlen: rows keep their blocks, rows past B are released first
    assert _code(h.prefill_varlen, [np.zeros(200, np.int32)]) == b.LLM_OK
    assert tab(0) == [6, 1, 0, 4, 2, 3, 5] and tab(1) == [] and h.kv_free_blocks() == 3
    h.destroy()
