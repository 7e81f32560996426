"""Paged KV cache on the GPU: the cache as a pool of blocks reached through
per-row block tables (nano-vllm notes: allocate_kv_cache, block tables and
slot mapping) computes exactly what the static cache computes.

* A paged handle's logits equal a static handle's (same parameters, seed and
  calls) bit for bit -- the kernels sum in the same order, only the cache
  addresses differ -- over prefill, decode steps that cross block
  boundaries, chunked prefill, varlen prefill and per-row decode, with blocks
  handed out on demand and with scrambled tables set by the caller; two
  cases also against the oracle.
* The attention and KV-write kernels alone, on scrambled tables, equal the
  static ones bit for bit for the decode kernel's three work-group shapes
  and the prefill kernel (32-position blocks put each 64-key tile in two).
* A pool sized from a memory budget fills that budget.
"""
import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import synth
from tests.gpu_util import cosine, dev, empty, host, randn_f16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


def small_kw(**kw):
    base = dict(n_layers=2, dim=512, n_heads=4, n_kv_heads=2, vocab_size=1024, multiple_of=64,
                ffn_dim_multiplier=0.0, max_batch_size=3, max_seq_len=256, dtype=1)
    base.update(kw)
    return base


def fp32_kw(**kw):
    base = dict(n_layers=2, dim=64, n_heads=4, n_kv_heads=2, vocab_size=256, multiple_of=32,
                ffn_dim_multiplier=0.0, max_batch_size=2, max_seq_len=96, dtype=0)
    base.update(kw)
    return base


def scramble(h, rows, seed):
    """Give rows 0..rows-1 full tables drawn from a random permutation of
    the pool (every row's blocks out of order and interleaved with the
    others')."""
    n, wdt = h.kv_num_blocks(), h.kv_table_width()
    assert n >= rows * wdt
    perm = np.random.default_rng(seed).permutation(n).astype(np.int32)
    for r in range(rows):
        h.kv_set_block_table(r, perm[r * wdt:(r + 1) * wdt])


def uniform_run(h, toks, chunks, steps):
    """Chunked prefill, then forced decode steps; logits after each."""
    out, pos = [], 0
    for c in chunks:
        h.prefill_at(pos, toks[:, pos:pos + c])
        pos += c
        out.append(h.get_logits())
    for p in range(pos, pos + steps):
        h.set_tokens(p, toks[:, p])
        h.decode(p)
        out.append(h.get_logits())
    return np.stack(out, 1)


def rows_run(h, toks, lens, steps):
    """Varlen prefill, then forced per-row decode steps."""
    h.prefill_varlen([toks[b, :lens[b]] for b in range(len(lens))])
    out = [h.get_logits()]
    for k in range(steps):
        h.set_tokens_rows([toks[b, lens[b] + k] for b in range(len(lens))])
        h.decode_rows()
        out.append(h.get_logits())
    return np.stack(out, 1)


CASES = {
    # name: (model kwargs, block size, scrambled tables, run, arguments)
    "fp32-bs32": (fp32_kw(), 32, False, "uniform", dict(chunks=[20], steps=40)),
    "fp32-rows-bs32": (fp32_kw(), 32, True, "rows", dict(lens=[3, 40], steps=30)),
    "fp16-bs32-scrambled": (small_kw(), 32, True, "uniform", dict(chunks=[40, 30], steps=20)),
    "fp16-bs64": (small_kw(), 64, False, "uniform", dict(chunks=[70], steps=70)),
    "fp16-rows-bs64": (small_kw(), 64, False, "rows", dict(lens=[5, 70, 130], steps=10)),
    "fp16-wide-rows-bs32": (small_kw(max_batch_size=20, max_seq_len=128), 32, True, "rows",
                            dict(lens=None, steps=6)),
    "fp16-tiled-bs256": (small_kw(max_batch_size=1, max_seq_len=1280), 256, False, "uniform",
                         dict(chunks=[1040], steps=3)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_paged_equals_static(B, case):
    kw, bs, scr, run, args = CASES[case]
    Bn = kw["max_batch_size"]
    if run == "rows" and args["lens"] is None:
        args = dict(args, lens=list(synth.prompt_lengths(61, Bn, 1, 60)))
    if run == "uniform":
        N = sum(args["chunks"]) + args["steps"]
        toks = synth.tokens(60, Bn, N, kw["vocab_size"])
        go = lambda h: uniform_run(h, toks, args["chunks"], args["steps"])
    else:
        Bn = len(args["lens"])
        N = max(args["lens"]) + args["steps"]
        toks = synth.tokens(60, Bn, N, kw["vocab_size"])
        go = lambda h: rows_run(h, toks, args["lens"], args["steps"])
    p = B.make_params(**kw)
    width = -(-kw["max_seq_len"] // bs)
    say("paged vs static", case)
    hs = B.llm_create(p, 99)
    want = go(hs)
    hs.destroy()
    hp = B.llm_create_paged(p, B.make_paging(bs, kw["max_batch_size"] * width), 99)
    if scr:
        scramble(hp, Bn, 7)
    got = go(hp)
    if not scr:  # on demand: each row holds exactly the blocks its positions reach
        ends = ([N] * Bn) if run == "uniform" else [n + args["steps"] for n in args["lens"]]
        for b in range(Bn):
            t = hp.kv_block_table(b)
            assert (t[:-(-ends[b] // bs)] >= 0).all() and (t[-(-ends[b] // bs):] < 0).all()
    hp.destroy()
    assert got.shape == want.shape
    assert np.array_equal(got, want), np.abs(got - want).max()
    if case in ("fp16-bs32-scrambled", "fp32-rows-bs32"):
        say("  oracle")
        if run == "uniform":
            full = oracle.forward_stream(oracle.Cfg(**kw), 99, toks, 0)
            ends = list(np.cumsum(args["chunks"]) - 1) + list(range(sum(args["chunks"]), N))
            ref = full[:, ends]
            d = np.abs(got - ref)
            cos = cosine(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]))
            assert d.max() <= 5e-2 and cos.min() >= 0.9999, (d.max(), cos.min())
        else:
            for b, n in enumerate(args["lens"]):
                ref = oracle.forward_stream(oracle.Cfg(**kw), 99, toks[b:b + 1, :n + args["steps"]], n - 1)[0]
                assert np.abs(got[b] - ref).max() <= 1e-3


@pytest.mark.parametrize("Bn,L,bs", [(16, 300, 32), (64, 300, 64), (160, 200, 32), (256, 77, 32), (256, 1, 32),
                                     (64, 33, 128)])
def test_paged_attention_decode_kernel(B, Bn, L, bs):
    """32 and 128, 320, and 512 (row, KV head) pairs: the eight-, four- and
    two-wave decode work-groups read scrambled tables; equal to the static
    cache."""
    kw = small_kw(max_batch_size=Bn, max_seq_len=320)
    H, Hkv, d = kw["n_heads"], kw["n_kv_heads"], 128
    rng = np.random.default_rng(70 + L)
    K = randn_f16(rng, (Bn, L, Hkv, d))
    V = randn_f16(rng, (Bn, L, Hkv, d))
    q = randn_f16(rng, (Bn, 1, H, d), 0.3)
    say("paged decode attention", Bn, L, bs)
    p = B.make_params(**kw)
    kd, vd, qd = dev(K), dev(V), dev(q)
    outs = []
    for paged in (False, True):
        if paged:
            h = B.llm_create_paged(p, B.make_paging(bs, Bn * (-(-320 // bs))), 78)
            scramble(h, Bn, L)
        else:
            h = B.llm_create(p, 78)
        h.op_kv_write(0, kd.data_ptr(), vd.data_ptr(), Bn, L, 0)
        od = empty((Bn, 1, H, d), np.float16)
        h.op_attention(0, qd.data_ptr(), Bn, 1, L - 1, od.data_ptr())
        outs.append(host(od))
        h.destroy()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("T,bs", [(63, 32), (129, 32), (200, 64), (300, 256)])
def test_paged_attention_prefill_kernel(B, T, bs):
    kw = small_kw(max_batch_size=2, max_seq_len=320)
    Bn, H, Hkv, d = 2, kw["n_heads"], kw["n_kv_heads"], 128
    rng = np.random.default_rng(80 + T)
    K = randn_f16(rng, (Bn, T, Hkv, d))
    V = randn_f16(rng, (Bn, T, Hkv, d))
    q = randn_f16(rng, (Bn, T, H, d), 0.3)
    say("paged prefill attention", T, bs)
    p = B.make_params(**kw)
    kd, vd, qd = dev(K), dev(V), dev(q)
    outs = []
    for paged in (False, True):
        if paged:
            h = B.llm_create_paged(p, B.make_paging(bs, Bn * (-(-320 // bs))), 79)
            scramble(h, Bn, T)
        else:
            h = B.llm_create(p, 79)
        h.op_kv_write(1, kd.data_ptr(), vd.data_ptr(), Bn, T, 0)
        od = empty((Bn, T, H, d), np.float16)
        h.op_attention(1, qd.data_ptr(), Bn, T, 0, od.data_ptr())
        outs.append(host(od))
        h.destroy()
    assert np.array_equal(outs[0], outs[1])


def test_paged_pool_from_budget(B):
    """num_blocks = 0: the pool takes total * utilisation minus what the
    process holds once weights, buffers and the largest pass's workspace are
    allocated (a 4-layer model of 7B width, 32 rows of 4096 positions, so
    that the budget and not the table size bounds the pool)."""
    import torch
    kw = dict(n_layers=4, dim=4096, n_heads=32, n_kv_heads=32, vocab_size=32000, multiple_of=256,
              ffn_dim_multiplier=0.0, max_batch_size=32, max_seq_len=4096, dtype=1)
    p = B.make_params(**kw)
    bs = 64
    per_block = B.llm_kv_block_bytes(p, bs)
    assert per_block == 2 * 4 * bs * 32 * 128 * 2
    free0, total = torch.cuda.mem_get_info()
    util = (total - free0 + (12 << 30)) / total
    say("paged pool from budget", f"util {util:.4f}")
    h = B.llm_create_paged(p, B.make_paging(bs, 0, util), 5)
    free1, _ = torch.cuda.mem_get_info()
    n = h.kv_num_blocks()
    cap = 32 * (4096 // bs)
    say(f"  {n} blocks of {per_block >> 20} MiB (table cap {cap})")
    assert 0 < n < cap
    used = total - free1
    assert used <= total * util + per_block
    assert used >= total * util - per_block - (256 << 20)
    # the handle works: a short prefill and a decode step
    toks = synth.tokens(62, 2, 70, kw["vocab_size"])
    h.prefill(toks[:, :65])
    h.set_tokens(65, toks[:, 65])
    h.decode(65)
    assert np.isfinite(h.get_logits()).all()
    assert n - h.kv_free_blocks() == 4
    h.destroy()
