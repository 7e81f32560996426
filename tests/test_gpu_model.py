"""End-to-end parity on the GPU: prefill + decode steps through the C ABI
against the oracle on the same seeded weights and tokens.

Protocol: the GPU consumes the oracle's token stream (teacher forcing via
llm_set_tokens), logits are compared at every step (max |delta| <= 5e-2,
cosine >= 0.9999 per row), and greedy ids must agree wherever the oracle's
top-1 margin exceeds 0.1."""
import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import configs, synth
from tests.gpu_util import cosine, say

pytestmark = pytest.mark.gpu

LOGIT_TOL = 5e-2
COS_TOL = 0.9999
MARGIN = 0.1


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


def ocfg(kw):
    return oracle.Cfg(**kw)


def gpu_forced_logits(h, tokens, T0, steps):
    """Prefill tokens[:, :T0], then decode steps at T0.. with the columns
    forced to `tokens`; returns logits [B][steps+1][V] and the GPU's argmax
    ids before forcing [B][steps+1]."""
    h.prefill(tokens[:, :T0])
    logits = [h.get_logits()]
    ids = [h.sample(0.0)]
    for p in range(T0, T0 + steps):
        h.set_tokens(p, tokens[:, p])
        h.decode(p)
        logits.append(h.get_logits())
        ids.append(h.sample(0.0))
    return np.stack(logits, 1), np.stack(ids, 1)


def oracle_greedy_stream(cfg, seed, prompt, steps):
    m = oracle.Model(cfg, seed)
    Bn, T0 = prompt.shape
    toks = np.zeros((Bn, T0 + steps + 1), np.int32)
    toks[:, :T0] = prompt
    lg = m.forward(prompt, 0)
    margins = []
    for p in range(T0, T0 + steps + 1):
        srt = np.sort(lg, -1)
        margins.append(srt[:, -1] - srt[:, -2])
        toks[:, p] = lg.argmax(-1)  # numpy argmax: lowest index on ties, like the oracle
        if p < T0 + steps:
            lg = m.forward(toks[:, p:p + 1], p)
    m.close()
    return toks, np.stack(margins, 1)


def check_logits(got, want):
    d = np.abs(got - want)
    cos = cosine(got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1]))
    say(f"  max|d|={d.max():.3e} min cos={cos.min():.7f}")
    assert d.max() <= LOGIT_TOL, d.max()
    assert cos.min() >= COS_TOL, cos.min()


def test_tiny_fp32_greedy(B):
    w = configs.TINY
    kw = w.model_kwargs()
    prompt = synth.tokens(w.token_seed, 1, w.prompt_len, w.vocab_size)
    say("tiny: oracle greedy stream")
    toks, margins = oracle_greedy_stream(ocfg(kw), w.weight_seed, prompt, w.decode_steps - 1)
    # 8 + 24 = 32 positions: the last sampled token has no column (S = 32)
    h = B.llm_create(B.make_params(**kw), w.weight_seed)
    say("tiny: gpu teacher forced")
    got, ids = gpu_forced_logits(h, toks, w.prompt_len, w.decode_steps)
    want = oracle.forward_stream(ocfg(kw), w.weight_seed, toks[:, :w.max_seq_len], w.prompt_len - 1)
    check_logits(got, want)
    ok = margins > MARGIN                       # [1][24]: logits at positions 7..30
    assert np.array_equal(ids[:, :-1][ok], toks[:, w.prompt_len:][ok])
    # free-running greedy on the GPU gives the oracle's stream up to the first
    # sub-margin step
    h.prefill(prompt)
    free = [h.sample(0.0)[0]]
    for p in range(w.prompt_len, w.prompt_len + w.decode_steps):
        h.decode(p)
        free.append(h.sample(0.0)[0])
    free = np.array(free)
    n_ok = int(np.argmin(ok[0])) if not ok[0].all() else ok.shape[1]
    assert np.array_equal(free[:n_ok], toks[0, w.prompt_len:][:n_ok])
    # the token buffer holds prompt + sampled tokens; the final sample (at
    # position S-1) is returned but has no column
    buf = h.get_tokens(w.max_seq_len)
    assert np.array_equal(buf[0, :w.prompt_len], prompt[0])
    assert np.array_equal(buf[0, w.prompt_len:], free[:-1])
    h.destroy()


def small_kw(**kw):
    base = dict(n_layers=2, dim=512, n_heads=4, n_kv_heads=2, vocab_size=1024, multiple_of=64,
                ffn_dim_multiplier=0.0, max_batch_size=3, max_seq_len=128, dtype=1)
    base.update(kw)
    return base


@pytest.mark.parametrize("rows,T0", [(3, 5), (3, 40), (1, 9), (2, 9), (1, 33)])
def test_small_fp16_forced(B, rows, T0):
    """GQA fp16 model: prompt 5 x 3 rows (M = 15, skinny products), 40 x 3
    (M = 120, tiled products), one or two rows (decode products that
    normalise their own input), then 12 decode steps."""
    kw = small_kw()
    steps = 12
    toks = synth.tokens(41, rows, T0 + steps, kw["vocab_size"])
    say("small fp16 forced", rows, T0)
    h = B.llm_create(B.make_params(**kw), 91)
    got, _ = gpu_forced_logits(h, toks, T0, steps)
    want = oracle.forward_stream(ocfg(kw), 91, toks, T0 - 1)
    check_logits(got, want)
    h.destroy()


@pytest.mark.parametrize("rows", [1, 3])
def test_fp16_decode_to_last_slot(B, rows):
    """fp16 GQA model at max_seq_len 64: a 52-token prompt, then forced decode
    steps up to position 63, the last slot of every cache stream (its K/V
    entry closes the stream's last 32-position block), against the oracle."""
    kw = small_kw(max_seq_len=64)
    T0, steps = 52, 12
    toks = synth.tokens(43, rows, T0 + steps, kw["vocab_size"])
    say("fp16 decode to the last slot", rows)
    h = B.llm_create(B.make_params(**kw), 93)
    got, _ = gpu_forced_logits(h, toks, T0, steps)
    h.destroy()
    want = oracle.forward_stream(ocfg(kw), 93, toks, T0 - 1)
    assert got.shape == want.shape
    check_logits(got, want)


@pytest.mark.parametrize("rows", [1, 2])
def test_fp16_prefill_fills_the_cache(B, rows):
    """A prompt of max_seq_len tokens (every cache slot written by one
    prefill), compared with the oracle at its last position; decoding after
    it is refused (no slot left)."""
    kw = small_kw(max_seq_len=64)
    toks = synth.tokens(47, rows, 64, kw["vocab_size"])
    h = B.llm_create(B.make_params(**kw), 97)
    h.prefill(toks)
    got = h.get_logits()
    with pytest.raises(RuntimeError):
        h.decode(64)
    h.destroy()
    want = oracle.forward_stream(ocfg(kw), 97, toks, 63)[:, 0]
    check_logits(got, want)


@pytest.mark.parametrize("rows", [5, 16, 17, 32])
def test_wide_batch_decode(B, rows):
    """Decode batches of 3..32 rows hand fragment-major activations between
    the RMSNorm, attention, SwiGLU and the products; dims chosen so that the
    head (768 row blocks), w1|w3 (352) and the rest (< 320) take the four-,
    two- and one-block-per-work-group products."""
    kw = small_kw(dim=1024, n_heads=8, n_kv_heads=2, vocab_size=12288, multiple_of=256,
                  max_batch_size=32, max_seq_len=64)
    T0, steps = 6, 6
    toks = synth.tokens(46, rows, T0 + steps, kw["vocab_size"])
    say("wide batch decode", rows)
    h = B.llm_create(B.make_params(**kw), 95)
    got, _ = gpu_forced_logits(h, toks, T0, steps)
    want = oracle.forward_stream(ocfg(kw), 95, toks, T0 - 1)
    check_logits(got, want)
    h.destroy()


@pytest.mark.parametrize("rows,T0", [(1, 1040), (2, 600)])
def test_long_prefill_tiled(B, rows, T0):
    """Prefills of >= 1024 rows hand activations to the 256 x 256 products in
    the weight tile layout; 1040 and 1200 rows leave ragged 256-row and
    16-row tails."""
    kw = small_kw(max_seq_len=1088, max_batch_size=2)
    steps = 3
    toks = synth.tokens(47, rows, T0 + steps, kw["vocab_size"])
    say("long prefill", rows, T0)
    h = B.llm_create(B.make_params(**kw), 96)
    got, _ = gpu_forced_logits(h, toks, T0, steps)
    want = oracle.forward_stream(ocfg(kw), 96, toks, T0 - 1)
    check_logits(got, want)
    h.destroy()


def chunked_forced_logits(h, tokens, chunks, steps):
    """Prefill tokens in consecutive chunks (prefill_at), then decode steps
    with forced columns; returns the logits after each chunk and each step,
    [B][len(chunks) + steps][V]."""
    out, pos = [], 0
    for c in chunks:
        h.prefill_at(pos, tokens[:, pos:pos + c])
        pos += c
        out.append(h.get_logits())
    h.sample(0.0)
    for p in range(pos, pos + steps):
        h.set_tokens(p, tokens[:, p])
        h.decode(p)
        out.append(h.get_logits())
        h.sample(0.0)
    return np.stack(out, 1)


@pytest.mark.parametrize("case", ["fp32", "fp16", "fp16-tiled", "fp16-mha"])
def test_prefill_at_offset(B, case):
    """Chunked prefill: each chunk attends to the cache prefix of the earlier
    chunks and causally to itself; logits at every chunk end and the decode
    steps after it match the oracle's one-pass forward."""
    if case == "fp32":
        kw = dict(n_layers=2, dim=64, n_heads=4, n_kv_heads=2, vocab_size=256, multiple_of=32,
                  ffn_dim_multiplier=0.0, max_batch_size=2, max_seq_len=32, dtype=0)
        rows, chunks, steps = 2, [5, 1, 7], 4
    elif case == "fp16":
        kw = small_kw()
        rows, chunks, steps = 3, [16, 24, 1, 9], 4
    elif case == "fp16-tiled":   # a >= 1024-row chunk after a prefix, then short ones
        kw = small_kw(max_seq_len=1216, max_batch_size=1)
        rows, chunks, steps = 1, [100, 1040, 33], 3
    else:
        kw = small_kw(n_kv_heads=4)
        rows, chunks, steps = 2, [63, 58], 3
    N = sum(chunks) + steps
    toks = synth.tokens(48, rows, N, kw["vocab_size"])
    say("prefill at offset", case, chunks)
    h = B.llm_create(B.make_params(**kw), 97)
    got = chunked_forced_logits(h, toks, chunks, steps)
    full = oracle.forward_stream(ocfg(kw), 97, toks, 0)
    ends = list(np.cumsum(chunks) - 1) + list(range(sum(chunks), N))
    want = full[:, ends]
    if case == "fp32":
        assert np.abs(got - want).max() <= 1e-3
    else:
        check_logits(got, want)
    h.destroy()


@pytest.mark.parametrize("case", ["fp32", "fp16", "fp16-tiled", "fp16-wide"])
def test_varlen_prefill_rows_decode(B, case):
    """Ragged prompts in one varlen prefill, then per-row decode steps with
    teacher-forced columns: every row's logits match the oracle's one-row
    forward over that row's tokens, and the token buffer holds each row's
    prompt and forced tokens."""
    if case == "fp32":
        kw = dict(n_layers=2, dim=64, n_heads=4, n_kv_heads=2, vocab_size=256, multiple_of=32,
                  ffn_dim_multiplier=0.0, max_batch_size=2, max_seq_len=32, dtype=0)
        lens, steps = [3, 8], 6
    elif case == "fp16":
        kw = small_kw()
        lens, steps = [5, 17, 40], 5
    elif case == "fp16-tiled":  # 1100 packed rows: weight-tile activation layout
        kw = small_kw(max_seq_len=768, max_batch_size=2)
        lens, steps = [700, 400], 3
    else:  # 20 rows: fragment-major decode steps with two row halves
        kw = small_kw(max_batch_size=20)
        lens, steps = list(synth.prompt_lengths(49, 20, 1, 40)), 3
    Bn = len(lens)
    N = max(lens) + steps
    toks = synth.tokens(50, Bn, N, kw["vocab_size"])
    say("varlen", case, lens[:4])
    h = B.llm_create(B.make_params(**kw), 98)
    h.prefill_varlen([toks[b, :lens[b]] for b in range(Bn)])
    got = [h.get_logits()]
    for k in range(steps):
        h.set_tokens_rows([toks[b, lens[b] + k] for b in range(Bn)])
        h.decode_rows()
        got.append(h.get_logits())
    got = np.stack(got, 1)                                   # [B][steps+1][V]
    buf = h.get_tokens(N)
    for b in range(Bn):
        n = lens[b] + steps
        assert np.array_equal(buf[b, :n], toks[b, :n])
        want = oracle.forward_stream(ocfg(kw), 98, toks[b:b + 1, :n], lens[b] - 1)[0]
        if case == "fp32":
            assert np.abs(got[b] - want).max() <= 1e-3
        else:
            check_logits(got[b:b + 1], want[None])
    h.destroy()


def test_small_fp16_sampled_and_deterministic(B):
    kw = small_kw()
    T0, steps = 9, 10
    prompt = synth.tokens(42, 3, T0, kw["vocab_size"])
    u = synth.uniforms(43, steps + 1, 3)
    h = B.llm_create(B.make_params(**kw), 92)

    def run():
        h.prefill(prompt)
        out = [h.sample(0.8, 0.9, u[0])]
        for i, p in enumerate(range(T0, T0 + steps)):
            h.decode(p)
            out.append(h.sample(0.8, 0.9, u[i + 1]))
        return np.stack(out, 1), h.get_tokens(T0 + steps + 1)

    a, ta = run()
    b, tb = run()
    assert np.array_equal(a, b) and np.array_equal(ta, tb)  # bit-identical reruns
    assert np.array_equal(ta[:, T0:], a)                      # sampled ids land in the buffer
    assert np.array_equal(ta[:, :T0], prompt)
    # the sampled stream, fed back teacher-forced, matches the oracle's logits
    want = oracle.forward_stream(ocfg(kw), 92, ta[:, :T0 + steps], T0 - 1)
    got, _ = gpu_forced_logits(h, ta, T0, steps)
    check_logits(got, want)
    h.destroy()


def test_mha_and_gqa_paths(B):
    """n_kv_heads = n_heads (MHA) and n_rep = 4 on the same dims."""
    for hkv in (4, 1):
        kw = small_kw(n_kv_heads=hkv)
        toks = synth.tokens(44, 2, 20, kw["vocab_size"])
        say("heads", hkv)
        h = B.llm_create(B.make_params(**kw), 93)
        got, _ = gpu_forced_logits(h, toks, 12, 8)
        check_logits(got, oracle.forward_stream(ocfg(kw), 93, toks, 11))
        h.destroy()


def test_profile_hooks(B):
    """The timing hooks run, report finite positive times, leave the weights
    alone, and the projection timer demands a fresh prefill afterwards."""
    kw = small_kw()
    toks = synth.tokens(45, 2, 16, kw["vocab_size"])
    h = B.llm_create(B.make_params(**kw), 94)
    want, _ = gpu_forced_logits(h, toks, 10, 5)
    prof = h.profile_decode(14, 2)
    assert all(np.isfinite(v) and v >= 0 for v in prof.values()) and prof["step"] > 0
    assert prof["qkv"] > 0 and prof["w13"] > 0 and prof["attention"] > 0
    us = h.profile_projections(2)
    say("  us per launch", us)
    assert all(np.isfinite(v) and v > 0 for v in us.values())
    with pytest.raises(B.LlmError):
        h.decode(15)
    got, _ = gpu_forced_logits(h, toks, 10, 5)
    assert np.array_equal(got, want)
    # the profiled prefill is a prefill: same logits as the plain one
    import torch
    td = torch.from_numpy(np.ascontiguousarray(toks[:, :10])).cuda()
    pp = h.profile_prefill_d(td.data_ptr(), 2, 10, 2)
    assert pp["step"] > 0 and pp["qkv"] > 0
    assert np.array_equal(h.get_logits(), want[:, 0])
    h.destroy()
