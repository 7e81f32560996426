"""Model-level pins for the oracle: causal masking, incremental decode equal to
a full recompute, GQA equal to MHA with replicated K/V heads, and fp32 vs
fp64 accumulation self-consistency.  All on the CPU with small models."""
import numpy as np
import pytest

import oracle
from oracle import F16, F32
from llama_decoder_forward_amd import synth
from llama_decoder_forward_amd.configs import TINY


def tiny_cfg(**kw):
    base = dict(n_layers=2, dim=64, n_heads=4, n_kv_heads=2, vocab_size=256, multiple_of=32,
                ffn_dim_multiplier=0.0, norm_eps=1e-5, rope_theta=10000.0, max_batch_size=2,
                max_seq_len=32, dtype=F32)
    base.update(kw)
    return oracle.Cfg(**base)


def small_f16_cfg(**kw):
    base = dict(n_layers=3, dim=256, n_heads=4, n_kv_heads=2, vocab_size=512, multiple_of=64,
                ffn_dim_multiplier=0.0, norm_eps=1e-5, rope_theta=10000.0, max_batch_size=2,
                max_seq_len=64, dtype=F16)
    base.update(kw)
    return oracle.Cfg(**base)


@pytest.mark.parametrize("mk", [tiny_cfg, small_f16_cfg])
def test_causal_mask_future_tokens_do_not_leak(mk):
    cfg = mk()
    N = 20
    tok = synth.tokens(7, 1, N, cfg.vocab_size)
    alt = tok.copy()
    alt[0, 12:] = (alt[0, 12:] + 17) % cfg.vocab_size
    a = oracle.forward_stream(cfg, 99, tok, 0)
    b = oracle.forward_stream(cfg, 99, alt, 0)
    assert np.array_equal(a[0, :12], b[0, :12])       # positions <= 11 unchanged, bit for bit
    assert not np.allclose(a[0, 12:], b[0, 12:])       # later positions do see their tokens


@pytest.mark.parametrize("mk", [tiny_cfg, small_f16_cfg])
def test_incremental_decode_equals_recompute(mk):
    cfg = mk()
    T, k = 6, 10
    tok = synth.tokens(8, 2, T + k, cfg.vocab_size)
    full = oracle.forward_stream(cfg, 5, tok, T - 1)    # logits at positions T-1 .. T+k-1
    m = oracle.Model(cfg, 5)
    inc = [m.forward(tok[:, :T], 0)]
    for p in range(T, T + k):
        inc.append(m.forward(tok[:, p:p + 1], p))
    inc = np.stack(inc, axis=1)
    assert np.array_equal(inc, full)
    # a prefill that resumes at an offset (zeros block before the causal
    # triangle, P1 section 3.8) gives the same logits again
    m2 = oracle.Model(cfg, 5)
    m2.forward(tok[:, :T], 0)
    chunk = m2.forward(tok[:, T:T + 4], T)
    assert np.array_equal(chunk, full[:, 4])


def test_rows_are_independent():
    cfg = small_f16_cfg()
    tok = synth.tokens(9, 2, 10, cfg.vocab_size)
    both = oracle.forward_stream(cfg, 3, tok, 9)
    one = oracle.forward_stream(cfg, 3, tok[1:], 9)
    assert np.array_equal(both[1], one[0])


def test_mha_is_gqa_with_one_group_each():
    # n_kv_heads = n_heads: repeat_kv is the identity (P1 section 3.4)
    cfg = tiny_cfg(n_kv_heads=4)
    tok = synth.tokens(10, 1, 8, 256)
    a = oracle.forward_stream(cfg, 11, tok, 0)
    b = oracle.forward_stream(tiny_cfg(n_kv_heads=0), 11, tok, 0)  # None -> MHA
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", [F32, F16])
def test_gqa_equals_mha_with_replicated_kv(dtype):
    """Query head h must read KV head h // n_rep (repeat_kv's expand+reshape,
    P1 section 3.4).  An MHA model whose wk/wv head blocks are copies of the
    GQA model's blocks h // n_rep gives identical logits; the mapping
    h % n_kv would not."""
    H, Hkv, hd, D = 4, 2, 16, 64
    gqa = oracle.Model(tiny_cfg(n_kv_heads=Hkv, dtype=dtype, max_batch_size=1), 21)
    mha = oracle.Model(tiny_cfg(n_kv_heads=H, dtype=dtype, max_batch_size=1), 21)
    n_rep = H // Hkv
    for l in range(2):
        for which in (1, 2):  # wk, wv
            tid = 16 + 8 * l + which
            w = gqa.weights(tid, 0, Hkv * hd * D).reshape(Hkv, hd, D)
            mha.set_weights(tid, np.concatenate([w[h // n_rep] for h in range(H)]))
    tok = synth.tokens(12, 1, 12, 256)
    a = gqa.forward(tok, 0)
    b = mha.forward(tok, 0)
    assert np.array_equal(a, b)
    # the other mapping (h % n_kv) gives a different model
    alt = oracle.Model(tiny_cfg(n_kv_heads=H, dtype=dtype, max_batch_size=1), 21)
    for l in range(2):
        for which in (1, 2):
            tid = 16 + 8 * l + which
            w = gqa.weights(tid, 0, Hkv * hd * D).reshape(Hkv, hd, D)
            alt.set_weights(tid, np.concatenate([w[h % Hkv] for h in range(H)]))
    assert not np.allclose(alt.forward(tok, 0), a)


def test_weights_match_generator():
    cfg = tiny_cfg()
    m = oracle.Model(cfg, 44)
    for tid, n in [(0, 256 * 64), (1, 256 * 64), (16 + 4, 192 * 64), (24 + 5, 64 * 192)]:
        assert np.array_equal(m.weights(tid, 0, n), oracle.gen_tensor(44, tid, 0, n, F32))


def test_fp64_accumulation_self_consistency():
    """Parity of the composed model is unpinned by the pages (no printed
    logits); fp32 and fp64 accumulation must agree closely."""
    cfg = tiny_cfg()
    tok = synth.tokens(TINY.token_seed, 1, 20, 256)
    a = oracle.forward_stream(cfg, TINY.weight_seed, tok, 0)
    b = oracle.forward_stream(cfg, TINY.weight_seed, tok, 0, acc64=True)
    assert np.max(np.abs(a - b)) < 1e-4
    cfg16 = small_f16_cfg()
    tok = synth.tokens(13, 1, 20, cfg16.vocab_size)
    a = oracle.forward_stream(cfg16, 77, tok, 0)
    b = oracle.forward_stream(cfg16, 77, tok, 0, acc64=True)
    assert np.max(np.abs(a - b)) < 2e-2
    cos = np.sum(a * b, -1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(b, axis=-1)
    assert cos.min() > 0.9999


def test_generate_slices_printed_example():
    """P2 section 1 prints the slices 0:8, 8:9, 9:10 for an 8-token prompt:
    one prefill over positions 0..7, then one-token steps at 8, 9, ...  The
    oracle's prefill+decode over those slices equals the full-sequence logits
    at positions 7, 8, 9."""
    from tests.conftest import golden
    slices = [tuple(map(int, s.split(":"))) for s in golden("printed_values.txt")["generate_slices_prompt8"].split(",")]
    assert slices == [(0, 8), (8, 9), (9, 10)]
    cfg = tiny_cfg()
    tok = synth.tokens(1, 1, 10, 256)
    m = oracle.Model(cfg, 1)
    got = np.stack([m.forward(tok[:, a:b], a)[0] for a, b in slices])
    assert np.array_equal(got, oracle.forward_stream(cfg, 1, tok, 7)[0])
