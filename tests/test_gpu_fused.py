"""The one-row decode layer in one launch (csrc/decode_fused.hip) against the
separate launches it replaces: every product, normalisation, epilogue and the
attention do the same arithmetic in the same order, so the logits of a
one-row decode are bit-identical with and without the fused layer (the
handle reads LLM_FUSED_LAYER when it is created; the fused layer is
opt-in).  Covered: GQA and MHA,
the static and the paged cache, uniform and per-row positions, contexts that
cross 32-key steps and blocks, a 7B-shaped layer (4096 / 11008 / 32 heads),
and the oracle on the fused handle."""
import os

import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import synth
from tests.gpu_util import cosine, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


def small_kw(**kw):
    base = dict(n_layers=2, dim=512, n_heads=4, n_kv_heads=2, vocab_size=1024, multiple_of=64,
                ffn_dim_multiplier=0.0, max_batch_size=1, max_seq_len=256, dtype=1)
    base.update(kw)
    return base


def create(B, kw, seed, fused, paging=None):
    old = os.environ.get("LLM_FUSED_LAYER")
    os.environ["LLM_FUSED_LAYER"] = "1" if fused else "0"
    try:
        p = B.make_params(**kw)
        return B.llm_create_paged(p, paging, seed) if paging else B.llm_create(p, seed)
    finally:
        if old is None:
            del os.environ["LLM_FUSED_LAYER"]
        else:
            os.environ["LLM_FUSED_LAYER"] = old


def uniform_run(h, toks, T0, steps):
    h.prefill(toks[:, :T0])
    out = [h.get_logits()]
    for p in range(T0, T0 + steps):
        h.set_tokens(p, toks[:, p])
        h.decode(p)
        out.append(h.get_logits())
    return np.stack(out, 1)


def rows_run(h, toks, n0, steps):
    h.prefill_varlen([toks[0, :n0]])
    out = [h.get_logits()]
    for k in range(steps):
        h.set_tokens_rows([toks[0, n0 + k]])
        h.decode_rows()
        out.append(h.get_logits())
    return np.stack(out, 1)


CASES = {
    "gqa": (small_kw(), None, "uniform", 9, 40),
    "mha": (small_kw(n_kv_heads=4), None, "uniform", 30, 40),
    "gqa-rep4": (small_kw(dim=1024, n_heads=8, n_kv_heads=2, multiple_of=256), None, "uniform", 5, 70),
    "paged-bs32": (small_kw(), 32, "uniform", 20, 50),
    "rows": (small_kw(), None, "rows", 33, 20),
    "7b-layer": (small_kw(n_layers=2, dim=4096, n_heads=32, n_kv_heads=32, vocab_size=32000, multiple_of=256,
                          max_seq_len=512), None, "uniform", 8, 40),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_layer_bit_identical(B, case):
    kw, bs, run, T0, steps = CASES[case]
    toks = synth.tokens(71, 1, T0 + steps, kw["vocab_size"])
    outs = []
    for fused in (False, True):
        say("fused layer", case, "fused" if fused else "separate launches")
        paging = B.make_paging(bs, -(-kw["max_seq_len"] // bs)) if bs else None
        h = create(B, kw, 77, fused, paging)
        outs.append(uniform_run(h, toks, T0, steps) if run == "uniform" else rows_run(h, toks, T0, steps))
        h.sync()
        h.destroy()
    d = np.abs(outs[0] - outs[1]).max()
    assert np.array_equal(outs[0], outs[1]), d
    if case == "gqa":
        want = oracle.forward_stream(oracle.Cfg(**kw), 77, toks, T0 - 1)
        got = outs[1]
        dd = np.abs(got - want)
        cos = cosine(got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1]))
        say(f"  oracle max|d|={dd.max():.3e} min cos={cos.min():.7f}")
        assert dd.max() <= 5e-2 and cos.min() >= 0.9999


def test_fused_layer_graph_replays(B):
    """The captured decode step with the fused layers replays many times with
    eager work between replays (sampling, token writes), each replay equal to
    the separate-launch handle's step."""
    kw = small_kw()
    toks = synth.tokens(72, 1, 150, kw["vocab_size"])
    got = []
    for fused in (False, True):
        h = create(B, kw, 78, fused)
        got.append(uniform_run(h, toks, 4, 140))
        h.sync()
        h.destroy()
    assert np.array_equal(got[0], got[1])
