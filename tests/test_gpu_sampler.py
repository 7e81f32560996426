"""The sampler from logits (llm_sample with temperature > 0) against the
oracle's sample on identical logits.

P = softmax(logits / t) in fp32 (the walkthrough "Meta Llama
源码深度剖析与生产应用教程", section 4.2; the course notes on generate,
section 4), then the exact top-p draw of section 4.3.  Both sides take each
softmax term and the normaliser as correctly rounded fp32 values (evaluated in
double, rounded once), so the probability vectors agree bit for bit whatever
the order of the sum, and the token ids must be equal.  A mismatch is allowed
only where the draw or the nucleus threshold lies within 1e-6 of an interval
edge (a double-rounding tie in one term could move it), at most one per test.

Logits come from the GPU forward of one-layer models of the workloads'
widths (logit standard deviation 0.02 sqrt(dim): 1.28, 1.43, 1.81), at the
workloads' (t, p), so the nuclei have the workloads' sizes.
"""
import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import configs, synth
from tests.gpu_util import say

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


def near_edge(logits, t, p, u, rel=1e-6):
    """True when the oracle's draw sits within rel (relative) of an interval
    edge or of the nucleus threshold, where a last-bit difference in P could
    change the token."""
    P = oracle.softmax_temp(logits, t).astype(np.float64)
    order = np.lexsort((np.arange(P.size), -P))
    Q = np.floor(P[order] * 2.0 ** 48)
    E = np.concatenate([[0.0], np.cumsum(Q)])
    thr = np.floor(np.float64(np.float32(p)) * 2.0 ** 48)
    k = int(np.sum(E[:-1] <= thr))
    S = E[k]
    tt = np.floor(np.floor(np.float64(np.float32(u)) * 2.0 ** 24) * S / 2.0 ** 24)
    near_draw = np.min(np.abs(E[1:k + 1] - tt)) <= rel * S
    near_thr = np.min(np.abs(E[max(k - 1, 0):k + 1] - thr)) <= rel * thr
    return bool(near_draw or near_thr)


def one_layer_logits(B, w, batch, seed_off=0, vocab=None):
    kw = w.model_kwargs(max_batch_size=batch, max_seq_len=64)
    kw["n_layers"] = 1
    if vocab:
        kw["vocab_size"] = vocab
    h = B.llm_create(B.make_params(**kw), w.weight_seed + seed_off)
    toks = synth.tokens(w.token_seed + seed_off, batch, 8, kw["vocab_size"])
    h.prefill(toks)
    return h, h.get_logits()


def compare_draws(h, logits, t, p, useed, draws):
    batch = logits.shape[0]
    mism = 0
    for k in range(draws):
        u = synth.uniforms(useed, draws, batch)[k]
        got = h.sample(t, p, u)
        want = np.array([oracle.sample(logits[b], t, p, float(u[b])) for b in range(batch)])
        for b in np.nonzero(got != want)[0]:
            mism += 1
            assert near_edge(logits[b], t, p, float(u[b])), (k, b, got[b], want[b])
        # sampling does not change the logits: draw again with the same u
        assert np.array_equal(h.sample(t, p, u), got)
    return mism


@pytest.mark.parametrize("name", ["llama2-7b-bs32", "llama2-13b-bs8", "llama2-70b-gqa-bs32"])
def test_sample_from_logits_matches_oracle(B, name):
    w = configs.WORKLOADS[name]
    say(name, "one-layer logits, t", w.temperature, "p", w.top_p)
    h, logits = one_layer_logits(B, w, 32)
    mism = compare_draws(h, logits, w.temperature, w.top_p, w.uniform_seed, 4)
    say(f"  {4 * 32} draws, {mism} at an interval edge")
    assert mism <= 1
    # greedy: argmax, lowest id on ties
    assert np.array_equal(h.sample(0.0), logits.argmax(-1))
    h.destroy()


@pytest.mark.parametrize("vocab,batch", [(40000, 8), (65536, 3)])
def test_sample_large_vocab_two_launch_path(B, vocab, batch):
    """Vocabularies above 32768 take the two-launch path (softmax into a
    probability buffer, then the radix select over global memory)."""
    w = configs.L7B_BS32
    say("vocab", vocab, "batch", batch)
    h, logits = one_layer_logits(B, w, batch, seed_off=11, vocab=vocab)
    for t, p in [(0.6, 0.9), (1.0, 0.5), (0.3, 1.0)]:
        compare_draws(h, logits, t, p, w.uniform_seed + vocab, 2)
    assert np.array_equal(h.sample(0.0), logits.argmax(-1))
    h.destroy()
