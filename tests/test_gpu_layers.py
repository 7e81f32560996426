"""Parity one layer at a time, at full depth.

For every layer l the GPU runs TransformerBlock l (llm_op_layer: the kernels
and launch forms of a whole pass for the same rows) on the residual rows the
oracle computed entering that layer, and its output is compared with the
oracle's output of the same layer.  An error therefore cannot build up over
depth: each comparison measures one layer's rounding noise, and a mistake in
any layer (a dropped term, a wrong head, a wrong position) shows up at that
layer, whatever the depth.  The walkthrough's TransformerBlock ("Meta Llama
源码深度剖析与生产应用教程", section 3.7) is what each call computes; the
llama2.zig article (section 5.1) checks its engine the same way, layer by
layer.

Rows: batch rows never mix, so the GPU runs many rows that are copies of the
few rows the oracle computes (row b is oracle row b % R).  The prefill runs at
256 rows of 4 tokens (1024 activation rows: the tiled prefill products of the
benchmark's prefills), the decode steps at the benchmark's batch (the decode
products' forms for that many rows).

Bound (per row and position, see the one-layer noise model in the design doc):
  max|gpu - oracle| <= max(4 ulp_fp16(max|y|), 4 * max|oracle_fp64 - oracle|)
and the cosine of the row >= 1 - 1e-5, where oracle_fp64 is the same layer
with float64 accumulation on the same input.
"""
import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import configs, synth
from tests.gpu_util import cosine, say

pytestmark = [pytest.mark.gpu]

F16 = 1
T0, STEPS, R = 4, 2, 2


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    import torch as t
    return t


def f16_ulp_at(v):
    return np.spacing(np.asarray(v, np.float16)).astype(np.float64)


def check_layer(l, got, want, want64_fn, stats):
    """got/want: [rows][tokens][D] float32 (the oracle rows the GPU rows
    copy).  Per (row, position): the max error against the bound; the
    oracle's fp64 spread (want64_fn, a float64-accumulation run of the same
    layer on the same input) is computed only where 4 fp16 steps of the row
    maximum do not already cover the error."""
    d = np.abs(got.astype(np.float64) - want)
    ymax = np.abs(want).max(-1)
    worst = d.max(-1)
    bound = 4 * f16_ulp_at(ymax)
    spread = np.zeros_like(worst)
    if np.any(worst > bound):
        spread = np.abs(want64_fn().astype(np.float64) - want).max(-1)
        bound = np.maximum(bound, 4 * spread)
    cos = cosine(got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1]))
    stats.append((l, float(worst.max()), float((worst / f16_ulp_at(ymax)).max()), float(spread.max()),
                  float(cos.min())))
    assert np.all(worst <= bound) and cos.min() >= 1 - 1e-5, (l, worst.max(), bound.min(), cos.min())


def per_layer_parity(B, torch, w, n_layers, dec_batches, prefill_rows=256, max_seq_len=64, seed_off=0):
    """Run every layer of workload w on the oracle's inputs; dec_batches: the
    decode batch sizes whose forms are checked at every step."""
    kw = w.model_kwargs(max_batch_size=prefill_rows, max_seq_len=max_seq_len)
    kw["n_layers"] = n_layers
    N = T0 + STEPS
    toks = synth.tokens(w.token_seed + seed_off, R, N, w.vocab_size)
    cfg = oracle.Cfg(**dict(kw, max_batch_size=R))
    say(f"{w.name} x{n_layers} layers: oracle stream (fp32) with residuals")
    _, res = oracle.forward_stream(cfg, w.weight_seed, toks, N - 1, resid=True)   # [NL+1][R][N][D]
    say(f"{w.name}: gpu create")
    h = B.llm_create(B.make_params(**kw), w.weight_seed)
    dt = np.float16 if w.dtype == F16 else np.float32
    stats = []
    try:
        for l in range(n_layers):
            cache = {}

            def want64(l=l, cache=cache):
                if "y" not in cache:
                    cache["y"] = oracle.layer_apply(cfg, w.weight_seed, l, res[l], acc64=True)
                return cache["y"]
            # prefill form: positions 0..T0-1 of prefill_rows rows
            rows = np.arange(prefill_rows) % R
            x = torch.from_numpy(np.ascontiguousarray(res[l][rows, :T0].astype(dt))).cuda()
            h.op_layer(l, x.data_ptr(), prefill_rows, T0, 0)
            got = x.cpu().numpy().astype(np.float32)
            check_layer(l, got[:R], res[l + 1][:, :T0], lambda: want64()[:, :T0], stats)
            assert all(np.array_equal(got[b], got[b % R]) for b in range(prefill_rows))
            # decode forms: one position at a time, for each batch size
            for p in range(T0, N):
                for nb in dec_batches:
                    rb = np.arange(nb) % R
                    x = torch.from_numpy(np.ascontiguousarray(res[l][rb, p:p + 1].astype(dt))).cuda()
                    h.op_layer(l, x.data_ptr(), nb, 1, p)
                    got = x.cpu().numpy().astype(np.float32)
                    for r in range(min(R, nb)):
                        sel = [b for b in range(nb) if b % R == r]
                        assert all(np.array_equal(got[b], got[sel[0]]) for b in sel)
                    k = min(R, nb)
                    check_layer(l, got[:k], res[l + 1][:k, p:p + 1], lambda: want64()[:k, p:p + 1], stats)
            if l % 10 == 0 or l == n_layers - 1:
                say(f"  layer {l}: max|d| {max(s[1] for s in stats[-1 - len(dec_batches) * STEPS:]):.3e}")
    finally:
        h.destroy()
    worst = max(stats, key=lambda s: s[2])
    say(f"  {w.name}: worst layer {worst[0]}: max|d| {worst[1]:.3e} = {worst[2]:.2f} ulp of the row max, "
        f"min cos {min(s[4] for s in stats):.8f}; oracle fp64 runs needed on "
        f"{sum(s[3] > 0 for s in stats)} of {len(stats)} checks")
    return stats


def test_per_layer_small_fp16(B, torch):
    """A 3-layer 7B-width GQA model: every decode row-count form (1, 2, 5,
    17, 32 rows) against the oracle, layer by layer."""
    w = configs.L7B_BS1
    small = configs.Workload("small-gqa", 9, n_layers=3, dim=1024, n_heads=8, n_kv_heads=2,
                             vocab_size=2048, multiple_of=256, ffn_dim_multiplier=0.0, dtype=F16,
                             batch=32, prompt_len=8)
    per_layer_parity(B, torch, small, 3, dec_batches=[1, 2, 5, 17, 32])
    del w


def test_per_layer_tiny_fp32(B, torch):
    w = configs.TINY
    per_layer_parity(B, torch, w, w.n_layers, dec_batches=[1, 3], prefill_rows=8, max_seq_len=32)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_per_layer_7b_full_depth(B, torch):
    """All 32 layers of the 7B model: decode forms of one row (the
    normalisation inside the products) and of 32 rows (split-K partials
    handed to the normalisation launch)."""
    per_layer_parity(B, torch, configs.L7B_BS1, 32, dec_batches=[1, 32])


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_per_layer_13b_full_depth(B, torch):
    """All 40 layers of the 13B model, decode at the workload's 8 rows."""
    per_layer_parity(B, torch, configs.L13B_BS8, 40, dec_batches=[8])


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_per_layer_70b_full_depth(B, torch):
    """All 80 layers of the 70B GQA model, decode at the workload's 32 rows."""
    per_layer_parity(B, torch, configs.L70B_BS32, 80, dec_batches=[32])
