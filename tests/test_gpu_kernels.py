"""Per-kernel parity on the GPU against the oracle: seeded weights (bit-exact),
RMSNorm, the skinny and tiled matrix products, decode and prefill attention,
and the exact top-p sampler (bit-exact).  Inputs are seeded synthetic
arrays; expected values come from oracle functions on the same inputs."""
import math

import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import configs
from tests.gpu_util import cosine, dev, empty, f16_ulp, host, randn_f16, say, within_one_f16_step

pytestmark = pytest.mark.gpu

F16, F32 = 1, 0


def small_f16(**kw):
    base = dict(n_layers=2, dim=512, n_heads=4, n_kv_heads=2, vocab_size=1024, multiple_of=64,
                ffn_dim_multiplier=0.0, max_batch_size=4, max_seq_len=512, dtype=F16)
    base.update(kw)
    return base


@pytest.fixture(scope="module")
def B():
    from llama_decoder_forward_amd import binding
    return binding


@pytest.fixture(scope="module")
def small(B):
    kw = small_f16()
    say("create small fp16 model", kw)
    h = B.llm_create(B.make_params(**kw), 77)
    yield h, kw
    h.destroy()


def tensor_shapes(kw):
    D, H, Hkv = kw["dim"], kw["n_heads"], kw["n_kv_heads"]
    hd = D // H
    F = oracle.ffn_hidden(D, kw["multiple_of"], kw["ffn_dim_multiplier"])
    shapes = {0: (kw["vocab_size"], D), 1: (kw["vocab_size"], D)}
    for l in range(kw["n_layers"]):
        base = 16 + 8 * l
        shapes.update({base: (H * hd, D), base + 1: (Hkv * hd, D), base + 2: (Hkv * hd, D),
                       base + 3: (D, H * hd), base + 4: (F, D), base + 5: (D, F), base + 6: (F, D)})
    return shapes, F


@pytest.mark.parametrize("which", ["f16", "f32"])
def test_weights_bit_equal(B, which):
    if which == "f16":
        kw = small_f16()
        seed = 77
    else:
        w = configs.TINY
        kw = w.model_kwargs()
        seed = w.weight_seed
    say("weights", which)
    h = B.llm_create(B.make_params(**kw), seed)
    shapes, _ = tensor_shapes(kw)
    rng = np.random.default_rng(1)
    for tid, (r, c) in shapes.items():
        n = r * c
        for first in [0, int(rng.integers(0, n - 300)), n - 300]:
            got = h.read_weights(tid, first, 300)
            want = oracle.gen_tensor(seed, tid, first, 300, kw["dtype"])
            assert np.array_equal(got, want), (tid, first)
    h.destroy()


def test_rmsnorm(B, small):
    h, kw = small
    rng = np.random.default_rng(2)
    for M, scale in [(1, 1.0), (37, 0.3), (5, 20.0)]:
        say("rmsnorm", M, scale)
        x = randn_f16(rng, (M, kw["dim"]), scale)
        xd, yd = dev(x), empty((M, kw["dim"]), np.float16)
        h.op_rmsnorm(xd.data_ptr(), M, yd.data_ptr())
        y = host(yd).astype(np.float32)
        want = np.stack([oracle.rmsnorm(x[m].astype(np.float32), 1e-5, F16) for m in range(M)])
        d = np.abs(y - want)
        assert np.all(within_one_f16_step(y, want)), d.max()
        assert np.mean(d == 0) > 0.97


def packed_weights(kw, seed, layer, mat):
    """The oracle's weights of a packed matrix in stored row order."""
    shapes, F = tensor_shapes(kw)
    base = 16 + 8 * layer
    g = lambda tid: oracle.gen_tensor(seed, tid, 0, shapes[tid][0] * shapes[tid][1], F16).reshape(shapes[tid])
    if mat == 0:
        return np.concatenate([g(base), g(base + 1), g(base + 2)])
    if mat == 1:
        return g(base + 3)
    if mat == 2:
        w1, w3 = g(base + 4), g(base + 6)
        blocks = [np.concatenate([w1[8 * j:8 * j + 8], w3[8 * j:8 * j + 8]]) for j in range(F // 8)]
        return np.concatenate(blocks)
    if mat == 3:
        return g(base + 5)
    return g(1)


@pytest.mark.parametrize("mat", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("M", [1, 2, 7, 16, 17, 32, 33, 200, 300, 1100, 2048])
def test_linear(B, small, mat, M):
    h, kw = small
    W = packed_weights(kw, 77, 1, mat)
    N, K = W.shape
    rng = np.random.default_rng(3 + M)
    x = randn_f16(rng, (M, K), 0.5)
    say("linear", mat, M, N, K)
    xd, yd = dev(x), empty((M, N), np.float16)
    h.op_linear(1, mat, xd.data_ptr(), M, yd.data_ptr())
    y = host(yd).astype(np.float32)
    want = oracle.linear(W, x.astype(np.float32), F16)
    d = np.abs(y - want)
    ok = accumulation_close(y, want, W, x)
    assert np.all(ok), [(m, n, y[m, n], want[m, n]) for m, n in np.argwhere(~ok)[:5]]
    assert np.mean(d == 0) > 0.9


def test_linear_odd_tile_count(B):
    """A head of 1040 rows (65 row tiles, odd) for M in the two-column-group
    range."""
    kw = small_f16(vocab_size=1040)
    h = B.llm_create(B.make_params(**kw), 79)
    W = packed_weights(kw, 79, 0, 4)
    rng = np.random.default_rng(16)
    for M in (20, 32):
        say("odd tiles", M)
        x = randn_f16(rng, (M, kw["dim"]), 0.5)
        xd, yd = dev(x), empty((M, 1040), np.float16)
        h.op_linear(0, 4, xd.data_ptr(), M, yd.data_ptr())
        y = host(yd).astype(np.float32)
        want = oracle.linear(W, x.astype(np.float32), F16)
        assert np.all(accumulation_close(y, want, W, x))
    h.destroy()


def accumulation_close(got, want, W, x):
    """Two results of the same fp32 dot products summed in different orders:
    within one fp16 rounding step, or within the fp32 accumulation error
    bound 2^-20 * sum_k |w_k x_k| (values near zero, where fp16 steps are
    finer than the fp32 sum's own rounding)."""
    absW = (np.ascontiguousarray(W) & np.uint16(0x7FFF)).astype(np.uint16)
    mag = oracle.linear(absW, np.abs(x.astype(np.float32)), F32)
    return within_one_f16_step(got, want) | (np.abs(got - want) <= mag * 2.0 ** -20)


def test_linear_7b_shapes_sampled(B):
    """7B-shaped layer 0 (one layer only: weights depend only on (seed,
    tensor)), skinny M=1 and tiled M=4480 (the batched prompt workload's
    rows); sampled outputs checked one by one."""
    w = configs.L7B_BS1
    kw = w.model_kwargs(max_batch_size=1, max_seq_len=64)
    kw["n_layers"] = 1
    say("create 7B-shaped single layer")
    h = B.llm_create(B.make_params(**kw), w.weight_seed)
    shapes, F = tensor_shapes(kw)
    rng = np.random.default_rng(4)
    for mat, tids in [(0, [16, 17, 18]), (2, None), (3, [21])]:
        for M in [1, 4480]:
            N = {0: 3 * 4096, 2: 2 * F, 3: 4096}[mat]
            K = {0: 4096, 2: 4096, 3: F}[mat]
            say("7B linear", mat, M)
            x = randn_f16(rng, (M, K), 0.5)
            xd, yd = dev(x), empty((M, N), np.float16)
            h.op_linear(0, mat, xd.data_ptr(), M, yd.data_ptr())
            y = host(yd)
            ms = rng.integers(0, M, 6)
            ns = np.unique(rng.integers(0, N, 40))
            rows = []
            for n in ns:
                if mat == 2:
                    j, r = n // 16, n % 16
                    tid, row = (16 + 4, 8 * j + r) if r < 8 else (16 + 6, 8 * j + r - 8)
                elif mat == 0:
                    tid, row = 16 + n // 4096, n % 4096
                else:
                    tid, row = 21, n
                rows.append(oracle.gen_tensor(w.weight_seed, tid, row * K, K, F16))
            want = oracle.linear(np.stack(rows), x[ms].astype(np.float32), F16)
            got = y[np.ix_(ms, ns)].astype(np.float32)
            assert np.all(accumulation_close(got, want, np.stack(rows), x[ms]))
    h.destroy()


def attention_reference(q, K, V, pos_list, n_rep):
    """Oracle attention per (row, position, head): q[B][T][H][d], K/V
    [B][L][Hkv][d]; query at position p sees keys 0..p."""
    Bn, T, H, d = q.shape
    out = np.empty_like(q, dtype=np.float32)
    for b in range(Bn):
        for t in range(T):
            p = pos_list[t]
            for hh in range(H):
                g = hh // n_rep
                out[b, t, hh] = oracle.attention_row(q[b, t, hh].astype(np.float32),
                                                     K[b, :p + 1, g].astype(np.float32),
                                                     V[b, :p + 1, g].astype(np.float32), F16)
    return out


@pytest.mark.parametrize("L", [1, 5, 64, 65, 300, 512])
def test_attention_decode(B, small, L):
    h, kw = small
    Bn, H, Hkv, d = 3, kw["n_heads"], kw["n_kv_heads"], kw["dim"] // kw["n_heads"]
    rng = np.random.default_rng(10 + L)
    K = randn_f16(rng, (Bn, L, Hkv, d))
    V = randn_f16(rng, (Bn, L, Hkv, d))
    q = randn_f16(rng, (Bn, 1, H, d), 0.3)
    say("attention decode", L)
    kd, vd = dev(K), dev(V)
    h.op_kv_write(0, kd.data_ptr(), vd.data_ptr(), Bn, L, 0)
    qd, od = dev(q), empty((Bn, 1, H, d), np.float16)
    h.op_attention(0, qd.data_ptr(), Bn, 1, L - 1, od.data_ptr())
    got = host(od).astype(np.float32)
    want = attention_reference(q, K, V, [L - 1], H // Hkv)
    assert np.max(np.abs(got - want)) < 4e-3, np.max(np.abs(got - want))
    assert cosine(got.reshape(-1, d), want.reshape(-1, d)).min() > 0.9999


@pytest.mark.parametrize("Bn,L,S", [(64, 300, 320), (64, 33, 320), (256, 77, 320), (256, 1, 320),
                                     (64, 700, 1024), (160, 1000, 1024), (160, 3, 1024)])
def test_attention_decode_many_pairs(B, Bn, L, S):
    """Bn * n_kv_heads (row, KV head) pairs: 128 pairs take the eight-wave
    work-groups with non-temporal K/V loads, 320 the four-wave ones, 512 the
    two-wave ones with the next step prefetched (non-temporal too); caches
    of 320 and 1024 positions, ragged last steps, long contexts and a single
    key included.  A second launch gives the same bits."""
    kw = small_f16(max_batch_size=Bn, max_seq_len=S)
    h = B.llm_create(B.make_params(**kw), 78)
    H, Hkv, d = kw["n_heads"], kw["n_kv_heads"], 128
    assert Bn * Hkv in (128, 320, 512)
    rng = np.random.default_rng(15 + L)
    K = randn_f16(rng, (Bn, L, Hkv, d))
    V = randn_f16(rng, (Bn, L, Hkv, d))
    q = randn_f16(rng, (Bn, 1, H, d), 0.3)
    say("attention decode many pairs", Bn, L)
    kd, vd = dev(K), dev(V)
    h.op_kv_write(0, kd.data_ptr(), vd.data_ptr(), Bn, L, 0)
    qd, od = dev(q), empty((Bn, 1, H, d), np.float16)
    h.op_attention(0, qd.data_ptr(), Bn, 1, L - 1, od.data_ptr())
    got = host(od).astype(np.float32)
    h.op_attention(0, qd.data_ptr(), Bn, 1, L - 1, od.data_ptr())
    assert np.array_equal(host(od).astype(np.float32), got)
    rows = [0, Bn // 2 + 1, Bn - 1]
    want = attention_reference(q[rows], K[rows], V[rows], [L - 1], H // Hkv)
    assert np.max(np.abs(got[rows] - want)) < 4e-3
    h.destroy()


@pytest.mark.parametrize("T", [1, 2, 63, 129, 200, 500])
def test_attention_prefill(B, small, T):
    h, kw = small
    Bn, H, Hkv, d = 2, kw["n_heads"], kw["n_kv_heads"], kw["dim"] // kw["n_heads"]
    rng = np.random.default_rng(20 + T)
    K = randn_f16(rng, (Bn, T, Hkv, d))
    V = randn_f16(rng, (Bn, T, Hkv, d))
    q = randn_f16(rng, (Bn, T, H, d), 0.3)
    say("attention prefill", T)
    kd, vd = dev(K), dev(V)
    h.op_kv_write(1, kd.data_ptr(), vd.data_ptr(), Bn, T, 0)
    qd, od = dev(q), empty((Bn, T, H, d), np.float16)
    h.op_attention(1, qd.data_ptr(), Bn, T, 0, od.data_ptr())
    got = host(od).astype(np.float32)
    want = attention_reference(q, K, V, list(range(T)), H // Hkv)
    assert np.max(np.abs(got - want)) < 4e-3, np.max(np.abs(got - want))


def test_top_p_bit_exact(B):
    w = configs.L70B_BS32
    kw = small_f16(max_batch_size=32, vocab_size=32000)
    h = B.llm_create(B.make_params(**kw), 5)
    rng = np.random.default_rng(30)
    for case, (t, p) in enumerate([(0.6, 0.9), (0.8, 0.95), (1.0, 1.0), (0.3, 0.5), (2.0, 0.999),
                                   (0.6, 1e-6)]):
        say("top-p", t, p)
        logits = (rng.standard_normal((32, 32000)) * 1.4).astype(np.float32)
        if case == 2:
            logits[:, ::7] = logits[:, :1]  # many exact ties
        probs = np.stack([oracle.softmax_temp(l, t) for l in logits])
        u = ((rng.integers(0, 2 ** 24, 32)) / 2 ** 24).astype(np.float32)
        got = h.sample_probs(probs, p, u)
        want = np.array([oracle.top_p(probs[i], p, float(u[i]))[0] for i in range(32)])
        assert np.array_equal(got, want), (case, got, want)
    h.destroy()
