"""Planted mistakes: each case edits one plausible mistake into a copy of
oracle/oracle.c, builds it with gcc into a temporary directory, and runs the
pin named for that mistake against the mutated build (ORACLE_LIB points the
oracle wrapper at it) in a child pytest process.  The pin must fail.  The
committed oracle is never touched; everything runs on the CPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

COMP = "tests/test_oracle_composition.py::"
MUTATIONS = [
    # (name, original text, replacement, occurrence, pin that must fail)
    ("silu applied to w3 x instead of w1 x",
     "a[i] = rnd(rnd(orc_silu(a[i]), dt) * b[i], dt);",
     "a[i] = rnd(rnd(orc_silu(b[i]), dt) * a[i], dt);", 0,
     COMP + "test_swiglu_is_linear_in_the_up_projection"),
    ("FFN residual add dropped",
     "x[i] = rnd(x[i] + t[i], dt);", "x[i] = rnd(t[i], dt);", 1,
     COMP + "test_block_is_identity_when_wo_and_w2_are_zero"),
    ("attention residual add dropped",
     "x[i] = rnd(x[i] + t[i], dt);", "x[i] = rnd(t[i], dt);", 0,
     COMP + "test_block_is_identity_when_wo_and_w2_are_zero"),
    ("final RMSNorm skipped before the output head",
     "orc_rmsnorm(h + (size_t)r * d->D, NULL, d->D, d->eps, d->dtype, acc64, xn + (size_t)r * d->D);",
     "memcpy(xn + (size_t)r * d->D, h + (size_t)r * d->D, sizeof(float) * d->D);", 0,
     COMP + "test_block_is_identity_when_wo_and_w2_are_zero"),
    ("V read from another KV head than K",
     "const float *Vb = vc + ((size_t)bb * d->S * Hkv + g) * hd;",
     "const float *Vb = vc + ((size_t)bb * d->S * Hkv + (g + 1) % Hkv) * hd;", 0,
     COMP + "test_query_heads_read_values_of_their_own_kv_head"),
    ("GQA head map h % n_kv instead of h // n_rep",
     "g = h / n_rep;", "g = h % Hkv;", 0,
     "tests/test_oracle_model.py::test_gqa_equals_mha_with_replicated_kv"),
    ("linear output stored transposed",
     "Y[(size_t)m * N + n] = rnd(", "Y[(size_t)n * M + m] = rnd(", 0,
     COMP + "test_linear_against_float64_matmul"),
    ("attention scores not scaled by 1/sqrt(d)",
     "float scale = (float)(1.0 / sqrt((double)d));", "float scale = 1.0f;", 0,
     "tests/test_oracle_pins.py::test_attention_textbook_float64"),
    ("FFN normalises the block input instead of h",
     "    /* ffn_norm, SwiGLU w2(silu(w1 x) * w3 x) (P1 section 3.6), residual */\n"
     "#pragma omp parallel for schedule(static)\n"
     "    for (int m = 0; m < M; m++) orc_rmsnorm(",
     "    /* ffn_norm, SwiGLU w2(silu(w1 x) * w3 x) (P1 section 3.6), residual */\n"
     "#pragma omp parallel for schedule(static)\n"
     "    for (int m = 0; m < M; m++) if (0) orc_rmsnorm(", 0,
     COMP + "test_whole_model_against_float64_numpy"),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,nth,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_its_pin(tmp_path, name, old, new, nth, pin):
    src = open(SRC).read()
    assert src.count(old) > nth, f"mutation site not found: {old!r}"
    mutated = _replace_nth(src, old, new, nth)
    c_path = tmp_path / "oracle.c"
    so_path = tmp_path / "liboracle.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                           "-shared", "-std=gnu11", str(c_path), "-o", str(so_path), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(so_path), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", pin],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 1 and " failed" in out, f"{name}: {pin} did not fail\n{out[-2000:]}"
