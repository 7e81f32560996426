"""The five workloads the decoder is measured and checked on.

Shapes are the Llama-2 model sizes listed in the walkthrough's model table
("Meta Llama 源码深度剖析与生产应用教程", section 2) plus a tiny fp32 GQA model
for exhaustive checks.  Each workload fixes the batch, the prompt, the number
of decode steps and the sampler settings; seeds are per workload index i:
weights 1000+i, prompt tokens 2000+i, sampler uniforms 3000+i.
"""
from __future__ import annotations

from dataclasses import dataclass, field

F32, F16 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_layers: int
    dim: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int
    multiple_of: int
    ffn_dim_multiplier: float
    dtype: int
    batch: int
    prompt_len: int            # fixed prompt length (0 when ragged)
    prompt_range: tuple = ()   # (lo, hi) for ragged prompts
    decode_steps: int = 0
    temperature: float = 0.0   # <= 0: greedy
    top_p: float = 1.0
    max_seq_len: int = 2048
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    note: str = field(default="", compare=False)

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def weight_seed(self) -> int:
        return 1000 + self.index

    @property
    def token_seed(self) -> int:
        return 2000 + self.index

    @property
    def uniform_seed(self) -> int:
        return 3000 + self.index

    def ffn_hidden(self) -> int:
        h = int(2 * (4 * self.dim) / 3)
        if self.ffn_dim_multiplier > 0:
            h = int(self.ffn_dim_multiplier * h)
        return self.multiple_of * ((h + self.multiple_of - 1) // self.multiple_of)

    def model_kwargs(self, max_batch_size: int | None = None, max_seq_len: int | None = None):
        return dict(n_layers=self.n_layers, dim=self.dim, n_heads=self.n_heads,
                    n_kv_heads=self.n_kv_heads, vocab_size=self.vocab_size,
                    multiple_of=self.multiple_of, ffn_dim_multiplier=self.ffn_dim_multiplier,
                    norm_eps=self.norm_eps, rope_theta=self.rope_theta,
                    max_batch_size=self.batch if max_batch_size is None else max_batch_size,
                    max_seq_len=self.max_seq_len if max_seq_len is None else max_seq_len,
                    dtype=self.dtype)

    def weight_bytes(self) -> int:
        """Bytes of every layer matrix plus the output head (what one decode
        step streams), excluding the embedding table (gathered, not streamed)."""
        es = 2 if self.dtype == F16 else 4
        D, hd, F = self.dim, self.head_dim, self.ffn_hidden()
        per_layer = (self.n_heads + 2 * self.n_kv_heads) * hd * D + D * self.n_heads * hd + 3 * F * D
        return es * (self.n_layers * per_layer + self.vocab_size * D)

    def layer_params(self) -> int:
        D, hd, F = self.dim, self.head_dim, self.ffn_hidden()
        return (self.n_heads + 2 * self.n_kv_heads) * hd * D + D * self.n_heads * hd + 3 * F * D


TINY = Workload("tiny-fp32", 1, n_layers=2, dim=64, n_heads=4, n_kv_heads=2, vocab_size=256,
                multiple_of=32, ffn_dim_multiplier=0.0, dtype=F32, batch=1, prompt_len=8,
                decode_steps=24, max_seq_len=32)
L7B_BS1 = Workload("llama2-7b-bs1", 2, n_layers=32, dim=4096, n_heads=32, n_kv_heads=32,
                   vocab_size=32000, multiple_of=256, ffn_dim_multiplier=0.0, dtype=F16, batch=1,
                   prompt_len=8, decode_steps=256, max_seq_len=2048)
L7B_BS32 = Workload("llama2-7b-bs32", 3, n_layers=32, dim=4096, n_heads=32, n_kv_heads=32,
                    vocab_size=32000, multiple_of=256, ffn_dim_multiplier=0.0, dtype=F16, batch=32,
                    prompt_len=0, prompt_range=(128, 512), decode_steps=128, temperature=0.6,
                    top_p=0.9, max_seq_len=2048)
L13B_BS8 = Workload("llama2-13b-bs8", 4, n_layers=40, dim=5120, n_heads=40, n_kv_heads=40,
                    vocab_size=32000, multiple_of=256, ffn_dim_multiplier=0.0, dtype=F16, batch=8,
                    prompt_len=1024, decode_steps=512, temperature=0.8, top_p=0.95,
                    max_seq_len=2048)
L70B_BS32 = Workload("llama2-70b-gqa-bs32", 5, n_layers=80, dim=8192, n_heads=64, n_kv_heads=8,
                     vocab_size=32000, multiple_of=4096, ffn_dim_multiplier=1.3, dtype=F16,
                     batch=32, prompt_len=2048, decode_steps=128, temperature=0.6, top_p=0.9,
                     max_seq_len=4096)

WORKLOADS = {w.name: w for w in (TINY, L7B_BS1, L7B_BS32, L13B_BS8, L70B_BS32)}
