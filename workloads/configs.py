"""Shapes and seeds of the five synthetic workloads.

The serving pages benchmark on models and tools that are not available here
(a Llama-2-7B chat model driven by a load generator, an OPT-13B throughput
script).  These configurations stand in for them with seeded synthetic data of
the same attention shapes: Llama-2-7B (32 heads of 128), a Llama-3-8B-like GQA
layer (32 query heads over 8 KV heads), a 13B-like 40x128 layer for the serving
trace, and generation lengths in the 10..500 token range the pages use as their
example.  Only shapes, sizes, distributions and seeds live here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import gen


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    title: str
    seed: int
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    ctx_kind: str                 # "fixed" | "uniform" | "loguniform" | "shared_prefix"
    ctx_lo: int = 0
    ctx_hi: int = 0
    ctx_fixed: tuple = ()
    shared_prefix: int = 0        # tokens in the shared prefix (shared_prefix kind)
    suffix_lo: int = 0
    suffix_hi: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def context_lens(self) -> np.ndarray:
        if self.ctx_kind == "fixed":
            return np.asarray(self.ctx_fixed, dtype=np.int32)
        if self.ctx_kind == "uniform":
            return gen.context_lens_uniform(self.seed, self.num_seqs, self.ctx_lo, self.ctx_hi)
        if self.ctx_kind == "loguniform":
            return gen.context_lens_loguniform(self.seed, self.num_seqs, self.ctx_lo, self.ctx_hi)
        if self.ctx_kind == "shared_prefix":
            suffix = gen.stream(self.seed, gen.TAG_CTX).integers(
                self.suffix_lo, self.suffix_hi + 1, self.num_seqs)
            return (self.shared_prefix + suffix).astype(np.int32)
        raise ValueError(self.ctx_kind)

    def pool_order(self) -> np.ndarray:
        return gen.pool_permutation(self.seed, self.num_blocks)

    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V one token holds over all KV heads."""
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes


@dataclass(frozen=True)
class TraceConfig:
    name: str
    title: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    steps: int
    arrival_mean: float
    prompt_lo: int
    prompt_hi: int
    out_p: float
    out_lo: int
    out_hi: int
    chunk: int
    # prefix caching: prompts open with one of `openings` shared system prompts
    # (0 = plain prompts of the lengths above, no token IDs)
    openings: int = 0
    open_lo: int = 0
    open_hi: int = 0
    suffix_lo: int = 0
    suffix_hi: int = 0
    vocab: int = 64

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def prefix(self) -> bool:
        return self.openings > 0

    def arrivals(self, step: int):
        """Requests arriving at `step`: (prompt length, out_len) pairs, or with shared
        openings (prompt token IDs, out_len) pairs."""
        p, o = gen.trace_arrivals(self.seed, step, self.arrival_mean, self.prompt_lo,
                                  self.prompt_hi, self.out_p, self.out_lo, self.out_hi)
        if not self.prefix:
            return list(zip(p.tolist(), o.tolist()))
        toks = gen.shared_opening_prompts(self.seed, step, len(p), self.openings, self.open_lo,
                                          self.open_hi, self.suffix_lo, self.suffix_hi, self.vocab)
        return list(zip(toks, o.tolist()))

    def gen_token(self, rid: int, position: int) -> int:
        return gen.generated_token(self.seed, rid, position, self.vocab)

    def gen_tokens(self, rid: int, first: int, count: int) -> np.ndarray:
        return gen.generated_tokens(self.seed, rid, first, count, self.vocab)


@dataclass(frozen=True)
class PrefillConfig:
    """Prompt chunks at the end of partly filled caches, as a serving step prefills them."""
    name: str
    title: str
    seed: int
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    chunk: int                    # tokens per chunk
    offset_lo: int                # tokens already cached before the chunk: U[lo, hi]
    offset_hi: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def offsets(self) -> np.ndarray:
        return gen.stream(self.seed, gen.TAG_CTX).integers(
            self.offset_lo, self.offset_hi + 1, self.num_seqs).astype(np.int32)

    def pool_order(self) -> np.ndarray:
        return gen.pool_permutation(self.seed, self.num_blocks)


CONFIGS = {
    "tiny_f32": DecodeConfig(
        name="tiny_f32", title="tiny paged decode, fp32, 4 seqs, ctx {1,15,16,33}",
        seed=1, dtype="f32", num_seqs=4, num_q_heads=2, num_kv_heads=2, head_dim=64,
        block_size=16, num_blocks=16, ctx_kind="fixed", ctx_fixed=(1, 15, 16, 33)),
    "llama2_7b_b64": DecodeConfig(
        name="llama2_7b_b64", title="Llama-2-7B-shaped decode, bf16, batch 64, ctx U[128,4096]",
        seed=2, dtype="bf16", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=20000, ctx_kind="uniform", ctx_lo=128, ctx_hi=4096),
    "gqa_b256": DecodeConfig(
        name="gqa_b256", title="GQA decode (32q/8kv, D=128), bf16, batch 256, ctx log-U[16,8192]",
        seed=3, dtype="bf16", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=200000, ctx_kind="loguniform", ctx_lo=16, ctx_hi=8192),
    "shared_prefix_b16": DecodeConfig(
        name="shared_prefix_b16", title="shared 1024-token prefix + private suffix, bf16, B=16",
        seed=4, dtype="bf16", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=20000, ctx_kind="shared_prefix", shared_prefix=1024,
        suffix_lo=16, suffix_hi=512),
    "shared_prefix_b32": DecodeConfig(
        name="shared_prefix_b32", title="shared 1024-token prefix + private suffix, bf16, B=32",
        seed=5, dtype="bf16", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=32, num_blocks=10000, ctx_kind="shared_prefix", shared_prefix=1024,
        suffix_lo=16, suffix_hi=512),
    "trace_13b": TraceConfig(
        name="trace_13b", title="continuous-batching trace, 200 steps, 40x128 heads, bf16",
        seed=6, dtype="bf16", num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
        num_blocks=50000, steps=200, arrival_mean=8.0, prompt_lo=32, prompt_hi=1024,
        out_p=0.01, out_lo=10, out_hi=500, chunk=512),
    "prefill_13b": PrefillConfig(
        name="prefill_13b", title="chunked prefill, 8 chunks of 512 after U[0,3584] cached tokens, "
        "40x128 heads, bf16", seed=7, dtype="bf16", num_seqs=8, num_q_heads=40, num_kv_heads=40,
        head_dim=128, block_size=16, num_blocks=4096, chunk=512, offset_lo=0, offset_hi=3584),
    "prefill_gqa": PrefillConfig(
        name="prefill_gqa", title="chunked prefill, 8 chunks of 512 after U[0,3584] cached tokens, "
        "32q/8kv x 128, bf16", seed=8, dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, num_blocks=4096, chunk=512, offset_lo=0, offset_hi=3584),
    # serving trace whose prompts open with one of 8 shared system prompts
    "trace_prefix": TraceConfig(
        name="trace_prefix", title="continuous-batching trace with prefix caching: 8 shared "
        "system prompts of 256-1024 tokens + private suffixes of 16-256, 40x128 heads, bf16",
        seed=9, dtype="bf16", num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
        num_blocks=50000, steps=200, arrival_mean=8.0, prompt_lo=0, prompt_hi=0,
        out_p=0.01, out_lo=10, out_hi=500, chunk=512, openings=8, open_lo=256, open_hi=1024,
        suffix_lo=16, suffix_hi=256, vocab=64),
    "trace_prefix_small": TraceConfig(
        name="trace_prefix_small", title="prefix-caching trace, 48 steps, small pool, bf16",
        seed=17, dtype="bf16", num_q_heads=8, num_kv_heads=4, head_dim=128, block_size=16,
        num_blocks=200, steps=48, arrival_mean=2.0, prompt_lo=0, prompt_hi=0,
        out_p=0.08, out_lo=2, out_hi=40, chunk=64, openings=3, open_lo=20, open_hi=120,
        suffix_lo=4, suffix_hi=60, vocab=64),
    # small trace for GPU parity tests: same loop, a pool small enough to preempt
    "trace_small": TraceConfig(
        name="trace_small", title="continuous-batching trace, 48 steps, small pool, bf16",
        seed=16, dtype="bf16", num_q_heads=8, num_kv_heads=4, head_dim=128, block_size=16,
        num_blocks=160, steps=48, arrival_mean=2.0, prompt_lo=8, prompt_hi=300,
        out_p=0.08, out_lo=2, out_hi=40, chunk=64),
}


def get_config(name: str):
    return CONFIGS[name]
