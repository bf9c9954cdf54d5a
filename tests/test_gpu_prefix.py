"""GPU: prefix caching end to end.  Prompts that open with one of two shared
system prompts are admitted with add_prefix; only their uncached tokens are
written; full blocks are registered; some requests leave and others reuse their
cached blocks from the free queue.  Decode attention and chunked-prefill
attention over the shared blocks must then equal the oracle over each request's
whole logical sequence (keys/values a pure function of token and position)."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import contiguous_decode, prefill_attention
from paged_kv_cache_397_amd import ops
from paged_kv_cache_397_amd.batch import PagedKVCache, to_device, to_storage
from tests.gpu_util import assert_close, to_f64
from workloads import gen

pytestmark = pytest.mark.gpu

SEED, VOCAB = 61, 64


def _admit(cache, rid, tokens, spec):
    cached = cache.alloc.add_prefix(rid, tokens)
    n = len(tokens)
    if cached < n:
        k, v = gen.token_kv(SEED, tokens[cached:], cached, spec.num_kv_heads, spec.head_dim,
                            spec.dtype, vocab=VOCAB)
        cache.write_tokens(k, v, cache.alloc.slots(rid, cached, n - cached))
    cache.alloc.register(rid, tokens)
    return cached


def test_prefix_reuse_end_to_end():
    spec = ops.CacheSpec(num_blocks=160, block_size=16, num_kv_heads=4, head_dim=128, dtype="bf16")
    Hq = 16
    cache = PagedKVCache(spec, gen.pool_permutation(SEED, 160), fill=float("nan"))
    prompts = gen.shared_opening_prompts(SEED, 0, 12, 2, 40, 100, 5, 40, VOCAB)
    toks, cached = {}, {}
    for r in range(6):
        toks[r] = prompts[r]
        cached[r] = _admit(cache, r, prompts[r], spec)
    for r in (0, 2, 4):                                # their cached blocks go back to the queue
        cache.alloc.free(r)
        del toks[r]
    for r in range(6, 12):
        toks[r] = prompts[r]
        cached[r] = _admit(cache, r, prompts[r], spec)
    lookups, hits, ncached = cache.alloc.prefix_stats()
    assert hits > 0 and sum(cached[r] > 0 for r in toks) >= 3, (lookups, hits, cached)
    # requests with the same opening share physical blocks
    tables = {r: cache.alloc.block_table(r) for r in toks}
    shared = [b for r in toks for b in tables[r] if cache.alloc.refcount(b) > 1]
    assert shared

    live = sorted(toks)
    S = len(live)
    tdev, ctx_dev, _, ctx = cache.metadata(live)
    scale = 1 / math.sqrt(spec.head_dim)
    q_host = gen.q_values(SEED, 1, S, Hq, spec.head_dim, spec.dtype)
    out = torch.empty(S, Hq, spec.head_dim, dtype=torch.bfloat16, device="cuda")
    ops.paged_attn_decode(spec, out, to_device(q_host, spec), cache.k, cache.v, tdev, ctx_dev,
                          scale, num_units=7)
    torch.cuda.synchronize()
    dec = to_f64(to_storage(out), "bf16")
    full = {r: gen.token_kv(SEED, toks[r], 0, spec.num_kv_heads, spec.head_dim, spec.dtype,
                            vocab=VOCAB) for r in live}
    for i, r in enumerate(live):
        K, V = full[r]
        ref = contiguous_decode(q_host[i], K, V, scale, "bf16")
        assert_close(dec[i], ref, "bf16", f"decode, request {r} (cached {cached[r]})")

    # each request's uncached tail as a prefill chunk over the shared blocks
    c = np.array([len(toks[r]) - cached[r] for r in live], dtype=np.int32)
    qs = np.zeros(S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(c)
    T = int(qs[-1])
    qp_host = gen.q_values(SEED, 2, T, Hq, spec.head_dim, spec.dtype)
    pout = torch.empty(T, Hq, spec.head_dim, dtype=torch.bfloat16, device="cuda")
    ops.paged_attn_prefill(spec, pout, to_device(qp_host, spec), cache.k, cache.v, tdev,
                           torch.from_numpy(qs).cuda(), ctx_dev, scale)
    torch.cuda.synchronize()
    pre = to_f64(to_storage(pout), "bf16")
    for i, r in enumerate(live):
        K, V = full[r]
        rows = slice(int(qs[i]), int(qs[i + 1]))
        ref = prefill_attention(to_f64(qp_host[rows], "bf16"), to_f64(K, "bf16"), to_f64(V, "bf16"),
                                scale, cached[r])
        assert_close(pre[rows], ref, "bf16", f"prefill tail, request {r} (cached {cached[r]})")
