"""GPU: the shared-prefix and serving-trace workloads at their full sizes, in the
benchmark's launch configuration (default unit count), against the fp64 oracle.

* Shared prefix (64 sequences forked at 1024 + B/2 tokens, 63 copy-on-write copies
  of the shared partial block, private suffixes of 16..512 tokens; B = 16 and 32):
  every sequence against the oracle, bit-identical under both load policies and to
  a batch holding private copies of the same logical data (hihuo.com "vLLM 原理：
  PagedAttention 和 Continuous Batching", 优势 > 3. 支持共享: sequences that share
  a prefix share its pages).
* The 13B-shaped serving trace (40 heads, 200 steps, Poisson arrivals, chunked
  prompts): every 20th step, every decoded sequence against the oracle; at the
  trace's own 50k-block pool and at 20k blocks, where the pool fills and the
  scheduler preempts (same page, Preemption（抢占）).

Margins (max-abs, max-rel over |ref| >= 1e-3) are printed per check."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import contiguous_decode
from oracle.layout import to_float64
from paged_kv_cache_397_amd import ops
from paged_kv_cache_397_amd.batch import PagedKVCache, to_device, to_storage
from paged_kv_cache_397_amd.scheduler import TraceScheduler
from tests.gpu_util import assert_close, parallel_map, report_margin
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


def _decode(spec, cache_k, cache_v, tables, ctx, q, scale, keep_cached=False):
    S, Hq, D = q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=spec.torch_dtype, device="cuda")
    ops.paged_attn_decode(spec, out, q, cache_k, cache_v, tables, ctx, scale, num_units=0,
                          keep_cached=keep_cached)
    torch.cuda.synchronize()
    return to_storage(out)


# ----------------------------------------------------------------------------- shared prefix
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["shared_prefix_b16", "shared_prefix_b32"])
def test_shared_prefix_full_size(name):
    cfg = CONFIGS[name]
    B, S, Hq, Hkv, D = cfg.block_size, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    spec = ops.CacheSpec(cfg.num_blocks, B, Hkv, D, cfg.dtype)
    cache = PagedKVCache(spec, cfg.pool_order(), fill=float("nan"))
    # the parent holds the shared prefix, ending in a partial block; 63 children fork it
    prefix = cfg.shared_prefix + B // 2
    Kp, Vp = gen.seq_kv(cfg.seed, 0, prefix, Hkv, D, cfg.dtype)
    cache.add_sequence(0, Kp, Vp)
    for c in range(1, S):
        cache.alloc.fork(0, c)
    shared_blocks = cache.alloc.block_table(0)
    assert all(cache.alloc.refcount(b) == S for b in shared_blocks)
    ctx = cfg.context_lens().astype(np.int64)
    extra = ctx - prefix
    logical = {}
    for i in range(S):
        Ks, Vs = gen.seq_kv(cfg.seed, 1000 + i, int(extra[i]), Hkv, D, cfg.dtype)
        logical[i] = (np.concatenate([Kp, Ks]), np.concatenate([Vp, Vs]))
    # suffixes appended round robin, so each sequence's first append meets the
    # shared partial block: 63 copy-on-write copies, the last sharer writes in place
    written = np.zeros(S, dtype=np.int64)
    n_cow = 0
    while (written < extra).any():
        active = np.nonzero(written < extra)[0]
        st, done, slots, cows, _, _ = cache.alloc.append_batch(active)
        assert st == 0 and done == len(active)
        pairs = cows[cows[:, 0] >= 0]
        n_cow += len(pairs)
        if len(pairs):
            ops.copy_blocks(spec, cache.k, cache.v,
                            torch.from_numpy(np.ascontiguousarray(pairs)).cuda())
        pos = prefix + written[active]
        kk = np.stack([logical[i][0][p] for i, p in zip(active, pos)])
        vv = np.stack([logical[i][1][p] for i, p in zip(active, pos)])
        cache.write_tokens(kk, vv, slots)
        written[active] += 1
    assert n_cow == S - 1
    assert all(cache.alloc.refcount(b) == S for b in shared_blocks[:-1])
    seqs = list(range(S))
    tables, ctx_dev, _, ctx_host = cache.metadata(seqs)
    assert np.array_equal(ctx_host, ctx)
    q_host = gen.q_values(cfg.seed, 0, S, Hq, D, cfg.dtype)
    q = to_device(q_host, spec)
    streamed = _decode(spec, cache.k, cache.v, tables, ctx_dev, q, cfg.scale)
    kept = _decode(spec, cache.k, cache.v, tables, ctx_dev, q, cfg.scale, keep_cached=True)
    assert np.array_equal(streamed.view(np.uint8), kept.view(np.uint8))
    ref = np.stack(parallel_map(
        lambda i: contiguous_decode(q_host[i], *logical[i], cfg.scale, cfg.dtype), seqs))
    margins = assert_close(to_float64(streamed, cfg.dtype), ref, cfg.dtype, name)
    report_margin(f"{name} (all {S} sequences, default units)", margins)
    # the same logical data in private blocks: the same bits
    del cache
    priv = PagedKVCache(spec, cfg.pool_order(), fill=float("nan"))
    for i in seqs:
        priv.add_sequence(i, *logical[i])
    t2, c2, _, _ = priv.metadata(seqs, tables.shape[1])
    private = _decode(spec, priv.k, priv.v, t2, c2, q, cfg.scale)
    assert np.array_equal(private.view(np.uint8), streamed.view(np.uint8))


# ----------------------------------------------------------------------------- serving trace
def _run_trace(num_blocks: int, check_every: int = 20):
    """The 13B-shaped trace through the library scheduler and kernels; returns
    (steps checked, sequences checked, preemptions, (max-abs, max-rel))."""
    cfg = CONFIGS["trace_13b"]
    B, D, Hq, Hkv, dtype = cfg.block_size, cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads, cfg.dtype
    spec = ops.CacheSpec(num_blocks, B, Hkv, D, dtype)
    kc, vc = ops.empty_cache(spec)
    kc.fill_(float("nan"))
    vc.fill_(float("nan"))
    sched = TraceScheduler(num_blocks, B, cfg.chunk, gen.pool_permutation(cfg.seed, num_blocks))
    max_blocks = -(-(cfg.prompt_hi + cfg.out_hi) // B)
    seed = cfg.seed
    checked = seqs_checked = preempted = 0
    worst = [0.0, 0.0]
    for n in range(cfg.steps):
        plan = sched.step(n, cfg.arrivals(n))
        preempted += len(plan.preempted)
        if plan.prefill:
            kv = [gen.trace_table_kv(seed, rid, range(s0, s0 + c), Hkv, D, dtype)
                  for rid, s0, c, _ in plan.prefill]
            ops.reshape_and_cache(spec, to_device(np.concatenate([k for k, _ in kv]), spec),
                                  to_device(np.concatenate([v for _, v in kv]), spec),
                                  torch.from_numpy(np.concatenate([sl for *_, sl in plan.prefill])).cuda(),
                                  kc, vc)
        S = len(plan.decode_rids)
        if S == 0:
            continue
        rids, pos = plan.decode_rids, plan.decode_pos
        kv = [gen.trace_table_kv(seed, int(r), [int(p)], Hkv, D, dtype) for r, p in zip(rids, pos)]
        ops.append_tokens(spec, to_device(np.concatenate([k for k, _ in kv]), spec),
                          to_device(np.concatenate([v for _, v in kv]), spec),
                          torch.from_numpy(plan.decode_slots).cuda(), kc, vc,
                          cow_pairs=torch.from_numpy(np.ascontiguousarray(plan.decode_cows)).cuda())
        if n % check_every != check_every - 1:
            continue
        tables, ctx = sched.alloc.batch_metadata(rids, max_blocks)
        assert np.array_equal(ctx, pos + 1)
        q_host = gen.trace_table_query(seed, rids.tolist(), pos.tolist(), Hq, D, dtype)
        got = to_float64(_decode(spec, kc, vc, torch.from_numpy(tables).cuda(),
                                 torch.from_numpy(ctx).cuda(), to_device(q_host, spec),
                                 cfg.scale), dtype)

        def one(i):
            K, V = gen.trace_table_kv(seed, int(rids[i]), range(int(pos[i]) + 1), Hkv, D, dtype)
            return contiguous_decode(q_host[i], K, V, cfg.scale, dtype)

        ref = np.stack(parallel_map(one, range(S)))
        m = assert_close(got, ref, dtype, f"trace_13b at {num_blocks} blocks, step {n}, {S} sequences")
        worst = [max(worst[0], m[0]), max(worst[1], m[1])]
        checked += 1
        seqs_checked += S
    return checked, seqs_checked, preempted, worst


@pytest.mark.timeout(900)
@pytest.mark.parametrize("num_blocks", [50000, 20000])
def test_serving_trace_full_size(num_blocks):
    checked, seqs, preempted, worst = _run_trace(num_blocks)
    report_margin(f"trace_13b at {num_blocks} blocks ({checked} steps, {seqs} sequence checks, "
                  f"{preempted} preemptions)", worst)
    assert checked == 10 and seqs > 3000
    if num_blocks < 50000:
        assert preempted > 0, "the 20k-block pool was meant to fill and preempt"
