"""GPU: paged decode attention through the C ABI against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import contiguous_decode
from oracle.cache import reshape_and_cache as oracle_reshape_and_cache
from oracle.layout import CacheLayout, to_float64
from paged_kv_cache_397_amd import ops
from paged_kv_cache_397_amd.batch import PagedKVCache, to_device, to_storage
from tests.gpu_util import Batch, assert_close, report_margin
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- the tiny fp32 config
def test_tiny_config_and_its_cache_write():
    cfg = CONFIGS["tiny_f32"]
    spec = ops.CacheSpec(cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
    b = Batch(spec, cfg.context_lens(), cfg.num_q_heads, cfg.seed, free_order=cfg.pool_order())
    out = b.run()
    assert_close(to_float64(out, "f32"), b.expected(), "f32", "tiny step 1")
    # one decode step more: reserve the next slot of every sequence (the third one
    # opens a new block), write 4 new tokens there, attend again over ctx + 1.
    status, done, slots, cows, new_blocks, _ = b.cache.alloc.append_batch(np.arange(4))
    assert status == 0 and done == 4 and (cows < 0).all()
    assert (new_blocks >= 0).tolist() == [False, False, True, False]
    kn, vn = gen.new_tokens(cfg.seed, 1, 4, spec.num_kv_heads, spec.head_dim, "f32")
    k_before, v_before = to_storage(b.cache.k), to_storage(b.cache.v)
    b.cache.write_tokens(kn, vn, slots)
    lay = CacheLayout(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, "f32")
    oracle_reshape_and_cache(lay, kn, vn, slots, k_before, v_before)
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(b.cache.k), k_before, equal_nan=True)
    assert np.array_equal(to_storage(b.cache.v), v_before, equal_nan=True)
    tables, ctx, _, ctx_host = b.cache.metadata(range(4))
    assert ctx_host.tolist() == [2, 16, 17, 34]
    q2h = gen.q_values(cfg.seed, 1, 4, cfg.num_q_heads, cfg.head_dim, "f32")
    q2 = to_device(q2h, spec)
    out2 = torch.empty_like(q2)
    ops.paged_attn_decode(spec, out2, q2, b.cache.k, b.cache.v, tables, ctx, cfg.scale)
    torch.cuda.synchronize()
    for i in range(4):
        K, V = gen.seq_kv(cfg.seed, i, int(b.ctx[i]), 2, 64, "f32")
        K = np.concatenate([K, kn[i:i + 1]])
        V = np.concatenate([V, vn[i:i + 1]])
        ref = contiguous_decode(q2h[i], K, V, cfg.scale, "f32")
        assert_close(to_float64(to_storage(out2)[i], "f32"), ref, "f32", f"tiny step 2 seq {i}")


# ----------------------------------------------------------------------------- shapes and edges
EDGE_CTX = [0, 1, 15, 16, 17, 33, 100, 257]


@pytest.mark.parametrize("dtype,D,B,Hq,Hkv", [
    ("bf16", 128, 16, 8, 8),   # per-head VALU path
    ("bf16", 128, 16, 16, 4),  # group MFMA path, G = 4
    ("bf16", 64, 32, 8, 4),    # group, G = 2, two tiles per block
    ("bf16", 128, 64, 16, 2),  # group, G = 8
    ("bf16", 64, 16, 16, 1),   # group, G = 16
    ("f32", 64, 16, 2, 2),     # fp32 per-head
    ("f32", 128, 32, 6, 2),    # fp32 with G = 3 (per-head path)
    ("bf16", 128, 8, 32, 8),   # blocks of 8 tokens: a tile reads two blocks; group, G = 4
    ("bf16", 128, 8, 8, 8),    # blocks of 8, per-head path
    ("f32", 64, 8, 4, 2),      # blocks of 8, fp32
])
@pytest.mark.parametrize("units", [0, 1, 3, 40])
def test_decode_matches_oracle(dtype, D, B, Hq, Hkv, units):
    spec = ops.CacheSpec(num_blocks=64, block_size=B, num_kv_heads=Hkv, head_dim=D, dtype=dtype)
    b = Batch(spec, EDGE_CTX, Hq, seed=100 + D + B + Hq, free_order=gen.pool_permutation(7, 64))
    out = b.run(num_units=units)
    ref = b.expected()
    assert not np.isnan(to_float64(out, dtype)).any()
    assert_close(to_float64(out, dtype), ref, dtype, f"{dtype} D{D} B{B} G{Hq // Hkv} units {units}")
    assert not to_float64(out[0], dtype).any()          # ctx 0 -> zeros


@pytest.mark.parametrize("dtype,Hq,Hkv,units", [("bf16", 16, 4, 0), ("bf16", 16, 4, 7),
                                                 ("bf16", 8, 8, 0), ("f32", 4, 2, 64)])
def test_batch_past_the_register_held_lengths(dtype, Hq, Hkv, units):
    """300 sequences: the kernel scans the context lengths 64 at a time, so a unit's
    first sequence is found several rounds into the scan, past the batch sizes of the
    other tests.  Zero-length sequences (also at 256 and 257) get zeros; every other
    output matches the oracle."""
    rng = gen.stream(61, 1)
    ctx = rng.integers(1, 80, 300)
    ctx[[0, 100, 255, 256, 257, 299]] = 0
    ctx[[1, 254, 258, 298]] = [700, 513, 640, 1]
    spec = ops.CacheSpec(num_blocks=2048, block_size=16, num_kv_heads=Hkv, head_dim=64, dtype=dtype)
    b = Batch(spec, ctx, Hq, seed=62, free_order=gen.pool_permutation(9, 2048))
    out = b.run(num_units=units)
    got = to_float64(out, dtype)
    assert not np.isnan(got).any()
    assert not got[ctx == 0].any()
    assert_close(got, b.expected(), dtype, f"{dtype} G{Hq // Hkv} units {units} S 300")


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 4, 4), ("bf16", 8, 2), ("f32", 2, 2)])
def test_single_token_returns_value_bitwise(dtype, Hq, Hkv):
    spec = ops.CacheSpec(num_blocks=8, block_size=16, num_kv_heads=Hkv, head_dim=128, dtype=dtype)
    b = Batch(spec, [1, 1, 1], Hq, seed=9)
    out = b.run(num_units=2)
    G = Hq // Hkv
    for i in range(3):
        _, V = gen.seq_kv(9, i, 1, Hkv, 128, dtype)
        for j in range(Hq):
            assert np.array_equal(out[i, j], V[0, j // G]), (i, j)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 8, 8), ("bf16", 16, 4), ("f32", 4, 4)])
def test_invariances_bitwise(dtype, Hq, Hkv):
    """Permuted physical IDs and identity vs scattered tables give bit-identical output."""
    ctx = [5, 300, 64, 1000, 17, 2]
    spec = ops.CacheSpec(num_blocks=128, block_size=16, num_kv_heads=Hkv, head_dim=128, dtype=dtype)
    base = Batch(spec, ctx, Hq, seed=21, free_order=gen.pool_permutation(1, 128)).run(num_units=7)
    perm = Batch(spec, ctx, Hq, seed=21, free_order=gen.pool_permutation(2, 128)).run(num_units=7)
    ident = Batch(spec, ctx, Hq, seed=21, free_order=None).run(num_units=7)
    assert np.array_equal(base, perm) and np.array_equal(base, ident)


def test_poisoned_padding_columns_change_nothing():
    spec = ops.CacheSpec(num_blocks=64, block_size=16, num_kv_heads=4, head_dim=128, dtype="bf16")
    b = Batch(spec, [20, 1, 47], 16, seed=31, free_order=gen.pool_permutation(3, 64), max_blocks=8)
    base = b.run(num_units=5)
    t = b.tables_host.copy()
    t[t < 0] = 123456789                                    # garbage past the valid columns
    poisoned = b.run(num_units=5, tables=torch.from_numpy(t).cuda())
    assert np.array_equal(base, poisoned)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 16, 4), ("bf16", 8, 8), ("f32", 4, 2)])
@pytest.mark.parametrize("units", [0, 3, 40])
def test_context_lengths_outside_the_table_are_clamped(dtype, Hq, Hkv, units):
    """Lengths past what a table row addresses (max_blocks_per_seq * B) act as that
    maximum and negative ones as zero: the output equals, bit for bit, the call with
    the clamped lengths, and the oracle on them."""
    true_ctx = [48, 16, 48, 0, 5, 47]
    spec = ops.CacheSpec(num_blocks=64, block_size=16, num_kv_heads=Hkv, head_dim=128, dtype=dtype)
    b = Batch(spec, true_ctx, Hq, seed=33, free_order=gen.pool_permutation(8, 64), max_blocks=3)
    wild = torch.tensor([49, 16, 2**31 - 1, -7, 5, 47], dtype=torch.int32, device="cuda")
    got = b.run(num_units=units, ctx=wild)
    assert np.array_equal(got.view(np.uint8), b.run(num_units=units).view(np.uint8))
    assert_close(to_float64(got, dtype), b.expected(), dtype, f"clamped lengths, units {units}")
    assert not to_float64(got[3], dtype).any()


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 16, 4), ("bf16", 8, 8), ("f32", 4, 2)])
@pytest.mark.parametrize("units", [0, 3, 40])
def test_blocks_of_8_with_an_odd_table_width(dtype, Hq, Hkv, units):
    """Blocks of 8 tokens and five table columns (a row addresses 40 tokens), so the
    last 16-token tile of a full row has one block only: lengths past 40 act as 40,
    equal bit for bit to the call with the clamped lengths and to the oracle, with
    the pool's unused blocks NaN-poisoned."""
    true_ctx = [40, 8, 33, 0, 5, 39, 16, 17]
    spec = ops.CacheSpec(num_blocks=64, block_size=8, num_kv_heads=Hkv, head_dim=128, dtype=dtype)
    b = Batch(spec, true_ctx, Hq, seed=34, free_order=gen.pool_permutation(9, 64), max_blocks=5)
    wild = torch.tensor([41, 8, 33, -1, 5, 39, 16, 17], dtype=torch.int32, device="cuda")
    got = b.run(num_units=units, ctx=wild)
    assert np.array_equal(got.view(np.uint8), b.run(num_units=units).view(np.uint8))
    assert not np.isnan(to_float64(got, dtype)).any()
    assert_close(to_float64(got, dtype), b.expected(), dtype, f"blocks of 8, units {units}")
    assert not to_float64(got[3], dtype).any()


@pytest.mark.parametrize("dtype,Hq,Hkv,B", [("bf16", 32, 8, 16), ("bf16", 8, 8, 16), ("bf16", 32, 8, 8)])
def test_unit_count_sweep(dtype, Hq, Hkv, B):
    """Every split of the work (one unit .. more units than tiles) stays within tolerance."""
    rng = gen.stream(41, 1)
    ctx = rng.integers(1, 700, 12)
    spec = ops.CacheSpec(num_blocks=2048, block_size=B, num_kv_heads=Hkv, head_dim=128, dtype=dtype)
    b = Batch(spec, ctx, Hq, seed=41, free_order=gen.pool_permutation(4, 2048))
    ref = b.expected()
    for units in (1, 2, 7, 64, 513, 5000, 0):
        assert_close(to_float64(b.run(num_units=units), dtype), ref, dtype, f"units {units}")


def test_shared_prefix_fork_and_copy_on_write():
    """Sequences forked from one parent share its blocks; their first write into the
    shared partial block goes through copy-on-write.  Output equals the oracle and
    is bit-identical to a batch holding private copies of the prefix."""
    B, Hkv, Hq, D = 16, 4, 4, 128
    spec = ops.CacheSpec(num_blocks=96, block_size=B, num_kv_heads=Hkv, head_dim=D, dtype="bf16")
    cache = PagedKVCache(spec, gen.pool_permutation(5, 96), fill=float("nan"))
    prefix = 2 * B + B // 2
    Kp, Vp = gen.seq_kv(61, 0, prefix, Hkv, D, "bf16")
    cache.add_sequence(0, Kp, Vp)
    kids = [1, 2, 3]
    for c in kids:
        cache.alloc.fork(0, c)
    suffix = {0: 5, 1: 20, 2: 9, 3: 1}
    logical = {}
    n_cow = 0
    for s, n in suffix.items():
        Ks, Vs = gen.seq_kv(61, 100 + s, n, Hkv, D, "bf16")
        logical[s] = (np.concatenate([Kp, Ks]), np.concatenate([Vp, Vs]))
    order = [1, 2, 3, 0]                                    # the parent writes last, in place
    for s in order:
        for p in range(suffix[s]):
            slot, cow = cache.alloc.append(s)
            if cow is not None:
                n_cow += 1
                ops.copy_blocks(spec, cache.k, cache.v,
                                torch.tensor([cow], dtype=torch.int32, device="cuda"))
            Ks, Vs = logical[s]
            cache.write_tokens(Ks[prefix + p:prefix + p + 1], Vs[prefix + p:prefix + p + 1], [slot])
    assert n_cow == 3
    seqs = [0, 1, 2, 3]
    tables, ctx, _, ctx_host = cache.metadata(seqs)
    q_host = gen.q_values(61, 0, 4, Hq, D, "bf16")
    q = to_device(q_host, spec)
    out = torch.empty_like(q)
    ops.paged_attn_decode(spec, out, q, cache.k, cache.v, tables, ctx, 1 / math.sqrt(D), num_units=6)
    torch.cuda.synchronize()
    got = to_storage(out)
    for k, s in enumerate(seqs):
        ref = contiguous_decode(q_host[k], *logical[s], 1 / math.sqrt(D), "bf16")
        assert_close(to_float64(got[k], "bf16"), ref, "bf16", f"shared seq {s}")
    # the load policy for shared blocks changes nothing but where lines are cached
    kept = torch.empty_like(q)
    ops.paged_attn_decode(spec, kept, q, cache.k, cache.v, tables, ctx, 1 / math.sqrt(D),
                          num_units=6, keep_cached=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(kept).view(np.uint8), got.view(np.uint8))
    # private copies of the same logical data
    priv = PagedKVCache(spec, None, fill=float("nan"))
    for s in seqs:
        priv.add_sequence(s, *logical[s])
    t2, c2, _, _ = priv.metadata(seqs)
    out2 = torch.empty_like(q)
    ops.paged_attn_decode(spec, out2, q, priv.k, priv.v, t2, c2, 1 / math.sqrt(D), num_units=6)
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(out2), got)


# ----------------------------------------------------------------------------- full-size configs
@pytest.mark.parametrize("name", ["gqa_b256", "llama2_7b_b64"])
def test_full_size_config_every_sequence(name):
    """The benchmark's configuration and launch (default units) on a NaN-poisoned
    pool: every sequence of the batch against the fp64 oracle, margins reported."""
    cfg = CONFIGS[name]
    spec = ops.CacheSpec(cfg.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
    b = Batch(spec, cfg.context_lens(), cfg.num_q_heads, cfg.seed, free_order=cfg.pool_order(),
              poison=True, keep_kv=True)
    out = b.run(num_units=0)
    got = to_float64(out, spec.dtype)
    assert np.isfinite(got).all()
    margins = assert_close(got, b.expected(), spec.dtype, f"{name}, all {b.S} sequences")
    report_margin(f"{name} (all {b.S} sequences, default units)", margins)
    # every sequence, merged in the kernel, equals the two-kernel path bit for bit
    units = ops.default_units()
    ws = ops.decode_workspace(spec, cfg.num_q_heads, units)
    two = torch.full((b.S, cfg.num_q_heads, cfg.head_dim), float("nan"), dtype=spec.torch_dtype,
                     device="cuda")
    args = (spec, two, b.q, b.cache.k, b.cache.v, b.tables, b.ctx_dev, cfg.scale, units, ws)
    ops.paged_attn_decode_partial(*args)
    ops.paged_attn_decode_merge(*args)
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(two).view(np.uint8), out.view(np.uint8))
    # ordinary loads (PA_DECODE_KEEP_CACHED) instead of non-temporal ones: same bits
    kept = torch.full_like(two, float("nan"))
    ops.paged_attn_decode(spec, kept, b.q, b.cache.k, b.cache.v, b.tables, b.ctx_dev, cfg.scale,
                          units, ws, keep_cached=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(kept).view(np.uint8), out.view(np.uint8))


# ----------------------------------------------------------------------------- two calls vs one


@pytest.mark.parametrize("dtype,Hq,Hkv,D,units", [("bf16", 32, 8, 128, 37), ("bf16", 16, 16, 128, 64),
                                                 ("bf16", 16, 8, 64, 19), ("f32", 4, 2, 128, 11)])
def test_partial_then_merge_equals_single_call_bitwise(dtype, Hq, Hkv, D, units):
    """_partial then _merge on one stream is the single call, bit for bit."""
    rng = gen.stream(51, 1)
    ctx = rng.integers(1, 900, 10)
    ctx[3] = 0
    spec = ops.CacheSpec(num_blocks=1024, block_size=16, num_kv_heads=Hkv, head_dim=D, dtype=dtype)
    b = Batch(spec, ctx, Hq, seed=51, free_order=gen.pool_permutation(5, 1024))
    single = b.run(num_units=units)
    ws = ops.decode_workspace(spec, Hq, units)
    out = torch.full((b.S, Hq, D), float("nan"), dtype=spec.torch_dtype, device="cuda")
    args = (spec, out, b.q, b.cache.k, b.cache.v, b.tables, b.ctx_dev, 1 / math.sqrt(D), units, ws)
    ops.paged_attn_decode_partial(*args)
    ops.paged_attn_decode_merge(*args)
    torch.cuda.synchronize()
    two = to_storage(out)
    assert np.array_equal(single.view(np.uint8), two.view(np.uint8))
    assert_close(to_float64(single, dtype), b.expected(), dtype, "single call")


def test_reused_workspace_across_calls():
    """One workspace serves many calls with different lengths and unit counts, and
    every output of every call is written (outputs start as NaN).  The arrival counts
    at the workspace's end (one int32 per unit, read by the single-call decode) are
    back at zero after every call."""
    spec = ops.CacheSpec(num_blocks=2048, block_size=16, num_kv_heads=8, head_dim=128, dtype="bf16")
    ws = ops.decode_workspace(spec, 32, 300)
    rng = gen.stream(52, 1)
    for trial in range(4):
        ctx = rng.integers(1, 1500, 9)
        b = Batch(spec, ctx, 32, seed=60 + trial, free_order=gen.pool_permutation(6, 2048))
        for units in (300, 41, 300, 7, 41, 299):
            out = torch.full((b.S, 32, 128), float("nan"), dtype=spec.torch_dtype, device="cuda")
            ops.paged_attn_decode(spec, out, b.q, b.cache.k, b.cache.v, b.tables, b.ctx_dev,
                                  1 / math.sqrt(128), units, ws)
            torch.cuda.synchronize()
            assert int(ws[-4 * 300:].count_nonzero()) == 0, (trial, units)
            fresh = b.run(num_units=units)
            assert np.array_equal(to_storage(out).view(np.uint8), fresh.view(np.uint8)), (trial, units)
        assert_close(to_float64(fresh, "bf16"), b.expected(), "bf16", f"trial {trial}")


@pytest.mark.parametrize("dtype,D,B,Hq,Hkv", [
    ("bf16", 128, 16, 8, 8),   # per-head VALU path
    ("bf16", 128, 16, 32, 8),  # group MFMA path, G = 4
    ("f32", 64, 16, 4, 2),     # fp32
])
@pytest.mark.parametrize("sign", [-1.0, 0.0])
def test_negative_and_zero_scale(dtype, D, B, Hq, Hkv, sign):
    """The softmax takes any finite scale: a negative one (the largest weight goes to
    the smallest product) and zero (every visible token weighs the same, so the row
    is the mean of V) match the oracle on a poisoned cache."""
    spec = ops.CacheSpec(num_blocks=64, block_size=B, num_kv_heads=Hkv, head_dim=D, dtype=dtype)
    b = Batch(spec, EDGE_CTX[1:], Hq, seed=61, free_order=gen.pool_permutation(61, 64))
    scale = sign / math.sqrt(D)
    out = to_float64(b.run(scale=scale), dtype)
    ref = b.expected(scale=scale)
    assert_close(out, ref, dtype, f"scale {scale}")
    if sign == 0.0:
        for i, L in enumerate(b.ctx):
            _, V = gen.seq_kv(61, i, int(L), Hkv, D, dtype)
            mean = to_float64(V, dtype).mean(axis=0)        # [Hkv, D]
            assert_close(out[i], np.repeat(mean, Hq // Hkv, axis=0), dtype, f"mean of V, seq {i}")
