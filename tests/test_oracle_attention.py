"""Pins of the oracle's decode attention (CPU only).

The oracle is tied to things other than itself: torch's float64 CPU
scaled-dot-product attention, closed forms, and invariances of paging.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention, paged_decode, contiguous_decode
from oracle.cache import reshape_and_cache
from oracle.layout import CacheLayout, to_float64
from workloads import gen


def _scatter_batch(layout, ctx, tables, Ks, Vs, fill=None):
    """Write each sequence's logical K/V into its blocks with the oracle writer."""
    kc = layout.empty_cache(fill)
    vc = layout.empty_cache(fill)
    B = layout.block_size
    for i, L in enumerate(ctx):
        slots = [tables[i][p // B] * B + p % B for p in range(L)]
        reshape_and_cache(layout, Ks[i], Vs[i], slots, kc, vc)
    return kc, vc


def _random_case(seed, dtype, S, Hq, Hkv, D, B, max_ctx, N):
    rng = gen.stream(seed, 7)
    ctx = rng.integers(0, max_ctx + 1, S)
    ctx[0] = max(ctx[0], 1)
    perm = rng.permutation(N)
    maxB = max(1, -(-int(ctx.max()) // B))
    tables = np.full((S, maxB), -1, dtype=np.int64)
    pos = 0
    for i, L in enumerate(ctx):
        nb = -(-int(L) // B)
        tables[i, :nb] = perm[pos:pos + nb]
        pos += nb
    assert pos <= N
    Ks, Vs = [], []
    for i, L in enumerate(ctx):
        K, V = gen.seq_kv(seed, i, int(L), Hkv, D, dtype)
        Ks.append(K)
        Vs.append(V)
    q = gen.q_values(seed, 0, S, Hq, D, dtype)
    return ctx, tables, Ks, Vs, q


def _sdpa(q64, K64, V64, scale):
    """torch CPU float64 SDPA for one decode query; q [Hq,D], K/V [L,Hkv,D]."""
    qt = torch.from_numpy(q64)[None, :, None, :]                 # [1,Hq,1,D]
    kt = torch.from_numpy(np.ascontiguousarray(K64.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V64.transpose(1, 0, 2)))[None]
    G = q64.shape[0] // K64.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B", [
    ("f32", 2, 2, 64, 16), ("bf16", 4, 1, 64, 16), ("bf16", 8, 2, 128, 32), ("f32", 6, 3, 128, 16)])
@pytest.mark.parametrize("seed", [11, 12])
def test_paged_matches_torch_sdpa(dtype, Hq, Hkv, D, B, seed):
    S, max_ctx, N = 4, 40, 64
    layout = CacheLayout(N, Hkv, B, D, dtype)
    ctx, tables, Ks, Vs, q = _random_case(seed, dtype, S, Hq, Hkv, D, B, max_ctx, N)
    kc, vc = _scatter_batch(layout, ctx, tables, Ks, Vs)
    scale = 1.0 / math.sqrt(D)
    out = paged_decode(layout, q, kc, vc, tables, ctx, scale)
    for i, L in enumerate(ctx):
        if L == 0:
            assert not out[i].any()
            continue
        ref = _sdpa(to_float64(q[i], dtype), to_float64(Ks[i], dtype), to_float64(Vs[i], dtype), scale)
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value_row():
    rng = gen.stream(5, 1)
    for dtype in ("f32", "bf16"):
        q = gen.draw_values(rng, (4, 64), dtype)
        K = gen.draw_values(rng, (1, 2, 64), dtype)
        V = gen.draw_values(rng, (1, 2, 64), dtype)
        out = contiguous_decode(q, K, V, 0.125, dtype)
        V64 = to_float64(V, dtype)
        assert np.array_equal(out[0], V64[0, 0]) and np.array_equal(out[1], V64[0, 0])
        assert np.array_equal(out[2], V64[0, 1]) and np.array_equal(out[3], V64[0, 1])


def test_constant_values_return_the_constant():
    rng = gen.stream(5, 2)
    q = rng.standard_normal((2, 64))
    K = rng.standard_normal((37, 1, 64))
    V = np.broadcast_to(rng.standard_normal((1, 1, 64)), (37, 1, 64))
    out = decode_attention(q, K, V, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(V[0, 0], (2, 64)), rtol=1e-14, atol=0)


def test_zero_query_averages_values():
    rng = gen.stream(5, 3)
    K = rng.standard_normal((29, 2, 32))
    V = rng.standard_normal((29, 2, 32))
    out = decode_attention(np.zeros((2, 32)), K, V, 1.0)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    # all keys equal has the same effect whatever the query is
    Keq = np.broadcast_to(K[:1], K.shape)
    out2 = decode_attention(rng.standard_normal((2, 32)), Keq, V, 0.7)
    np.testing.assert_allclose(out2, V.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_two_tokens_logistic_weights():
    rng = gen.stream(5, 4)
    q = rng.standard_normal((1, 16))
    K = rng.standard_normal((2, 1, 16))
    V = rng.standard_normal((2, 1, 16))
    scale = 0.25
    s0 = scale * float(K[0, 0] @ q[0])
    s1 = scale * float(K[1, 0] @ q[0])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    expect = w0 * V[0, 0] + w1 * V[1, 0]
    np.testing.assert_allclose(decode_attention(q, K, V, scale)[0], expect, rtol=1e-14, atol=1e-15)


def test_softmax_is_shift_safe():
    """Huge scores do not overflow: the max shift keeps the weights finite."""
    q = np.full((1, 4), 100.0)
    K = np.array([[[100.0] * 4], [[99.0] * 4]])
    V = np.array([[[1.0] * 4], [[0.0] * 4]])
    out = decode_attention(q, K, V, 1.0)
    w0 = 1.0 / (1.0 + math.exp(-400.0))
    np.testing.assert_allclose(out[0], w0, rtol=1e-15)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_invariances(dtype):
    """Permuting physical IDs, identity vs scattered tables, and shared vs private
    prefix blocks all give bit-identical oracle outputs."""
    S, Hq, Hkv, D, B, N = 3, 4, 2, 64, 16, 48
    layout = CacheLayout(N, Hkv, B, D, dtype)
    ctx, tables, Ks, Vs, q = _random_case(21, dtype, S, Hq, Hkv, D, B, 70, N)
    kc, vc = _scatter_batch(layout, ctx, tables, Ks, Vs)
    base = paged_decode(layout, q, kc, vc, tables, ctx, 0.125)
    # 1. relabel every physical block by a permutation
    perm = gen.stream(21, 8).permutation(N)
    tables_p = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    kc_p, vc_p = _scatter_batch(layout, ctx, tables_p, Ks, Vs)
    assert np.array_equal(paged_decode(layout, q, kc_p, vc_p, tables_p, ctx, 0.125), base)
    # 2. identity tables: sequence i owns a contiguous run of blocks
    tables_i = np.full_like(tables, -1)
    pos = 0
    for i, L in enumerate(ctx):
        nb = -(-int(L) // B)
        tables_i[i, :nb] = np.arange(pos, pos + nb)
        pos += nb
    kc_i, vc_i = _scatter_batch(layout, ctx, tables_i, Ks, Vs)
    assert np.array_equal(paged_decode(layout, q, kc_i, vc_i, tables_i, ctx, 0.125), base)


def test_shared_prefix_equals_private_copies():
    dtype, Hq, Hkv, D, B, N = "bf16", 2, 2, 64, 16, 32
    layout = CacheLayout(N, Hkv, B, D, dtype)
    prefix = 2 * B
    Kp, Vp = gen.seq_kv(31, 0, prefix, Hkv, D, dtype)
    suffix = [5, 19]
    Ks, Vs = [], []
    for i, s in enumerate(suffix):
        Kx, Vx = gen.seq_kv(31, 10 + i, s, Hkv, D, dtype)
        Ks.append(np.concatenate([Kp, Kx]))
        Vs.append(np.concatenate([Vp, Vx]))
    ctx = [prefix + s for s in suffix]
    q = gen.q_values(31, 0, 2, Hq, D, dtype)
    # shared: both tables start with physical blocks 3, 9
    shared = [[3, 9, 20, -1], [3, 9, 21, 22]]
    kc, vc = layout.empty_cache(), layout.empty_cache()
    for p in range(prefix):
        layout.write_token(kc, vc, shared[0][p // B], p % B, Kp[p], Vp[p])
    for i, s in enumerate(suffix):
        for p in range(prefix, prefix + s):
            layout.write_token(kc, vc, shared[i][p // B], p % B, Ks[i][p], Vs[i][p])
    out_shared = paged_decode(layout, q, kc, vc, np.array(shared), ctx, 0.125)
    private = [[0, 1, 2, -1], [4, 5, 6, 7]]
    kc2, vc2 = _scatter_batch(layout, ctx, private, Ks, Vs)
    out_private = paged_decode(layout, q, kc2, vc2, np.array(private), ctx, 0.125)
    assert np.array_equal(out_shared, out_private)


def test_unused_slots_and_table_entries_are_not_read():
    """NaN in every unwritten slot and block, and out-of-range IDs in the padding
    columns of the tables, change nothing."""
    dtype, Hq, Hkv, D, B, N = "f32", 2, 1, 64, 16, 16
    layout = CacheLayout(N, Hkv, B, D, dtype)
    ctx, tables, Ks, Vs, q = _random_case(41, dtype, 3, Hq, Hkv, D, B, 40, N)
    kc, vc = _scatter_batch(layout, ctx, tables, Ks, Vs)
    base = paged_decode(layout, q, kc, vc, tables, ctx, 0.125)
    kcn, vcn = _scatter_batch(layout, ctx, tables, Ks, Vs, fill=np.nan)
    assert np.isnan(kcn).any() and np.isnan(vcn).any()
    padded = np.where(tables >= 0, tables, 10 ** 6)
    out = paged_decode(layout, q, kcn, vcn, padded, ctx, 0.125)
    assert np.array_equal(out, base)


def test_zero_and_negative_scales():
    """scale = 0 weighs every token equally (the mean of V); a negative scale is the
    positive one with the query negated; two tokens at a negative scale follow the
    logistic weights of the negated score difference."""
    rng = gen.stream(5, 9)
    q = rng.standard_normal((4, 32))
    K = rng.standard_normal((23, 2, 32))
    V = rng.standard_normal((23, 2, 32))
    np.testing.assert_allclose(decode_attention(q, K, V, 0.0), np.repeat(V.mean(axis=0), 2, axis=0),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(decode_attention(q, K, V, -0.3), decode_attention(-q, K, V, 0.3),
                               rtol=1e-13, atol=1e-14)
    s = -0.5 * (K[:2, 0] @ q[0])
    w1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
    expect = (1.0 - w1) * V[0, 0] + w1 * V[1, 0]
    np.testing.assert_allclose(decode_attention(q[:1], K[:2, :1], V[:2, :1], -0.5)[0], expect,
                               rtol=1e-13, atol=1e-14)
