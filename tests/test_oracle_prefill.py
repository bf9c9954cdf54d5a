"""Pins of the oracle's chunked-prefill attention (CPU only).

Tied to things other than the oracle itself: torch's float64 CPU
scaled-dot-product attention under an explicit causal mask offset by the chunk
start, closed forms, the oracle's decode attention (pinned on its own), and the
fact that cutting a prompt into chunks must not change any row.  Planted
mistakes (a dropped diagonal, chunk positions counted from zero, a reversed
mask) must fail the pins.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle.attention import decode_attention, paged_decode, paged_prefill, prefill_attention
from oracle.cache import reshape_and_cache
from oracle.layout import CacheLayout, to_float64
from workloads import gen


def _sdpa_causal(q, K, V, scale, start):
    """torch float64 SDPA: q [c,Hq,D] at positions start.., K/V [L,Hkv,D]."""
    c, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]        # [1,Hq,c,D]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    rows = torch.arange(c)[:, None] + start
    mask = torch.arange(L)[None, :] <= rows                                         # [c, L]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _chunk_case(seed, dtype, Hq, Hkv, D, B, specs, N):
    """specs: list of (L, c) per sequence.  Returns everything paged_prefill needs
    plus the logical K/V of each sequence."""
    rng = gen.stream(seed, 9)
    perm = rng.permutation(N)
    layout = CacheLayout(N, Hkv, B, D, dtype)
    S = len(specs)
    maxB = max(1, max(-(-L // B) for L, _ in specs))
    tables = np.full((S, maxB), -1, dtype=np.int64)
    kc, vc = layout.empty_cache(None), layout.empty_cache(None)
    pos = 0
    Ks, Vs = [], []
    for i, (L, _) in enumerate(specs):
        nb = -(-L // B)
        tables[i, :nb] = perm[pos:pos + nb]
        pos += nb
        K, V = gen.seq_kv(seed, i, L, Hkv, D, dtype)
        slots = [tables[i][p // B] * B + p % B for p in range(L)]
        reshape_and_cache(layout, K, V, slots, kc, vc)
        Ks.append(K)
        Vs.append(V)
    assert pos <= N
    qs = np.zeros(S + 1, dtype=np.int64)
    qs[1:] = np.cumsum([c for _, c in specs])
    q = gen.q_values(seed, 1, int(qs[-1]), Hq, D, dtype)
    ctx = np.array([L for L, _ in specs], dtype=np.int64)
    return layout, q, kc, vc, tables, qs, ctx, Ks, Vs


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B", [
    ("f32", 2, 2, 64, 16), ("bf16", 4, 1, 64, 16), ("bf16", 8, 2, 128, 32), ("f32", 6, 3, 128, 16)])
def test_paged_prefill_matches_torch_sdpa(dtype, Hq, Hkv, D, B):
    specs = [(1, 1), (37, 37), (40, 9), (16, 16), (33, 1), (70, 23), (5, 0)]
    layout, q, kc, vc, tables, qs, ctx, Ks, Vs = _chunk_case(31, dtype, Hq, Hkv, D, B, specs, 64)
    scale = 1.0 / math.sqrt(D)
    out = paged_prefill(layout, q, kc, vc, tables, qs, ctx, scale)
    for i, (L, c) in enumerate(specs):
        if c == 0:
            continue
        rows = slice(int(qs[i]), int(qs[i + 1]))
        ref = _sdpa_causal(to_float64(q[rows], dtype), to_float64(Ks[i], dtype),
                           to_float64(Vs[i], dtype), scale, L - c)
        np.testing.assert_allclose(out[rows], ref, rtol=1e-12, atol=1e-12)


def test_first_prompt_token_returns_its_value_row():
    """Position 0 sees only itself: softmax over one key is 1, whatever the query."""
    rng = gen.stream(32, 1)
    Hq, Hkv, D = 8, 2, 64
    K = rng.standard_normal((12, Hkv, D))
    V = rng.standard_normal((12, Hkv, D))
    q = 50.0 * rng.standard_normal((12, Hq, D))
    out = prefill_attention(q, K, V, 0.125, 0)
    for j in range(Hq):
        np.testing.assert_array_equal(out[0, j], V[0, j // (Hq // Hkv)])


def test_zero_query_gives_running_mean():
    """Equal scores: row i is the mean of the value rows 0 .. start + i."""
    rng = gen.stream(33, 1)
    Hq, Hkv, D, L, start = 4, 4, 32, 30, 11
    V = rng.standard_normal((L, Hkv, D))
    K = rng.standard_normal((L, Hkv, D))
    q = np.zeros((L - start, Hq, D))
    out = prefill_attention(q, K, V, 1.0, start)
    cum = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None, None]
    np.testing.assert_allclose(out, cum[start:], rtol=1e-13, atol=1e-13)


def test_any_chunking_gives_the_same_rows():
    """A 61-token prompt prefilled at once, or in chunks of 16/20/25, writing each
    chunk before attending with it: every row agrees to float64 rounding."""
    dtype, Hq, Hkv, D, B = "bf16", 8, 2, 64, 16
    L = 61
    layout, q, kc, vc, tables, qs, ctx, Ks, Vs = _chunk_case(34, dtype, Hq, Hkv, D, B, [(L, L)], 8)
    scale = 1.0 / math.sqrt(D)
    whole = paged_prefill(layout, q, kc, vc, tables, qs, ctx, scale)
    start = 0
    for c in (16, 20, 25):
        # the cache holds start + c tokens when this chunk attends (later tokens
        # are not written yet): give the call exactly that length
        part = paged_prefill(layout, q[start:start + c], kc, vc, tables,
                             np.array([0, c]), np.array([start + c]), scale)
        np.testing.assert_allclose(part, whole[start:start + c], rtol=1e-13, atol=1e-13)
        start += c
    assert start == L


def test_last_row_of_a_chunk_is_decode():
    """The chunk's last token sees the whole cache, as a decode query does."""
    dtype, Hq, Hkv, D, B = "f32", 6, 3, 64, 16
    specs = [(50, 7), (17, 17), (3, 1)]
    layout, q, kc, vc, tables, qs, ctx, Ks, Vs = _chunk_case(35, dtype, Hq, Hkv, D, B, specs, 16)
    scale = 0.2
    out = paged_prefill(layout, q, kc, vc, tables, qs, ctx, scale)
    last = np.stack([q[int(qs[i + 1]) - 1] for i in range(len(specs))])
    dec = paged_decode(layout, last, kc, vc, tables, ctx, scale)
    for i in range(len(specs)):
        np.testing.assert_allclose(out[int(qs[i + 1]) - 1], dec[i], rtol=1e-12, atol=1e-12)


# ---- planted mistakes -------------------------------------------------------------

def _mutant_no_diagonal(q, K, V, scale, start):
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape)
    for i in range(q.shape[0]):
        n = max(start + i, 1)                      # wrong: a token does not see itself
        out[i] = decode_attention(q[i], K[:n], V[:n], scale)
    return out


def _mutant_positions_from_zero(q, K, V, scale, start):
    return prefill_attention(q, K, V, scale, 0)     # wrong: ignores the cached prefix


def _mutant_reversed_mask(q, K, V, scale, start):
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape)
    L = K.shape[0]
    for i in range(q.shape[0]):
        lo = start + i                             # wrong: sees itself and the future
        out[i] = decode_attention(q[i], K[lo:L], V[lo:L], scale)
    return out


@pytest.mark.parametrize("mutant", [_mutant_no_diagonal, _mutant_positions_from_zero,
                                    _mutant_reversed_mask])
def test_prefill_pins_reject_mutants(mutant, monkeypatch):
    monkeypatch.setattr(oa, "prefill_attention", mutant)
    dtype, Hq, Hkv, D, B = "f32", 4, 2, 64, 16
    specs = [(40, 9), (23, 23)]
    layout, q, kc, vc, tables, qs, ctx, Ks, Vs = _chunk_case(36, dtype, Hq, Hkv, D, B, specs, 16)
    out = oa.paged_prefill(layout, q, kc, vc, tables, qs, ctx, 0.125)
    bad = False
    for i, (L, c) in enumerate(specs):
        rows = slice(int(qs[i]), int(qs[i + 1]))
        ref = _sdpa_causal(to_float64(q[rows], dtype), to_float64(Ks[i], dtype),
                           to_float64(Vs[i], dtype), 0.125, L - c)
        bad |= not np.allclose(out[rows], ref, rtol=1e-6, atol=1e-6)
    assert bad, mutant.__name__


def test_zero_scale_gives_running_mean():
    """A zero scale equalises the scores whatever the query: row i is the mean of
    the value rows 0 .. start + i."""
    rng = gen.stream(33, 7)
    Hq, Hkv, D, L, start = 4, 2, 32, 27, 9
    V = rng.standard_normal((L, Hkv, D))
    K = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((L - start, Hq, D))
    out = prefill_attention(q, K, V, 0.0, start)
    cum = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None, None]
    np.testing.assert_allclose(out, np.repeat(cum[start:], Hq // Hkv, axis=1), rtol=1e-13, atol=1e-13)
