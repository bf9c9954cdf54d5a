"""Pins of the oracle's cache-layout reader/writer (CPU only)."""

import os

import numpy as np
import pytest

from oracle.layout import CacheLayout, to_float64
from workloads import gen


def _golden_rows(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "layout_offsets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            shape, coord, offs = (p.split() for p in line.split("|"))
            rows.append((shape[0], *map(int, shape[1:]), *map(int, coord), *map(int, offs)))
    return rows


def _index_cache(layout):
    """A cache whose element at flat offset n holds the value n."""
    n = layout.cache_elems
    if layout.dtype == "f32":
        return np.arange(n, dtype=np.float32)
    assert n < 65536
    return np.arange(n, dtype=np.uint16)


def test_hand_derived_offsets(golden_dir):
    rows = _golden_rows(golden_dir)
    assert len(rows) >= 6
    for dtype, N, H, B, D, b, h, o, d, k_off, v_off in rows:
        lay = CacheLayout(N, H, B, D, dtype)
        kc, vc = _index_cache(lay), _index_cache(lay)
        K, V = lay.gather(kc, vc, [b], B)
        assert int(K[o, h, d]) == k_off, (dtype, b, h, o, d)
        assert int(V[o, h, d]) == v_off, (dtype, b, h, o, d)


@pytest.mark.parametrize("dtype,N,H,B,D", [("bf16", 3, 2, 16, 64), ("bf16", 2, 3, 32, 128),
                                          ("f32", 2, 2, 16, 64), ("f32", 2, 1, 48, 128)])
def test_offsets_are_a_bijection(dtype, N, H, B, D):
    lay = CacheLayout(N, H, B, D, dtype)
    kc, vc = _index_cache(lay).astype(np.int64), _index_cache(lay).astype(np.int64)
    K, V = lay.gather(kc, vc, list(range(N)), N * B)
    for arr in (K, V):
        flat = np.sort(arr.reshape(-1))
        assert np.array_equal(flat, np.arange(lay.cache_elems))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sixteen_byte_groups(dtype):
    """Each 16-byte group holds what the contract says: K = X dims of one token;
    V = 4 consecutive tokens of E dims spaced 16 apart, all in one block/head."""
    N, H, B, D = 2, 2, 32, 128
    lay = CacheLayout(N, H, B, D, dtype)
    X, E = lay.X, lay.E
    kc = np.arange(lay.cache_elems, dtype=np.int64)
    vc = kc.copy()
    K, V = lay.gather(kc, vc, list(range(N)), N * B)   # logical (token, head, dim) -> offset
    inv_k = np.empty((lay.cache_elems, 3), dtype=np.int64)
    inv_v = np.empty((lay.cache_elems, 3), dtype=np.int64)
    t, h, d = np.meshgrid(np.arange(N * B), np.arange(H), np.arange(D), indexing="ij")
    inv_k[K.reshape(-1)] = np.stack([t.reshape(-1), h.reshape(-1), d.reshape(-1)], 1)
    inv_v[V.reshape(-1)] = np.stack([t.reshape(-1), h.reshape(-1), d.reshape(-1)], 1)
    for g in range(0, lay.cache_elems, X):
        kt, kh, kd = inv_k[g:g + X].T
        assert len(set(kt)) == 1 and len(set(kh)) == 1
        assert list(kd) == list(range(kd[0], kd[0] + X)) and kd[0] % X == 0
        vt, vh, vd = inv_v[g:g + X].T
        assert len(set(vh)) == 1 and len(set(vt // B)) == 1
        toks = vt.reshape(E, 4)
        dims = vd.reshape(E, 4)
        for e in range(E):
            assert list(toks[e]) == list(range(toks[e][0], toks[e][0] + 4)) and toks[e][0] % 4 == 0
            assert len(set(dims[e])) == 1
            assert dims[e][0] == dims[0][0] + 16 * e
        assert np.array_equal(toks, np.broadcast_to(toks[0], toks.shape))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_write_then_gather_round_trip(dtype):
    N, H, B, D = 6, 2, 32, 64
    lay = CacheLayout(N, H, B, D, dtype)
    kc, vc = lay.empty_cache(), lay.empty_cache()
    rng = gen.stream(123, 99)
    blocks = [4, 1, 5]
    L = 70
    K = gen.draw_values(rng, (L, H, D), dtype)
    V = gen.draw_values(rng, (L, H, D), dtype)
    for p in range(L):
        lay.write_token(kc, vc, blocks[p // B], p % B, K[p], V[p])
    K2, V2 = lay.gather(kc, vc, blocks, L)
    assert np.array_equal(K2, K) and np.array_equal(V2, V)
    # untouched blocks stay zero
    K0, V0 = lay.gather(kc, vc, [0, 2, 3], 3 * B)
    assert not K0.any() and not V0.any()


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = to_float64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and vals[3] == 0.0
    assert vals[4] == 3.140625                      # 0x4049: 1.5703125 * 2
    assert vals[5] == (2 - 2 ** -7) * 2.0 ** 127    # largest finite bf16
    assert vals[6] == 2.0 ** -133                   # smallest subnormal bf16
