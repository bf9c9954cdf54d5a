"""Swap preemption in the oracle (CPU): a hand-worked run with a shared block and a
host pool too small for a second swap, a data round trip through different
device blocks that must gather back unchanged, and pool invariants over random runs."""

import numpy as np
import pytest

from oracle.allocator_model import AllocatorModel, BadState, OutOfBlocks
from oracle.cache import reshape_and_cache, swap_blocks
from oracle.layout import CacheLayout
from workloads import gen


def test_hand_worked_run():
    m = AllocatorModel(6, 4, num_host_blocks=4)
    assert m.add(0, 10) == [0, 1, 2]
    m.fork(0, 1)
    assert m.swap_out(0) == [(0, 0), (1, 1), (2, 2)]
    assert [m.refcount(b) for b in range(6)] == [1, 1, 1, 0, 0, 0]   # sequence 1 still holds them
    assert m.free_list() == [3, 4, 5] and m.snapshot()["host_free"] == [3]
    before = m.snapshot()
    with pytest.raises(OutOfBlocks):                  # three host blocks needed, one free
        m.swap_out(1)
    assert m.snapshot() == before
    for op in (lambda: m.append(0), lambda: m.fork(0, 5), lambda: m.slots(0, 0, 1),
               lambda: m.swap_out(0), lambda: m.add(0, 1), lambda: m.swap_in(1)):
        with pytest.raises(BadState):
            op()
    m.release(1)
    assert m.free_list() == [3, 4, 5, 0, 1, 2]
    assert m.swap_in(0) == [(0, 3), (1, 4), (2, 5)]
    assert m.snapshot()["host_free"] == [3, 0, 1, 2] and m.length(0) == 10
    assert m.block_table(0) == [3, 4, 5] and m.free_list() == [0, 1, 2]
    assert m.swap_out(0) == [(3, 3), (4, 0), (5, 1)]
    m.release(0)                                      # a swapped sequence frees its host blocks
    assert m.snapshot()["host_free"] == [2, 3, 0, 1] and not m.swapped


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_data_round_trip_through_other_blocks(dtype):
    Hkv, D, B, N, H = 2, 64, 16, 12, 8
    dev, host = CacheLayout(N, Hkv, B, D, dtype), CacheLayout(H, Hkv, B, D, dtype)
    kc, vc = dev.empty_cache(0), dev.empty_cache(0)
    hk, hv = host.empty_cache(0), host.empty_cache(0)
    m = AllocatorModel(N, B, gen.pool_permutation(5, N), num_host_blocks=H)
    L = 37
    m.add(0, L)
    K, V = gen.seq_kv(5, 0, L, Hkv, D, dtype)
    reshape_and_cache(dev, K, V, m.slots(0, 0, L), kc, vc)
    swap_blocks(dev, kc, vc, host, hk, hv, m.swap_out(0))
    m.add(1, 60)                                      # another sequence overwrites the freed blocks
    K1, V1 = gen.seq_kv(6, 1, 60, Hkv, D, dtype)
    reshape_and_cache(dev, K1, V1, m.slots(1, 0, 60), kc, vc)
    m.release(1)
    swap_blocks(host, hk, hv, dev, kc, vc, m.swap_in(0))
    Kg, Vg = dev.gather(kc, vc, np.asarray(m.block_table(0)), L)
    assert np.array_equal(Kg, K) and np.array_equal(Vg, V)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_pool_invariants_random_runs(seed):
    rng = gen.stream(seed, 5)
    N, H = 16, 10
    m = AllocatorModel(N, 2, rng.permutation(N), num_host_blocks=H)
    swaps = 0
    for _ in range(500):
        op = int(rng.integers(0, 6))
        s = int(rng.integers(0, 6))
        try:
            if op == 0:
                m.add(s, int(rng.integers(0, 9)))
            elif op == 1:
                m.append(s)
            elif op == 2:
                m.fork(s, int(rng.integers(0, 6)))
            elif op == 3:
                m.swap_out(s)
                swaps += 1
            elif op == 4:
                m.swap_in(s)
            else:
                m.release(s)
        except (OutOfBlocks, BadState):
            pass
        held = {b for t in m.tables.values() for b in t}
        assert len(held) + m.num_free() == N
        assert sum(m.ref) == sum(len(t) for t in m.tables.values())
        on_host = [h for t in m.swapped.values() for h in t]
        assert len(on_host) == len(set(on_host)) and len(on_host) + len(m.host_free) == H
        assert set(m.lengths) == set(m.tables) | set(m.swapped)
        for s2, t in m.swapped.items():
            assert len(t) == -(-m.lengths[s2] // 2)
    assert swaps > 0
