"""Pins of the oracle cache writes and the allocator model (CPU only)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import allocator_model as am
from oracle.cache import copy_blocks, reshape_and_cache
from oracle.layout import CacheLayout
from workloads import gen


# ----------------------------------------------------------------------------- cache writes
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reshape_and_cache_writes_only_its_slots(dtype):
    lay = CacheLayout(8, 2, 32, 64, dtype)
    rng = gen.stream(3, 3)
    kc = gen.draw_values(rng, lay.cache_elems, dtype)
    vc = gen.draw_values(rng, lay.cache_elems, dtype)
    k0, v0 = kc.copy(), vc.copy()
    T = 9
    k = gen.draw_values(rng, (T, 2, 64), dtype)
    v = gen.draw_values(rng, (T, 2, 64), dtype)
    slots = np.array([5, -1, 33, 255, 0, -1, 100, 101, 31], dtype=np.int64)
    reshape_and_cache(lay, k, v, slots, kc, vc)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        K, V = lay.gather(kc, vc, [s // 32], 32)
        assert np.array_equal(K[s % 32], k[t]) and np.array_equal(V[s % 32], v[t])
    # every element that no slot covers keeps its old bits
    mark_k = lay.empty_cache()
    mark_v = lay.empty_cache()
    ones = np.ones((2, 64), dtype=mark_k.dtype)
    for s in slots[slots >= 0]:
        lay.write_token(mark_k, mark_v, s // 32, s % 32, ones, ones)
    assert mark_k.sum() == 7 * 2 * 64 and mark_v.sum() == 7 * 2 * 64
    assert np.array_equal(kc[mark_k == 0], k0[mark_k == 0])
    assert np.array_equal(vc[mark_v == 0], v0[mark_v == 0])


def test_copy_blocks_copies_whole_blocks():
    lay = CacheLayout(6, 2, 16, 64, "bf16")
    rng = gen.stream(3, 4)
    kc = gen.draw_values(rng, lay.cache_elems, "bf16")
    vc = gen.draw_values(rng, lay.cache_elems, "bf16")
    k0, v0 = kc.copy(), vc.copy()
    copy_blocks(lay, kc, vc, [[1, 4], [2, 0]])
    for src, dst in [(1, 4), (2, 0)]:
        a = lay.gather(kc, vc, [dst], 16)
        b = lay.gather(k0, v0, [src], 16)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for keep in (1, 2, 3, 5):
        a = lay.gather(kc, vc, [keep], 16)
        b = lay.gather(k0, v0, [keep], 16)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- allocator pages' examples
@pytest.fixture(scope="module")
def examples(golden_dir):
    with open(os.path.join(golden_dir, "allocator_examples.json")) as f:
        return json.load(f)


def test_pages_for_tokens(examples):
    ex = examples["pages_for_tokens"]
    for n, pages in ex["cases"]:
        m = am.AllocatorModel(200, ex["block_size"])
        assert len(m.add(0, n)) == pages


def test_on_demand_growth(examples):
    ex = examples["on_demand_growth"]
    B = ex["block_size"]
    m = am.AllocatorModel(64, B)
    m.add(7, ex["start_tokens"])
    assert len(m.block_table(7)) == ex["start_pages"]
    slot, cow = m.append(7)                              # token 501
    assert cow is None
    assert m.block_table(7).index(slot // B) + 1 == ex["token_501_page"]
    while m.length(7) < 512:
        m.append(7)
    assert len(m.block_table(7)) == ex["pages_after_512_tokens"]
    slot, _ = m.append(7)                                # token 513
    assert len(m.block_table(7)) == ex["token_513_page"]
    assert m.block_table(7).index(slot // B) + 1 == ex["token_513_page"]
    assert slot % B == 0


def test_preallocation_waste_vs_paging(examples):
    ex = examples["preallocation_waste"]
    waste = (ex["reserved"] - ex["used"]) / ex["reserved"]
    assert round(100 * waste) == ex["waste_percent_rounded"]
    # the same request under paging wastes only the unused tail of its last page
    m = am.AllocatorModel(512, 16)
    held = len(m.add(0, ex["used"])) * 16
    assert held - ex["used"] < 16


def test_fifo_sample(examples):
    ex = examples["fifo_sample"]
    m = am.AllocatorModel(ex["num_blocks"], ex["block_size"])
    for (seq, n), want in zip(ex["requests"], ex["expected_tables"]):
        assert m.add(seq, n) == want


def test_release_reuse(examples):
    ex = examples["release_reuse"]
    m = am.AllocatorModel(ex["num_blocks"], ex["block_size"])
    for step in ex["steps"]:
        if step[0] == "add":
            m.add(step[1], step[2])
        else:
            m.release(step[1])
    assert m.block_table(12) == ex["expected_table_12"]
    assert m.free_list() == ex["expected_free_after"]


# ----------------------------------------------------------------------------- allocator semantics
def test_oom_leaves_state_unchanged():
    m = am.AllocatorModel(5, 16)
    m.add(0, 40)                                         # 3 blocks
    snap = m.snapshot()
    with pytest.raises(am.OutOfBlocks):
        m.add(1, 33)                                     # needs 3, 2 free
    assert m.snapshot() == snap
    m.add(1, 16)                                         # 1 block, 1 left
    for _ in range(16):
        m.append(1)                                      # the first opens the last block
    assert m.length(1) == 32 and m.num_free() == 0
    snap = m.snapshot()
    with pytest.raises(am.OutOfBlocks):
        m.append(1)                                      # the 33rd token needs a block
    assert m.snapshot() == snap
    with pytest.raises(am.BadState):
        m.add(0, 1)
    with pytest.raises(am.BadState):
        m.release(99)
    with pytest.raises(am.BadState):
        m.fork(99, 5)
    with pytest.raises(am.BadState):
        m.fork(0, 1)
    with pytest.raises(am.BadArgument):
        m.slots(0, 30, 20)


def test_fork_and_copy_on_write():
    B = 16
    m = am.AllocatorModel(10, B)
    m.add(0, 20)                                         # blocks 0, 1 (block 1 partial)
    m.fork(0, 1)
    m.fork(0, 2)
    assert m.refcount(0) == 3 and m.refcount(1) == 3
    slot, cow = m.append(1)                              # writes into shared partial block 1
    assert cow == (1, 2) and slot == 2 * B + 4
    assert m.block_table(1) == [0, 2] and m.refcount(1) == 2 and m.refcount(2) == 1
    slot, cow = m.append(2)
    assert cow == (1, 3) and m.refcount(1) == 1
    slot, cow = m.append(0)                              # last holder writes in place
    assert cow is None and slot == 1 * B + 4
    m.release(1)
    assert m.refcount(0) == 2 and m.free_list()[-1] == 2


def _check_invariants(m):
    held = {b for t in m.tables.values() for b in t}
    assert len(m.free) + len(held) == m.num_blocks
    assert len(set(m.free)) == len(m.free) and not (set(m.free) & held)
    assert sum(m.ref) == sum(len(t) for t in m.tables.values())
    for b in range(m.num_blocks):
        assert m.ref[b] == sum(t.count(b) for t in m.tables.values())
    for s, t in m.tables.items():
        assert len(t) == -(-m.lengths[s] // m.block_size)
        assert len(set(t)) == len(t)


def test_brute_force_all_short_op_sequences():
    """Every sequence of <= 6 operations on a 4-block pool of 2-token blocks keeps
    the invariants, and freeing everything at the end restores the whole pool."""
    ops = [("add", 0, 1), ("add", 1, 3), ("append", 0), ("append", 1),
           ("fork", 0, 2), ("release", 0), ("release", 1), ("append", 2)]
    count = 0
    for n in range(1, 7):
        for seqops in itertools.product(ops, repeat=n):
            m = am.AllocatorModel(4, 2)
            for op in seqops:
                snap = m.snapshot()
                try:
                    getattr(m, op[0])(*op[1:])
                except am.AllocError:
                    assert m.snapshot() == snap
                _check_invariants(m)
            for s in list(m.tables):
                m.release(s)
            assert sorted(m.free) == [0, 1, 2, 3] and not any(m.ref)
            count += 1
    assert count == sum(len(ops) ** n for n in range(1, 7))


def test_shared_prefix_workload_counts():
    """64 sequences sharing a 1024+B/2 token prefix: every prefix block is held 64
    times, and the first append of 63 of them copies the shared partial block."""
    for B in (16, 32):
        m = am.AllocatorModel(20000 if B == 16 else 10000, B)
        m.add(0, 1024 + B // 2)
        for c in range(1, 64):
            m.fork(0, c)
        assert all(m.refcount(b) == 64 for b in m.block_table(0))
        cows = [m.append(s)[1] for s in range(64)]
        assert sum(c is not None for c in cows) == 63
        assert cows[63] is None
        _check_invariants(m)
