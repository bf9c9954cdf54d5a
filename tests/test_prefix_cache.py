"""Prefix caching in the allocator model (CPU): published FNV-1a-64 test vectors,
a hand-worked run on a six-block pool, and content safety over random runs (a
reused block always holds exactly the tokens the new prompt has at that place)."""

import numpy as np
import pytest

from oracle.allocator_model import AllocatorModel, OutOfBlocks, chain_hash, fnv1a64
from workloads import gen


def test_fnv1a64_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_chain_hash_depends_on_order_and_parent():
    a = chain_hash(0, [1, 2, 3, 4])
    assert a == fnv1a64(bytes(8) + b"".join(t.to_bytes(4, "little") for t in (1, 2, 3, 4)))
    assert chain_hash(0, [2, 1, 3, 4]) != a
    assert chain_hash(a, [5, 6, 7, 8]) != chain_hash(0, [5, 6, 7, 8])


def test_hand_worked_run():
    m = AllocatorModel(6, 4)
    h0 = chain_hash(0, [1, 2, 3, 4])
    h1 = chain_hash(h0, [5, 6, 7, 8])
    A = list(range(1, 11))
    assert m.add_prefix(0, A) == 0 and m.block_table(0) == [0, 1, 2]
    m.register(0, A)                                  # blocks 0 and 1 are full
    assert m.snapshot()["cached"] == {0: h0, 1: h1}
    B = list(range(1, 9)) + [99, 100]
    assert m.add_prefix(1, B) == 8 and m.block_table(1) == [0, 1, 3]
    assert [m.refcount(b) for b in range(6)] == [2, 2, 1, 1, 0, 0] and m.free_list() == [4, 5]
    m.release(0)
    m.release(1)
    assert m.free_list() == [4, 5, 2, 0, 1, 3]        # cached blocks stay findable in the queue
    C = [1, 2, 3, 4, 7, 7, 7, 7, 5]
    assert m.add_prefix(2, C) == 4                    # block 0 hits, block 1 misses
    assert m.block_table(2) == [0, 4, 5] and m.free_list() == [2, 1, 3]
    assert m.add(3, 8) == [2, 1]                      # taking block 1 evicts its hash
    assert m.snapshot()["cached"] == {0: h0}
    before = m.snapshot()
    with pytest.raises(OutOfBlocks):                  # block 0 hits, two more needed, one free
        m.add_prefix(4, list(range(1, 10)))
    assert m.snapshot() == before
    assert m.add_prefix(5, [1, 2, 3, 4]) == 0         # the block of the last token is never reused
    assert m.block_table(5) == [3]
    assert (m.lookups, m.hits) == (2 + 2 + 2, 0 + 2 + 1)


def test_duplicate_content_stays_uncached_and_each_block_is_considered_once():
    m = AllocatorModel(8, 2)
    assert m.add(0, 4) == [0, 1] and m.add(1, 4) == [2, 3]
    m.register(0, [1, 2, 3, 4])
    m.register(1, [1, 2, 3, 4])                       # same content: sequence 0's blocks stay cached
    assert sorted(m.snapshot()["cached"]) == [0, 1]
    m.release(0)
    assert m.free_list() == [4, 5, 6, 7, 0, 1]
    assert m.add(2, 12) == [4, 5, 6, 7, 0, 1]         # taking 0 and 1 evicts both hashes
    assert m.snapshot()["cached"] == {}
    m.register(1, [1, 2, 3, 4])                       # blocks 2, 3 were considered already
    assert m.snapshot()["cached"] == {}


def _content_safety_run(seed, steps=400):
    rng = gen.stream(seed, 3)
    B, N = 4, 24
    m = AllocatorModel(N, B, rng.permutation(N))
    toks, content = {}, {}                            # seq -> tokens; block -> tokens written
    nxt = 0
    for _ in range(steps):
        op = rng.integers(0, 5)
        live = sorted(toks)
        if op == 0 or not live:
            # prompts from a 3-token alphabet with a few shared openings -> real reuse
            opening = [[1, 2, 1, 2, 3, 3, 1, 2], [2, 2, 2, 2, 1, 1, 1, 1], []][rng.integers(0, 3)]
            tail = rng.integers(1, 4, rng.integers(1, 12)).tolist()
            t = opening + tail
            try:
                cached = m.add_prefix(nxt, t)
            except OutOfBlocks:
                continue
            table = m.block_table(nxt)
            for i in range(cached // B):              # reused blocks hold exactly our tokens
                assert content[table[i]] == t[i * B:(i + 1) * B]
            for p in range(cached, len(t)):           # the rest is written now
                content.setdefault(table[p // B], [None] * B)[p % B] = t[p]
            toks[nxt] = t
            nxt += 1
        elif op == 1:
            s = live[rng.integers(0, len(live))]
            tok = int(rng.integers(1, 4))
            try:
                slot, cow = m.append(s)
            except OutOfBlocks:
                continue
            if cow is not None:
                content[cow[1]] = list(content[cow[0]])
            b, off = divmod(slot, B)
            content.setdefault(b, [None] * B)
            if off == 0:
                content[b] = [None] * B
            content[b][off] = tok
            toks[s].append(tok)
        elif op == 2:
            s = live[rng.integers(0, len(live))]
            m.register(s, toks[s][:rng.integers(0, len(toks[s]) + 1)])
        elif op == 3:
            s = live[rng.integers(0, len(live))]
            m.release(s)
            del toks[s]
        else:
            s = live[rng.integers(0, len(live))]
            m.fork(s, nxt)
            toks[nxt] = list(toks[s])
            nxt += 1
        # invariants
        held = {b for t in m.tables.values() for b in t}
        assert len(held) + m.num_free() == N and held.isdisjoint(m.free_list())
        assert sum(m.ref) == sum(len(t) for t in m.tables.values())
        for b, h in m.block_hash.items():
            assert m.cached[h] == b and len(content[b]) == B and None not in content[b]
    return m


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_content_safety_random_runs(seed):
    m = _content_safety_run(seed)
    assert m.hits > 0                                  # the runs did exercise reuse


def test_progress_after_a_partial_hit_continues_the_chain():
    """A prompt whose first block hits and second misses registers its second block
    under the key chained from the first (the reused one), not from the miss."""
    m = AllocatorModel(8, 2)
    m.add_prefix(0, [1, 2, 3])
    m.register(0, [1, 2, 3])
    assert m.add_prefix(1, [1, 2, 5, 6, 7]) == 2
    m.register(1, [1, 2, 5, 6, 7])
    h0 = chain_hash(0, [1, 2])
    assert m.snapshot()["cached"][m.block_table(1)[1]] == chain_hash(h0, [5, 6])
