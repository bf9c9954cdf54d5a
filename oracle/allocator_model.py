"""Oracle model of the block manager (test infrastructure).

What the pages fix:

* The cache is split into fixed-size pages of ``block_size`` tokens (16 by
  default) taken from a list of free pages, so no contiguous region is ever
  searched for (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
  Batching原理与实践", sections 2.2 and 3.4 on ``--block-size``).
* Each request keeps a page table listing its physical pages in logical order
  (hihuo.com "vLLM 原理：PagedAttention 和 Continuous Batching", PagedAttention >
  工作原理 > 1. 页表管理).
* Allocation is on demand: a request of n tokens holds ceil(n / block_size)
  pages, and a new page is taken only when a token falls past the last page
  (same page, 工作原理 > 2. 按需分配, with the 500 -> 32 pages, 1000 -> 63 pages,
  501st token stays in page 32, 513th token opens page 33 examples).
* A finished request returns all its pages at once (same page, 工作原理 > 3.
  及时释放).
* The free pool is a FIFO queue initialised with every block ID, and an
  allocation takes ceil(n / block_size) blocks from its head
  (blog.gitcode.com "如何通过PagedAttention实现LLM高性能推理：实战指南",
  section 2.2, the sample data structure).
* Pages may be shared by several sequences (shared prompt prefixes, parallel
  sampling, beam search) without copying (hihuo.com page, 优势 > 3. 支持共享).

Readings where the pages are silent or disagree:

* allocation is all-or-nothing: when too few blocks are free the call fails
  with OOM and changes nothing (the sample would raise half-way and leak);
* freed blocks go to the tail of the free queue, in the sequence's logical
  order; a block is freed when its last holder lets go (reference count 0);
* ``fork`` gives a new sequence the same table as its parent and adds one
  reference to each block;
* writing a token into a block held by more than one sequence first moves the
  writer onto a fresh block (copy-on-write of the whole block); the other
  holders keep the old one, and the last holder writes in place.

Pins: the worked examples above (``tests/golden/allocator_examples.json``);
conservation (free + held = N; sum of reference counts = total table length);
freeing everything restores the pool; brute force over every operation sequence
of length <= 6 on a 4-block pool against these invariants.
"""

from __future__ import annotations

from collections import deque


class AllocError(Exception):
    """Base of the allocator model's failures."""


class OutOfBlocks(AllocError):
    """Not enough free blocks; the state is unchanged."""


class BadState(AllocError):
    """Unknown, duplicate or already-freed sequence; the state is unchanged."""


class BadArgument(AllocError):
    """Argument out of range; the state is unchanged."""


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise BadArgument("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BadArgument("initial free order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}

    # -- queries ---------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        return self.ref[block] if 0 <= block < self.num_blocks else -1

    def free_list(self) -> list[int]:
        return list(self.free)

    def block_table(self, seq: int) -> list[int]:
        self._need(seq)
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        self._need(seq)
        return self.lengths[seq]

    def slots(self, seq: int, start: int, count: int) -> list[int]:
        """Slot (block * B + offset) of positions start .. start+count-1."""
        self._need(seq)
        if start < 0 or count < 0 or start + count > self.lengths[seq]:
            raise BadArgument("positions outside the sequence")
        B = self.block_size
        t = self.tables[seq]
        return [t[p // B] * B + p % B for p in range(start, start + count)]

    # -- operations ------------------------------------------------------------
    def add(self, seq: int, num_tokens: int) -> list[int]:
        """Admit a new sequence holding ``num_tokens`` tokens."""
        if seq in self.tables:
            raise BadState(f"sequence {seq} already exists")
        if num_tokens < 0:
            raise BadArgument("negative token count")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        blocks = [self.free.popleft() for _ in range(need)]
        for b in blocks:
            self.ref[b] = 1
        self.tables[seq] = blocks
        self.lengths[seq] = num_tokens
        return list(blocks)

    def append(self, seq: int):
        """Reserve the slot of the sequence's next token.

        Returns (slot, cow) where cow is None or the (src, dst) block pair the
        caller must copy before writing.
        """
        self._need(seq)
        B = self.block_size
        pos = self.lengths[seq]
        table = self.tables[seq]
        j = pos // B
        cow = None
        if j == len(table):
            if not self.free:
                raise OutOfBlocks("no free block for a new page")
            nb = self.free.popleft()
            self.ref[nb] = 1
            table.append(nb)
        elif self.ref[table[j]] > 1:
            if not self.free:
                raise OutOfBlocks("no free block for copy-on-write")
            old = table[j]
            nb = self.free.popleft()
            self.ref[nb] = 1
            self.ref[old] -= 1
            table[j] = nb
            cow = (old, nb)
        self.lengths[seq] = pos + 1
        return table[j] * B + pos % B, cow

    def fork(self, parent: int, child: int) -> None:
        """New sequence ``child`` sharing every block of ``parent``."""
        self._need(parent)
        if child in self.tables:
            raise BadState(f"sequence {child} already exists")
        t = list(self.tables[parent])
        for b in t:
            self.ref[b] += 1
        self.tables[child] = t
        self.lengths[child] = self.lengths[parent]

    def release(self, seq: int) -> None:
        """Drop the sequence; blocks whose count reaches zero join the free tail."""
        self._need(seq)
        for b in self.tables[seq]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lengths[seq]

    # -- helpers ---------------------------------------------------------------
    def _need(self, seq: int) -> None:
        if seq not in self.tables:
            raise BadState(f"unknown sequence {seq}")

    def snapshot(self):
        """Everything observable, for bit-exact comparison."""
        return {
            "free": list(self.free),
            "ref": list(self.ref),
            "tables": {s: list(t) for s, t in sorted(self.tables.items())},
            "lengths": dict(sorted(self.lengths.items())),
        }
