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

Prefix caching.  Requests whose prompts start with the same tokens (a shared
system prompt) can share those tokens' cache pages instead of computing them
again (hihuo.com page, 优势 > 3. 支持共享; ksqn.cn page, 3.4 and 5.2 item 4 on
``--enable-prefix-caching``).  The pages give no mechanism; the readings here:

* Only full blocks are shared.  A full block is identified by a chain hash over
  its tokens and its predecessor's hash, so equal hashes mean equal prefixes (up
  to 64-bit hash collisions): h_i = FNV-1a-64(le64(h_{i-1}) || le32(tokens of
  block i)), h_{-1} = 0, FNV-1a-64 as published by its authors (offset basis
  0xcbf29ce484222325, prime 0x100000001b3, xor then multiply per byte).
* ``add_prefix`` reuses the longest run of cached blocks from the start of the
  prompt, but never a block holding the prompt's last token (that token must be
  computed to produce the next one); the rest is allocated as usual.  A reused
  block with no holder leaves the free queue; all-or-nothing as ``add``.
* ``register`` is called once a sequence's blocks hold written K/V; it considers
  each full block once, in order: a block whose hash is not cached yet becomes
  the cached block for it; a duplicate of a cached hash stays uncached.
* A cached block whose last holder lets go joins the free queue's tail like any
  other block and stays findable; it is evicted (its hash forgotten) only when
  an allocation takes it from the head of the queue.  The FIFO queue is thereby
  least-recently-freed-first.

Swapping.  A suspended request's pages can be moved to CPU memory and brought
back later instead of being recomputed (hihuo.com page, Preemption（抢占）: the
two modes Recompute and Swap; ksqn.cn page, 3.4 on ``--swap-space``).  Readings:
a host pool of fixed-size blocks with its own FIFO free queue; ``swap_out`` is
all-or-nothing, gives the sequence one host block per table entry (in logical
order, taken from the host queue's head), and drops its device references as
``release`` would (a shared block stays for its other holders); ``swap_in``
takes fresh device blocks from the queue's head and returns the host blocks to
the host queue's tail in logical order.  A swapped sequence keeps its length and
prefix-cache progress; anything but ``swap_in`` or ``release`` on it is BadState.

Prefix-cache pins: published FNV-1a-64 test vectors; a hand-worked run on a
six-block pool (tests/test_prefix_cache.py); content safety over random runs
(every reused block holds exactly the tokens the new prompt has at that place).
"""

from __future__ import annotations

from collections import deque


FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64 bits: for each byte, xor it in, then multiply by the prime."""
    h = FNV64_OFFSET
    for byte in data:
        h = ((h ^ byte) * FNV64_PRIME) & MASK64
    return h


def chain_hash(parent: int, block_tokens) -> int:
    """Identity of a full block: its tokens after its predecessor's identity."""
    data = parent.to_bytes(8, "little") + b"".join(
        (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in block_tokens)
    return fnv1a64(data)


class AllocError(Exception):
    """Base of the allocator model's failures."""


class OutOfBlocks(AllocError):
    """Not enough free blocks; the state is unchanged."""


class BadState(AllocError):
    """Unknown, duplicate or already-freed sequence; the state is unchanged."""


class BadArgument(AllocError):
    """Argument out of range; the state is unchanged."""


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None,
                 num_host_blocks: int = 0):
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
        # prefix cache: chain hash -> block, block -> chain hash, and per sequence
        # (leading full blocks already considered, chain hash after them)
        self.cached: dict[int, int] = {}
        self.block_hash: dict[int, int] = {}
        self.progress: dict[int, tuple[int, int]] = {}
        self.lookups = 0
        self.hits = 0
        self.host_free = deque(range(num_host_blocks))
        self.swapped: dict[int, list[int]] = {}   # sequence -> host blocks, logical order

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
        if seq in self.tables or seq in self.swapped:
            raise BadState(f"sequence {seq} already exists")
        if num_tokens < 0:
            raise BadArgument("negative token count")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        blocks = [self._take() for _ in range(need)]
        self.tables[seq] = blocks
        self.lengths[seq] = num_tokens
        self.progress[seq] = (0, 0)
        return list(blocks)

    def add_prefix(self, seq: int, tokens) -> int:
        """Admit a new sequence whose prompt is ``tokens``, reusing cached blocks
        for the longest cached run of its leading full blocks.  Returns the number
        of prompt tokens whose K/V are already in the cache."""
        if seq in self.tables or seq in self.swapped:
            raise BadState(f"sequence {seq} already exists")
        tokens = [int(t) for t in tokens]
        n, B = len(tokens), self.block_size
        eligible = (n - 1) // B if n > 0 else 0   # never the block of the last token
        hits, h = [], 0          # h: chain key after the reused blocks
        for i in range(eligible):
            hi = chain_hash(h, tokens[i * B:(i + 1) * B])
            if hi not in self.cached:
                break
            hits.append(self.cached[hi])
            h = hi
        need = -(-n // B) - len(hits)
        idle = sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free) - idle:
            raise OutOfBlocks(f"need {need} blocks, {len(self.free) - idle} free")
        self.lookups += eligible
        self.hits += len(hits)
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        blocks = hits + [self._take() for _ in range(need)]
        self.tables[seq] = blocks
        self.lengths[seq] = n
        self.progress[seq] = (len(hits), h)
        return len(hits) * B

    def register(self, seq: int, tokens) -> None:
        """Offer the sequence's full blocks covered by ``tokens`` (its first
        len(tokens) tokens, K/V written) to the prefix cache, each block once."""
        self._need(seq)
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.lengths[seq]:
            raise BadArgument("more tokens than the sequence holds")
        B = self.block_size
        done, h = self.progress[seq]
        table = self.tables[seq]
        for i in range(done, len(tokens) // B):
            h = chain_hash(h, tokens[i * B:(i + 1) * B])
            b = table[i]
            if b not in self.block_hash and h not in self.cached:
                self.cached[h] = b
                self.block_hash[b] = h
            done = i + 1
        self.progress[seq] = (done, h)

    def _take(self) -> int:
        """The head of the free queue for a new use; a cached block is evicted."""
        b = self.free.popleft()
        if b in self.block_hash:
            del self.cached[self.block_hash.pop(b)]
        self.ref[b] = 1
        return b

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
            nb = self._take()
            table.append(nb)
        elif self.ref[table[j]] > 1:
            if not self.free:
                raise OutOfBlocks("no free block for copy-on-write")
            old = table[j]
            nb = self._take()
            self.ref[old] -= 1
            table[j] = nb
            cow = (old, nb)
        self.lengths[seq] = pos + 1
        return table[j] * B + pos % B, cow

    def fork(self, parent: int, child: int) -> None:
        """New sequence ``child`` sharing every block of ``parent``."""
        self._need(parent)
        if child in self.tables or child in self.swapped:
            raise BadState(f"sequence {child} already exists")
        t = list(self.tables[parent])
        for b in t:
            self.ref[b] += 1
        self.tables[child] = t
        self.lengths[child] = self.lengths[parent]
        self.progress[child] = self.progress[parent]

    def swap_out(self, seq: int) -> list[tuple[int, int]]:
        """Move the sequence to host blocks; returns (device block, host block) pairs
        to copy, in logical order."""
        self._need(seq)
        table = self.tables[seq]
        if len(table) > len(self.host_free):
            raise OutOfBlocks(f"need {len(table)} host blocks, {len(self.host_free)} free")
        pairs = [(b, self.host_free.popleft()) for b in table]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        self.swapped[seq] = [h for _, h in pairs]
        del self.tables[seq]
        return pairs

    def swap_in(self, seq: int) -> list[tuple[int, int]]:
        """Bring a swapped sequence back to fresh device blocks; returns (host block,
        device block) pairs to copy, in logical order."""
        if seq not in self.swapped:
            raise BadState(f"sequence {seq} is not swapped out")
        host = self.swapped[seq]
        if len(host) > len(self.free):
            raise OutOfBlocks(f"need {len(host)} blocks, {len(self.free)} free")
        blocks = [self._take() for _ in host]
        self.host_free.extend(host)
        self.tables[seq] = blocks
        del self.swapped[seq]
        return list(zip(host, blocks))

    def release(self, seq: int) -> None:
        """Drop the sequence; blocks whose count reaches zero join the free tail."""
        if seq in self.swapped:
            self.host_free.extend(self.swapped.pop(seq))
            del self.lengths[seq]
            del self.progress[seq]
            return
        self._need(seq)
        for b in self.tables[seq]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lengths[seq]
        del self.progress[seq]

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
            "cached": dict(sorted(self.block_hash.items())),
            "host_free": list(self.host_free),
            "swapped": {s: list(t) for s, t in sorted(self.swapped.items())},
        }
