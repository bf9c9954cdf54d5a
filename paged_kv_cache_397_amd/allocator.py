"""Python handle on the library's host block allocator (pa_alloc_* / pa_seq_*)."""

from __future__ import annotations

import ctypes

import numpy as np

from . import _native as N


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockAllocator:
    """FIFO free list, per-sequence block tables, reference counts, fork and
    copy-on-write; every call runs in libpagedkv's C++ allocator."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        self._lib = N.lib()
        h = ctypes.c_void_p()
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
        N.check(self._lib.pa_alloc_create(num_blocks, block_size,
                                          None if order is None else _ptr(order),
                                          ctypes.byref(h)), "pa_alloc_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    @classmethod
    def borrowed(cls, handle, num_blocks: int, block_size: int, owner) -> "BlockAllocator":
        """A handle on an allocator another object owns (a scheduler's); `owner` is
        kept alive with it, and closing it destroys nothing."""
        self = cls.__new__(cls)
        self._lib = N.lib()
        self._h = ctypes.c_void_p(handle)
        self._owner = owner
        self.num_blocks = num_blocks
        self.block_size = block_size
        return self

    def close(self):
        if self._h and getattr(self, "_owner", None) is None:
            self._lib.pa_alloc_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- queries --------------------------------------------------------------
    def num_free(self) -> int:
        return int(self._lib.pa_alloc_num_free(self._h))

    def num_seqs(self) -> int:
        return int(self._lib.pa_alloc_num_seqs(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_alloc_refcount(self._h, block))

    def free_list(self) -> list[int]:
        n = ctypes.c_int32()
        N.check(self._lib.pa_alloc_free_list(self._h, None, 0, ctypes.byref(n)), "free_list")
        out = np.empty(n.value, dtype=np.int32)
        N.check(self._lib.pa_alloc_free_list(self._h, _ptr(out), n.value, ctypes.byref(n)),
                "free_list")
        return out.tolist()

    def info(self, seq: int):
        nt, nb = ctypes.c_int32(), ctypes.c_int32()
        N.check(self._lib.pa_seq_info(self._h, seq, ctypes.byref(nt), ctypes.byref(nb)), "seq_info")
        return nt.value, nb.value

    def length(self, seq: int) -> int:
        return self.info(seq)[0]

    def block_table(self, seq: int) -> list[int]:
        _, nb = self.info(seq)
        out = np.empty(max(nb, 1), dtype=np.int32)
        N.check(self._lib.pa_seq_block_table(self._h, seq, _ptr(out), nb), "seq_block_table")
        return out[:nb].tolist()

    def slots(self, seq: int, start: int, count: int) -> np.ndarray:
        out = np.empty(max(count, 1), dtype=np.int64)
        N.check(self._lib.pa_seq_slots(self._h, seq, start, count, _ptr(out)), "seq_slots")
        return out[:count]

    def batch_metadata(self, seqs, max_blocks_per_seq: int, tables=None, ctx=None):
        """Block tables [n, max_blocks_per_seq] (padding -1) and context lengths [n],
        into `tables` / `ctx` when given (C-contiguous int32 of those shapes)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.shape[0]
        if tables is None:
            tables = np.empty((n, max_blocks_per_seq), dtype=np.int32)
        if ctx is None:
            ctx = np.empty(n, dtype=np.int32)
        if (tables.shape != (n, max_blocks_per_seq) or tables.dtype != np.int32 or
                not tables.flags.c_contiguous or ctx.shape != (n,) or ctx.dtype != np.int32):
            raise ValueError("tables / ctx do not match the batch")
        N.check(self._lib.pa_batch_metadata(self._h, _ptr(seqs), n, max_blocks_per_seq,
                                            _ptr(tables), _ptr(ctx)), "batch_metadata")
        return tables, ctx

    # -- operations -----------------------------------------------------------
    def add(self, seq: int, num_tokens: int) -> None:
        N.check(self._lib.pa_seq_add(self._h, seq, num_tokens), "seq_add")

    def append(self, seq: int):
        """Returns (slot, cow) with cow None or the (src, dst) block copy to do first."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        N.check(self._lib.pa_seq_append(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                        ctypes.byref(dst)), "seq_append")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seqs):
        """Append one token to each sequence in order.

        Returns (status, done, slots[n], cow_pairs[n, 2], new_blocks[n], new_cols[n]);
        entries past `done` are unspecified.  status is PA_OK, PA_ERR_OOM or PA_ERR_STATE.
        """
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.shape[0]
        slots = np.empty(n, dtype=np.int64)
        cows = np.empty((n, 2), dtype=np.int32)
        nb = np.empty(n, dtype=np.int32)
        nc = np.empty(n, dtype=np.int32)
        done = ctypes.c_int32()
        st = self._lib.pa_seq_append_batch(self._h, _ptr(seqs), n, _ptr(slots), _ptr(cows),
                                           _ptr(nb), _ptr(nc), ctypes.byref(done))
        if st not in (N.PA_OK, N.PA_ERR_OOM, N.PA_ERR_STATE):
            N.check(st, "seq_append_batch")
        return st, done.value, slots, cows, nb, nc

    def bind_append_batch(self, seqs, slots, cow_pairs, new_blocks, new_cols):
        """append_batch for a fixed list of sequences, with its outputs written into
        the given arrays (int64 [n], int32 [n, 2], int32 [n], int32 [n]; C-contiguous,
        e.g. views of a pinned staging buffer).  The arguments are converted once; the
        returned callable makes one library call per step and returns (status, done).
        The arrays must outlive the callable."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.shape[0]
        for arr, dt, shape in ((slots, np.int64, (n,)), (cow_pairs, np.int32, (n, 2)),
                               (new_blocks, np.int32, (n,)), (new_cols, np.int32, (n,))):
            if arr.dtype != dt or arr.shape != shape or not arr.flags.c_contiguous:
                raise ValueError(f"output array must be C-contiguous {np.dtype(dt).name} {shape}")
        done = ctypes.c_int32()
        fn = self._lib.pa_seq_append_batch
        args = (self._h, _ptr(seqs), n, _ptr(slots), _ptr(cow_pairs), _ptr(new_blocks),
                _ptr(new_cols), ctypes.byref(done))
        keep = (seqs, slots, cow_pairs, new_blocks, new_cols)

        def call():
            st = fn(*args)
            if st not in (N.PA_OK, N.PA_ERR_OOM, N.PA_ERR_STATE):
                N.check(st, "seq_append_batch")
            return st, done.value

        call.keep = keep  # the arrays the pointers refer to
        return call

    def fork(self, parent: int, child: int) -> None:
        N.check(self._lib.pa_seq_fork(self._h, parent, child), "seq_fork")

    def free(self, seq: int) -> None:
        N.check(self._lib.pa_seq_free(self._h, seq), "seq_free")

    # -- prefix cache ---------------------------------------------------------
    def add_prefix(self, seq: int, tokens) -> int:
        """Admit a prompt, reusing cached full blocks of its opening; returns the
        number of leading tokens whose K/V are already cached."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32()
        N.check(self._lib.pa_seq_add_prefix(self._h, seq, _ptr(t), t.shape[0], ctypes.byref(cached)),
                "seq_add_prefix")
        return cached.value

    def register(self, seq: int, tokens) -> None:
        """Offer the full blocks covered by the sequence's first len(tokens) tokens
        (their K/V written) to the prefix cache."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        N.check(self._lib.pa_seq_register_blocks(self._h, seq, _ptr(t), t.shape[0]),
                "seq_register_blocks")

    def prefix_stats(self):
        """(blocks looked up, blocks reused, blocks cached now)."""
        lk, ht, nc = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        N.check(self._lib.pa_alloc_prefix_stats(self._h, ctypes.byref(lk), ctypes.byref(ht),
                                                ctypes.byref(nc)), "alloc_prefix_stats")
        return lk.value, ht.value, nc.value

    def cached_blocks(self) -> dict[int, int]:
        """{block: key} for every cached block."""
        key = ctypes.c_uint64()
        out = {}
        for b in range(self.num_blocks):
            if self._lib.pa_alloc_block_cached(self._h, b, ctypes.byref(key)) == 1:
                out[b] = key.value
        return out

    # -- swapping -------------------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        N.check(self._lib.pa_alloc_set_host_pool(self._h, num_host_blocks), "alloc_set_host_pool")

    def num_free_host(self) -> int:
        return int(self._lib.pa_alloc_num_free_host(self._h))

    def host_free_list(self) -> list[int]:
        n = ctypes.c_int32()
        N.check(self._lib.pa_alloc_host_free_list(self._h, None, 0, ctypes.byref(n)), "host_free_list")
        out = np.empty(max(n.value, 1), dtype=np.int32)
        N.check(self._lib.pa_alloc_host_free_list(self._h, _ptr(out), n.value, ctypes.byref(n)),
                "host_free_list")
        return out[:n.value].tolist()

    def host_blocks(self, seq: int) -> list[int]:
        _, nb = self.info(seq)
        out = np.empty(max(nb, 1), dtype=np.int32)
        N.check(self._lib.pa_seq_host_blocks(self._h, seq, _ptr(out), nb), "seq_host_blocks")
        return out[:nb].tolist()

    def is_swapped(self, seq: int) -> bool:
        r = int(self._lib.pa_seq_is_swapped(self._h, seq))
        if r < 0:
            raise N.PagedKVError(N.PA_ERR_STATE, "seq_is_swapped")
        return bool(r)

    def _swap(self, fn: str, seq: int) -> np.ndarray:
        _, nb = self.info(seq)
        pairs = np.empty((max(nb, 1), 2), dtype=np.int32)
        n = ctypes.c_int32()
        N.check(getattr(self._lib, fn)(self._h, seq, _ptr(pairs), nb, ctypes.byref(n)), fn)
        return pairs[:n.value]

    def swap_out(self, seq: int) -> np.ndarray:
        """Move the sequence to host blocks; returns (device, host) block pairs [n, 2]."""
        return self._swap("pa_seq_swap_out", seq)

    def swap_in(self, seq: int) -> np.ndarray:
        """Bring the sequence back; returns (host, device) block pairs [n, 2]."""
        return self._swap("pa_seq_swap_in", seq)
