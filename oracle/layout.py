"""Oracle reader/writer of the physical KV-cache layout (test infrastructure).

The source pages fix only the logical picture: a sequence's keys and values are
cut into fixed-size blocks of tokens that may sit anywhere in one pool, and a
per-sequence table maps logical block j to its physical block
(ksqn.cn "大模型推理性能优化：PagedAttention与Continuous Batching原理与实践",
section 2.2; hihuo.com "vLLM 原理：PagedAttention 和 Continuous Batching",
section PagedAttention > 工作原理 > 1. 页表管理).  The byte layout inside a block
is this library's own contract, stated in ``include/pagedkv.h``:

* a block of B tokens is cut into B/TT tiles of TT = min(B, 16) tokens (a block
  of 8 tokens is one tile of 8);
* K tile   = [D/X][TT][X]             (X = 16 bytes / element size)
* V tile   = [D/(16E)][TT/4][16][E][4] (E = X/4): each 16-byte group holds four
  consecutive tokens of E head-dim positions spaced 16 apart;
* tiles are ordered block -> tile -> kv head (the Hkv heads' tiles of one tile
  slot of a block are adjacent).

This module expresses that contract as numpy reshapes/transposes of the flat
cache arrays (no index arithmetic is shared with the HIP code).  Values stay in
their storage format: ``float32`` for f32 caches, ``uint16`` bit patterns for
bf16 caches.  ``to_float64`` is the oracle's exact decoder.

Pins: the hand-derived offsets in ``tests/golden/layout_offsets.txt``; every
element lands at a distinct offset and the offsets cover the pool exactly; each
16-byte group holds the elements the header says it holds; write-then-read
returns the written tokens.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TILE = 16  # tokens per tile


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored data (bf16 bits -> high half of a float32)."""
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float64)
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class CacheLayout:
    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    dtype: str  # "f32" | "bf16"

    def __post_init__(self):
        if self.block_size != 8 and self.block_size % TILE:
            raise ValueError("block_size must be 8 or a multiple of 16")
        if self.head_dim % (TILE * self.E):
            raise ValueError("head_dim must be a multiple of 16*E")

    # -- derived sizes --------------------------------------------------------
    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def X(self) -> int:
        """Elements per 16-byte group."""
        return 16 // self.elem_bytes

    @property
    def E(self) -> int:
        """Head-dim positions per 16-byte V group (each with 4 tokens)."""
        return self.X // 4

    @property
    def tile_tokens(self) -> int:
        """Tokens per tile: 16, or 8 for a block of 8."""
        return min(self.block_size, TILE)

    @property
    def tiles_per_block(self) -> int:
        return self.block_size // self.tile_tokens

    @property
    def cache_elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim

    def empty_cache(self, fill=None) -> np.ndarray:
        c = np.zeros(self.cache_elems, dtype=storage_dtype(self.dtype))
        if fill is not None:
            c[...] = fill
        return c

    # -- views of the flat arrays ---------------------------------------------
    def _k6(self, k_cache):
        """K as [block, head, tile, d//X, token%TT, d%X] (stored tile-major)."""
        N, H, T, D, X, TT = (self.num_blocks, self.num_kv_heads, self.tiles_per_block,
                             self.head_dim, self.X, self.tile_tokens)
        return k_cache.reshape(N, T, H, D // X, TT, X).transpose(0, 2, 1, 3, 4, 5)

    def _v8(self, v_cache):
        """V as [block, head, tile, m, j, i, e, r]: token 4j+r of the tile, dim
        16E*m + 16e + i (stored tile-major)."""
        N, H, T, D, E, TT = (self.num_blocks, self.num_kv_heads, self.tiles_per_block,
                             self.head_dim, self.E, self.tile_tokens)
        return v_cache.reshape(N, T, H, D // (TILE * E), TT // 4, TILE, E, 4).transpose(
            0, 2, 1, 3, 4, 5, 6, 7)

    # -- reads ----------------------------------------------------------------
    def gather(self, k_cache, v_cache, blocks, length):
        """Keys and values of the first ``length`` tokens held by ``blocks``.

        Returns two [length, Hkv, D] arrays in storage format; only the listed
        blocks are read.
        """
        H, D = self.num_kv_heads, self.head_dim
        blocks = np.asarray(blocks, dtype=np.int64)
        nb = blocks.shape[0]
        k = self._k6(k_cache)[blocks]                     # [nb, H, T, D/X, 16, X]
        k = k.transpose(0, 2, 4, 1, 3, 5).reshape(nb * self.block_size, H, D)
        v = self._v8(v_cache)[blocks]                     # [nb, H, T, m, j, i, e, r]
        v = v.transpose(0, 2, 4, 7, 1, 3, 6, 5).reshape(nb * self.block_size, H, D)
        return k[:length].copy(), v[:length].copy()

    # -- writes ---------------------------------------------------------------
    def write_token(self, k_cache, v_cache, block, offset, k_tok, v_tok):
        """Store one token's [Hkv, D] key and value at (block, offset in block)."""
        H, D, X, E = self.num_kv_heads, self.head_dim, self.X, self.E
        t, o = divmod(int(offset), self.tile_tokens)
        self._k6(k_cache)[block, :, t, :, o, :] = np.asarray(k_tok).reshape(H, D // X, X)
        j, r = divmod(o, 4)
        vt = np.asarray(v_tok).reshape(H, D // (TILE * E), E, TILE).transpose(0, 1, 3, 2)
        self._v8(v_cache)[block, :, t, :, j, :, :, r] = vt

    def block_elems(self) -> int:
        """Elements one physical block holds in each of the K and V arrays."""
        return self.num_kv_heads * self.block_size * self.head_dim
