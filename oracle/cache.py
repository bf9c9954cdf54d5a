"""Oracle cache writes: scatter of new tokens and whole-block copy (test infrastructure).

* New tokens' keys and values are written into the slots of their blocks
  (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous Batching原理与实践",
  section 2.2, the scatter that pairs with the gather; hihuo.com "vLLM 原理：
  PagedAttention 和 Continuous Batching", section 调度流程, step 4 which updates
  the cache after each forward step).  A slot is ``block * B + offset``; slot -1
  means "no write".  The bits are copied unchanged; every other byte of the
  cache keeps its value.
* Blocks shared by several sequences are mapped without copying (hihuo.com page,
  PagedAttention > 优势 > 3. 支持共享).  When one sharer must write into a shared
  block, the whole block is first copied to a fresh block (copy-on-write; the
  pages name sharing but not this mechanism, so its form is this library's
  reading).  ``copy_blocks`` copies every byte of the K and V data of ``src``
  onto ``dst``, pair by pair in the order given.

* Preemption by swapping moves a suspended request's K/V blocks to CPU memory
  and back (hihuo.com page, Preemption（抢占）: Swap; ksqn.cn page, 3.4 on
  ``--swap-space``).  ``swap_blocks`` copies whole blocks from one pool to another
  pool of the same block geometry (device to host, or back), pair by pair.

Pins: write-then-gather returns the written tokens; bytes of untouched slots are
unchanged; slot -1 writes nothing; a copied block reads back equal to its source;
a sequence swapped out and in through different blocks gathers back unchanged.
"""

from __future__ import annotations

import numpy as np

from .layout import CacheLayout


def reshape_and_cache(layout: CacheLayout, k, v, slot_mapping, k_cache, v_cache) -> None:
    """Write token t's k[t], v[t] ([Hkv, D], storage format) at slot_mapping[t]."""
    B = layout.block_size
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), B)
        layout.write_token(k_cache, v_cache, block, offset, k[t], v[t])


def copy_blocks(layout: CacheLayout, k_cache, v_cache, pairs) -> None:
    """For each (src, dst) pair, in order, copy block src's K and V bytes onto dst."""
    n = layout.block_elems()
    kb = k_cache.reshape(layout.num_blocks, n)
    vb = v_cache.reshape(layout.num_blocks, n)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        kb[dst] = kb[src]
        vb[dst] = vb[src]


def swap_blocks(src_layout: CacheLayout, src_k, src_v, dst_layout: CacheLayout, dst_k, dst_v,
                pairs) -> None:
    """For each (src, dst) pair, copy block src of one pool onto block dst of another
    pool with the same block geometry."""
    n = src_layout.block_elems()
    assert dst_layout.block_elems() == n
    sk = src_k.reshape(src_layout.num_blocks, n)
    sv = src_v.reshape(src_layout.num_blocks, n)
    dk = dst_k.reshape(dst_layout.num_blocks, n)
    dv = dst_v.reshape(dst_layout.num_blocks, n)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        dk[dst] = sk[src]
        dv[dst] = sv[src]
