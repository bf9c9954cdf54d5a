"""A device-resident paged KV cache together with its host block allocator.

Glue for callers (tests, benchmark, serving loops): tokens are placed by the
library allocator and written by the library's cache-write kernel; decode
metadata (block tables, context lengths) is exported by the allocator and
copied to the device.  No arithmetic of the method lives here.
"""

from __future__ import annotations

import numpy as np
import torch

from . import ops
from .allocator import BlockAllocator


def to_device(x, spec: ops.CacheSpec, device="cuda") -> torch.Tensor:
    """Storage-format numpy data (float32, or uint16 bf16 bits) -> device tensor."""
    if isinstance(x, torch.Tensor):
        return x.to(device)
    x = np.ascontiguousarray(x)
    if spec.dtype == "bf16":
        if x.dtype != np.uint16:
            raise ValueError("bf16 data must be given as uint16 bit patterns")
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    if x.dtype != np.float32:
        raise ValueError("f32 data must be float32")
    return torch.from_numpy(x).to(device)


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage-format numpy array (bf16 as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class PagedKVCache:
    def __init__(self, spec: ops.CacheSpec, initial_free_order=None, device="cuda",
                 fill: float | None = 0.0):
        self.spec = spec
        self.device = device
        self.k, self.v = ops.empty_cache(spec, device)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)
        self.alloc = BlockAllocator(spec.num_blocks, spec.block_size, initial_free_order)

    def write_tokens(self, k, v, slots, stream=None):
        """Write token t's k[t], v[t] ([T, Hkv, D]) at slots[t]."""
        kd = to_device(k, self.spec, self.device)
        vd = to_device(v, self.spec, self.device)
        sd = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        ops.reshape_and_cache(self.spec, kd, vd, sd, self.k, self.v, stream)

    def add_sequence(self, seq_id: int, k, v, stream=None):
        """Admit a sequence whose first len(k) tokens have keys k and values v."""
        n = int(k.shape[0])
        self.alloc.add(seq_id, n)
        if n:
            self.write_tokens(k, v, self.alloc.slots(seq_id, 0, n), stream)

    def metadata(self, seq_ids, max_blocks: int | None = None):
        """Device (block_tables [n, maxB] int32, context_lens [n] int32) and host copies."""
        seq_ids = list(seq_ids)
        if max_blocks is None:
            max_blocks = max([self.alloc.info(s)[1] for s in seq_ids] + [1])
        tables, ctx = self.alloc.batch_metadata(seq_ids, max_blocks)
        return (torch.from_numpy(tables).to(self.device), torch.from_numpy(ctx).to(self.device),
                tables, ctx)
