"""Plant plausible mistakes in copies of the oracle and check that the pins notice.

Each mutant is a small edit of the oracle's arithmetic (a wrong head index, a
dropped scale, swapped operands, a transposed layout read, a LIFO free list).
The pins used by the other CPU tests must reject every one of them.
"""

import math

import numpy as np
import torch

from oracle import allocator_model as am
from oracle.attention import decode_attention
from workloads import gen


def _sdpa(q, K, V, scale):
    G = q.shape[0] // K.shape[1]
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None].repeat_interleave(G, 1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()


def _mutant_head_mod(q, K, V, scale):
    Hq, Hkv = q.shape[0], K.shape[1]
    out = np.zeros_like(q)
    for j in range(Hq):
        h = j % Hkv                                   # wrong: should be j // G
        s = scale * (K[:, h] @ q[j])
        p = np.exp(s - s.max())
        out[j] = p @ V[:, h] / p.sum()
    return out


def _mutant_no_scale(q, K, V, scale):
    return decode_attention(q, K, V, 1.0)


def _mutant_swap_kv(q, K, V, scale):
    return decode_attention(q, V, K, scale)


def _mutant_last_token_dropped(q, K, V, scale):
    return decode_attention(q, K[:-1], V[:-1], scale)


def test_attention_pins_reject_mutants():
    rng = gen.stream(77, 1)
    q = rng.standard_normal((8, 64))
    K = rng.standard_normal((23, 2, 64))
    V = rng.standard_normal((23, 2, 64))
    scale = 1 / math.sqrt(64)
    ref = _sdpa(q, K, V, scale)
    np.testing.assert_allclose(decode_attention(q, K, V, scale), ref, rtol=1e-12, atol=1e-12)
    for mutant in (_mutant_head_mod, _mutant_no_scale, _mutant_swap_kv, _mutant_last_token_dropped):
        assert not np.allclose(mutant(q, K, V, scale), ref, rtol=1e-6, atol=1e-6), mutant.__name__


def test_layout_pin_rejects_a_transposed_read(golden_dir):
    """Reading K tiles as token-major [16][D] instead of [D/X][16][X] misses the
    hand-derived offsets."""
    import os
    rows = [l for l in open(os.path.join(golden_dir, "layout_offsets.txt"))
            if l.strip() and not l.startswith("#")]
    misses = 0
    for line in rows:
        shape, coord, offs = (p.split() for p in line.split("|"))
        dtype, N, H, B, D = shape[0], *map(int, shape[1:])
        b, h, o, d = map(int, coord)
        k_off = int(offs[0])
        wrong = ((b * H + h) * B + o) * D + d     # token-major reading
        misses += wrong != k_off
    assert misses >= 3


def test_allocator_pins_reject_lifo():
    class Lifo(am.AllocatorModel):
        def add(self, seq, num_tokens):
            need = -(-num_tokens // self.block_size)
            if seq in self.tables or need > len(self.free):
                raise am.AllocError()
            blocks = [self.free.pop() for _ in range(need)]
            for b in blocks:
                self.ref[b] = 1
            self.tables[seq] = blocks
            self.lengths[seq] = num_tokens
            return blocks
    m = Lifo(1024, 16)
    assert m.add(0, 40) != [0, 1, 2]          # the FIFO sample's first allocation
